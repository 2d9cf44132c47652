"""The comparison rule of the device numerics tests, on the CPU: the oracle's
own results pass it, and planted differences (a flipped bit, a NaN turned
into a number, a NaN sign flipped where it is determined, a NaN that is not
quiet) are rejected.  Also checks that the special cases really hold what
they are meant to hold (every scenario present, NaNs with a determined sign
and NaNs from invalid operations both occur)."""

import copy

import numpy as np
import pytest

import numerics_cases as nc
import oracle
import pins


@pytest.fixture(scope="module")
def case():
    idx, w, Y, n_sp = nc.build_case(40, 136, 16, 4, 4, seed=5, shifted=False)
    ref = nc.oracle_results(oracle.get(), idx, w, Y, 136, 16, 4)
    dev = {key: ref[key] for key in ("out", "partial", "out_partial", "partial32", "out_partial32", "grad_xr",
                                      "grad_x", "grad_ye")}
    dev["out_range"] = ref["out"]
    # grad_w on the device is fp32; the oracle's fp64 value rounded to fp32 is within the bound
    dev["grad_w"] = ref["grad_w"].astype(np.float32).ravel()
    return idx, w, Y, n_sp, ref, dev


def _run(case, dev):
    idx, w, Y, n_sp, ref, _ = case
    nc.compare_all(dev, ref, idx, w, Y, 16, 4, n_sp, "cpu", log=lambda *a: None)


def test_oracle_results_pass_the_rule(case):
    _run(case, case[5])


def test_cases_hold_every_scenario_and_both_kinds_of_nan(case):
    idx, w, Y, n_sp, ref, dev = case
    spc = np.nonzero(np.arange(136) % 3 != 2)[0]
    seen = set()
    for t in range(n_sp):
        for h in spc:
            seen.add(tuple(int(v) for v in Y[t, :4, h]))
    assert set(nc.SCENARIOS) <= seen
    out_nan = pins.bf16_is_nan(ref["out"])
    assert out_nan.sum() > 50
    T, H = ref["out"].shape
    wv = np.broadcast_to(w[:n_sp, :, None], (n_sp, 4, H)).astype(np.float32)
    yv = nc.f32_of(Y[:n_sp])
    m = nc.nan_sign_mask([yv[:, j] for j in range(4)] + [wv[:, j] for j in range(4)])
    determined = out_nan[:n_sp] & m
    assert determined.sum() > 20 and (out_nan[:n_sp] & ~m).sum() > 20
    # both signs among the determined NaNs
    signs = ref["out"][:n_sp][determined] >> 15
    assert set(signs.tolist()) == {0, 1}
    # subnormal results and infinities occur too
    o = ref["out"]
    assert np.any(((o & 0x7F80) == 0) & ((o & 0x7F) != 0))
    assert np.any(o == 0x7F80) and np.any(o == 0xFF80)


def _planted(case, key, fn):
    dev = copy.deepcopy(case[5])
    dev[key] = fn(np.array(dev[key]))
    with pytest.raises(AssertionError):
        _run(case, dev)


def test_flipped_low_bit_is_caught(case):
    def f(a):
        i = np.argwhere(~pins.bf16_is_nan(a))[7]
        a[tuple(i)] ^= 1
        return a
    for key in ("out", "out_range", "partial", "grad_xr", "grad_x", "grad_ye", "out_partial32"):
        _planted(case, key, f)


def test_subnormal_flushed_is_caught(case):
    def f(a):
        sub = ((a & 0x7F80) == 0) & ((a & 0x7F) != 0)
        a[sub] &= 0x8000
        return a
    _planted(case, "out", f)


def test_nan_made_a_number_is_caught(case):
    def f(a):
        a[pins.bf16_is_nan(a)] = 0x7F80
        return a
    _planted(case, "out", f)


def test_determined_nan_sign_flip_is_caught(case):
    idx, w, Y, n_sp, ref, _ = case
    H = ref["out"].shape[1]
    wv = np.broadcast_to(w[:n_sp, :, None], (n_sp, 4, H)).astype(np.float32)
    yv = nc.f32_of(Y[:n_sp])
    m = np.zeros(ref["out"].shape, bool)
    m[:n_sp] = nc.nan_sign_mask([yv[:, j] for j in range(4)] + [wv[:, j] for j in range(4)])

    def f(a):
        a[m & pins.bf16_is_nan(a)] ^= 0x8000
        return a
    _planted(case, "out", f)


def test_undetermined_nan_sign_flip_is_accepted(case):
    idx, w, Y, n_sp, ref, dev0 = case
    H = ref["out"].shape[1]
    wv = np.broadcast_to(w[:n_sp, :, None], (n_sp, 4, H)).astype(np.float32)
    yv = nc.f32_of(Y[:n_sp])
    m = np.zeros(ref["out"].shape, bool)
    m[:n_sp] = nc.nan_sign_mask([yv[:, j] for j in range(4)] + [wv[:, j] for j in range(4)])
    dev = copy.deepcopy(dev0)
    flip = ~m & pins.bf16_is_nan(dev["out"])
    assert flip.sum() > 0
    dev["out"] = np.where(flip, dev["out"] ^ 0x8000, dev["out"]).astype(np.uint16)
    _run(case, dev)


def test_signalling_nan_is_caught(case):
    def f(a):
        n = pins.bf16_is_nan(a)
        a[n] = (a[n] & 0xFF80) | 0x0001
        return a
    _planted(case, "out", f)


def test_fp32_partial_bit_is_caught(case):
    def f(a):
        u = a.view(np.uint32)
        i = np.argwhere(np.isfinite(a) & (a != 0))[3]
        u[tuple(i)] ^= 1
        return a
    _planted(case, "partial32", f)


def test_grad_w_error_is_caught(case):
    def f(a):
        i = np.argwhere(np.isfinite(a) & (np.abs(a) > 1e-3))[0]
        a[tuple(i)] *= 1.01
        return a
    _planted(case, "grad_w", f)
