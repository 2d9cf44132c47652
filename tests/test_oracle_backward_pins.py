"""Pins for the oracle's training-direction and rank-partial functions (CPU)."""

import numpy as np
import pytest

import oracle
import pins
import synth


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _int_bf16(rng, shape, lo=-8, hi=8):
    return synth.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


CASES = [(40, 8, 3, 4), (33, 16, 5, 2), (25, 12, 4, 12), (17, 8, 8, 2), (0, 8, 2, 4), (50, 6, 2, 1)]


@pytest.mark.parametrize("T,E,k,R", CASES)
def test_dispatch_backward_integer_sums_are_plain_sums(orc, T, E, k, R):
    """Small integers add exactly: grad_xr[p] is the sum of the expert rows p
    fed, grad_x[t] the sum of all of t's expert rows (np.add.at)."""
    rng = np.random.default_rng(T + 7 * E + k + R)
    idx, _ = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, 16, E, R)
    g = _int_bf16(rng, (T * k, 16))
    gxr, gx = orc.dispatch_backward(p, g, T, E, k, R)
    gf = synth.bf16_bits_to_f32(g).astype(np.float64)
    exr = np.zeros((p["N"], 16))
    np.add.at(exr, p["fan_src"], gf)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(gxr), exr)
    ex = np.zeros((T, 16))
    perm = np.argsort(idx.ravel(), kind="stable")
    np.add.at(ex, perm // k, gf)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(gx), ex)


@pytest.mark.parametrize("T,E,k,R", CASES[:4])
def test_dispatch_backward_is_the_adjoint_of_dispatch(orc, T, E, k, R):
    """<dispatch(x), g> == <x, dispatch^T(g)> (integers: exact)."""
    rng = np.random.default_rng(3 * T + E)
    idx, _ = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, 16, E, R)
    x = _int_bf16(rng, (T, 16), -3, 3)
    g = _int_bf16(rng, (T * k, 16), -3, 3)
    _, xe = orc.dispatch(p, x, E, k, R)
    _, gx = orc.dispatch_backward(p, g, T, E, k, R)
    lhs = (synth.bf16_bits_to_f32(xe).astype(np.float64) * synth.bf16_bits_to_f32(g)).sum()
    rhs = (synth.bf16_bits_to_f32(x).astype(np.float64) * synth.bf16_bits_to_f32(gx)).sum()
    assert lhs == rhs


@pytest.mark.parametrize("seed", range(3))
def test_backward_and_rank_partial_exact_replay(orc, seed):
    rng = np.random.default_rng(50 + seed)
    T, E, k, R = 6, 16, 5, 4
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    rc, p = orc.plan(idx, 8, E, R)
    ye = synth.wide_bf16(rng, (T * k, 8), -10, 10)
    gxr, gx = orc.dispatch_backward(p, ye, T, E, k, R)
    pins.check_dispatch_backward_exact(p, ye, gxr, gx)
    part, out = orc.combine_rank_partial(p, ye, w, E, R)
    pins.check_rank_partial_exact(p, ye, w, part, out)


def test_order_sensitive_cases(orc):
    for case in pins.order_sensitive_backward_case():
        rc, p = orc.plan(case["idx"], 8, case["E"], case["R"])
        _, gx = orc.dispatch_backward(p, case["g"], 1, case["E"], 3, case["R"])
        assert synth.bf16_bits_to_f32(gx)[0, 0] == np.float32(2.0 ** -30)


def test_rank_partial_equals_direct_combine_when_exact(orc):
    """Power-of-two gates and small integers: no rounding anywhere, so the
    two-stage sum equals the direct combine bit for bit."""
    rng = np.random.default_rng(9)
    T, E, k, R = 64, 32, 6, 8
    idx, _ = synth.random_routing(rng, T, E, k)
    w = (2.0 ** -rng.integers(0, 4, size=(T, k))).astype(np.float32)
    rc, p = orc.plan(idx, 32, E, R)
    ye = _int_bf16(rng, (T * k, 32), -4, 4)
    _, out = orc.combine_rank_partial(p, ye, w, E, R)
    np.testing.assert_array_equal(out, orc.combine(p["comb_row"], ye, w, E, R))


def test_rank_partial_error_bound(orc):
    """Random values: within two bf16 roundings plus the fp32 chain bound of
    the exact weighted sum."""
    rng = np.random.default_rng(10)
    T, E, k, R = 128, 64, 8, 8
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    rc, p = orc.plan(idx, 64, E, R)
    ye = synth.random_bf16(rng, (T * k, 64))
    part, out = orc.combine_rank_partial(p, ye, w, E, R)
    yf = synth.bf16_bits_to_f32(ye).astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * yf[p["comb_row"]]
    exact = terms.sum(axis=1)
    pf = synth.bf16_bits_to_f32(part).astype(np.float64)
    part_abs = np.zeros((T, 64))
    for t in range(T):
        for pp in p["tok_rank_row"][t]:
            if pp >= 0:
                part_abs[t] += np.abs(pf[pp])
    got = synth.bf16_bits_to_f32(out).astype(np.float64)
    bound = 2.0 ** -8 * (part_abs + np.abs(exact)) + 2 * k * 2.0 ** -24 * np.abs(terms).sum(axis=1) + 2.0 ** -132
    assert np.all(np.abs(got - exact) <= bound)


def test_combine_backward_against_products_and_dot(orc):
    rng = np.random.default_rng(11)
    T, E, k, R = 12, 16, 4, 4
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    rc, p = orc.plan(idx, 24, E, R)
    ye = synth.random_bf16(rng, (T * k, 24))
    g = synth.random_bf16(rng, (T, 24))
    gye, gw = orc.combine_backward(p["comb_row"], g, ye, w, E, R)
    pins.check_combine_backward(p["comb_row"], g, ye, w, gye, gw)


def test_combine_backward_adjoint_identity(orc):
    """d/dw of <combine(ye, w), g> is grad_w, and <combine(ye, w), g> =
    sum_tj w_tj grad_w_tj (exact in fp64 for bf16 inputs of this size)."""
    rng = np.random.default_rng(12)
    T, E, k, R = 30, 16, 4, 8
    idx, w = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, 16, E, R)
    ye = _int_bf16(rng, (T * k, 16), -5, 5)
    g = _int_bf16(rng, (T, 16), -5, 5)
    _, gw = orc.combine_backward(p["comb_row"], g, ye, w, E, R)
    yf = synth.bf16_bits_to_f32(ye).astype(np.float64)
    exact_out = (w.astype(np.float64)[:, :, None] * yf[p["comb_row"]]).sum(axis=1)
    lhs = (exact_out * synth.bf16_bits_to_f32(g)).sum()
    rhs = (w.astype(np.float64) * gw).sum()
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


@pytest.mark.parametrize("seed", range(3))
def test_rank_partial_f32_exact_replay(orc, seed):
    rng = np.random.default_rng(60 + seed)
    T, E, k, R = 6, 16, 5, 4
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    rc, p = orc.plan(idx, 8, E, R)
    ye = synth.wide_bf16(rng, (T * k, 8), -10, 10)
    part, out = orc.combine_rank_partial_f32(p, ye, w, E, R)
    pins.check_rank_partial_f32_exact(p, ye, w, part, out)


def test_rank_partial_f32_equals_direct_combine_when_exact(orc):
    """Power-of-two gates and small integers: nothing rounds, so the fp32
    partials sum to the direct combine bit for bit."""
    rng = np.random.default_rng(11)
    T, E, k, R = 64, 32, 6, 8
    idx, _ = synth.random_routing(rng, T, E, k)
    w = (2.0 ** -rng.integers(0, 4, size=(T, k))).astype(np.float32)
    rc, p = orc.plan(idx, 32, E, R)
    ye = _int_bf16(rng, (T * k, 32), -4, 4)
    _, out = orc.combine_rank_partial_f32(p, ye, w, E, R)
    np.testing.assert_array_equal(out, orc.combine(p["comb_row"], ye, w, E, R))


def test_rank_partial_f32_error_bound(orc):
    """Random values: within one bf16 rounding plus the fp32 chain bound of
    the exact weighted sum (the partials are not rounded to bf16), and on
    average no farther from it than the bf16-partial path."""
    rng = np.random.default_rng(12)
    T, E, k, R = 128, 64, 8, 8
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    rc, p = orc.plan(idx, 64, E, R)
    ye = synth.random_bf16(rng, (T * k, 64))
    part, out = orc.combine_rank_partial_f32(p, ye, w, E, R)
    yf = synth.bf16_bits_to_f32(ye).astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * yf[p["comb_row"]]
    exact = terms.sum(axis=1)
    got = synth.bf16_bits_to_f32(out).astype(np.float64)
    chain = 2 * k * 2.0 ** -24 * np.abs(terms).sum(axis=1)   # fp32 fma chains and the fp32 sum of partials
    bound = 2.0 ** -8 * (np.abs(exact) + chain) + chain + 2.0 ** -133   # plus one bf16 rounding (half ulp <= 2^-8 rel.)
    assert np.all(np.abs(got - exact) <= bound)
    # the fp32 path is at least as close to the exact sum as the bf16-partial path, on average
    _, out16 = orc.combine_rank_partial(p, ye, w, E, R)
    e16 = np.abs(synth.bf16_bits_to_f32(out16).astype(np.float64) - exact).mean()
    e32 = np.abs(got - exact).mean()
    assert e32 <= e16
