"""The oracle against what the pages and the mathematics fix (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
import pins
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


# ---------------------------------------------------------------- worked example

def test_fig3_worked_example(orc):
    """Hand-derived fixture from the DySHARP write-up's Fig. 3 (tokens A, B)."""
    g = json.load(open(os.path.join(GOLDEN, "fig3_two_tokens.json")))
    d, ex = g["dims"], g["expected"]
    idx = np.array(g["topk_idx"], np.int32)
    rc, p = orc.plan(idx, d["H"], d["E"], d["R"])
    assert rc == 0
    for key in ("expert_count", "expert_offset", "rank_count", "rank_offset", "send_token",
                "tok_rank_row", "fan_src", "fan_dst", "comb_row", "rank_segs", "expert_segs"):
        np.testing.assert_array_equal(p[key], np.array(ex[key]), err_msg=key)
    assert p["N"] == ex["N"]

    c = g["combine"]
    x = synth.f32_to_bf16_bits(np.array(c["x"], np.float32))
    xr, xe = orc.dispatch(p, x, d["E"], d["k"], d["R"])
    np.testing.assert_array_equal(xr, x[ex["xr_token_of_row"]])
    np.testing.assert_array_equal(xe, x[ex["xe_token_of_row"]])
    w = np.array(c["topk_w"], np.float32)
    # identity expert: out == x
    np.testing.assert_array_equal(orc.combine(p["comb_row"], xe, w, d["E"], d["R"]), x)
    # ye[q] = (q+1) * c
    cc = np.array(c["c"], np.float32)
    ye = synth.f32_to_bf16_bits((np.arange(1, 7, dtype=np.float32)[:, None] * cc[None, :]))
    out = orc.combine(p["comb_row"], ye, w, d["E"], d["R"])
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(out), np.array(c["out_with_ye_scaled_c"], np.float32))


# ---------------------------------------------------------------- plan pins

TINY = [(T, E, k, R) for T in (0, 1, 2, 5, 17, 40) for (E, k, R) in
        ((8, 2, 4), (8, 3, 4), (8, 8, 2), (6, 2, 3), (16, 4, 16), (16, 5, 1), (12, 3, 2))]


@pytest.mark.parametrize("T,E,k,R", TINY)
def test_plan_tiny_brute_force(orc, T, E, k, R):
    rng = np.random.default_rng(1000 * T + 10 * E + k + R)
    idx, _ = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, 8, E, R)
    assert rc == 0
    pins.check_plan_all(p, idx, E, R, brute=True)


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_plan_configs_library_pins(orc, cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    idx, _ = synth.make_routing(cfg, 0)
    rc, p = orc.plan(idx, cfg.H, cfg.E, cfg.R)
    assert rc == 0
    pins.check_plan_all(p, idx, cfg.E, cfg.R)


def test_allgather_special_case(orc):
    """k = E: every token goes to every rank, so every rank segment is
    arange(T) and xr is R stacked copies of x (the static all-gather pattern
    of the DySHARP write-up, section 3)."""
    T, H, E, R = 37, 16, 8, 4
    rng = np.random.default_rng(7)
    idx, _ = synth.random_routing(rng, T, E, E)
    rc, p = orc.plan(idx, H, E, R)
    assert rc == 0
    np.testing.assert_array_equal(p["send_token"], np.tile(np.arange(T), R))
    x = synth.random_bf16(rng, (T, H))
    xr, xe = orc.dispatch(p, x, E, E, R)
    np.testing.assert_array_equal(xr, np.tile(x, (R, 1)))


def test_single_rank_special_case(orc):
    """R = 1: one rank holds every expert; xr == x, send_token == arange(T)."""
    T, H, E, k = 29, 24, 8, 3
    rng = np.random.default_rng(8)
    idx, _ = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, H, E, 1)
    assert rc == 0
    np.testing.assert_array_equal(p["send_token"], np.arange(T))
    x = synth.random_bf16(rng, (T, H))
    xr, _ = orc.dispatch(p, x, E, k, 1)
    np.testing.assert_array_equal(xr, x)


def test_one_expert_per_rank(orc):
    """E = R: no two experts share a rank, nothing to deduplicate: N = T*k and
    every rank row feeds exactly one expert row."""
    T, E, k = 50, 8, 3
    rng = np.random.default_rng(9)
    idx, _ = synth.random_routing(rng, T, E, k)
    rc, p = orc.plan(idx, 8, E, E)
    assert rc == 0 and p["N"] == T * k
    assert np.all(p["fan_dst"][:, 0] >= 0)


def test_all_tokens_one_expert(orc):
    """Every token's first slot is expert 0: segment 0 holds all tokens in order."""
    T, E, k, R = 33, 8, 2, 4
    idx = np.stack([np.zeros(T, np.int32), 1 + (np.arange(T) % 7)], axis=1).astype(np.int32)
    rc, p = orc.plan(idx, 8, E, R)
    assert rc == 0
    assert p["expert_count"][0] == T
    np.testing.assert_array_equal(p["comb_row"][:, 0], np.arange(T))
    pins.check_plan_all(p, idx, E, R, brute=True)


# ---------------------------------------------------------------- dispatch pins

@pytest.mark.parametrize("T,E,k,R,H", [(0, 8, 2, 4, 8), (19, 8, 3, 4, 16), (64, 16, 4, 8, 8), (7, 6, 6, 3, 32)])
def test_dispatch_library_pins(orc, T, E, k, R, H):
    rng = np.random.default_rng(T + E + k + R + H)
    idx, _ = synth.random_routing(rng, T, E, k)
    x = synth.random_bf16(rng, (T, H))
    rc, p = orc.plan(idx, H, E, R)
    assert rc == 0
    xr, xe = orc.dispatch(p, x, E, k, R)
    pins.check_dispatch(p, idx, x, xr, xe)


def test_dispatch_config0_full(orc):
    cfg = synth.CONFIGS[0]
    inp = synth.make_inputs(cfg, 0)
    rc, p = orc.plan(inp["topk_idx"], cfg.H, cfg.E, cfg.R)
    xr, xe = orc.dispatch(p, inp["x"], cfg.E, cfg.k, cfg.R)
    pins.check_dispatch(p, inp["topk_idx"], inp["x"], xr, xe)


# ---------------------------------------------------------------- combine pins

def _hard_case(rng, T, H, k, Q):
    """Values spread over many binades with mixed signs so that term order,
    fusing and the final rounding all change the result somewhere."""
    mant = rng.standard_normal((Q, H))
    expo = rng.integers(-12, 13, size=(Q, H))
    ye = synth.f32_to_bf16_bits((mant * 2.0 ** expo).astype(np.float32))
    w = (rng.standard_normal((T, k)) * 2.0 ** rng.integers(-6, 7, size=(T, k))).astype(np.float32)
    return ye, w


@pytest.mark.parametrize("seed", range(4))
def test_combine_exact_rational_replay(orc, seed):
    rng = np.random.default_rng(100 + seed)
    T, H, k, Q = 6, 16, 5, 40
    ye, w = _hard_case(rng, T, H, k, Q)
    comb_row = np.stack([rng.choice(Q, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    got = orc.combine(comb_row, ye, w, 8, 1)
    np.testing.assert_array_equal(got, pins.combine_exact(comb_row, ye, w))


def test_combine_order_and_fusing_visible(orc):
    comb_row, ye, w = pins.edge_combine_case()
    got = orc.combine(comb_row, ye, w, 4, 1)
    np.testing.assert_array_equal(got, pins.combine_exact(comb_row, ye, w))
    f = synth.bf16_bits_to_f32(got)
    assert f[0, 0] == np.float32(2.0 ** -30)
    assert f[1, 0] == np.float32(2.0 ** -23 + 2.0 ** -30)


def test_combine_ties_to_even(orc):
    r0, r1 = pins.tie_rows()
    ye = synth.f32_to_bf16_bits(np.stack([r0, r1]))
    got = synth.bf16_bits_to_f32(orc.combine(np.array([[0, 1]], np.int32), ye, np.ones((1, 2), np.float32), 4, 1))
    expect = np.array([1.0, 1.0 + 2.0 ** -6, 2.0, -1.0, -(1.0 + 2.0 ** -6), 0.5, 3.0, 1.0], np.float32)
    np.testing.assert_array_equal(got[0], expect)


def test_combine_subnormal_and_ties(orc):
    """Gradual underflow kept (no flush to zero) and ties rounded to even."""
    # ye values: tiny bf16 subnormal-range numbers and values whose weighted sum
    # lands exactly half-way between two bf16 values.
    tiny = np.array([2.0 ** -130, -2.0 ** -131, 2.0 ** -133, 3 * 2.0 ** -128], np.float32)
    tie = np.array([1.0, 2.0 ** -8, 1.0 + 2.0 ** -7, 3 * 2.0 ** -9], np.float32)
    ye = synth.f32_to_bf16_bits(np.tile(np.stack([tiny, tie, tie * 3, tiny * 5]), (1, 2)))
    comb_row = np.array([[0, 3], [1, 2], [2, 1]], np.int32)
    w = np.array([[0.5, 0.25], [1.0, 1.0], [0.5, 1.0]], np.float32)
    got = orc.combine(comb_row, ye, w, 4, 1)
    np.testing.assert_array_equal(got, pins.combine_exact(comb_row, ye, w))
    assert np.any(got[0] != 0)          # a flush-to-zero mistake would zero row 0


def test_combine_k1_unit_gate_is_a_permutation(orc):
    rng = np.random.default_rng(11)
    T, H = 31, 24
    perm = rng.permutation(T).astype(np.int32)[:, None]
    ye = synth.random_bf16(rng, (T, H))
    got = orc.combine(perm, ye, np.ones((T, 1), np.float32), 4, 1)
    np.testing.assert_array_equal(got, ye[perm[:, 0]])


def test_combine_error_bound_vs_fp64(orc):
    """Larger case: within the fp32 chain's error bound of the fp64 sum plus
    half a bf16 ulp of the result."""
    rng = np.random.default_rng(12)
    T, H, k, Q = 64, 256, 8, 512
    ye = synth.random_bf16(rng, (Q, H))
    w = rng.standard_normal((T, k)).astype(np.float32)
    comb_row = np.stack([rng.choice(Q, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    got = synth.bf16_bits_to_f32(orc.combine(comb_row, ye, w, 8, 1)).astype(np.float64)
    yf = synth.bf16_bits_to_f32(ye).astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * yf[comb_row]
    exact = terms.sum(axis=1)
    bound = k * 2.0 ** -24 * np.abs(terms).sum(axis=1) + np.abs(exact) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(got - exact) <= bound)


def plus_zero(x):
    """The fp32 sum starts at +0 and can never end at -0 (an exact zero sum
    rounds to +0), so a -0 input comes back as +0; every other value comes
    back unchanged."""
    return np.where(x == 0x8000, np.uint16(0), x).astype(np.uint16)


@pytest.mark.parametrize("cfg_id", [0, 1])
def test_round_trip_identity_expert(orc, cfg_id):
    """dispatch -> identity expert -> combine with gates summing to 1 returns x
    bit for bit (fp32 error ~k*2^-24 is far below half a bf16 ulp)."""
    cfg = synth.CONFIGS[cfg_id]
    inp = synth.make_inputs(cfg, 0)
    rc, p = orc.plan(inp["topk_idx"], cfg.H, cfg.E, cfg.R)
    xr, xe = orc.dispatch(p, inp["x"], cfg.E, cfg.k, cfg.R)
    out = orc.combine(p["comb_row"], xe, inp["topk_w"], cfg.E, cfg.R)
    np.testing.assert_array_equal(out, plus_zero(inp["x"]))


def test_round_trip_deepseek_slice(orc):
    cfg = synth.CONFIGS[2]
    idx, w = synth.make_routing(cfg, 0)
    T = 256
    x = synth.make_x(cfg, 0)[:T]
    idx, w = idx[:T], w[:T]
    rc, p = orc.plan(idx, cfg.H, cfg.E, cfg.R)
    xr, xe = orc.dispatch(p, x, cfg.E, cfg.k, cfg.R)
    np.testing.assert_array_equal(orc.combine(p["comb_row"], xe, w, cfg.E, cfg.R), plus_zero(x))


# ---------------------------------------------------------------- errors

def test_error_codes(orc):
    assert orc.check_dims(4, 8, 8, 2, 4) == oracle.OK
    assert orc.check_dims(0, 8, 8, 2, 4) == oracle.OK
    assert orc.check_dims(-1, 8, 8, 2, 4) == oracle.E_INVALID_ARG
    assert orc.check_dims(4, 0, 8, 2, 4) == oracle.E_INVALID_ARG
    assert orc.check_dims(4, 8, 8, 9, 4) == oracle.E_INVALID_ARG      # k > E
    assert orc.check_dims(4, 8, 8, 2, 3) == oracle.E_INVALID_ARG      # E % R
    assert orc.check_dims(4, 12, 8, 2, 4) == oracle.E_ALIGN           # H % 8
    assert orc.check_dims(1 << 28, 8, 16, 8, 4) == oracle.E_OVERFLOW  # T*k >= 2^31
    bad = np.array([[0, 8]], np.int32)
    assert orc.plan(bad, 8, 8, 4)[0] == oracle.E_BAD_INDEX
    assert orc.plan(np.array([[3, 3]], np.int32), 8, 8, 4)[0] == oracle.E_BAD_INDEX
    assert orc.plan(np.array([[-1, 2]], np.int32), 8, 8, 4)[0] == oracle.E_BAD_INDEX


# ---------------------------------------------------------------- the rounding step

def test_round_bf16_ieee_table_and_definition(orc):
    """fp32 -> bf16 on its own: an IEEE table (ties to even, overflow to
    infinity with the sign, a NaN whose payload sits only in the low half
    stays a NaN, NaNs keep their sign and come out quiet) and the
    nearest-even rule decided by float64 distances on 2^18 random patterns."""
    pins.check_round_bf16(orc)


def test_round_bf16_low_payload_nan_is_not_infinity(orc):
    """The classic slip of adding the rounding bias to a NaN: 0x7f800001 has
    its payload in the dropped half and would carry into infinity."""
    got = orc.round_bf16(np.array([0x7F800001, 0xFF800001, 0x7F80FFFF], np.uint32))
    assert np.all(pins.bf16_is_nan(got)) and list(got >> 15) == [0, 1, 0]
