"""Independent checks that pin the oracle to something other than itself.

Each check derives the expected result a different way from the oracle:
closed forms (bincount, prefix sums), library routines (a stable argsort,
nonzero of the token x rank hit matrix), O(T^2) brute force, and an exact
rational replay of the fp32 fused-multiply-add chain.  Every function raises
AssertionError on a mismatch; test_oracle_mutants.py plants mistakes in a
copy of the oracle and requires that some check here fails.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


# --------------------------------------------------------------------------
# plan
# --------------------------------------------------------------------------

def hit_matrix(idx: np.ndarray, E: int, R: int) -> np.ndarray:
    T = idx.shape[0]
    hit = np.zeros((T, R), dtype=bool)
    if T:
        hit[np.repeat(np.arange(T), idx.shape[1]), (idx // (E // R)).ravel()] = True
    return hit


def check_counts(p: dict, idx: np.ndarray, E: int, R: int):
    """Closed forms: histogram, distinct ranks per token, prefix sums."""
    T, k = idx.shape
    np.testing.assert_array_equal(p["expert_count"], np.bincount(idx.ravel(), minlength=E))
    hit = hit_matrix(idx, E, R)
    np.testing.assert_array_equal(p["rank_count"], hit.sum(axis=0))
    np.testing.assert_array_equal(p["expert_offset"], np.concatenate([[0], np.cumsum(p["expert_count"])]))
    np.testing.assert_array_equal(p["rank_offset"], np.concatenate([[0], np.cumsum(p["rank_count"])]))
    N = int(hit.sum())
    assert p["N"] == N
    assert int(p["expert_count"].sum()) == T * k
    assert N <= T * min(k, R)
    Epr = E // R
    for r in range(R):
        assert p["rank_count"][r] <= min(T, int(p["expert_count"][r * Epr:(r + 1) * Epr].sum()))


def check_expert_side_argsort(p: dict, idx: np.ndarray, E: int, R: int):
    """Expert-major placement == a stable sort of the flattened top-k ids."""
    T, k = idx.shape
    perm = np.argsort(idx.ravel(), kind="stable")          # expert row q holds pair perm[q]
    cr = p["comb_row"].ravel()
    np.testing.assert_array_equal(cr[perm], np.arange(T * k))
    if T * k:
        tok_of_q = perm // k
        np.testing.assert_array_equal(p["send_token"][p["fan_src"]], tok_of_q)
        rank_of_q = idx.ravel()[perm] // (E // R)
        ro = p["rank_offset"]
        p_of_q = p["fan_src"]
        assert np.all((p_of_q >= ro[rank_of_q]) & (p_of_q < ro[rank_of_q + 1]))


def check_rank_side_nonzero(p: dict, idx: np.ndarray, E: int, R: int):
    """Rank-major placement == nonzero() of the hit matrix read rank-major."""
    T, k = idx.shape
    hit = hit_matrix(idx, E, R)
    r_list, t_list = np.nonzero(hit.T)
    np.testing.assert_array_equal(p["send_token"], t_list)
    KR = min(k, R)
    expect = np.full((T, KR), -1, np.int32)
    order = np.argsort(t_list, kind="stable")              # rows grouped by token, rank ascending
    ts = t_list[order]
    slot = np.arange(len(ts)) - np.searchsorted(ts, ts, side="left")
    expect[ts, slot] = order
    np.testing.assert_array_equal(p["tok_rank_row"], expect)


def check_fan_dst(p: dict, idx: np.ndarray, E: int, R: int):
    """The receiver map lists, per rank row, exactly the expert rows whose source it is."""
    T, k = idx.shape
    D = min(k, E // R)
    N = p["N"]
    expect = np.full((N, D), -1, np.int32)
    order = np.argsort(p["fan_src"], kind="stable")          # expert rows grouped by source, q ascending
    fs = p["fan_src"][order]
    j = np.arange(len(fs)) - np.searchsorted(fs, fs, side="left")
    assert np.all(j < D), "a rank row feeds more expert rows than experts per rank"
    expect[fs, j] = order
    np.testing.assert_array_equal(p["fan_dst"], expect)


def check_segments(p: dict, E: int, R: int):
    Epr = E // R
    rs = np.stack([np.arange(R), -np.ones(R, int), p["rank_offset"][:-1], p["rank_count"]], axis=1)
    es = np.stack([np.arange(E) // Epr, np.arange(E), p["expert_offset"][:-1], p["expert_count"]], axis=1)
    np.testing.assert_array_equal(p["rank_segs"], rs)
    np.testing.assert_array_equal(p["expert_segs"], es)


def check_brute_force(p: dict, idx: np.ndarray, E: int, R: int):
    """O(T^2) definition of every row position, for tiny T."""
    T, k = idx.shape
    Epr = E // R
    ranks = [sorted({int(e) // Epr for e in idx[t]}) for t in range(T)]
    for t in range(T):
        for i, r in enumerate(ranks[t]):
            before = sum(1 for u in range(t) if r in ranks[u])
            assert p["tok_rank_row"][t, i] == p["rank_offset"][r] + before
        for j in range(k):
            e = int(idx[t, j])
            before = sum(1 for u in range(t) if e in set(idx[u].tolist()))
            q = p["expert_offset"][e] + before
            assert p["comb_row"][t, j] == q
            assert p["fan_src"][q] == p["tok_rank_row"][t, ranks[t].index(e // Epr)]


def check_plan_all(p: dict, idx: np.ndarray, E: int, R: int, brute: bool = False):
    check_counts(p, idx, E, R)
    check_expert_side_argsort(p, idx, E, R)
    check_rank_side_nonzero(p, idx, E, R)
    check_fan_dst(p, idx, E, R)
    check_segments(p, E, R)
    if brute:
        check_brute_force(p, idx, E, R)


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

def check_dispatch(p: dict, idx: np.ndarray, x: np.ndarray, xr: np.ndarray, xe: np.ndarray):
    """Every rank row is its token's x row; every expert row is its token's x
    row (the token of expert row q is perm[q] // k for the stable sort perm)."""
    T, k = idx.shape
    np.testing.assert_array_equal(xr, x[p["send_token"]])
    perm = np.argsort(idx.ravel(), kind="stable")
    np.testing.assert_array_equal(xe, x[perm // k] if T * k else xe)


# --------------------------------------------------------------------------
# combine: exact replay of the fp32 chain with rationals
# --------------------------------------------------------------------------

def _round_fraction(x: Fraction, prec: int, emin: int, emax: int) -> float:
    """Round a rational to the nearest value of a binary format with `prec`
    significand bits (ties to even), gradual underflow below 2**emin and
    overflow to infinity above the largest finite value."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = -x if x < 0 else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - prec + 1)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * float(val)


def f32_fma_exact(a: float, b: float, c: float) -> float:
    """fp32 fused multiply-add: the exact a*b+c rounded once to binary32."""
    return _round_fraction(Fraction(a) * Fraction(b) + Fraction(c), 24, -126, 127)


def bf16_bits_of_exact(v: float) -> int:
    """bf16 (round to nearest even) of an fp32 value, as bits."""
    if v != v:
        raise ValueError("nan")
    if v in (float("inf"), float("-inf")):
        r = v
    else:
        r = _round_fraction(Fraction(v), 8, -126, 127)
    bits = int(np.array([r], dtype=np.float32).view(np.uint32)[0]) >> 16
    return bits


def combine_exact(comb_row: np.ndarray, ye_bits: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t,h] for the chain acc=+0; acc=fma(w[t,j], ye[q,h], acc), j ascending."""
    T, k = comb_row.shape
    H = ye_bits.shape[1]
    yf = (ye_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    out = np.zeros((T, H), np.uint16)
    for t in range(T):
        for h in range(H):
            acc = 0.0
            for j in range(k):
                acc = f32_fma_exact(float(w[t, j]), float(yf[comb_row[t, j], h]), acc)
            out[t, h] = bf16_bits_of_exact(acc)
    return out


# --------------------------------------------------------------------------
# the fp32 -> bf16 rounding step on its own
# --------------------------------------------------------------------------

def bf16_is_nan(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def bf16_nearest_even(bits: np.ndarray) -> np.ndarray:
    """bf16 of finite or infinite fp32 values (uint32 bit patterns), decided
    by value: the two bf16 neighbours of |v| (the truncation, and the next
    value away from zero one bf16 ulp further, 2^128 past the largest finite
    one) are compared by their float64 distance to |v|; a tie goes to the
    neighbour with an even last significand bit; 2^128 is infinity.  Every
    quantity is exact in float64.  NaN inputs are not handled here."""
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    assert not np.any(((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x007FFFFF) != 0))
    sign = (bits >> 16) & 0x8000
    mag = bits & np.uint32(0x7FFFFFFF)
    v = mag.view(np.float32).astype(np.float64)
    lo_bits = mag & np.uint32(0xFFFF0000)
    lo = lo_bits.view(np.float32).astype(np.float64)
    expo = (lo_bits >> 23).astype(np.int64)
    ulp = np.ldexp(1.0, np.maximum(expo, 1) - 127 - 7)        # bf16 spacing at lo (subnormals: 2^-133)
    inf = np.isinf(v)
    v = np.where(inf, 0.0, v)                                  # decided below; keeps the distances finite
    lo = np.where(inf, 0.0, lo)
    d_lo, d_hi = v - lo, (lo + ulp) - v
    lo16 = (lo_bits >> 16).astype(np.uint32)
    up = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo16 & 1) == 1))
    res = np.where(inf, 0x7F80, np.where(up, lo16 + 1, lo16))   # lo16 + 1 past 0x7F7F is 0x7F80: infinity
    return (res | sign).astype(np.uint16)


# (fp32 bits, bf16 bits) fixed by the IEEE 754 rules for a narrowing
# conversion: nearest, ties to even, overflow to infinity with the sign,
# a NaN stays a NaN (made quiet) with its sign.
ROUND_TABLE = [
    (0x00000000, 0x0000), (0x80000000, 0x8000),          # zeros keep their sign
    (0x3F808000, 0x3F80), (0x3F818000, 0x3F82),          # ties: even stays, odd goes up
    (0x3F808001, 0x3F81), (0xBF808001, 0xBF81),          # just above a tie
    (0x00008000, 0x0000), (0x00018000, 0x0002),          # ties among fp32 subnormals
    (0x00017FFF, 0x0001), (0x80008001, 0x8001),
    (0x007FFFFF, 0x0080),                                 # largest fp32 subnormal rounds up to 2^-126
    (0x7F7F7FFF, 0x7F7F),                                 # below the half-way point: the largest bf16
    (0x7F7F8000, 0x7F80), (0xFF7F8000, 0xFF80),          # half-way, odd: to infinity
    (0x7F7FFFFF, 0x7F80), (0xFF7FFFFF, 0xFF80),          # the largest fp32 overflows bf16
    (0x7F800000, 0x7F80), (0xFF800000, 0xFF80),          # infinities
]
# fp32 NaN bits -> (sign of the bf16 NaN): every one must stay a quiet NaN
NAN_TABLE = [(0x7F800001, 0), (0xFF800001, 1), (0x7FC00000, 0), (0xFFC00000, 1), (0x7F80FFFF, 0),
             (0x7FBFFFFF, 0), (0xFFFFFFFF, 1), (0x7F810000, 0)]


def check_round_bf16(orc) -> None:
    """The oracle's rounding step against the IEEE table above and against
    bf16_nearest_even on 2^18 random finite fp32 patterns (every binade, both
    signs, subnormals, and patterns next to each tie)."""
    src = np.array([a for a, _ in ROUND_TABLE], np.uint32)
    np.testing.assert_array_equal(orc.round_bf16(src), np.array([b for _, b in ROUND_TABLE], np.uint16))
    np.testing.assert_array_equal(bf16_nearest_even(src), np.array([b for _, b in ROUND_TABLE], np.uint16))
    nan = np.array([a for a, _ in NAN_TABLE], np.uint32)
    got = orc.round_bf16(nan)
    assert np.all(bf16_is_nan(got)), [hex(v) for v in got]
    assert np.all((got & 0x0040) != 0), "NaN not made quiet"
    np.testing.assert_array_equal(got >> 15, np.array([s for _, s in NAN_TABLE], np.uint16))
    rng = np.random.default_rng(4242)
    r = rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    r = r[((r & 0x7F800000) != 0x7F800000)]                    # finite only
    near = (r & np.uint32(0xFFFF0000)) | np.uint32(0x8000)     # exact ties and their neighbours
    near = np.concatenate([near, near + 1, near - 1])
    near = near[((near & 0x7F800000) != 0x7F800000)]
    r = np.concatenate([r, near])
    np.testing.assert_array_equal(orc.round_bf16(r), bf16_nearest_even(r))


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ord(a) - ord(b)| on bf16 bit patterns; +0 and -0 are equal."""
    def ordkey(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(ordkey(a) - ordkey(b))


# --------------------------------------------------------------------------
# the whole battery, as one function (used on planted-mistake oracle copies)
# --------------------------------------------------------------------------

def tie_rows():
    """Two bf16 rows whose sum (gates 1, 1) lands exactly half-way between
    two bf16 values in every column: even and odd neighbours, both signs."""
    r0 = np.array([1.0, 1.0 + 2.0 ** -7, 2.0, -1.0, -(1.0 + 2.0 ** -7), 0.5, 3.0, 1.0], np.float32)
    r1 = np.array([2.0 ** -8, 2.0 ** -8, 2.0 ** -7, -(2.0 ** -8), -(2.0 ** -8), 2.0 ** -9, 2.0 ** -7, 0.0], np.float32)
    return r0, r1


def edge_combine_case():
    """Hand-built rows where the order, the fusing and the gate index of the
    fp32 chain each change the bf16 result (the rows hold bf16 values):
      token 0: y = [1, -1, 2^-30], w = [1, 1, 1]: ascending gives 2^-30, any
               other order loses the small term (cancellation);
      token 1: w = [-1, 1+2^-23], y = [1+2^-7, 1+2^-7]: the fused step keeps
               the product's low bits (2^-23 + 2^-30), an unfused one gives 2^-23.
    """
    import synth
    rows = np.array([[1.0] * 8, [-1.0] * 8, [2.0 ** -30] * 8, [1.0 + 2.0 ** -7] * 8], np.float32)
    ye = synth.f32_to_bf16_bits(rows)
    comb_row = np.array([[0, 1, 2], [3, 3, 3]], np.int32)
    w = np.array([[1.0, 1.0, 1.0], [-1.0, 1.0 + 2.0 ** -23, 0.0]], np.float32)
    return comb_row, ye, w


def run_battery(orc) -> None:
    import json
    import os
    import synth
    here = os.path.dirname(os.path.abspath(__file__))
    check_round_bf16(orc)
    g = json.load(open(os.path.join(here, "golden", "fig3_two_tokens.json")))
    d, ex = g["dims"], g["expected"]
    idx = np.array(g["topk_idx"], np.int32)
    rc, p = orc.plan(idx, d["H"], d["E"], d["R"])
    assert rc == 0
    for key in ("expert_count", "rank_count", "send_token", "tok_rank_row", "fan_src", "fan_dst", "comb_row"):
        np.testing.assert_array_equal(p[key], np.array(ex[key]))
    for (T, E, k, R) in ((17, 8, 3, 4), (40, 12, 3, 2), (23, 16, 4, 16), (9, 8, 8, 2)):
        rng = np.random.default_rng(T * 31 + E)
        idx, _ = synth.random_routing(rng, T, E, k)
        rc, p = orc.plan(idx, 16, E, R)
        assert rc == 0
        check_plan_all(p, idx, E, R, brute=True)
        x = synth.random_bf16(rng, (T, 16))
        xr, xe = orc.dispatch(p, x, E, k, R)
        check_dispatch(p, idx, x, xr, xe)
    for cfg_id in (0, 1):
        cfg = synth.CONFIGS[cfg_id]
        inp = synth.make_inputs(cfg, 0)
        rc, p = orc.plan(inp["topk_idx"], cfg.H, cfg.E, cfg.R)
        check_plan_all(p, inp["topk_idx"], cfg.E, cfg.R)
        xr, xe = orc.dispatch(p, inp["x"], cfg.E, cfg.k, cfg.R)
        out = orc.combine(p["comb_row"], xe, inp["topk_w"], cfg.E, cfg.R)
        np.testing.assert_array_equal(out, np.where(inp["x"] == 0x8000, 0, inp["x"]).astype(np.uint16))
    for seed in range(3):
        rng = np.random.default_rng(100 + seed)
        T, H, k, Q = 6, 16, 5, 40
        ye = synth.f32_to_bf16_bits((rng.standard_normal((Q, H)) * 2.0 ** rng.integers(-12, 13, size=(Q, H))).astype(np.float32))
        w = (rng.standard_normal((T, k)) * 2.0 ** rng.integers(-6, 7, size=(T, k))).astype(np.float32)
        comb_row = np.stack([rng.choice(Q, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        np.testing.assert_array_equal(orc.combine(comb_row, ye, w, 8, 1), combine_exact(comb_row, ye, w))
    comb_row, ye, w = edge_combine_case()
    np.testing.assert_array_equal(orc.combine(comb_row, ye, w, 4, 1), combine_exact(comb_row, ye, w))
    r0, r1 = tie_rows()
    tiny = np.array([2.0 ** -130, -2.0 ** -131, 2.0 ** -133, 3 * 2.0 ** -128] * 2, np.float32)
    ye = synth.f32_to_bf16_bits(np.stack([r0, r1, tiny, tiny * 5]))
    comb_row = np.array([[0, 1], [2, 3]], np.int32)
    w = np.array([[1.0, 1.0], [0.5, 0.25]], np.float32)
    np.testing.assert_array_equal(orc.combine(comb_row, ye, w, 4, 1), combine_exact(comb_row, ye, w))


# --------------------------------------------------------------------------
# backward and rank-partial combine
# --------------------------------------------------------------------------
    run_battery_backward(orc)


def f32_add_exact(a: float, b: float) -> float:
    return _round_fraction(Fraction(a) + Fraction(b), 24, -126, 127)


def bf16_of_f32_bits(v: float) -> int:
    return bf16_bits_of_exact(v)


def _f(bits):
    return float((np.uint32(bits) << np.uint32(16)).view(np.float32))


def staged_sum_exact(groups, rows_bits):
    """bf16( fp32 running sum from +0 over rows_bits[g] for g in groups ), per column, exactly."""
    H = rows_bits.shape[1]
    out = np.zeros(H, np.uint16)
    for h in range(H):
        acc = 0.0
        for g in groups:
            acc = f32_add_exact(acc, _f(rows_bits[g, h]))
        out[h] = bf16_bits_of_exact(acc)
    return out


def check_dispatch_backward_exact(plan, grad_xe, gxr, gx):
    """Exact replay of both stages with rationals (tiny inputs)."""
    N = plan["N"]
    for p in range(N):
        qs = [int(q) for q in plan["fan_dst"][p] if q >= 0]
        np.testing.assert_array_equal(gxr[p], staged_sum_exact(qs, grad_xe))
    for t in range(plan["tok_rank_row"].shape[0]):
        ps = [int(p) for p in plan["tok_rank_row"][t] if p >= 0]
        np.testing.assert_array_equal(gx[t], staged_sum_exact(ps, gxr))


def check_rank_partial_exact(plan, ye, w, part, out):
    T, k = plan["comb_row"].shape
    gate = np.zeros(T * k, np.float32)
    gate[plan["comb_row"].ravel()] = w.ravel()
    H = ye.shape[1]
    for p in range(plan["N"]):
        qs = [int(q) for q in plan["fan_dst"][p] if q >= 0]
        for h in range(H):
            acc = 0.0
            for q in qs:
                acc = f32_fma_exact(float(gate[q]), _f(ye[q, h]), acc)
            assert part[p, h] == bf16_bits_of_exact(acc), (p, h)
    for t in range(T):
        ps = [int(p) for p in plan["tok_rank_row"][t] if p >= 0]
        np.testing.assert_array_equal(out[t], staged_sum_exact(ps, part))


def check_rank_partial_f32_exact(plan, ye, w, part, out):
    """Exact replay of the fp32-partial return path: each partial is the
    correctly rounded fp32 fma chain over its expert rows (compared as fp32
    bits), each output the fp32 running sum of its partials, then bf16."""
    T, k = plan["comb_row"].shape
    gate = np.zeros(T * k, np.float32)
    gate[plan["comb_row"].ravel()] = w.ravel()
    H = ye.shape[1]
    for p in range(plan["N"]):
        qs = [int(q) for q in plan["fan_dst"][p] if q >= 0]
        for h in range(H):
            acc = 0.0
            for q in qs:
                acc = f32_fma_exact(float(gate[q]), _f(ye[q, h]), acc)
            assert np.float32(acc).view(np.uint32) == part[p, h].view(np.uint32), (p, h)
    for t in range(T):
        ps = [int(p) for p in plan["tok_rank_row"][t] if p >= 0]
        for h in range(H):
            acc = 0.0
            for pp in ps:
                acc = f32_add_exact(acc, float(part[pp, h]))
            assert out[t, h] == bf16_bits_of_exact(acc), (t, h)


def order_sensitive_backward_case():
    """Tiny plans where summation order decides the bf16 result:
    (a) one token, three experts on one rank: the receiver sums three rows;
    (b) one token, one expert on each of three ranks: the sender sums three.
    Row values 1, -1, 2^-30: ascending order keeps 2^-30, any other loses it."""
    import synth
    vals = np.array([[1.0] * 8, [-1.0] * 8, [2.0 ** -30] * 8], np.float32)
    rows = synth.f32_to_bf16_bits(vals)
    case_a = dict(idx=np.array([[0, 1, 2]], np.int32), E=8, R=1, g=rows)
    case_b = dict(idx=np.array([[0, 2, 4]], np.int32), E=6, R=3, g=rows)
    return case_a, case_b


def run_battery_backward(orc) -> None:
    import synth
    for case in order_sensitive_backward_case():
        rc, p = orc.plan(case["idx"], 8, case["E"], case["R"])
        assert rc == 0
        gxr, gx = orc.dispatch_backward(p, case["g"], 1, case["E"], 3, case["R"])
        check_dispatch_backward_exact(p, case["g"], gxr, gx)
        assert float((np.uint32(gx[0, 0]) << np.uint32(16)).view(np.float32)) == 2.0 ** -30
        w = np.array([[1.0, 1.0, 1.0]], np.float32)
        part, out = orc.combine_rank_partial(p, case["g"], w, case["E"], case["R"])
        check_rank_partial_exact(p, case["g"], w, part, out)
        assert float((np.uint32(out[0, 0]) << np.uint32(16)).view(np.float32)) == 2.0 ** -30
        part32, out32 = orc.combine_rank_partial_f32(p, case["g"], w, case["E"], case["R"])
        check_rank_partial_f32_exact(p, case["g"], w, part32, out32)
        assert float((np.uint32(out32[0, 0]) << np.uint32(16)).view(np.float32)) == 2.0 ** -30
    for (T, E, k, R) in ((9, 8, 3, 4), (7, 12, 4, 2), (6, 16, 5, 16)):
        rng = np.random.default_rng(T * 101 + E)
        idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
        rc, p = orc.plan(idx, 8, E, R)
        ye = synth.wide_bf16(rng, (T * k, 8), -6, 6)
        gxr, gx = orc.dispatch_backward(p, ye, T, E, k, R)
        check_dispatch_backward_exact(p, ye, gxr, gx)
        part, out = orc.combine_rank_partial(p, ye, w, E, R)
        check_rank_partial_exact(p, ye, w, part, out)
        part32, out32 = orc.combine_rank_partial_f32(p, ye, w, E, R)
        check_rank_partial_f32_exact(p, ye, w, part32, out32)
        g = synth.wide_bf16(rng, (T, 8), -6, 6)
        gye, gw = orc.combine_backward(p["comb_row"], g, ye, w, E, R)
        check_combine_backward(p["comb_row"], g, ye, w, gye, gw)


def check_combine_backward(comb_row, g, ye, w, gye, gw):
    """grad_ye[q] = bf16(fp32(w * g)) element by element; grad_w = fp64 dot
    (numpy) of the bf16 rows."""
    T, k = comb_row.shape
    gf = (g.astype(np.uint32) << np.uint32(16)).view(np.float32)
    yf = (ye.astype(np.uint32) << np.uint32(16)).view(np.float32)
    for t in range(T):
        for j in range(k):
            q = comb_row[t, j]
            prod = (np.float32(w[t, j]) * gf[t]).astype(np.float32)       # IEEE fp32 products
            expect = np.array([bf16_bits_of_exact(float(v)) for v in prod], np.uint16)
            np.testing.assert_array_equal(gye[q], expect)
            dot = float(np.dot(gf[t].astype(np.float64), yf[q].astype(np.float64)))
            assert abs(gw[t, j] - dot) <= 1e-12 * max(1.0, float(np.abs(gf[t].astype(np.float64) * yf[q]).sum()))
