"""Numerical edge cases for the reductions of the shuffle: the inputs, the
oracle's results for them, and the comparison rule (test helpers).

The combine is the per-token sum of the DySHARP write-up (section 2 /
Fig. 1); its arithmetic (fp32 from +0, ascending order, one fused
multiply-add per term, one round-to-nearest-even to bf16, subnormals kept, a
NaN stays a quiet NaN) is the reading the oracle is pinned to.  The cases
hold what random activations never produce: bf16 subnormals, sums that land
among the fp32 and bf16 subnormals, exact ties, the order- and
fusing-sensitive rows of the oracle pins, infinities, finite sums that
overflow (in fp32, or only in the rounding to bf16), NaN inputs, Inf - Inf,
signed zeros, and NaN / infinite / zero / huge / tiny gates.

Comparison: every element whose oracle value is not a NaN must match bit for
bit.  A NaN must come out as a quiet NaN in the same place.  Its sign is
compared where it is determined: where exactly one operand of the element is
a NaN and no operand is infinite or huge.  IEEE 754 leaves the sign of a NaN
that an invalid operation creates unspecified (x86 makes Inf - Inf a
negative NaN, CDNA a positive one); payloads are not compared.
"""

from __future__ import annotations

import numpy as np

import pins
import synth


def bf(v: float) -> int:
    """bf16 bits of a value that bf16 holds exactly."""
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, f"{v} is not a bf16 value"
    return b >> 16


PINF, NINF, QNAN, NQNAN, SNAN, MAXF = 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0x7F7F

# Column scenarios: the values of the four special slots in one column.
SCENARIOS = [
    (0x0001, 0x0002, 0x8001, 0x007F),              # bf16 subnormals
    (0x0080, 0x8001, 0x0000, 0x0000),              # 2^-126 - 2^-133: just below the normal range
    (bf(1.0), bf(2.0 ** -8), 0, 0),                # a tie, even neighbour: 1
    (bf(1 + 2.0 ** -7), bf(2.0 ** -8), 0, 0),      # a tie, odd neighbour: rounds up
    (bf(-1.0), bf(-(2.0 ** -8)), 0, 0),            # a negative tie
    (bf(1.0), bf(-1.0), bf(2.0 ** -30), 0),        # ascending order keeps 2^-30
    (bf(1 + 2.0 ** -7), bf(1 + 2.0 ** -7), 0, 0),  # with gates (-1, 1 + 2^-23) only fusing keeps 2^-30
    (bf(3 * 2.0 ** -128), bf(-(2.0 ** -126)), bf(2.0 ** -133), 0),  # sums among the fp32 subnormals
    (PINF, bf(1.0), bf(2.0), bf(3.0)),             # +Inf
    (NINF, bf(1.0), 0, 0),                         # -Inf
    (MAXF, MAXF, 0, 0),                            # a finite sum past the fp32 range
    (MAXF, bf(2.0 ** 119), 0, 0),                  # exact in fp32, half-way in bf16: to Inf (even)
    (MAXF, bf(2.0 ** 118), 0, 0),                  # below half-way: stays the largest bf16
    (QNAN, bf(1.0), bf(2.0), 0),                   # a NaN input
    (NQNAN, bf(1.0), 0, 0),                        # a negative NaN input
    (SNAN, bf(-1.0), 0, 0),                        # a signalling NaN: quiet after the first operation
    (PINF, NINF, 0, 0),                            # Inf - Inf
    (QNAN, PINF, 0, 0),                            # NaN with Inf
    (0x8000, 0x8000, 0x8000, 0x8000),              # -0 terms: the sum starts at +0
    (bf(-(2.0 ** -126)), bf(2.0 ** -126), 0x8000, 0),  # an exact zero sum: +0
    (bf(-3.0), bf(1.0), bf(1.0), bf(1.0)),         # cancels to exactly 0 on the last term
]
NS = len(SCENARIOS)


def gate_patterns(k: int):
    """Per-token gates: the first four slots carry the special gates, the rest 1."""
    pats = [
        [1.0, 1.0, 1.0, 1.0],
        [0.5, 0.25, 0.125, 1.0],                 # halvings push tiny normals into subnormals
        [-1.0, 1 + 2.0 ** -23, 1.0, 1.0],        # the fusing-sensitive pair
        [2.0 ** -100, 2.0 ** -20, 1.0, -1.0],    # products underflow
        [float("inf"), 1.0, 1.0, 1.0],           # Inf gate (Inf * 0 is NaN)
        [float("nan"), 1.0, 1.0, 1.0],           # NaN gate
        [0.0, -0.0, 0.0, 0.0],                   # zero gates
        [2.0 ** 100, 2.0 ** 100, 1.0, 1.0],      # products overflow
    ]
    return [np.array(p + [1.0] * (k - 4), np.float32) for p in pats]


def route_patterns(k: int, E: int, R: int):
    """Slot -> expert patterns with different groupings by rank, and slot
    orders that differ from the ascending expert order the receiver sums in."""
    Epr = E // R
    pats = []
    if k <= Epr:
        pats.append(list(range(k)))                          # one rank, ascending
        pats.append(list(range(k))[::-1])                    # one rank, descending
    spread = [((j + 1) % R) * Epr + j // R for j in range(k)]  # across ranks, rotated
    pats.append(spread)
    if 1 + 2 * ((k - 1) // (2 * R)) < Epr:
        pairs = [((j // 2) % R) * Epr + (j % 2) + 2 * (j // (2 * R)) for j in range(k)]
        pats.append(pairs[::-1])                             # two per rank, descending
    rng = np.random.default_rng(E * 131 + k * 7 + R)
    for _ in range(2):
        pats.append(list(rng.permutation(E)[:k]))
    out = []
    for p in pats:
        p = np.array(p, np.int32)
        assert len(set(p.tolist())) == k and p.min() >= 0 and p.max() < E, p
        out.append(p)
    return out


def build_case(T_pad: int, H: int, E: int, k: int, R: int, seed: int, shifted: bool = False):
    """Special tokens (every gate pattern x every route pattern), then T_pad
    random tokens.  Returns (idx [T,k], w [T,k], Y [T,k,H] bf16 bits, n_sp):
    Y[t, j] is the row the expert of slot j returns for token t.  Two of
    every three columns of a special token hold scenarios (in turn) in four
    of its slots (slots 0..3, or the last four for odd tokens when shifted)
    and +0 in the other slots; the third column holds random normals."""
    assert k >= 4
    rng = np.random.default_rng(seed)
    gates, routes = gate_patterns(k), route_patterns(k, E, R)
    idx = np.array([r for _ in gates for r in routes], np.int32).reshape(-1, k)
    w = np.array([g for g in gates for _ in routes], np.float32).reshape(-1, k)
    n_sp = idx.shape[0]
    ridx, rw = synth.random_routing(rng, T_pad, E, k, signed_gates=True)
    idx = np.concatenate([idx, ridx]).astype(np.int32)
    w = np.concatenate([w, rw]).astype(np.float32)
    T = idx.shape[0]
    Y = synth.random_bf16(rng, (T, k, H))
    scen = np.array(SCENARIOS, np.uint16)                    # [NS, 4]
    spc = np.nonzero(np.arange(H) % 3 != 2)[0]               # the special columns
    for t in range(n_sp):
        which = (np.arange(len(spc)) + 5 * t) % NS           # every scenario in turn, shifted per token
        slots = np.arange(4) + (k - 4 if shifted and t % 2 else 0)
        Y[t][:, spc] = 0
        for s, j in enumerate(slots):
            Y[t, j, spc] = scen[which, s]
    return idx, w, Y, n_sp


def nan_sign_mask(op_groups):
    """op_groups: float32 arrays of one shape, the operands of each output
    element.  True where exactly one operand is a NaN and none is infinite
    or of magnitude 2^60 or more (so no operation on the way can create a
    NaN of its own)."""
    nan = sum(np.isnan(a).astype(np.int32) for a in op_groups)
    wild = sum((~np.isfinite(a) & ~np.isnan(a)) | (np.abs(np.nan_to_num(a)) >= 2.0 ** 60) for a in op_groups)
    return (nan == 1) & (wild == 0)


def f32_of(bits16):
    return (np.asarray(bits16, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def assert_bf16_same(got, exp, sign_mask, what):
    """The comparison rule for bf16 results; returns the number of NaNs."""
    got = np.asarray(got, np.uint16)
    exp = np.asarray(exp, np.uint16)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    gn, en = pins.bf16_is_nan(got), pins.bf16_is_nan(exp)
    bad = np.argwhere(gn != en)
    assert bad.size == 0, f"{what}: NaN placement differs at {bad[:5].tolist()}"
    assert np.all(got[gn] & 0x0040), f"{what}: a NaN that is not quiet"
    diff = np.argwhere((got != exp) & ~en)
    assert diff.size == 0, (f"{what}: {diff.shape[0]} elements differ, first at {diff[:3].tolist()}: "
                            f"{[hex(int(got[tuple(i)])) for i in diff[:3]]} vs "
                            f"{[hex(int(exp[tuple(i)])) for i in diff[:3]]}")
    m = gn & np.broadcast_to(sign_mask, got.shape)
    sdiff = np.argwhere(m & ((got >> 15) != (exp >> 15)))
    assert sdiff.size == 0, f"{what}: NaN sign differs where it is determined, at {sdiff[:5].tolist()}"
    return int(gn.sum())


def assert_f32_same(got, exp, sign_mask, what):
    """The same rule for fp32 results (compared as bits)."""
    got = np.ascontiguousarray(got, np.float32).view(np.uint32)
    exp = np.ascontiguousarray(exp, np.float32).view(np.uint32)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)

    def isnan(u):
        return ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    gn, en = isnan(got), isnan(exp)
    assert np.array_equal(gn, en), f"{what}: NaN placement differs"
    assert np.all(got[gn] & 0x00400000), f"{what}: a NaN that is not quiet"
    diff = np.argwhere((got != exp) & ~en)
    assert diff.size == 0, f"{what}: {diff.shape[0]} elements differ, first at {diff[:3].tolist()}"
    m = gn & np.broadcast_to(sign_mask, got.shape)
    assert not np.any(m & ((got >> 31) != (exp >> 31))), f"{what}: NaN sign differs where it is determined"


# ---------------------------------------------------------------- the oracle side

ALL_PARTS = ("combine", "rank_partial", "rank_partial_f32", "dispatch_backward", "combine_backward")


def oracle_results(orc, idx, w, Y, H, E, R, parts=ALL_PARTS):
    """Lays the rows out by the oracle's plan and runs the oracle's reductions
    named in `parts` on them.  ye[comb_row[t, j]] = Y[t, j]; grad_out = Y[:, 0]."""
    T, k = idx.shape
    rc, o = orc.plan(idx, H, E, R)
    assert rc == 0
    ye = np.empty((T * k, H), np.uint16)
    ye[o["comb_row"].ravel()] = Y.reshape(T * k, H)
    grad_out = np.ascontiguousarray(Y[:, 0, :])
    res = {"plan": o, "ye": ye, "grad_out": grad_out, "parts": tuple(parts)}
    if "combine" in parts:
        res["out"] = orc.combine(o["comb_row"], ye, w, E, R)
    if "rank_partial" in parts:
        res["partial"], res["out_partial"] = orc.combine_rank_partial(o, ye, w, E, R)
    if "rank_partial_f32" in parts:
        res["partial32"], res["out_partial32"] = orc.combine_rank_partial_f32(o, ye, w, E, R)
    if "dispatch_backward" in parts:
        res["grad_xr"], res["grad_x"] = orc.dispatch_backward(o, ye, T, E, k, R)
    if "combine_backward" in parts:
        res["grad_ye"], res["grad_w"] = orc.combine_backward(o["comb_row"], grad_out, ye, w, E, R)
    return res


def abs_dot(comb_row, g_bits, ye_bits, chunk=256, finite_only=False):
    """sum_h |grad_out[t,h] * ye[q,h]| for every (t, j), in float64, chunked;
    with finite_only the infinite and NaN products count as 0."""
    T, k = comb_row.shape
    out = np.zeros((T, k))
    with np.errstate(invalid="ignore"):
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            g = np.abs(f32_of(g_bits[t0:t1])).astype(np.float64)
            for j in range(k):
                p = g * np.abs(f32_of(ye_bits[comb_row[t0:t1, j]]))
                if finite_only:
                    p = np.where(np.isfinite(p), p, 0.0)
                out[t0:t1, j] = p.sum(axis=1)
    return out


def compare_all(dev, ref, idx, w, Y, E, R, n_sp, name, log=print):
    """Every device result against the oracle's under the rule above, for the
    parts the oracle ran.  `dev` holds numpy arrays: out, out_range
    (optional), partial, out_partial, partial32, out_partial32, grad_xr,
    grad_x, grad_ye, grad_w; the first N rows of the rank-row results.  The
    NaN-sign masks are built for the first n_sp tokens, the only ones that
    hold special values."""
    parts = ref["parts"]
    o = ref["plan"]
    T, k = idx.shape
    H = Y.shape[2]
    N = o["N"]
    Epr = E // R
    wv = np.broadcast_to(w[:n_sp, :, None], (n_sp, k, H)).astype(np.float32)
    yv = f32_of(Y[:n_sp])
    rank_of = idx[:n_sp] // Epr

    def token_mask(use_gates):
        m = np.zeros((T, H), bool)
        groups = [yv[:, j, :] for j in range(k)] + ([wv[:, j, :] for j in range(k)] if use_gates else [])
        m[:n_sp] = nan_sign_mask(groups)
        return m

    st = o["send_token"]
    rank_p = np.searchsorted(o["rank_offset"], np.arange(N), side="right") - 1
    sp_rows = np.nonzero(st < n_sp)[0]                       # rank rows of the special tokens

    def partial_mask(use_gates):
        m = np.zeros((N, H), bool)
        t_of, r_of = st[sp_rows], rank_p[sp_rows]
        sel = rank_of[t_of] == r_of[:, None]                 # [rows, k]: the token's slots on that rank
        groups = []
        for j in range(k):
            groups.append(np.where(sel[:, j:j + 1], yv[t_of, j, :], 0.0).astype(np.float32))
            if use_gates:
                groups.append(np.where(sel[:, j:j + 1], wv[t_of, j, :], 0.0).astype(np.float32))
        m[sp_rows] = nan_sign_mask(groups)
        return m

    m_tok_w = token_mask(True)
    if "combine" in parts:
        nn = assert_bf16_same(dev["out"], ref["out"], m_tok_w, f"{name} combine")
        nd = int((m_tok_w & pins.bf16_is_nan(ref["out"])).sum())
        log(f"[numerics] {name} combine bit-exact: {nn} NaNs, {nd} with a determined sign")
        if dev.get("out_range") is not None:
            assert_bf16_same(dev["out_range"], ref["out"], m_tok_w, f"{name} combine_range")
    if "rank_partial" in parts or "rank_partial_f32" in parts:
        m_part_w = partial_mask(True)
    if "rank_partial" in parts:
        assert_bf16_same(dev["partial"], ref["partial"], m_part_w, f"{name} rank-partial partials")
        assert_bf16_same(dev["out_partial"], ref["out_partial"], m_tok_w, f"{name} rank-partial out")
    if "rank_partial_f32" in parts:
        assert_f32_same(dev["partial32"], ref["partial32"], m_part_w, f"{name} fp32 partials")
        assert_bf16_same(dev["out_partial32"], ref["out_partial32"], m_tok_w, f"{name} fp32-partial out")
    if "dispatch_backward" in parts:
        assert_bf16_same(dev["grad_xr"], ref["grad_xr"], partial_mask(False), f"{name} grad_xr")
        assert_bf16_same(dev["grad_x"], ref["grad_x"], token_mask(False), f"{name} grad_x")
    if "combine_backward" not in parts:
        log(f"[numerics] {name} {', '.join(parts)}: every result matches")
        return
    # grad_ye[q(t, j)] = bf16(w[t, j] * grad_out[t]): operands w and grad_out
    g32 = f32_of(ref["grad_out"][:n_sp])
    gmask = np.zeros((T * k, H), bool)
    gm = np.stack([nan_sign_mask([wv[:, j, :], g32]) for j in range(k)], axis=1)   # [n_sp, k, H]
    gmask[o["comb_row"][:n_sp].ravel()] = gm.reshape(n_sp * k, H)
    assert_bf16_same(dev["grad_ye"], ref["grad_ye"], gmask, f"{name} grad_ye")
    # grad_w: within its fp32 summation bound where no path can overflow;
    # NaN where the oracle's fp64 value is NaN; the same infinity where the
    # oracle's is infinite
    got_w = np.asarray(dev["grad_w"], np.float64).reshape(T, k)
    o_gw = ref["grad_w"]
    ad = abs_dot(o["comb_row"], ref["grad_out"], ref["ye"])
    V = H // 8
    terms = max(8 * u + 6 + -(-V // (64 * u)) + 2 for u in (1, 2))
    tame = np.isfinite(ad) & (ad < 2.0 ** 120)
    bound = terms * 2.0 ** -24 * ad + 2.0 ** -126
    err = np.abs(got_w - o_gw)
    assert np.all(err[tame] <= bound[tame]), f"{name} grad_w outside its bound"
    assert np.all(np.isnan(got_w[np.isnan(o_gw)])), f"{name} grad_w: a NaN of the oracle is not a NaN"
    ad_fin = abs_dot(o["comb_row"], ref["grad_out"], ref["ye"], finite_only=True)
    inf = np.isinf(o_gw) & (ad_fin < 2.0 ** 120)               # the finite terms cannot overflow
    assert np.array_equal(got_w[inf], o_gw[inf]), f"{name} grad_w: an infinity differs"
    log(f"[numerics] {name} every reduction matches (grad_w: {int(tame.sum())} finite checked, "
        f"{int(np.isnan(o_gw).sum())} NaN, {int(inf.sum())} infinite)")
