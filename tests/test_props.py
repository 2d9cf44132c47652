"""Property tests of the oracle over random shapes (hypothesis, CPU only).

The invariants are the ones the pages fix: every routed (token, expert) pair
is placed exactly once, segment sizes equal the routing histogram, a token is
sent to a given rank at most once, and dispatch -> identity expert ->
combine with gates summing to 1 returns the input."""

import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import pins
import synth


@st.composite
def routing_case(draw):
    R = draw(st.integers(1, 8))
    Epr = draw(st.integers(1, 6))
    E = R * Epr
    k = draw(st.integers(1, E))
    T = draw(st.integers(0, 48))
    H = 8 * draw(st.integers(1, 4))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    skew = draw(st.booleans())
    rng = np.random.default_rng(seed)
    if skew and T:
        # every token's first slot is the same expert
        hot = int(rng.integers(E))
        rest = [int(e) for e in rng.permutation(E) if e != hot]
        idx = np.array([[hot] + list(rng.permutation(rest)[:k - 1]) for _ in range(T)], np.int32).reshape(T, k)
        g = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
        w = (g / g.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    else:
        idx, w = synth.random_routing(rng, T, E, k)
    x = synth.random_bf16(rng, (T, H))
    return T, H, E, k, R, idx, w, x


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(routing_case())
def test_oracle_invariants(case):
    T, H, E, k, R, idx, w, x = case
    orc = oracle.get()
    rc, p = orc.plan(idx, H, E, R)
    assert rc == 0
    # every routed pair placed exactly once
    assert sorted(p["comb_row"].ravel().tolist()) == list(range(T * k))
    # segment sizes equal the histogram; offsets are their prefix sums
    pins.check_counts(p, idx, E, R)
    # at most one rank row per (token, rank), ranks ascending
    Epr = E // R
    for t in range(T):
        rows = [int(q) for q in p["tok_rank_row"][t] if q >= 0]
        ranks = [int(np.searchsorted(p["rank_offset"], q, side="right") - 1) for q in rows]
        assert ranks == sorted(set(ranks)) == sorted({int(e) // Epr for e in idx[t]})
    pins.check_plan_all(p, idx, E, R, brute=T <= 16)
    # dispatch is a bit copy and the identity-expert round trip returns x
    xr, xe = orc.dispatch(p, x, E, k, R)
    pins.check_dispatch(p, idx, x, xr, xe)
    out = orc.combine(p["comb_row"], xe, w, E, R)
    np.testing.assert_array_equal(out, np.where(x == 0x8000, 0, x).astype(np.uint16))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(routing_case())
def test_oracle_backward_adjoint(case):
    """<dispatch(x), g> == <x, dispatch^T(g)> for small integers (exact)."""
    T, H, E, k, R, idx, w, x = case
    orc = oracle.get()
    rc, p = orc.plan(idx, H, E, R)
    rng = np.random.default_rng(T * 7 + E)
    xi = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(T, H)).astype(np.float32))
    gi = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(T * k, H)).astype(np.float32))
    _, xe = orc.dispatch(p, xi, E, k, R)
    _, gx = orc.dispatch_backward(p, gi, T, E, k, R)
    lhs = (synth.bf16_bits_to_f32(xe).astype(np.float64) * synth.bf16_bits_to_f32(gi)).sum()
    rhs = (synth.bf16_bits_to_f32(xi).astype(np.float64) * synth.bf16_bits_to_f32(gx)).sum()
    assert lhs == rhs
