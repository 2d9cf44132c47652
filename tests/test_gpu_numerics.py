"""Numerical edge cases through every HIP reduction, bit for bit against the
oracle (MI355X).

The inputs and the comparison rule are in numerics_cases.py: subnormals,
ties, order- and fusing-sensitive sums, infinities, overflow, NaNs,
Inf - Inf and signed zeros, with special gates.  Entry points: combine,
combine over token ranges, the rank-partial combine with bf16 and with fp32
partials, dispatch backward (receiver and sender sums), combine backward
(grad_ye bit for bit, grad_w within its bound where finite), and the
identity-expert round trip of rows that hold subnormals.  Each runs on small
ragged shapes (1 KiB units, top-k above 8) and on a batch whose row buffers
pass 2 GiB, where combine and the sender's sum take whole 8 KiB rows per
wave.
"""

from __future__ import annotations

import numpy as np
import pytest

import numerics_cases as nc
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_token_amd as ms
    ms.load()


def device_results(idx, w, ye, grad_out, H, E, R, N, ranges=None, parts=nc.ALL_PARTS):
    """The reduction entry points named in `parts` on the device, on rows laid
    out as the oracle's plan lays them out.  Returns numpy copies; rank-row
    results cut to their first N rows."""
    import torch

    import gpu_harness as h
    import moe_expert_token_amd as ms
    T, k = idx.shape
    KR = min(k, R)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(np.ascontiguousarray(idx)).cuda(), ws)
    info = ms.moe_shuffle_plan_query(plan)
    assert info["status"] == 0 and info["N"] == N, info
    ye_d = h.to_dev16(ye)
    w_d = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    full = lambda r: torch.full((max(r, 1), H), h.SENTINEL, dtype=torch.int16, device="cuda")  # noqa: E731
    rows = T * KR
    res = {"comb_row": ms.plan_array_views(plan, N)["comb_row"].cpu().numpy()}

    out = full(T)
    if "combine" in parts:
        ms.moe_shuffle_combine(plan, ye_d, w_d, out)
        res["out"] = h.to_host16(out)[:T]
        if ranges:
            out.fill_(h.SENTINEL)
            for t0, t1 in ranges:
                ms.moe_shuffle_combine_range(plan, ye_d, w_d, out, t0, t1)
            res["out_range"] = h.to_host16(out)[:T]
    if "rank_partial" in parts:
        out.fill_(h.SENTINEL)
        part = full(rows)
        ms.moe_shuffle_combine_rank_partial(plan, ye_d, w_d, part, out)
        res["partial"], res["out_partial"] = h.to_host16(part)[:N], h.to_host16(out)[:T]
        del part
    if "rank_partial_f32" in parts:
        out.fill_(h.SENTINEL)
        part32 = torch.full((max(rows, 1), H), float("nan"), dtype=torch.float32, device="cuda")
        ms.moe_shuffle_combine_rank_partial_f32(plan, ye_d, w_d, part32, out)
        res["partial32"], res["out_partial32"] = part32[:N].cpu().numpy(), h.to_host16(out)[:T]
        del part32
    if "dispatch_backward" in parts:
        out.fill_(h.SENTINEL)
        gxr = full(rows)
        ms.moe_shuffle_dispatch_backward(plan, ye_d, gxr, out)
        res["grad_xr"], res["grad_x"] = h.to_host16(gxr)[:N], h.to_host16(out)[:T]
        del gxr
    if "combine_backward" in parts:
        gye = full(T * k)
        gw = torch.full((max(T * k, 1),), float("nan"), dtype=torch.float32, device="cuda")
        ms.moe_shuffle_combine_backward(plan, h.to_dev16(grad_out), ye_d, w_d, gye, gw)
        res["grad_ye"], res["grad_w"] = h.to_host16(gye)[:T * k], gw.cpu().numpy()[:T * k]
    torch.cuda.synchronize()
    ms.moe_shuffle_plan_destroy(plan)
    return res


def run_case(idx, w, Y, H, E, R, n_sp, ranges=None, name="", parts=nc.ALL_PARTS):
    import gpu_harness as h
    import oracle
    T, k = idx.shape
    h.say(f"[numerics] {name} T={T} H={H} E={E} k={k} R={R} special tokens {n_sp}")
    ref = nc.oracle_results(oracle.get(), idx, w, Y, H, E, R, parts)
    dev = device_results(idx, w, ref["ye"], ref["grad_out"], H, E, R, ref["plan"]["N"], ranges, parts)
    np.testing.assert_array_equal(dev["comb_row"], ref["plan"]["comb_row"])
    nc.compare_all(dev, ref, idx, w, Y, E, R, n_sp, name, log=h.say)


@pytest.mark.parametrize("T_pad,H,E,k,R,shifted", [
    (152, 520, 16, 4, 4, False),    # ragged rows (65 vectors: one full unit and one vector), 4 token tiles
    (41, 512, 48, 12, 4, True),     # top-12: a 12-wide receiver map and more than 8 combine terms
    (0, 64, 8, 4, 1, False),        # a single rank: the sender sums one partial
    (100, 32, 8, 8, 8, True),       # one expert per rank, rows of four 16-byte vectors
])
def test_special_values_small(T_pad, H, E, k, R, shifted):
    idx, w, Y, n_sp = nc.build_case(T_pad, H, E, k, R, seed=T_pad * 7 + H + k, shifted=shifted)
    T = idx.shape[0]
    ranges = [(a, min(T, a + 64)) for a in range(0, T, 64)] if T > 64 else None
    run_case(idx, w, Y, H, E, R, n_sp, ranges=ranges, name=f"special-{T}x{H}-k{k}-R{R}")


def test_special_values_large_buffers():
    """33000 tokens, top-8, H = 4096: the expert rows and the rank rows pass
    2 GiB, so combine and the sender's sum read whole 8 KiB rows per wave.
    The special tokens come first; random tokens (rows drawn from a pool of
    512 random rows) fill the rest.  Only the calls whose units change with
    the buffer size run here (the fp32-partial sums and the combine backward
    keep their unit at every size and run in the small cases)."""
    rng = np.random.default_rng(33)
    T, H, E, k, R = 33000, 4096, 64, 8, 8
    idx_s, w_s, Y_s, n_sp = nc.build_case(0, H, E, k, R, seed=3, shifted=True)
    n_rand = T - n_sp
    ridx, rw = synth.random_routing(rng, n_rand, E, k, signed_gates=True)
    pool = synth.random_bf16(rng, (512, H))
    Y = np.concatenate([Y_s, pool[rng.integers(0, 512, size=(n_rand, k))]])
    idx = np.concatenate([idx_s, ridx]).astype(np.int32)
    w = np.concatenate([w_s, rw]).astype(np.float32)
    assert T * k * H * 2 > (2 << 30) and T * min(k, R) * H * 2 > (2 << 30)
    run_case(idx, w, Y, H, E, R, n_sp, ranges=[(0, 64 * 200), (64 * 200, T)], name="special-large",
             parts=("combine", "rank_partial", "dispatch_backward"))


def test_order_sensitive_pin_cases_on_device():
    """The two hand-built plans of the oracle pins where only the ascending
    order keeps a 2^-30 term (three experts on one rank: the receiver sums
    three rows; one expert on each of three ranks: the sender sums three),
    through every reduction on the device."""
    import oracle
    import pins
    for case in pins.order_sensitive_backward_case():
        idx, E, R, g = case["idx"], case["E"], case["R"], case["g"]
        k = idx.shape[1]
        rc, o = oracle.get().plan(idx, 8, E, R)
        Y = g[o["comb_row"][0]][None]                      # Y[0, j] = the pin's row of slot j
        run_case(idx, np.ones((1, k), np.float32), Y, 8, E, R, 1, name=f"order-pin-R{R}")


@pytest.mark.parametrize("k", [2, 8])
def test_round_trip_with_subnormal_rows(k):
    """dispatch -> identity expert -> combine with gates summing to 1 returns
    x bit for bit for every finite x, bf16 subnormals and the largest finite
    values included (-0 comes back as +0), infinities as themselves, NaNs as
    quiet NaNs."""
    import gpu_harness as h
    import oracle
    import pins
    rng = np.random.default_rng(90 + k)
    T, H, E, R = 700, 136, 16, 4
    idx, w = synth.random_routing(rng, T, E, k)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)     # every bf16 pattern ...
    sub = rng.random((T, H)) < 0.3
    x = np.where(sub, x & np.uint16(0x807F), x).astype(np.uint16)  # ... 30 % of them subnormals or zeros
    x[:, 0], x[:, 1], x[:, 2], x[:, 3] = 0x0001, 0x8001, nc.MAXF, 0xFF7F
    x[:, 4], x[:, 5] = 0x8000, nc.PINF
    g = h.run_hip(idx, x, w, H, E, R)
    orc = oracle.get()
    rc, o = orc.plan(idx, H, E, R)
    oxr, oxe = orc.dispatch(o, x, E, k, R)
    np.testing.assert_array_equal(g["xe"], oxe)                   # a bit copy: signalling NaNs stay as they are
    o_out = orc.combine(o["comb_row"], oxe, w, E, R)
    nc.assert_bf16_same(g["out_rt"], o_out, np.ones((T, H), bool), f"round trip out k={k}")
    fin = ~pins.bf16_is_nan(x)
    expect = np.where(x == 0x8000, 0, x).astype(np.uint16)
    np.testing.assert_array_equal(g["out_rt"][fin], expect[fin])
    assert np.all(pins.bf16_is_nan(g["out_rt"][~fin]))
    h.say(f"[numerics] round trip k={k}: {int(sub.sum())} subnormal or zero inputs came back exactly")
