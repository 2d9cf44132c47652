"""The allocation-free plan (moe_shuffle_plan_static) against the plan in a
caller's workspace (moe_shuffle_plan), through the C ABI on the MI355X.

Two static plans in a row, the second on a smaller batch with other dims:
each must give the same plan arrays, and the same dispatch, combine,
rank-partial combine and combine backward results, bit for bit, as the
workspace plan on the same inputs.  The static workspace is read back
through the library's reference copy (its address comes from the plan's
array pointers).  An oversize batch is refused without touching the static
workspace."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_token_amd as ms
    ms.load()


PLAN_KEYS = ("expert_count", "expert_offset", "rank_count", "rank_offset", "send_token", "tok_rank_row",
             "fan_src", "fan_dst", "comb_row", "rank_segs", "expert_segs")


def plan_arrays(plan, dims, N):
    """The plan arrays of any plan, copied out of its workspace with the
    library's reference copy (the workspace starts at the status word)."""
    import torch

    import moe_expert_token_amd as ms
    a = ms.moe_shuffle_plan_arrays_get(plan)
    T, k, E, R = dims.num_tokens, dims.top_k, dims.num_experts, dims.num_ranks
    KR, D = a["tok_rank_width"], a["fan_dst_width"]
    base = a["status"]
    assert base == min(a[n] for n in PLAN_KEYS + ("status", "n_rank_rows"))
    total = ms.moe_shuffle_workspace_size(dims)
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    ms.moe_shuffle_copy_reference(base, buf, total)
    i32 = buf.view(torch.int32)
    shapes = {"expert_count": (E,), "expert_offset": (E + 1,), "rank_count": (R,), "rank_offset": (R + 1,),
              "send_token": (N,), "tok_rank_row": (T, KR), "fan_src": (T * k,), "fan_dst": (N, D),
              "comb_row": (T, k), "rank_segs": (R, 4), "expert_segs": (E, 4)}
    out = {}
    for name, shape in shapes.items():
        off = (a[name] - base) // 4
        n = int(np.prod(shape))
        out[name] = i32[off:off + n].view(*shape).cpu().numpy()
    return out


def run_path(ms, torch, plan, dims, x, w, ye, gout):
    """Dispatch, combine, rank-partial combine and combine backward on a plan;
    returns host copies."""
    T, H, k, R = dims.num_tokens, dims.hidden, dims.top_k, dims.num_ranks
    rows = T * min(k, R)
    xr = torch.full((rows, H), 0x7FC1, dtype=torch.int16, device="cuda")
    xe = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    part = torch.empty((rows, H), dtype=torch.int16, device="cuda")
    out_p = torch.empty((T, H), dtype=torch.int16, device="cuda")
    gye = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    gw = torch.empty((T * k,), dtype=torch.float32, device="cuda")
    ms.moe_shuffle_dispatch(plan, x, xr, xe)
    ms.moe_shuffle_combine(plan, ye, w, out)
    ms.moe_shuffle_combine_rank_partial(plan, ye, w, part, out_p)
    ms.moe_shuffle_combine_backward(plan, gout, ye, w, gye, gw)
    info = ms.moe_shuffle_plan_query(plan)
    torch.cuda.synchronize()
    N = info["N"]
    return {"N": N, "status": info["status"], "xr": xr[:N].cpu().numpy(), "xe": xe.cpu().numpy(),
            "out": out.cpu().numpy(), "partial": part[:N].cpu().numpy(), "out_partial": out_p.cpu().numpy(),
            "grad_ye": gye.cpu().numpy(), "grad_w": gw.cpu().numpy().view(np.uint32)}


def compare_static_with_workspace_plan(T, H, E, k, R, seed):
    import gpu_harness as h
    import torch

    import moe_expert_token_amd as ms
    h.say(f"[no-alloc] T={T} H={H} E={E} k={k} R={R}")
    rng = np.random.default_rng(seed)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    dims = ms.dims_of(T, H, E, k, R)
    idx_d = torch.from_numpy(idx).cuda()
    x = h.to_dev16(synth.random_bf16(rng, (T, H)))
    w_d = torch.from_numpy(w).cuda()
    ye = h.to_dev16(synth.wide_bf16(rng, (T * k, H)))
    gout = h.to_dev16(synth.wide_bf16(rng, (T, H), -8, 8))

    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    ref_plan = ms.moe_shuffle_plan(dims, idx_d, ws)
    ref = run_path(ms, torch, ref_plan, dims, x, w_d, ye, gout)
    ref_arrays = plan_arrays(ref_plan, dims, ref["N"])

    st_plan = ms.moe_shuffle_plan_static(dims, idx_d)
    got = run_path(ms, torch, st_plan, dims, x, w_d, ye, gout)
    assert got["status"] == 0 and got["N"] == ref["N"]
    got_arrays = plan_arrays(st_plan, dims, got["N"])
    for key in PLAN_KEYS:
        np.testing.assert_array_equal(got_arrays[key], ref_arrays[key], err_msg=key)
    for key in ("xr", "xe", "out", "partial", "out_partial", "grad_ye", "grad_w"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    # the static workspace lies outside every caller buffer
    a = ms.moe_shuffle_plan_arrays_get(st_plan)
    assert not (ws.data_ptr() <= a["status"] < ws.data_ptr() + ws.numel())
    ms.moe_shuffle_plan_destroy(ref_plan)
    h.say(f"[no-alloc] static plan = workspace plan, N={got['N']}, every result bit-exact")
    return st_plan, dims, got


def test_static_plan_matches_workspace_plan_twice_then_refuses_oversize():
    import torch

    import moe_expert_token_amd as ms
    # first call, then a smaller batch with other dims (the static workspace
    # keeps the first call's contents and must be fully rewritten)
    compare_static_with_workspace_plan(4096, 1032, 64, 8, 8, seed=1)
    plan2, dims2, got2 = compare_static_with_workspace_plan(700, 520, 16, 4, 4, seed=2)
    # oversize dims are refused before any launch: the second plan stays intact
    big = ms.dims_of(262144, 7168, 256, 8, 32)
    assert ms.moe_shuffle_workspace_size(big) > ms.STATIC_WORKSPACE_BYTES
    with pytest.raises(ms.MoeShuffleError) as e:
        ms.moe_shuffle_plan_static(big, torch.zeros((262144, 8), dtype=torch.int32, device="cuda"))
    assert e.value.code == ms.E_WORKSPACE
    arrays = plan_arrays(plan2, dims2, got2["N"])
    assert arrays["rank_offset"][-1] == got2["N"]
    info = ms.moe_shuffle_plan_query(plan2)
    assert info["status"] == 0 and info["N"] == got2["N"]


def test_static_plan_replays_in_a_graph():
    """The allocation-free plan under HIP graph capture, its purpose: plan,
    dispatch and combine captured once (the device's first static plan made
    before the capture) and replayed with new routing and activations in the
    captured buffers; every replay must give the bits of the same step run
    eagerly with a workspace plan."""
    import gpu_harness as h
    import torch

    import moe_expert_token_amd as ms
    T, H, E, k, R = 1000, 1032, 32, 4, 8
    rng = np.random.default_rng(31)
    dims = ms.dims_of(T, H, E, k, R)
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    x_d = torch.empty((T, H), dtype=torch.int16, device="cuda")
    bufs = [torch.zeros(shape, dtype=torch.int16, device="cuda") for shape in ((T * min(k, R), H), (T * k, H), (T, H))]
    ref = [torch.zeros_like(b) for b in bufs]
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")

    def load_inputs():
        idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
        idx_d.copy_(torch.from_numpy(idx))
        w_d.copy_(torch.from_numpy(w))
        x_d.copy_(h.to_dev16(synth.random_bf16(rng, (T, H))))

    def step(plan, out_bufs):
        xr, xe, out = out_bufs
        ms.moe_shuffle_dispatch(plan, x_d, xr, xe)
        ms.moe_shuffle_combine(plan, xe, w_d, out)
        return plan

    load_inputs()
    step(ms.moe_shuffle_plan_static(dims, idx_d), bufs)   # the first call on the device, outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step(ms.moe_shuffle_plan_static(dims, idx_d), bufs)
    torch.cuda.synchronize()
    for replay in range(4):
        load_inputs()
        eager = step(ms.moe_shuffle_plan(dims, idx_d, ws), ref)
        N = ms.moe_shuffle_plan_query(eager)["N"]
        for b in bufs:
            b.fill_(0x3F80)                   # eager work between the replays, and stale contents
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ms.moe_shuffle_plan_query(captured)["N"] == N
        for name, got, want in zip(("xr", "xe", "out"), bufs, ref):
            n = N if name == "xr" else got.shape[0]
            assert torch.equal(got[:n], want[:n]), f"replay {replay}: {name}"
        h.say(f"[no-alloc] graph replay {replay} N={N} matches the eager step")
        ms.moe_shuffle_plan_destroy(eager)
