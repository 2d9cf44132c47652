"""Stream and graph use.  The forward step (plan, dispatch, combine), the
combine backward, and the dispatch backward with both rank-partial
combines, each captured once in a HIP graph and replayed: every replay must give the
bits of the same calls run eagerly, with eager work and synchronisations
between the replays.  The library records no memset or host copy in these
calls, so a captured step is the step."""

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


def test_forward_step_replays_in_a_graph():
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    T, H, E, k, R = 1000, 1032, 32, 4, 8
    rng = np.random.default_rng(21)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    x_d = torch.empty((T, H), dtype=torch.int16, device="cuda")
    xr = torch.zeros((T * min(k, R), H), dtype=torch.int16, device="cuda")
    xe = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")

    def load_inputs(seed_rng):
        idx, w = synth.random_routing(seed_rng, T, E, k, signed_gates=True)
        x = synth.random_bf16(seed_rng, (T, H))
        idx_d.copy_(torch.from_numpy(idx))
        w_d.copy_(torch.from_numpy(w))
        x_d.copy_(h.to_dev16(x))

    def step():
        plan = ms.moe_shuffle_plan(dims, idx_d, ws)
        ms.moe_shuffle_dispatch(plan, x_d, xr, xe)
        ms.moe_shuffle_combine(plan, xe, w_d, out)
        return plan

    load_inputs(rng)
    ms.moe_shuffle_plan_destroy(step())   # every kernel launched once before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured_plan = step()
    torch.cuda.synchronize()

    for replay in range(4):
        load_inputs(rng)                  # new routing and activations in the captured buffers
        torch.cuda.synchronize()
        eager_plan = step()
        info = ms.moe_shuffle_plan_query(eager_plan)
        want = {"xr": xr[:info["N"]].clone(), "xe": xe.clone(), "out": out.clone()}
        ms.moe_shuffle_plan_destroy(eager_plan)
        for t in (xr, xe, out):
            t.fill_(0x3F80)               # eager work between the replays, and stale contents
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ms.moe_shuffle_plan_query(captured_plan)["N"] == info["N"]
        for name, t in (("xr", xr[:info["N"]]), ("xe", xe), ("out", out)):
            assert torch.equal(t, want[name]), f"replay {replay}: {name}"
        h.say(f"[graph] replay {replay} N={info['N']} matches the eager step")
    ms.moe_shuffle_plan_destroy(captured_plan)


def test_combine_backward_replays_in_a_graph():
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    T, H, E, k, R = 700, 1024, 64, 6, 16
    rng = np.random.default_rng(22)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    w_d = torch.from_numpy(w).cuda()
    g_d = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ye_d = h.to_dev16(synth.wide_bf16(rng, (T * k, H)))
    gye = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    gw = torch.zeros((T * k,), dtype=torch.float32, device="cuda")
    g_d.copy_(h.to_dev16(synth.wide_bf16(rng, (T, H))))
    ms.moe_shuffle_combine_backward(plan, g_d, ye_d, w_d, gye, gw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ms.moe_shuffle_combine_backward(plan, g_d, ye_d, w_d, gye, gw)
    for replay in range(3):
        g_d.copy_(h.to_dev16(synth.wide_bf16(rng, (T, H))))
        ms.moe_shuffle_combine_backward(plan, g_d, ye_d, w_d, gye, gw)
        torch.cuda.synchronize()
        want_gye, want_gw = gye.clone(), gw.clone()
        gye.fill_(0)
        gw.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gye, want_gye), f"replay {replay}: grad_ye"
        assert torch.equal(gw.view(torch.int32), want_gw.view(torch.int32)), f"replay {replay}: grad_w"
    ms.moe_shuffle_plan_destroy(plan)


def test_dispatch_backward_and_rank_partial_replay_in_a_graph():
    """The receiver and sender sums in all three forms (dispatch backward,
    rank-partial combine with bf16 and with fp32 partials; the last two
    include the per-row gate kernel) captured in one graph."""
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    T, H, E, k, R = 900, 1032, 48, 6, 8
    rng = np.random.default_rng(23)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    KR = min(k, R)
    w_d = torch.from_numpy(w).cuda()
    src = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    bufs = {"grad_xr": torch.empty((T * KR, H), dtype=torch.int16, device="cuda"),
            "grad_x": torch.empty((T, H), dtype=torch.int16, device="cuda"),
            "partial": torch.empty((T * KR, H), dtype=torch.int16, device="cuda"),
            "out": torch.empty((T, H), dtype=torch.int16, device="cuda"),
            "partial32": torch.empty((T * KR, H), dtype=torch.float32, device="cuda"),
            "out32": torch.empty((T, H), dtype=torch.int16, device="cuda")}

    def calls():
        ms.moe_shuffle_dispatch_backward(plan, src, bufs["grad_xr"], bufs["grad_x"])
        ms.moe_shuffle_combine_rank_partial(plan, src, w_d, bufs["partial"], bufs["out"])
        ms.moe_shuffle_combine_rank_partial_f32(plan, src, w_d, bufs["partial32"], bufs["out32"])

    N = ms.moe_shuffle_plan_query(plan)["N"]
    src.copy_(h.to_dev16(synth.wide_bf16(rng, (T * k, H))))
    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for replay in range(3):
        src.copy_(h.to_dev16(synth.wide_bf16(rng, (T * k, H))))
        calls()
        torch.cuda.synchronize()
        want = {key: b.clone() for key, b in bufs.items()}
        for b in bufs.values():
            b.view(torch.int16).fill_(0x7F7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, b in bufs.items():
            rows = N if key in ("grad_xr", "partial", "partial32") else T
            got, ref = b[:rows], want[key][:rows]
            if b.dtype == torch.float32:
                got, ref = got.view(torch.int32), ref.view(torch.int32)
            assert torch.equal(got, ref), f"replay {replay}: {key}"
    ms.moe_shuffle_plan_destroy(plan)


def test_two_plans_on_two_streams_at_once():
    """Two independent shuffles, each with its own workspace and buffers,
    issued on two streams without waits between them, give the bits each
    gives alone on the default stream."""
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    shapes = [(900, 1032, 32, 4, 8), (700, 2048, 64, 6, 16)]
    rng = np.random.default_rng(23)
    problems = []
    for T, H, E, k, R in shapes:
        idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
        x = synth.random_bf16(rng, (T, H))
        dims = ms.dims_of(T, H, E, k, R)
        problems.append(dict(
            dims=dims, idx=torch.from_numpy(idx).cuda(), w=torch.from_numpy(w).cuda(), x=h.to_dev16(x),
            ws=torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda"),
            xr=torch.zeros((T * min(k, R), H), dtype=torch.int16, device="cuda"),
            xe=torch.zeros((T * k, H), dtype=torch.int16, device="cuda"),
            out=torch.zeros((T, H), dtype=torch.int16, device="cuda")))

    def run(p, stream):
        plan = ms.moe_shuffle_plan(p["dims"], p["idx"], p["ws"], stream=stream)
        ms.moe_shuffle_dispatch(plan, p["x"], p["xr"], p["xe"], stream=stream)
        ms.moe_shuffle_combine(plan, p["xe"], p["w"], p["out"], stream=stream)
        return plan

    want = []
    for p in problems:
        plan = run(p, None)
        torch.cuda.synchronize()
        n = ms.moe_shuffle_plan_query(plan)["N"]
        want.append((n, p["xr"][:n].clone(), p["xe"].clone(), p["out"].clone()))
        ms.moe_shuffle_plan_destroy(plan)
    for p in problems:
        for t in (p["xr"], p["xe"], p["out"]):
            t.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        plans = [run(p, s) for p, s in zip(problems, streams)]
        torch.cuda.synchronize()
        for p, plan, (n, xr, xe, out) in zip(problems, plans, want):
            assert ms.moe_shuffle_plan_query(plan)["N"] == n
            assert torch.equal(p["xr"][:n], xr) and torch.equal(p["xe"], xe) and torch.equal(p["out"], out)
            ms.moe_shuffle_plan_destroy(plan)
