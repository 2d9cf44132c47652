"""Token ranges (dispatch and combine per chunk of tokens, pipelined on two
streams) on the MI355X: the result equals the oracle's bit for bit."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def chunk_bounds(T, chunks, tile=256):
    b = sorted({min(T, -(-(i * T // chunks) // tile) * tile) for i in range(chunks)} | {T})
    return [0] + [x for x in b if x > 0]


def run_pipelined(idx, x, w, H, E, R, bounds):
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    T, k = idx.shape
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    xr = torch.full((T * min(k, R), H), h.SENTINEL, dtype=torch.int16, device="cuda")
    xe = torch.full((T * k, H), h.SENTINEL, dtype=torch.int16, device="cuda")
    out = torch.full((T, H), h.SENTINEL, dtype=torch.int16, device="cuda")
    x_d = h.to_dev16(x)
    w_d = torch.from_numpy(w).cuda()
    a = torch.cuda.current_stream()
    b = torch.cuda.Stream()
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        ms.moe_shuffle_dispatch_range(plan, x_d, xr, xe, t0, t1, stream=a)
        ev = torch.cuda.Event()
        ev.record(a)
        b.wait_event(ev)
        ms.moe_shuffle_combine_range(plan, xe, w_d, out, t0, t1, stream=b)
    a.wait_stream(b)
    N = ms.moe_shuffle_plan_query(plan)["N"]
    torch.cuda.synchronize()
    res = (h.to_host16(xr), h.to_host16(xe), h.to_host16(out), N)
    ms.moe_shuffle_plan_destroy(plan)
    return res


@pytest.mark.parametrize("cfg_id,chunks", [(0, 1), (1, 3), (2, 4), (3, 4), (4, 8)])
def test_pipelined_ranges_match_oracle(cfg_id, chunks):
    import gpu_harness as h
    import oracle
    cfg = synth.CONFIGS[cfg_id]
    inp = synth.make_inputs(cfg, 0)
    bounds = chunk_bounds(cfg.T, chunks)
    h.say(f"[pipe] {cfg.name} bounds {bounds}")
    xr, xe, out, N = run_pipelined(inp["topk_idx"], inp["x"], inp["topk_w"], cfg.H, cfg.E, cfg.R, bounds)
    orc = oracle.get()
    rc, o = orc.plan(inp["topk_idx"], cfg.H, cfg.E, cfg.R)
    assert o["N"] == N
    oxr, oxe = orc.dispatch(o, inp["x"], cfg.E, cfg.k, cfg.R)
    np.testing.assert_array_equal(xr[:N], oxr)
    assert np.all(xr[N:] == h.SENTINEL)
    np.testing.assert_array_equal(xe, oxe)
    np.testing.assert_array_equal(out, orc.combine(o["comb_row"], oxe, inp["topk_w"], cfg.E, cfg.R))


@pytest.mark.parametrize("T,H,E,k,R,bounds", [
    (1000, 1032, 32, 4, 8, [0, 256, 768, 1000]),
    (700, 7168, 256, 8, 32, [0, 512, 700]),
    (513, 264, 24, 24, 6, [0, 256, 512, 513]),
    (300, 96, 12, 3, 1, [0, 300]),
    (1000, 1032, 32, 4, 8, [0, 64, 192, 640, 1000]),   # ranges on the 64-token plan tile
    (130, 64, 16, 4, 4, [0, 64, 128, 130]),
    (300, 64, 56, 2, 8, [0, 128, 300]),                 # a plan made in one block (64 columns)
    (1000, 64, 8, 2, 4, [0, 448, 1000]),                # a plan made one block per tile (recount)
    (2500, 64, 8, 2, 8, [0, 1088, 2048, 2500]),         # recount with up to 3 tiles per wave
])
def test_ragged_ranges(T, H, E, k, R, bounds):
    import gpu_harness as h
    import oracle
    rng = np.random.default_rng(T + H + E)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    xr, xe, out, N = run_pipelined(idx, x, w, H, E, R, bounds)
    orc = oracle.get()
    rc, o = orc.plan(idx, H, E, R)
    oxr, oxe = orc.dispatch(o, x, E, k, R)
    np.testing.assert_array_equal(xr[:N], oxr)
    np.testing.assert_array_equal(xe, oxe)
    np.testing.assert_array_equal(out, orc.combine(o["comb_row"], oxe, w, E, R))


def test_range_arguments():
    import torch
    import moe_expert_token_amd as ms
    T, H, E, k, R = 600, 64, 8, 2, 4
    rng = np.random.default_rng(3)
    idx, w = synth.random_routing(rng, T, E, k)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    xr = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    xe = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    w_d = torch.from_numpy(w).cuda()
    for t0, t1 in [(100, 256), (0, 300), (256, 128), (0, 601), (-256, 0), (32, 64), (0, 96)]:
        with pytest.raises(ms.MoeShuffleError) as e:
            ms.moe_shuffle_dispatch_range(plan, x, xr, xe, t0, t1)
        assert e.value.code == ms.E_INVALID_ARG
        with pytest.raises(ms.MoeShuffleError) as e:
            ms.moe_shuffle_combine_range(plan, xe, w_d, out, t0, t1)
        assert e.value.code == ms.E_INVALID_ARG
    ms.moe_shuffle_dispatch_range(plan, x, xr, xe, 256, 256)   # empty range: nothing to do
    ms.moe_shuffle_dispatch_range(plan, x, xr, xe, 512, 600)   # up to T
    torch.cuda.synchronize()


def _random_ranges(n=10, seed=79):
    """Seeded shapes with random range boundaries on the 64-token tile."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        R = int(rng.choice([1, 2, 4, 8, 16]))
        E = R * int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, 3000))
        H = 8 * int(rng.integers(1, 200))
        cuts = sorted({64 * int(c) for c in rng.integers(1, max(2, -(-T // 64)), size=int(rng.integers(0, 6)))
                       if 64 * int(c) < T})
        cases.append((T, H, E, k, R, [0] + cuts + [T]))
    return cases


@pytest.mark.parametrize("T,H,E,k,R,bounds", _random_ranges())
def test_random_ranges(T, H, E, k, R, bounds):
    import oracle
    rng = np.random.default_rng(T + 3 * H + 5 * E + 7 * k + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    xr, xe, out, N = run_pipelined(idx, x, w, H, E, R, bounds)
    orc = oracle.get()
    rc, o = orc.plan(idx, H, E, R)
    oxr, oxe = orc.dispatch(o, x, E, k, R)
    np.testing.assert_array_equal(xr[:N], oxr)
    np.testing.assert_array_equal(xe, oxe)
    np.testing.assert_array_equal(out, orc.combine(o["comb_row"], oxe, w, E, R))
