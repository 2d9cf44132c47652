"""Error behaviour of the C ABI on the device (MI355X)."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _setup(idx, H=64, E=8, R=4):
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    T, k = idx.shape
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    return ms, h, torch, dims, ws, plan


@pytest.mark.parametrize("bad", ["out_of_range", "negative", "duplicate"])
def test_bad_index_sets_status_and_blocks_writes(bad):
    rng = np.random.default_rng(1)
    idx, w = synth.random_routing(rng, 300, 8, 2)
    idx[137] = {"out_of_range": [1, 8], "negative": [-1, 3], "duplicate": [5, 5]}[bad]
    ms, h, torch, dims, ws, plan = _setup(idx)
    info = ms.moe_shuffle_plan_query(plan)
    assert info["status"] == ms.E_BAD_INDEX
    xr = torch.full((300 * 2, 64), h.SENTINEL, dtype=torch.int16, device="cuda")
    xe = torch.full((300 * 2, 64), h.SENTINEL, dtype=torch.int16, device="cuda")
    out = torch.full((300, 64), h.SENTINEL, dtype=torch.int16, device="cuda")
    x = h.to_dev16(synth.random_bf16(rng, (300, 64)))
    ms.moe_shuffle_dispatch(plan, x, xr, xe)
    ms.moe_shuffle_combine(plan, xe, torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    for t in (xr, xe, out):
        assert bool((t == h.SENTINEL).all())


def test_host_side_argument_errors():
    rng = np.random.default_rng(2)
    idx, w = synth.random_routing(rng, 100, 8, 2)
    ms, h, torch, dims, ws, plan = _setup(idx)
    x = h.to_dev16(synth.random_bf16(rng, (101, 64)))
    xr = torch.empty((200, 64), dtype=torch.int16, device="cuda")
    xe = torch.empty((200, 64), dtype=torch.int16, device="cuda")
    w_d = torch.from_numpy(w).cuda()
    out = torch.empty((100, 64), dtype=torch.int16, device="cuda")

    def code(f, *a):
        with pytest.raises(ms.MoeShuffleError) as e:
            f(*a)
        return e.value.code

    # one element (2 bytes) off a 16-byte boundary
    assert code(ms.moe_shuffle_dispatch, plan, x.view(-1)[1:], xr, xe) == ms.E_ALIGN
    assert code(ms.moe_shuffle_dispatch, plan, x, xr[:150], xe) == ms.E_INVALID_ARG      # xr below T*min(k,R)
    assert code(ms.moe_shuffle_dispatch, plan, x, xr, xr) == ms.E_INVALID_ARG           # xr overlaps xe
    assert code(ms.moe_shuffle_combine, plan, xe, w_d, xe) == ms.E_INVALID_ARG          # out overlaps ye
    assert code(ms.moe_shuffle_combine, plan, xe, w_d, out.view(-1)[4:]) == ms.E_ALIGN
    small = torch.empty(ws.numel() - 256, dtype=torch.uint8, device="cuda")
    assert code(ms.moe_shuffle_plan, dims, torch.from_numpy(idx).cuda(), small) == ms.E_WORKSPACE
    assert code(ms.moe_shuffle_plan, dims, torch.from_numpy(idx).cuda(), ws[16:]) == ms.E_ALIGN
    # after a query N is known, and xr may be sized exactly
    info = ms.moe_shuffle_plan_query(plan)
    ms.moe_shuffle_dispatch(plan, x[:100], xr[:info["N"]], xe)
    torch.cuda.synchronize()


def test_empty_plan_writes_zero_descriptors():
    ms, h, torch, dims, ws, plan = _setup(np.zeros((0, 2), np.int32))
    info = ms.moe_shuffle_plan_query(plan)
    assert info["status"] == 0 and info["N"] == 0
    v = ms.plan_array_views(plan, 0)
    assert int(v["expert_offset"].abs().sum()) == 0 and int(v["rank_offset"].abs().sum()) == 0
    np.testing.assert_array_equal(v["rank_segs"].cpu().numpy(), [[r, -1, 0, 0] for r in range(4)])
