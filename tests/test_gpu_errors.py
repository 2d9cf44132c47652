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


# Bad rows for every form of the plan: recount (one block per tile, each
# counting every tile again, a wave up to 3 tiles), one block of one wave
# per tile, and three launches (count, scan, place), where the status
# travels from the count kernel's error column through the scan to the
# place kernel's early exit.
BAD_CASES = [
    # name, T, E, k, R, rows made bad
    ("recount", 300, 8, 2, 4, (137,)),
    ("recount-last-tile", 1024, 8, 2, 4, (1023,)),             # 16 tiles, the bad row in the last
    ("recount-first-tile", 1024, 8, 2, 4, (0,)),               # ... and in tile 0
    ("recount-topk12", 500, 12, 12, 4, (499,)),                # 16 ids per lane
    ("one-block", 300, 56, 2, 8, (137,)),                      # 64 columns, 64 + 6 > 66
    ("one-block-last-tile", 512, 56, 4, 8, (511,)),            # 8 tiles x top-4
    ("recount-second-trip", 1100, 8, 2, 4, (1050,)),           # 18 tiles, the bad row in tile 16 (wave 0's second)
    ("recount-last-trip", 3072, 8, 2, 4, (3071,)),             # 48 tiles, the bad row in wave 15's third
    ("recount-trips-topk8", 1100, 8, 8, 1, (1099,)),           # 18 tiles at top-8, the bad row in the last
    ("three-launch", 1100, 32, 2, 8, (1050,)),                 # 18 tiles x 40 columns, the bad row in tile 16
    ("three-launch-last-tile", 4096, 8, 2, 4, (4095,)),        # 64 tiles, the bad row in the last
    ("three-launch-first-tile", 4096, 8, 2, 4, (0,)),          # ... and in tile 0
    ("three-launch-topk17-first", 500, 32, 17, 4, (3,)),       # top-17, the bad row in tile 0
    ("three-launch-topk17-last", 500, 32, 17, 4, (499,)),      # ... and in the last, ragged tile
    ("three-launch-mid-size", 4200, 8, 2, 4, (4150,)),         # 66 tiles, the bad row in tile 64
    ("three-launch-wide", 1100, 960, 2, 64, (5,)),             # 18 tiles x 1024 columns
]

WS_FILL = 0x5A  # workspace bytes before the plan: index arrays must keep them


@pytest.mark.parametrize("form,T,E,k,R,rows", BAD_CASES)
@pytest.mark.parametrize("bad", ["out_of_range", "negative", "duplicate"])
def test_bad_index_sets_status_and_blocks_writes(form, T, E, k, R, rows, bad):
    import torch
    import moe_expert_token_amd as ms
    import gpu_harness as h
    rng = np.random.default_rng(T + k)
    H = 64
    idx, w = synth.random_routing(rng, T, E, k)
    for r in rows:
        if bad == "out_of_range":
            idx[r, k - 1] = E
        elif bad == "negative":
            idx[r, 0] = -1
        else:
            idx[r, k - 1] = idx[r, 0]
    h.say(f"[errors] bad ids ({bad}) in rows {rows}, {form}: T={T} E={E} k={k} R={R}")
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.full((ms.moe_shuffle_workspace_size(dims),), WS_FILL, dtype=torch.uint8, device="cuda")
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    info = ms.moe_shuffle_plan_query(plan)
    assert info["status"] == ms.E_BAD_INDEX
    KR = min(k, R)
    xr = torch.full((T * KR, H), h.SENTINEL, dtype=torch.int16, device="cuda")
    xe = torch.full((T * k, H), h.SENTINEL, dtype=torch.int16, device="cuda")
    out = torch.full((T, H), h.SENTINEL, dtype=torch.int16, device="cuda")
    x = h.to_dev16(synth.random_bf16(rng, (T, H)))
    ms.moe_shuffle_dispatch(plan, x, xr, xe)
    ms.moe_shuffle_combine(plan, xe, torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    for t in (xr, xe, out):
        assert bool((t == h.SENTINEL).all())
    # the place step wrote no row index either
    fill = int(np.array([WS_FILL] * 4, np.uint8).view(np.int32)[0])
    v = ms.plan_array_views(plan, T * KR)
    for key in ("comb_row", "fan_dst", "fan_src", "send_token", "tok_rank_row", "expert_offset", "rank_offset"):
        assert bool((v[key] == fill).all()), f"{key} was written"
    ms.moe_shuffle_plan_destroy(plan)


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
