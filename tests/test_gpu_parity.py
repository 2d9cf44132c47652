"""HIP path vs the oracle through the C ABI, on the MI355X.

Bar: plan arrays, segment descriptors, xr[0:N] and xe bit-exact; combine
within 1 bf16 ulp (0 expected: both sides run the same fp32 fma chain);
rank rows past N left untouched."""

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


def harness():
    import gpu_harness
    return gpu_harness


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_config_full_size(cfg_id):
    """Every workload at full size, in the launch configuration the bench times:
    plan + dispatch bit-exact, combine of random expert outputs and the
    identity-expert round trip."""
    cfg = synth.CONFIGS[cfg_id]
    inp = synth.make_inputs(cfg, 0)
    ye = synth.make_expert_outputs(cfg, 0)
    h = harness()
    # the bench's launch configuration: no host sync, fan-out grid on the bound
    g, o = h.check_case(inp["topk_idx"], inp["x"], inp["topk_w"], cfg.H, cfg.E, cfg.R, ye=ye, name=cfg.name,
                        query_first=False)
    # the round trip returns x (with -0 read as +0)
    np.testing.assert_array_equal(g["out_rt"], np.where(inp["x"] == 0x8000, 0, inp["x"]).astype(np.uint16))
    # after a query the fan-out grid is the exact N: the same bits
    q = h.run_hip(inp["topk_idx"], inp["x"], inp["topk_w"], cfg.H, cfg.E, cfg.R, ye, query_first=True)
    for key in ("xr", "xe", "out", "out_rt"):
        np.testing.assert_array_equal(q[key], g[key], err_msg=key)


RAGGED = [
    # T, H, E, k, R
    (0, 64, 8, 2, 4),         # empty
    (1, 8, 8, 2, 4),          # one token, one 16-byte vector per row
    (63, 136, 8, 3, 4),       # ragged tile, ragged row (17 vectors)
    (64, 1024, 16, 4, 8),
    (65, 1032, 16, 4, 4),     # 129 vectors: more than one lane pass, ragged
    (255, 512, 32, 8, 8),
    (256, 2048, 32, 8, 32),   # one expert per rank: no dedup
    (257, 7168, 64, 6, 16),
    (700, 1152, 48, 5, 3),    # 16 experts per rank, wider than k
    (1000, 16384, 8, 2, 2),   # long rows: two chunks per row
    (513, 264, 24, 24, 6),    # k == E: every token to every rank (all-gather)
    (300, 96, 12, 3, 1),      # a single rank
    (129, 128, 1024 - 64, 8, 64),  # the largest histogram (E + R = 1024)
    (77, 64, 128, 64, 8),     # the largest top-k
    (333, 64, 16, 1, 4),      # top-1: one expert row per token, combine is a scaled copy
    (50, 32, 1, 1, 1),        # a single expert on a single rank
]


@pytest.mark.parametrize("T,H,E,k,R", RAGGED)
def test_ragged_and_edge_shapes(T, H, E, k, R):
    rng = np.random.default_rng(T * 7919 + H * 31 + E * 7 + k + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    ye = synth.wide_bf16(rng, (T * k, H))
    harness().check_case(idx, x, w, H, E, R, ye=ye, name=f"ragged-{T}x{H}")


# Either side of the limits of the three plan forms, which must all give
# the oracle's arrays bit for bit:
# - recount: one block per tile, each block counting every tile again; at
#   most 48 tiles of 64 tokens (up to 3 per wave of 16), E + R <= 64, top-k
#   <= 16 up to 16 tiles and <= 8 above, trips x (E + R + 3k) <= 66;
# - one block, one wave per tile: at most 16 tiles, 48 KiB of LDS, top-k
#   <= 16, tiles x top-k <= 32;
# - three launches (count, scan, place): everything else.
PLAN_FORMS = [
    # T, H, E, k, R
    (1024, 64, 32, 8, 8),       # 16 tiles x 40 columns, 40 + 24 = 64: recount
    (1024, 64, 32, 9, 8),       # 40 + 27 > 66, 144 slots: three launches
    (1025, 64, 8, 2, 8),        # 17 tiles x 16 columns, 2 x 22: recount, wave 0 counts tiles 0 and 16
    (2048, 64, 16, 2, 8),       # 32 tiles, 2 x 30: recount
    (2048, 64, 20, 2, 10),      # 32 tiles, 2 x 36 > 66: three launches
    (3000, 64, 8, 2, 8),        # 47 tiles, 3 x 22: recount, waves with 2 and 3 tiles
    (3072, 64, 8, 2, 8),        # 48 tiles: recount, 3 tiles per wave
    (3073, 64, 8, 2, 8),        # 49 tiles: three launches
    (1100, 64, 8, 8, 1),        # 18 tiles at top-8 of 8 experts, 2 x 33: recount, 8 ids per lane in two 16-byte loads
    (2500, 64, 8, 4, 2),        # 40 tiles at top-4, 3 x 22: recount
    (500, 64, 12, 12, 4),       # top-12, 16 + 36 <= 66: recount with 16 ids per lane
    (1025, 64, 32, 8, 8),       # 17 tiles: three launches
    (256, 64, 56, 2, 8),        # 4 tiles x 64 columns, 64 + 6 > 66: one block
    (512, 64, 56, 4, 8),        # 8 tiles x top-4 = 32 slots: one block
    (576, 64, 56, 4, 8),        # 9 tiles x top-4 = 36 slots: three launches
    (500, 64, 16, 16, 4),       # top-16, 8 x 16 slots: three launches
    (2000, 64, 32, 8, 8),       # 32 tiles, ragged last tile: three launches
    (4096, 64, 8, 2, 8),        # 64 tiles (the Mixtral-like shape): three launches
    (4096, 64, 56, 8, 8),       # 64 tiles x 64 columns: three launches
    (128, 64, 1024 - 64, 8, 64),  # 2 tiles x 1024 columns, 36 KiB of LDS: one block
    (129, 64, 1024 - 64, 8, 64),  # 3 tiles, 52 KiB: three launches
    (500, 64, 64, 17, 8),       # top-17: three launches
    (4200, 64, 32, 17, 8),      # top-17, 66 tiles: three launches
]


@pytest.mark.parametrize("T,H,E,k,R", PLAN_FORMS)
def test_both_plan_forms(T, H, E, k, R):
    rng = np.random.default_rng(T * 17 + E + k)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    harness().check_case(idx, x, w, H, E, R, name=f"plan-form-{T}-{E}-{k}")


# The plan reads a row of 4n (2n) ids 16 (8) bytes at a time when the ids
# start on such a boundary, else one id at a time: ids placed 4 and 8 bytes
# past a boundary, through every plan form, give the oracle's arrays too.
ID_ALIGN = [
    # T, E, k, R, shift in int32
    (300, 16, 8, 4, 1), (300, 16, 8, 4, 2), (300, 16, 2, 4, 1),       # recount
    (300, 56, 4, 8, 1), (300, 56, 2, 8, 1),                           # one block
    (3000, 16, 8, 4, 1), (3000, 16, 8, 4, 2), (3000, 16, 2, 4, 1),    # three launches
    (5000, 64, 8, 8, 1), (5000, 64, 12, 8, 2), (5000, 64, 2, 8, 1),   # three launches
]


@pytest.mark.parametrize("T,E,k,R,shift", ID_ALIGN)
def test_ids_off_the_vector_boundary(T, E, k, R, shift):
    rng = np.random.default_rng(T * 3 + E + k * 5 + shift)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, 64))
    harness().check_case(idx, x, w, 64, E, R, name=f"id-align-{T}-{E}-{k}+{shift}", idx_shift=shift)


def _plan_form_shapes(n=40, seed=91):
    """Seeded shapes around the plan forms' limits: up to 18 tiles, top-k up
    to 20, histograms up to 1024 columns; then 16 to 66 tiles at top-k up to
    10 and up to 160 columns."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        R = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        E = R * int(rng.integers(1, 17))
        if E + R > 1024:
            continue
        k = int(rng.integers(1, min(E, 20) + 1))
        shapes.append((int(rng.integers(0, 18 * 64 + 1)), 8 * int(rng.integers(1, 40)), E, k, R))
    while len(shapes) < n + n // 2:
        R = int(rng.choice([1, 2, 4, 8, 16]))
        E = R * int(rng.integers(1, 9))
        if E + R > 160:
            continue
        k = int(rng.integers(1, min(E, 10) + 1))
        shapes.append((int(rng.integers(16 * 64, 66 * 64 + 1)), 8 * int(rng.integers(1, 20)), E, k, R))
    return shapes


@pytest.mark.parametrize("T,H,E,k,R", _plan_form_shapes())
def test_random_shapes_around_plan_forms(T, H, E, k, R):
    rng = np.random.default_rng(T * 13 + H * 5 + E * 3 + k + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    harness().check_case(idx, x, w, H, E, R, name=f"plan-rand-{T}-{E}-{k}", query_first=bool(T % 2))


def test_all_tokens_one_expert_skew():
    """Every token picks expert 0 first: one segment holds all T rows."""
    rng = np.random.default_rng(5)
    T, H, E, k, R = 3000, 256, 64, 4, 16
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        idx[t, 0] = 0
        idx[t, 1:] = 1 + rng.choice(E - 1, size=k - 1, replace=False)
    w = rng.random((T, k)).astype(np.float32)
    x = synth.random_bf16(rng, (T, H))
    harness().check_case(idx, x, w, H, E, R, name="one-hot-expert")


def test_all_experts_on_one_rank():
    """Every token sends to one rank only: N = T, an eighth of the host-side
    bound T*min(k,R), so most blocks of the fan-out grid find no row."""
    rng = np.random.default_rng(8)
    T, H, E, k, R = 1000, 520, 64, 8, 8
    epr = E // R
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        r = rng.integers(R)
        idx[t] = r * epr + rng.permutation(epr)[:k]
    w = rng.random((T, k)).astype(np.float32)
    x = synth.random_bf16(rng, (T, H))
    g, o = harness().check_case(idx, x, w, H, E, R, name="one-rank-per-token")
    assert o["N"] == T


def test_plan_without_query_uses_upper_bound():
    """Dispatch sized by T*min(k,R) without a host sync gives the same bits."""
    h = harness()
    rng = np.random.default_rng(6)
    T, H, E, k, R = 900, 256, 32, 4, 8
    idx, w = synth.random_routing(rng, T, E, k)
    x = synth.random_bf16(rng, (T, H))
    a = h.run_hip(idx, x, w, H, E, R, query_first=False)
    b = h.run_hip(idx, x, w, H, E, R, query_first=True)
    for key in ("send_token", "fan_dst", "comb_row"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(a["xr"], b["xr"])
    np.testing.assert_array_equal(a["xe"], b["xe"])
    np.testing.assert_array_equal(a["out"], b["out"])


def test_repeat_runs_bitwise_identical():
    """No result depends on scheduling: ten runs of the whole skewed workload
    (16384 tokens, H = 7168, 64 ranks) in the bench's launch configuration
    (no host sync, fan-out grid on the bound) give the same plan arrays, xr,
    xe and out bit for bit; compared on the device."""
    import torch
    import moe_expert_token_amd as ms
    h = harness()
    cfg = synth.CONFIGS[3]
    inp = synth.make_inputs(cfg, 0)
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    KR = min(k, R)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    x = h.to_dev16(inp["x"])
    w = torch.from_numpy(inp["topk_w"]).cuda()
    xr = torch.empty((T * KR, H), dtype=torch.int16, device="cuda")
    xe = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ref = None
    for rep in range(10):
        xr.fill_(h.SENTINEL)
        xe.fill_(h.SENTINEL)
        out.fill_(h.SENTINEL)
        ws.fill_(0x5A)
        plan = ms.moe_shuffle_plan(dims, idx, ws)
        ms.moe_shuffle_dispatch_send(plan, x, xr)
        ms.moe_shuffle_dispatch_fanout(plan, xr, xe)
        ms.moe_shuffle_combine(plan, xe, w, out)
        N = ms.moe_shuffle_plan_query(plan)["N"]
        v = ms.plan_array_views(plan, N)
        got = {key: v[key].clone() for key in h.PLAN_KEYS}
        got.update(xr=xr[:N].clone(), xe=xe.clone(), out=out.clone())
        ms.moe_shuffle_plan_destroy(plan)
        if ref is None:
            ref = got
            continue
        for key, t in got.items():
            assert torch.equal(t, ref[key]), f"run {rep}: {key} differs from run 0"
    h.say(f"[determinism] 10 runs of {cfg.name} identical (N={N})")


def _random_shapes(n=24, seed=77):
    """Seeded shapes inside the limits: H a multiple of 8, R dividing E,
    k <= min(E, 64), E + R <= 1024."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        R = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
        E = R * int(rng.integers(1, 17))
        if E + R > 1024:
            continue
        k = int(rng.integers(1, min(E, 64) + 1))
        T = int(rng.integers(0, 2500))
        H = 8 * int(rng.integers(1, 300))
        shapes.append((T, H, E, k, R))
    return shapes


@pytest.mark.parametrize("T,H,E,k,R", _random_shapes())
def test_random_shapes(T, H, E, k, R):
    rng = np.random.default_rng(T * 31 + H * 7 + E * 3 + k + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    x = synth.random_bf16(rng, (T, H))
    ye = synth.wide_bf16(rng, (T * k, H))
    harness().check_case(idx, x, w, H, E, R, ye=ye, name=f"random-{T}x{H}", query_first=bool(T % 2))


def test_largest_batch_against_oracle_plan_and_properties():
    """A batch four times the largest workload's rows (262144 tokens, H = 7168,
    256 experts, top-8, 32 ranks: xr and xe 30 GB each), in the bench's launch
    configuration.  The plan is compared bit for bit with the oracle's; the
    row buffers, too large to copy out, are checked on the device against
    what the oracle's plan says each row holds (xr[p] = x[send_token[p]],
    xe[q] = x[token of q]); the identity-expert round trip returns x."""
    import torch
    import moe_expert_token_amd as ms
    import oracle
    T, H, E, k, R = 262144, 7168, 256, 8, 32
    rng = np.random.default_rng(262144)
    idx, w = synth.random_routing(rng, T, E, k)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    xr = torch.empty((T * min(k, R), H), dtype=torch.int16, device="cuda")
    xe = torch.empty((T * k, H), dtype=torch.int16, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    w_d = torch.from_numpy(w).cuda()
    plan = ms.moe_shuffle_plan(dims, torch.from_numpy(idx).cuda(), ws)
    ms.moe_shuffle_dispatch_send(plan, x, xr)
    ms.moe_shuffle_dispatch_fanout(plan, xr, xe)
    ms.moe_shuffle_combine(plan, xe, w_d, out)
    N = ms.moe_shuffle_plan_query(plan)["N"]
    torch.cuda.synchronize()
    rc, o = oracle.get().plan(idx, H, E, R)
    assert rc == 0 and o["N"] == N
    v = ms.plan_array_views(plan, N)
    for key in ("send_token", "tok_rank_row", "fan_src", "fan_dst", "comb_row", "expert_offset", "rank_offset"):
        np.testing.assert_array_equal(v[key].cpu().numpy(), o[key], err_msg=key)
    send_token = torch.from_numpy(o["send_token"].astype(np.int64)).cuda()
    tok_of_q = send_token[torch.from_numpy(o["fan_src"].astype(np.int64)).cuda()]
    step = 32768
    for p0 in range(0, N, step):
        p1 = min(N, p0 + step)
        assert torch.equal(xr[p0:p1], x[send_token[p0:p1]]), f"xr rows {p0}..{p1}"
    for q0 in range(0, T * k, step):
        q1 = min(T * k, q0 + step)
        assert torch.equal(xe[q0:q1], x[tok_of_q[q0:q1]]), f"xe rows {q0}..{q1}"
    assert torch.equal(out, torch.where(x == -32768, torch.zeros_like(x), x)), "round trip"
    ms.moe_shuffle_plan_destroy(plan)


def test_row_count_at_the_int32_limit_closed_form():
    """The largest batch the index limit admits: H = 8 (one 16-byte vector
    per row), E = R = 8 and k = 8, so every token reaches every rank and
    rank r's segment is the tokens in order, r * T + t; with T = 2^28 - 69
    the fan-out has T * k = 2^31 - 552 units, within 512 of the int32 unit
    limit (T * k * ceil(H / 512) + 64 < 2^31).  The plan is the definition
    written out for this case (rows ascending by token inside every
    segment), the row buffers are x repeated, and with gates 1/8 the
    combine returns x exactly (-0 read as +0); the training direction on
    the same plan, the token ranges and the rank-partial combines have
    closed forms too (below).  About 210 GiB of device memory at the peak;
    everything is checked on the device in slices."""
    import torch
    import moe_expert_token_amd as ms
    T, H, E, k, R = (1 << 28) - 69, 8, 8, 8, 8
    assert (1 << 31) - 1024 < T * k + 64 < (1 << 31)  # at the limit the host check enforces
    dev = torch.device("cuda:0")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()  # blocks cached by earlier tests count as free here
    free, _ = torch.cuda.mem_get_info(dev)
    if free < (215 << 30):
        pytest.skip(f"needs about 210 GiB of free device memory, {free / 2**30:.0f} GiB free")
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device=dev)
    t_all = torch.arange(T, dtype=torch.int32, device=dev)
    # token t names experts (t + j) mod 8, j = 0..7: distinct in every row
    idx = ((t_all[:, None] + torch.arange(k, dtype=torch.int32, device=dev)[None, :]) % E).contiguous()
    w = torch.full((T, k), 0.125, dtype=torch.float32, device=dev)
    gen = torch.Generator(device="cuda").manual_seed(31)
    x = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    xr = torch.empty((T * R, H), dtype=torch.int16, device=dev)
    xe = torch.empty((T * k, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    h = harness()
    h.say(f"[int32-limit] T={T} H={H} E={E} k={k} R={R}: plan, dispatch, combine")
    plan = ms.moe_shuffle_plan(dims, idx, ws)
    ms.moe_shuffle_dispatch(plan, x, xr, xe)
    ms.moe_shuffle_combine(plan, xe, w, out)
    assert ms.moe_shuffle_plan_query(plan)["N"] == T * R
    v = ms.plan_array_views(plan, T * R)
    seg = torch.arange(R + 1, dtype=torch.int64, device=dev) * T
    assert torch.equal(v["rank_offset"].long(), seg) and torch.equal(v["expert_offset"].long(), seg)
    step = 1 << 25
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        tt = t_all[t0:t1]
        rows = tt[:, None].long() + seg[None, :R]                  # rank (= expert) r's row of token t
        assert torch.equal(v["tok_rank_row"][t0:t1].long(), rows), f"tok_rank_row {t0}"
        assert torch.equal(v["comb_row"][t0:t1].long(), idx[t0:t1].long() * T + tt[:, None].long()), \
            f"comb_row {t0}"
        ref = torch.where(x[t0:t1] == -32768, torch.zeros_like(x[t0:t1]), x[t0:t1])
        assert torch.equal(out[t0:t1], ref), f"out {t0}"
        for r in range(R):
            p0 = r * T
            assert torch.equal(v["send_token"][p0 + t0:p0 + t1], tt), f"send_token rank {r} at {t0}"
            assert torch.equal(v["fan_src"][p0 + t0:p0 + t1].long(), tt.long() + p0), f"fan_src {r} at {t0}"
            assert torch.equal(xr[p0 + t0:p0 + t1], x[t0:t1]), f"xr rank {r} at {t0}"
            assert torch.equal(xe[p0 + t0:p0 + t1], x[t0:t1]), f"xe expert {r} at {t0}"
    h.say("[int32-limit] plan, xr, xe and out as the closed form gives; now the training direction")

    # Training direction on the same plan, with xe (x[t] in all 8 expert
    # rows of t) as both grad_xe and ye and x as grad_out: the receiver sum
    # of a rank row is its one expert row (x[t]), the sender sum of token t
    # is 8 x[t] (exact), grad_ye = bf16(x[t] / 8) (exact) and grad_w[t][j]
    # = sum_h x[t][h]^2 summed in fp32.
    xr.fill_(0x7F7F)
    out.fill_(0x7F7F)
    ms.moe_shuffle_dispatch_backward(plan, xe, xr, out)
    gye = torch.empty((T * k, H), dtype=torch.int16, device=dev)
    gw = torch.empty((T, k), dtype=torch.float32, device=dev)
    ms.moe_shuffle_combine_backward(plan, x, xe, w, gye, gw)
    torch.cuda.synchronize()
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        xs = x[t0:t1]
        x0 = torch.where(xs == -32768, torch.zeros_like(xs), xs)   # fma(1, -0, +0) = +0
        xf = xs.view(torch.bfloat16).float()
        eight = torch.where(xs == -32768, torch.zeros_like(xs), (xf * 8).to(torch.bfloat16).view(torch.int16))
        eighth = (xf * 0.125).to(torch.bfloat16).view(torch.int16)
        assert torch.equal(out[t0:t1], eight), f"grad_x {t0}"
        ss = (xf.double() ** 2).sum(1, keepdim=True)
        assert bool(((gw[t0:t1].double() - ss).abs() <= 1e-6 * ss + 1e-30).all()), f"grad_w {t0}"
        for r in range(R):
            p0 = r * T
            assert torch.equal(xr[p0 + t0:p0 + t1], x0), f"grad_xr rank {r} at {t0}"
            assert torch.equal(gye[p0 + t0:p0 + t1], eighth), f"grad_ye expert {r} at {t0}"
    h.say("[int32-limit] grad_xr, grad_x, grad_ye and grad_w as the closed form gives; now two token ranges")

    # The token-range calls over [0, cut) and [cut, T) give the forward
    # closed form again.
    del gye, gw
    cut = (T // 128) * 64
    for buf in (xr, xe, out):
        buf.fill_(0x7F7F)
    for t0, t1 in ((0, cut), (cut, T)):
        ms.moe_shuffle_dispatch_range(plan, x, xr, xe, t0, t1)
        ms.moe_shuffle_combine_range(plan, xe, w, out, t0, t1)
    torch.cuda.synchronize()
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        ref = torch.where(x[t0:t1] == -32768, torch.zeros_like(x[t0:t1]), x[t0:t1])
        assert torch.equal(out[t0:t1], ref), f"range out {t0}"
        for r in range(R):
            p0 = r * T
            assert torch.equal(xr[p0 + t0:p0 + t1], x[t0:t1]), f"range xr rank {r} at {t0}"
            assert torch.equal(xe[p0 + t0:p0 + t1], x[t0:t1]), f"range xe expert {r} at {t0}"
    h.say("[int32-limit] token ranges as the closed form gives; now the rank-partial combines")

    # Rank-partial combine (xe as ye): each rank row's partial is its one
    # expert row times 1/8, exact in bf16 and in fp32, and out is x again.
    p32 = torch.empty((T * R, H), dtype=torch.float32, device=dev)
    for f32 in (False, True):
        xr.fill_(0x7F7F)
        out.fill_(0x7F7F)
        if f32:
            ms.moe_shuffle_combine_rank_partial_f32(plan, xe, w, p32, out)
        else:
            ms.moe_shuffle_combine_rank_partial(plan, xe, w, xr, out)
        torch.cuda.synchronize()
        for t0 in range(0, T, step):
            t1 = min(T, t0 + step)
            xs = x[t0:t1]
            ref = torch.where(xs == -32768, torch.zeros_like(xs), xs)
            assert torch.equal(out[t0:t1], ref), f"rank-partial (fp32 {f32}) out {t0}"
            eighth = xs.view(torch.bfloat16).float() * 0.125
            for r in range(R):
                p0 = r * T
                if f32:
                    got = p32[p0 + t0:p0 + t1]
                    assert torch.equal(got, eighth + 0.0), f"fp32 partial rank {r} at {t0}"  # -0 -> +0
                else:
                    want = torch.where(xs == -32768, torch.zeros_like(xs), eighth.to(torch.bfloat16).view(torch.int16))
                    assert torch.equal(xr[p0 + t0:p0 + t1], want), f"partial rank {r} at {t0}"
    ms.moe_shuffle_plan_destroy(plan)
    h.say("[int32-limit] rank-partial combines as the closed form gives")
    del ws, idx, w, x, xr, xe, out, t_all, v, p32
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
