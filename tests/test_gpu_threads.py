"""Host threads calling the library at once, each on a stream of its own
with its own workspace and buffers (the calls release the GIL, so the
library's host code really runs concurrently): every thread's results
equal the same batch run alone, bit for bit."""

import threading

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

SHAPES = [(1000, 1024, 64, 8, 8), (700, 2048, 32, 4, 4), (2048, 512, 128, 8, 16), (64, 7168, 256, 8, 32)]


def _run(ms, torch, case, stream):
    T, H, E, k, R, idx, x, w = case
    dev = torch.device("cuda:0")
    with torch.cuda.stream(stream):
        dims = ms.dims_of(T, H, E, k, R)
        ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device=dev)
        idx_d, x_d, w_d = idx.to(dev, non_blocking=False), x.to(dev), w.to(dev)
        xr = torch.empty((T * min(k, R), H), dtype=torch.int16, device=dev)
        xe = torch.empty((T * k, H), dtype=torch.int16, device=dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
        grad_x = torch.empty((T, H), dtype=torch.int16, device=dev)
        plan = ms.moe_shuffle_plan(dims, idx_d, ws, stream=stream)
        ms.moe_shuffle_dispatch(plan, x_d, xr, xe, stream=stream)
        ms.moe_shuffle_combine(plan, xe, w_d, out, stream=stream)
        ms.moe_shuffle_dispatch_backward(plan, xe, xr.clone(), grad_x, stream=stream)
        stream.synchronize()
        res = {"xe": xe.cpu(), "out": out.cpu(), "grad_x": grad_x.cpu()}
        ms.moe_shuffle_plan_destroy(plan)
    return res


def test_concurrent_host_threads_on_their_own_streams():
    import torch
    import moe_expert_token_amd as ms
    cases = []
    for i, (T, H, E, k, R) in enumerate(SHAPES):
        rng = np.random.default_rng(900 + i)
        idx, w = synth.random_routing(rng, T, E, k)
        x = synth.random_bf16(rng, (T, H))
        cases.append((T, H, E, k, R, torch.from_numpy(idx), torch.from_numpy(x.view(np.int16)),
                      torch.from_numpy(w)))
    alone = [_run(ms, torch, c, torch.cuda.Stream()) for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    got = [[None] * len(cases) for _ in range(3)]
    errors = []

    def worker(j):
        try:
            for rep in range(3):
                got[rep][j] = _run(ms, torch, cases[j], streams[j])
        except Exception as e:  # reported below, with the thread's case
            errors.append((j, repr(e)))

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for rep in range(3):
        for j in range(len(cases)):
            for key, ref in alone[j].items():
                assert torch.equal(got[rep][j][key], ref), f"case {SHAPES[j]} repetition {rep}: {key}"
