"""The library driven from C on the GPU (tests/c/abi_gpu_drive.c): HIP
allocations made by a C program, the default stream, no PyTorch.  The hand
fixture of the DySHARP write-up's Fig. 3 (tests/golden) must come out
exactly, and a random batch must match the oracle bit for bit."""

import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests"))

import c_driver  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu

FIXTURE = os.path.join(ROOT, "tests", "golden", "fig3_two_tokens.json")


def _bits(values):
    """bf16 bits of float32 values that are exact in bf16."""
    u = np.asarray(values, np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any()
    return (u >> 16).astype(np.uint16)


def _check_plan(got, exp, T, k):
    for key in ("expert_count", "expert_offset", "rank_count", "rank_offset", "send_token", "fan_src"):
        np.testing.assert_array_equal(got[key], np.asarray(exp[key]).ravel(), err_msg=key)
    for key in ("tok_rank_row", "comb_row", "fan_dst", "rank_segs", "expert_segs"):
        np.testing.assert_array_equal(got[key], np.asarray(exp[key]).ravel(), err_msg=key)


def test_fig3_fixture_from_c():
    fx = json.load(open(FIXTURE))
    d, exp, cb = fx["dims"], fx["expected"], fx["combine"]
    T, H, E, k, R = d["T"], d["H"], d["E"], d["k"], d["R"]
    x = np.asarray(cb["x"], np.float32)
    w = np.asarray(cb["topk_w"], np.float32)
    # identity expert: the gates sum to 1, so out = x
    got = c_driver.run(T, H, E, k, R, fx["topk_idx"], x, w)
    assert got["returncode"] == 0, (got.get("ERROR"), got["stderr"])
    assert got["status"][0] == 0 and got["N"][0] == exp["N"]
    _check_plan(got, exp, T, k)
    np.testing.assert_array_equal(got["xr"].reshape(-1, H), x[exp["xr_token_of_row"]])
    np.testing.assert_array_equal(got["xe"].reshape(-1, H), x[exp["xe_token_of_row"]])
    np.testing.assert_array_equal(got["out"].reshape(T, H), x)
    # expert outputs ye[q] = (q + 1) * c give the fixture's combine values
    c = np.asarray(cb["c"], np.float32)
    ye = np.arange(1, T * k + 1, dtype=np.float32)[:, None] * c[None, :]
    got = c_driver.run(T, H, E, k, R, fx["topk_idx"], x, w, ye=ye)
    assert got["returncode"] == 0, (got.get("ERROR"), got["stderr"])
    np.testing.assert_array_equal(got["out"].reshape(T, H), np.asarray(cb["out_with_ye_scaled_c"], np.float32))


@pytest.mark.parametrize("T,H,E,k,R", [(300, 136, 16, 4, 4), (1100, 64, 32, 8, 8)])
def test_random_batch_from_c_matches_the_oracle(T, H, E, k, R):
    import oracle
    rng = np.random.default_rng(T + H)
    idx, w = synth.random_routing(rng, T, E, k)
    xb = synth.random_bf16(rng, (T, H))
    x = (xb.astype(np.uint32) << 16).view(np.float32)
    got = c_driver.run(T, H, E, k, R, idx, x, w)
    assert got["returncode"] == 0, (got.get("ERROR"), got["stderr"])
    orc = oracle.get()
    rc, o = orc.plan(idx, H, E, R)
    assert rc == 0 and got["status"][0] == 0 and got["N"][0] == o["N"]
    for key in ("expert_count", "expert_offset", "rank_count", "rank_offset", "send_token", "tok_rank_row",
                "fan_src", "fan_dst", "comb_row"):
        np.testing.assert_array_equal(got[key], np.asarray(o[key]).ravel(), err_msg=key)
    oxr, oxe = orc.dispatch(o, xb, E, k, R)
    np.testing.assert_array_equal(_bits(got["xr"]), oxr.ravel())
    np.testing.assert_array_equal(_bits(got["xe"]), oxe.ravel())
    oout = orc.combine(o["comb_row"], oxe, w, E, R)
    np.testing.assert_array_equal(_bits(got["out"]), oout.ravel())
