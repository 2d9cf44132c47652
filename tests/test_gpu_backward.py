"""Training direction and the deduplicated return path on the MI355X:
dispatch backward, rank-partial combine, combine backward vs the oracle."""

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


def _h():
    import gpu_harness
    return gpu_harness


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_backward_config_full_size(cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    idx, w = synth.make_routing(cfg, 0)
    ye = synth.make_expert_outputs(cfg, 0)
    rng = np.random.default_rng(1000 + cfg_id)
    grad_xe = synth.wide_bf16(rng, (cfg.T * cfg.k, cfg.H), -8, 8)
    grad_out = synth.wide_bf16(rng, (cfg.T, cfg.H), -8, 8)
    _h().check_backward_case(idx, w, cfg.H, cfg.E, cfg.R, ye, grad_xe, grad_out, name=cfg.name)


@pytest.mark.parametrize("T,H,E,k,R", [
    (0, 64, 8, 2, 4), (1, 8, 8, 2, 4), (63, 136, 8, 3, 4), (65, 1032, 16, 4, 4), (300, 96, 12, 3, 1),
    (257, 7168, 64, 6, 16), (513, 264, 24, 24, 6), (77, 64, 128, 64, 8), (200, 2048, 32, 8, 32),
    (333, 64, 16, 1, 4), (50, 32, 1, 1, 1),
])
def test_backward_ragged_shapes(T, H, E, k, R):
    rng = np.random.default_rng(T * 31 + H + E * 3 + k * 5 + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    ye = synth.wide_bf16(rng, (T * k, H), -10, 10)
    grad_xe = synth.wide_bf16(rng, (T * k, H), -10, 10)
    grad_out = synth.wide_bf16(rng, (T, H), -10, 10)
    _h().check_backward_case(idx, w, H, E, R, ye, grad_xe, grad_out, name=f"ragged-{T}x{H}")


def _random_shapes(n=12, seed=78):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        R = int(rng.choice([1, 2, 4, 8, 16, 32]))
        E = R * int(rng.integers(1, 17))
        if E + R > 1024:
            continue
        k = int(rng.integers(1, min(E, 64) + 1))
        shapes.append((int(rng.integers(1, 1500)), 8 * int(rng.integers(1, 260)), E, k, R))
    return shapes


@pytest.mark.parametrize("T,H,E,k,R", _random_shapes())
def test_backward_random_shapes(T, H, E, k, R):
    rng = np.random.default_rng(T * 13 + H + E * 5 + k * 3 + R)
    idx, w = synth.random_routing(rng, T, E, k, signed_gates=True)
    ye = synth.wide_bf16(rng, (T * k, H), -8, 8)
    grad_xe = synth.wide_bf16(rng, (T * k, H), -8, 8)
    grad_out = synth.wide_bf16(rng, (T, H), -8, 8)
    _h().check_backward_case(idx, w, H, E, R, ye, grad_xe, grad_out, name=f"random-{T}x{H}")
