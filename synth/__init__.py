"""Seeded synthetic inputs for the MoE token shuffle.

This module is the only code shared by the oracle side and the HIP side of
the tests and the bench: it draws inputs and holds none of the shuffle's own
arithmetic (no counting, placement, copying or reduction of rows).

Workloads (no page prints routing draws, so these stand in for the pages'
benchmarks; the shapes follow the MoE models the pages evaluate):

  0  tiny:      T=256,   H=128,  E=8,   k=2, R=4   softmax router
  1  Mixtral:   T=4096,  H=4096, E=8,   k=2, R=8   softmax router
  2  DeepSeek:  T=8192,  H=7168, E=256, k=8, R=32  sigmoid, 8 groups, top-4 groups
  3  skewed:    T=16384, H=7168, E=256, k=8, R=64  softmax over logits + ln Zipf(1.2)
  4  prefill:   T=65536, H=4096, E=128, k=8, R=16  softmax router

Recipe (identical for every consumer):
  * ``SeedSequence(seed).spawn(2)`` gives two PCG64 streams, one for the
    activations and one for the router.
  * activations: standard normal float32, rounded to bf16 (round to nearest
    even); returned as the raw uint16 bit patterns.
  * router logits: standard normal float32 of shape [T, E].
  * top-k: by score descending, ties to the lower expert id; gates are the
    selected scores renormalised to sum to 1 in float32.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Config", "CONFIGS", "make_x", "make_routing", "make_inputs",
           "random_routing", "random_bf16", "f32_to_bf16_bits", "bf16_bits_to_f32", "make_expert_outputs",
           "wide_bf16"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    k: int
    R: int
    router: str              # "softmax" | "sigmoid_group" | "softmax_zipf"
    groups: int = 0          # sigmoid_group: number of expert groups
    topk_groups: int = 0     # sigmoid_group: groups kept per token
    zipf_s: float = 0.0      # softmax_zipf: popularity exponent

    @property
    def Epr(self) -> int:
        return self.E // self.R


CONFIGS = {
    0: Config("tiny-T256-H128-E8-k2-R4", 256, 128, 8, 2, 4, "softmax"),
    1: Config("mixtral-T4096-H4096-E8-k2-R8", 4096, 4096, 8, 2, 8, "softmax"),
    2: Config("deepseekv3-T8192-H7168-E256-k8-R32", 8192, 7168, 256, 8, 32,
              "sigmoid_group", groups=8, topk_groups=4),
    3: Config("skewed-zipf1.2-T16384-H7168-E256-k8-R64", 16384, 7168, 256, 8, 64,
              "softmax_zipf", zipf_s=1.2),
    4: Config("prefill-T65536-H4096-E128-k8-R16", 65536, 4096, 128, 8, 16, "softmax"),
}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.

    Used only to draw bf16 activations; NaN never occurs in drawn data.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_x(cfg: Config, seed: int = 0, chunk_rows: int = 4096) -> np.ndarray:
    """Token-major activations x[T, H] as bf16 bit patterns (uint16)."""
    rng_x, _ = _streams(seed)
    out = np.empty((cfg.T, cfg.H), dtype=np.uint16)
    for r0 in range(0, cfg.T, chunk_rows):
        r1 = min(cfg.T, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(rng_x.standard_normal((r1 - r0, cfg.H), dtype=np.float32))
    return out


def _topk_desc(score: np.ndarray, k: int) -> np.ndarray:
    # descending score, ties to the lower id: a stable sort of the negated score
    order = np.argsort(-score, axis=1, kind="stable")
    return order[:, :k]


def make_routing(cfg: Config, seed: int = 0):
    """Router top-k: returns (topk_idx int32 [T,k], topk_w float32 [T,k])."""
    _, rng_r = _streams(seed)
    logits = rng_r.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.router == "softmax" or cfg.router == "softmax_zipf":
        if cfg.router == "softmax_zipf":
            ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
            p = ranks ** (-cfg.zipf_s)
            p /= p.sum()
            logits = logits + np.log(p).astype(np.float32)
        m = logits.max(axis=1, keepdims=True)
        ex = np.exp(logits - m, dtype=np.float32)
        score = ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)
        idx = _topk_desc(score, cfg.k)
    elif cfg.router == "sigmoid_group":
        score = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
        gsz = cfg.E // cfg.groups
        gscore = score.reshape(cfg.T, cfg.groups, gsz).max(axis=2)
        keep = _topk_desc(gscore, cfg.topk_groups)
        mask = np.zeros((cfg.T, cfg.groups), dtype=bool)
        np.put_along_axis(mask, keep, True, axis=1)
        masked = np.where(np.repeat(mask, gsz, axis=1), score, np.float32(-1.0))
        idx = _topk_desc(masked, cfg.k)
    else:
        raise ValueError(cfg.router)
    sel = np.take_along_axis(score, idx, axis=1).astype(np.float32)
    w = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(idx, dtype=np.int32), np.ascontiguousarray(w, dtype=np.float32)


def make_inputs(cfg: Config, seed: int = 0):
    idx, w = make_routing(cfg, seed)
    return {"x": make_x(cfg, seed), "topk_idx": idx, "topk_w": w}


def random_routing(rng: np.random.Generator, T: int, E: int, k: int, signed_gates: bool = False):
    """Tiny random routing: k distinct experts per token in random slot order."""
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    if signed_gates:
        w = rng.standard_normal((T, k)).astype(np.float32)
    else:
        g = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
        w = (g / g.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def random_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def wide_bf16(rng: np.random.Generator, shape, emin: int = -15, emax: int = 15) -> np.ndarray:
    """Random finite bf16 bit patterns: random sign and mantissa, exponent
    uniform in [emin, emax] (so sums cancel and round in many binades)."""
    r = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    e = rng.integers(127 + emin, 127 + emax + 1, size=shape, dtype=np.uint16)
    return ((r & np.uint16(0x807F)) | (e << np.uint16(7))).astype(np.uint16)


def make_expert_outputs(cfg: Config, seed: int = 0, chunk_rows: int = 16384) -> np.ndarray:
    """Stand-in expert outputs ye[T*k, H] (bf16 bits) for combine tests: the
    pages' experts are dense FFNs with trained weights, which are not here."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(3)[2]))
    rows = cfg.T * cfg.k
    out = np.empty((rows, cfg.H), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = wide_bf16(rng, (r1 - r0, cfg.H))
    return out
