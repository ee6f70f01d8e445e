"""Seeded synthetic inputs for the fused MoE expert layer.

This module is shared by the HIP path's tests and bench and by the CPU
oracle's tests.  It draws random numbers and lays them out; it holds none of
the layer's arithmetic (no quantiser, no rounding rule, no GEMM): the bf16
and fp8 casts it needs to *make* inputs are torch's own CPU casts.

Workload shapes follow the model the vLLM pages serve (Qwen3-30B-A3B-FP8:
hidden 2048, expert intermediate 768, 128 experts, top-8), per PR #20903
"[Kernel] DeepGemm MoE : Integrate triton permute / unpermute kernels"
(Test Plan / Performance), and the profiled modular-kernel shape of the same
page (Optimizations: M=64, topk=4, fp8 e4m3, 128x128 blocks).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

GROUP = 128  # quantisation group / weight block edge


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    K: int
    N: int
    Eg: int
    El: int
    topk: int
    chunk_size: int
    routing: str          # "softmax" | "zipf" | "hot"
    seed: int
    ep_rank_of_2: Optional[int] = None   # None: all experts local (null map)
    apply_router_weight_on_input: int = 0
    align: int = 128


CONFIGS = {
    # tiny, the oracle's whole-layer brute force runs on it
    "C1": LayerConfig("tiny", 64, 256, 128, 8, 8, 2, 64, "softmax", 1),
    # profiled modular-kernel shape: M=64, topk=4, half the experts local
    "C2": LayerConfig("profiling", 64, 2048, 768, 128, 64, 4, 64, "softmax", 2, ep_rank_of_2=1),
    "C3": LayerConfig("prefill", 4096, 2048, 768, 128, 128, 8, 4096, "softmax", 3),
    "C4": LayerConfig("chunk_stress", 8192, 2048, 768, 128, 64, 8, 64, "zipf", 4, ep_rank_of_2=1),
    "C4b": LayerConfig("chunk_tail", 130, 2048, 768, 128, 64, 8, 128, "zipf", 41, ep_rank_of_2=1),
    "C5u": LayerConfig("large_uniform", 16384, 2048, 768, 128, 128, 8, 16384, "softmax", 5),
    "C5u_on": LayerConfig("large_uniform_on_input", 16384, 2048, 768, 128, 128, 8, 16384, "softmax", 5,
                          apply_router_weight_on_input=1),
    "C5h": LayerConfig("large_hot", 16384, 2048, 768, 128, 128, 8, 16384, "hot", 6),
    "C5h_on": LayerConfig("large_hot_on_input", 16384, 2048, 768, 128, 128, 8, 16384, "hot", 6,
                          apply_router_weight_on_input=1),
}


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray              # [M, K] uint16 (bf16 bits)
    topk_ids: np.ndarray       # [M, T] int32 global expert ids (-1 = not routed)
    topk_weights: np.ndarray   # [M, T] float32
    expert_map: Optional[np.ndarray]  # [Eg] int32 or None (identity, El == Eg)
    w13: np.ndarray            # [El, 2N, K] uint8 (e4m3 bits)
    w13_s: np.ndarray          # [El, 2N/128, K/128] float32
    w2: np.ndarray             # [El, K, N] uint8
    w2_s: np.ndarray           # [El, K/128, N/128] float32
    extra: dict = field(default_factory=dict)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_bits(a: np.ndarray) -> np.ndarray:
    """float32 array (already within +-448) -> e4m3fn bit patterns via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def expert_map_for(cfg: LayerConfig) -> Optional[np.ndarray]:
    """EP rank r of 2 owns globals [r*El, (r+1)*El); every other id maps to -1."""
    if cfg.ep_rank_of_2 is None:
        return None
    m = np.full(cfg.Eg, -1, dtype=np.int32)
    lo = cfg.ep_rank_of_2 * cfg.El
    m[lo:lo + cfg.El] = np.arange(cfg.El, dtype=np.int32)
    return m


def _gumbel_topk(rng, log_p: np.ndarray, M: int, T: int):
    g = rng.gumbel(size=(M, log_p.shape[-1])).astype(np.float64)
    scores = log_p[None, :] + g
    ids = np.argsort(-scores, axis=1, kind="stable")[:, :T]
    return ids, np.take_along_axis(scores, ids, axis=1)


def _renorm_softmax(scores: np.ndarray) -> np.ndarray:
    s = scores - scores.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routing(rng, cfg: LayerConfig, M: Optional[int] = None):
    """topk ids/weights for cfg.routing.

    softmax: topk of N(0,1) logits over all Eg experts, weights = softmax over
    all Eg then renormalised over the chosen T.  zipf: popularity ~ rank^-1.2
    over a seeded permutation of ranks, Gumbel-top-k (distinct ids).  hot: 10%
    of experts carry a log-bias b chosen by bisection so that they receive 50%
    of the picks.
    """
    M = cfg.M if M is None else M
    Eg, T = cfg.Eg, cfg.topk
    info = {}
    if cfg.routing == "softmax":
        logits = rng.standard_normal((M, Eg)).astype(np.float64)
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :T]
        full = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(full)
        p /= p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
        w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    elif cfg.routing == "zipf":
        ranks = rng.permutation(Eg) + 1
        log_p = -1.2 * np.log(ranks.astype(np.float64))
        ids, sc = _gumbel_topk(rng, log_p, M, T)
        w = _renorm_softmax(sc)
    elif cfg.routing == "hot":
        n_hot = int(round(0.1 * Eg))
        hot = rng.choice(Eg, size=n_hot, replace=False)
        is_hot = np.zeros(Eg, dtype=bool)
        is_hot[hot] = True
        g = rng.gumbel(size=(M, Eg)).astype(np.float64)
        lo, hi = 0.0, 10.0
        for _ in range(40):
            b = 0.5 * (lo + hi)
            sc = g + b * is_hot[None, :]
            idx = np.argpartition(-sc, T - 1, axis=1)[:, :T]
            frac = is_hot[idx].mean()
            if frac < 0.5:
                lo = b
            else:
                hi = b
        b = 0.5 * (lo + hi)
        sc = g + b * is_hot[None, :]
        ids = np.argsort(-sc, axis=1, kind="stable")[:, :T]
        w = _renorm_softmax(np.take_along_axis(sc, ids, axis=1))
        info = {"hot_bias": b, "hot_experts": np.sort(hot), "hot_frac": float(is_hot[ids].mean())}
    else:
        raise ValueError(cfg.routing)
    return ids.astype(np.int32), w.astype(np.float32), info


def block_weights(rng, E: int, rows: int, cols: int, std: float = 0.02):
    """[E, rows, cols] fp8 e4m3 weights with one fp32 scale per 128x128 block.

    Values are N(0, std); each block's scale is its amax/448 and the codes are
    torch's e4m3fn cast of value/scale.
    """
    assert rows % GROUP == 0 and cols % GROUP == 0
    q = np.empty((E, rows, cols), dtype=np.uint8)
    s = np.empty((E, rows // GROUP, cols // GROUP), dtype=np.float32)
    for e in range(E):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
        blk = w.reshape(rows // GROUP, GROUP, cols // GROUP, GROUP)
        amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
        sc = np.maximum(amax, np.float32(1e-10)) / np.float32(448.0)
        s[e] = sc
        q[e] = e4m3_bits((blk / sc[:, None, :, None]).reshape(rows, cols))
    return q, s


def make_inputs(cfg: LayerConfig, M: Optional[int] = None) -> LayerInputs:
    """Draws x, then routing, then w13, then w2 from PCG64(cfg.seed)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    M = cfg.M if M is None else M
    x = bf16_bits(rng.standard_normal((M, cfg.K), dtype=np.float32))
    ids, w, info = routing(rng, cfg, M)
    w13, w13_s = block_weights(rng, cfg.El, 2 * cfg.N, cfg.K)
    w2, w2_s = block_weights(rng, cfg.El, cfg.K, cfg.N)
    return LayerInputs(cfg, x, ids, w, expert_map_for(cfg), w13, w13_s, w2, w2_s, info)


def small_config(name="small", M=200, K=512, N=256, Eg=16, El=16, topk=4, chunk_size=0,
                 routing="softmax", seed=11, ep_rank_of_2=None, on_input=0, align=128):
    return LayerConfig(name, M, K, N, Eg, El, topk, chunk_size, routing, seed, ep_rank_of_2,
                       on_input, align)


def random_ids(rng, M, T, Eg, p_minus1=0.0, p_invalid=0.0):
    """Arbitrary (not necessarily distinct) ids with injected -1 and invalid ids."""
    ids = rng.integers(0, Eg, size=(M, T), dtype=np.int64)
    u = rng.random((M, T))
    ids[u < p_minus1] = -1
    bad = (u >= p_minus1) & (u < p_minus1 + p_invalid)
    ids[bad] = rng.choice(np.array([-7, -2, Eg, Eg + 5, 2**30], dtype=np.int64), size=int(bad.sum()))
    return ids.astype(np.int32)


def random_codes(rng, shape, exclude_nan=True):
    """Uniform random e4m3 bytes (NaN codes 0x7F/0xFF excluded)."""
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    if exclude_nan:
        c[(c & 0x7F) == 0x7F] = 0x7E
    return c
