"""Workload table and seeded generators.

Every random draw comes from numpy's PCG64 seeded through
``SeedSequence(entropy=seed, spawn_key=key)``; each logical stream (weights,
outlier positions, activations, activation norms, routes, expert-down inputs)
has its own spawn key, so any slice of any stream can be regenerated on its own.
Weights are drawn in blocks of ``ROW_BLOCK`` rows, one key per block, which lets
a test regenerate a few rows of a large matrix without drawing the rest.

Floating-point samples are rounded float64 -> float32 (numpy, round to nearest
even) -> bf16 (round to nearest even on the float32 bits).  The shapes and
distributions follow the five workloads the hot path is measured on:

* ``ternary_1k``      1024 x 1024, N(0, 0.02^2), 1% of positions x10, batch 1
* ``int4_8k``         8192 x 8192, Student-t(4) * 0.015, batch 1 and 4
* ``ternary_moe``     64 experts of (up 1536x4096, down 4096x1536), t(4) * 0.02,
                      8 of 64 experts per token, 1 and 8 tokens
* ``cassandra_spec``  4096 x 14336, t(4) * 0.02, act norms LogNormal(0, 1), batch 1
* ``cassandra_verify`` 8192 x 28672, same distributions, batch 16

Block-sparse ternary weights (the skip format) take a dense draw and set whole
128-value blocks to zero, each block independently with probability
``ZERO_BLOCK_FRAC`` (its own stream, one key per row block).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROW_BLOCK = 512

# Stream identifiers (first element of the spawn key).
S_W, S_OUTLIER, S_X, S_NORM, S_ROUTE, S_DOWN_X, S_ZERO, S_XCH = 0, 1, 2, 3, 4, 5, 6, 7

# Fraction of all-zero 128-blocks in block-sparse ternary weights: 2 (1 - z) code
# bits plus 0.14 bits of scales and tables gives 1.74 bits per weight, under the
# 1.78 a 27B ternary package averages with its higher-precision embedding.
ZERO_BLOCK_FRAC = 0.2


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1-based workload number; seed = 20260000 + index
    fmt: str                   # "ternary", "int4", "ternary_moe", "cassandra"
    M: int
    K: int
    dist: str                  # "normal" or "t4"
    scale: float
    batches: tuple = (1,)
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    experts: int = 0
    topk: int = 0
    tokens: tuple = ()
    keep_num: int = 3
    keep_den: int = 10
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 20260000 + self.index


WORKLOADS = {
    "ternary_1k": Workload("ternary_1k", 1, "ternary", 1024, 1024, "normal", 0.02,
                           batches=(1,), outlier_frac=0.01, outlier_mult=10.0),
    "int4_8k": Workload("int4_8k", 2, "int4", 8192, 8192, "t4", 0.015, batches=(1, 4)),
    # M/K describe the up projection (4096 -> 1536, i.e. 1536 x 4096); the down
    # projection is the transpose shape 4096 x 1536.
    "ternary_moe": Workload("ternary_moe", 3, "ternary_moe", 1536, 4096, "t4", 0.02,
                            experts=64, topk=8, tokens=(1, 8)),
    "cassandra_spec": Workload("cassandra_spec", 4, "cassandra", 4096, 14336, "t4", 0.02,
                               batches=(1,)),
    "cassandra_verify": Workload("cassandra_verify", 5, "cassandra", 8192, 28672, "t4", 0.02,
                                 batches=(16,)),
}


def stream(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 generator for spawn key ``key`` under ``seed``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key)))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _draw(rng: np.random.Generator, dist: str, scale: float, n: int) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(n) * scale
    if dist == "t4":
        return rng.standard_t(4, n) * scale
    raise ValueError(dist)


def gen_weight_rows(seed: int, M: int, K: int, dist: str, scale: float,
                    r0: int = 0, r1: int | None = None, key_prefix: tuple = ()) -> np.ndarray:
    """Float64 samples for rows [r0, r1) of an M x K weight (before bf16 rounding)."""
    r1 = M if r1 is None else r1
    out = np.empty((r1 - r0, K), dtype=np.float64)
    b0, b1 = r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK
    for b in range(b0, b1 + 1):
        lo, hi = b * ROW_BLOCK, min(M, (b + 1) * ROW_BLOCK)
        rng = stream(seed, S_W, *key_prefix, b)
        blk = _draw(rng, dist, scale, (hi - lo) * K).reshape(hi - lo, K)
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = blk[s0 - lo:s1 - lo]
    return out


def gen_weights(wl: Workload, r0: int = 0, r1: int | None = None) -> np.ndarray:
    """bf16 bits [rows][K] of the workload's (dense) weight matrix, rows [r0, r1)."""
    M, K = wl.M, wl.K
    r1 = M if r1 is None else r1
    w = gen_weight_rows(wl.seed, M, K, wl.dist, wl.scale, r0, r1)
    if wl.outlier_frac > 0:
        n_out = int(np.floor(wl.outlier_frac * M * K))
        pos = stream(wl.seed, S_OUTLIER).choice(M * K, n_out, replace=False)
        rows = pos // K
        sel = (rows >= r0) & (rows < r1)
        flat = w.reshape(-1)
        flat[pos[sel] - r0 * K] *= wl.outlier_mult
    return f32_to_bf16_bits(w.astype(np.float32))


def gen_expert(wl: Workload, e: int, which: str) -> np.ndarray:
    """bf16 bits of expert ``e``'s up (1536 x 4096) or down (4096 x 1536) matrix."""
    j = {"up": 0, "down": 1}[which]
    M, K = (wl.M, wl.K) if j == 0 else (wl.K, wl.M)
    w = gen_weight_rows(wl.seed, M, K, wl.dist, wl.scale, key_prefix=(e, j))
    return f32_to_bf16_bits(w.astype(np.float32))


def gen_x(wl: Workload, B: int, K: int | None = None) -> np.ndarray:
    """bf16 bits [B][K] of N(0, 1) activations."""
    K = wl.K if K is None else K
    x = stream(wl.seed, S_X, B).standard_normal((B, K))
    return f32_to_bf16_bits(x.astype(np.float32))


def gen_x_outlier_channels(seed: int, B: int, K: int, n_big: int = 8, big: float = 100.0) -> np.ndarray:
    """bf16 bits [B][K] of activations with uneven input channels: N(0, 1) times a
    per-channel LogNormal(0, 1) scale (the spread the activation norms have), and
    ``n_big`` channels (distinct, seeded) ``big`` times larger still."""
    rng = stream(seed, S_XCH, B)
    scale = rng.lognormal(0.0, 1.0, K)
    scale[rng.choice(K, n_big, replace=False)] *= big
    x = rng.standard_normal((B, K)) * scale[None, :]
    return f32_to_bf16_bits(x.astype(np.float32))


def gen_act_norms(wl: Workload) -> np.ndarray:
    """float32 [K] per-input-channel activation L2 norms ~ LogNormal(0, 1)."""
    return stream(wl.seed, S_NORM).lognormal(0.0, 1.0, wl.K).astype(np.float32)


def gen_routes(wl: Workload, T: int) -> np.ndarray:
    """int32 [T][topk]: for each token, topk distinct experts drawn uniformly."""
    rng = stream(wl.seed, S_ROUTE, T)
    return np.stack([rng.choice(wl.experts, wl.topk, replace=False) for _ in range(T)]).astype(np.int32)


def gen_down_inputs(wl: Workload, T: int) -> np.ndarray:
    """bf16 bits [T][topk][M_up]: an independent N(0, 1) input per (token, expert slot)."""
    a = stream(wl.seed, S_DOWN_X, T).standard_normal((T, wl.topk, wl.M))
    return f32_to_bf16_bits(a.astype(np.float32))


def gen_zero_blocks(seed: int, M: int, K: int, frac: float = ZERO_BLOCK_FRAC,
                    r0: int = 0, r1: int | None = None) -> np.ndarray:
    """bool [rows][K/128] for rows [r0, r1): block (row, g) is zeroed."""
    r1 = M if r1 is None else r1
    G = K // 128
    out = np.empty((r1 - r0, G), dtype=bool)
    for b in range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1):
        lo, hi = b * ROW_BLOCK, min(M, (b + 1) * ROW_BLOCK)
        blk = stream(seed, S_ZERO, b).random((hi - lo, G)) < frac
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = blk[s0 - lo:s1 - lo]
    return out


def zero_out_blocks(w_bits: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """Copy of bf16 bits [rows][K] with the flagged 128-blocks set to +0."""
    rows, K = w_bits.shape
    out = np.array(w_bits, dtype=np.uint16, copy=True).reshape(rows, K // 128, 128)
    out[zero] = 0
    return out.reshape(rows, K)
