"""Seeded synthetic inputs, shared by the GPU path's callers and the oracle.

This module holds none of the MLP's arithmetic: it draws normal samples,
rounds them to bfloat16 (round-to-nearest-even) and slices shards out of
them.  Both sides consume exactly the same bf16 bit patterns; the oracle
decodes them to float64 itself and the GPU reads them as they are.

Recipe (the shapes come from the workload table in ``configs.py``):

* X and dY ~ N(0, 1); weights and the output bias ~ N(0, 0.02).
* Generator: numpy PCG64 seeded with ``[workload_id, tensor_id, block]``,
  ``standard_normal(dtype=float32) * sigma``, then RNE to bf16.
* tensor ids: X = 0, W_up (W1) = 1, W_gate = 2, W_down (W2) = 3, dY = 4,
  b2 = 5, LayerNorm weight = 6, LayerNorm bias = 7.
* LayerNorm parameters: weight ~ 1 + N(0, 0.1), bias ~ N(0, 0.02) (a
  trained-looking spread around the initial 1 and 0).
* Weights are generated one rank block at a time (block = rank): W1 and
  W_gate column blocks [h, F/t], W2 row blocks [F/t, h].  The full matrix is
  the concatenation of the blocks in rank order, so a rank's shard can be
  produced without drawing the others.
"""
from __future__ import annotations

import numpy as np

X_ID, WUP_ID, WGATE_ID, WDOWN_ID, DY_ID, B2_ID, LNW_ID, LNB_ID = 0, 1, 2, 3, 4, 5, 6, 7
WEIGHT_SIGMA = 0.02


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, nearest-even; NaN maps
    to a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def normal_bf16(seed, shape, sigma=1.0) -> np.ndarray:
    """bf16 bit patterns of ``sigma * N(0,1)`` float32 samples."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def gen_x(wid: int, N: int, h: int) -> np.ndarray:
    return normal_bf16([wid, X_ID, 0], (N, h))


def gen_dy(wid: int, N: int, h: int) -> np.ndarray:
    return normal_bf16([wid, DY_ID, 0], (N, h))


def gen_b2(wid: int, h: int) -> np.ndarray:
    return normal_bf16([wid, B2_ID, 0], (h,), WEIGHT_SIGMA)


def gen_ln_weight(wid: int, h: int) -> np.ndarray:
    """LayerNorm weight [h]: bf16 of 1 + 0.1 * N(0, 1)."""
    rng = np.random.default_rng([wid, LNW_ID, 0])
    return f32_to_bf16_bits(np.float32(1.0) + np.float32(0.1) * rng.standard_normal(size=(h,), dtype=np.float32))


def gen_ln_bias(wid: int, h: int) -> np.ndarray:
    return normal_bf16([wid, LNB_ID, 0], (h,), WEIGHT_SIGMA)


def gen_w_up_shard(wid: int, h: int, Fi: int, rank: int) -> np.ndarray:
    """Rank ``rank``'s column block of W_up (= W1), shape [h, Fi]."""
    return normal_bf16([wid, WUP_ID, rank], (h, Fi), WEIGHT_SIGMA)


def gen_w_gate_shard(wid: int, h: int, Fi: int, rank: int) -> np.ndarray:
    """Rank ``rank``'s column block of W_gate, shape [h, Fi]."""
    return normal_bf16([wid, WGATE_ID, rank], (h, Fi), WEIGHT_SIGMA)


def gen_w_down_shard(wid: int, h: int, Fi: int, rank: int) -> np.ndarray:
    """Rank ``rank``'s row block of W_down (= W2), shape [Fi, h]."""
    return normal_bf16([wid, WDOWN_ID, rank], (Fi, h), WEIGHT_SIGMA)


def gen_full_weights(wid: int, h: int, F: int, t: int, swiglu: bool):
    """Full W1 [h, F], W2 [F, h] and (SwiGLU) W_gate [h, F] as the rank-order
    concatenation of the per-rank blocks."""
    Fi = F // t
    W1 = np.concatenate([gen_w_up_shard(wid, h, Fi, r) for r in range(t)], axis=1)
    W2 = np.concatenate([gen_w_down_shard(wid, h, Fi, r) for r in range(t)], axis=0)
    Wg = (np.concatenate([gen_w_gate_shard(wid, h, Fi, r) for r in range(t)], axis=1)
          if swiglu else None)
    return W1, W2, Wg
