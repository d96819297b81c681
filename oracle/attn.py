"""fp64 CPU oracle for one tensor-parallel rank's attention projections.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone; shares no code with
the HIP path).  The attention core (scores, softmax, the weighted sum) is not
part of this path: its output O is an input here, and its gradient dQKV too.

What is computed is the plain definition of the attention block's
tensor-parallel split, in float64 with no intermediate rounding:

* the Q, K and V projections are split along their output dimension, by
  head: rank r takes n_heads/t query heads and the key/value heads of those
  heads' groups, and computes its own QKV = X @ W_qkv_r with no
  communication ("02 -- Tensor Parallelism", section "The attention
  pairing"; "Megatron-LM: Tensor Parallelism", section "Attention Block");
* with grouped-query attention the split is by key/value group; when there
  are fewer key/value heads than ranks they are replicated, each on
  t/n_kv ranks, every rank keeping only its own query heads ("Tensor and
  sequence parallelism", exercise 1 of the closing questions);
* the output projection is split along its input dimension: rank r
  multiplies its heads' attention output O_r by the matching rows of W_o
  into a full-shape partial sum, and the partials are added (the all-reduce)
  ("02 -- Tensor Parallelism", section "The attention pairing");
* the backward is that of the two products on each rank: dO_r = dY @ W_o_r^T,
  dW_o_r = O_r^T @ dY, dX_r = dQKV_r @ W_qkv_r^T (summed over ranks),
  dW_qkv_r = X^T @ dQKV_r; a replicated key/value head's weight gradient is
  the sum of its replicas' contributions.

Layouts (math layout, input dim first): X [N, h]; W_q [h, n_heads*d];
W_k, W_v [h, n_kv*d]; W_o [n_heads*d, h]; head j owns columns
[j*d, (j+1)*d).  Rank r's fused projection weight is
W_qkv_r = [W_q columns of its query heads | W_k columns of its key/value
heads | W_v columns of the same], shape [h, (q_r + 2*kv_r)*d].

Every function here is pinned in ``tests/test_oracle_attn_pins.py``.
"""
from __future__ import annotations

import numpy as np


def check_heads(t: int, n_heads: int, n_kv: int) -> None:
    """The splits the pages describe: query heads in equal blocks, key/value
    heads either in equal blocks (n_kv >= t) or replicated (n_kv < t, each on
    t/n_kv ranks); every key/value head serves n_heads/n_kv query heads."""
    if t < 1 or n_heads < 1 or n_kv < 1:
        raise ValueError("t, n_heads and n_kv must be positive")
    if n_heads % n_kv != 0:
        raise ValueError(f"n_heads={n_heads} must be a multiple of n_kv={n_kv}")
    if n_heads % t != 0:
        raise ValueError(f"n_heads={n_heads} must be a multiple of t={t}")
    if n_kv >= t and n_kv % t != 0:
        raise ValueError(f"n_kv={n_kv} must be a multiple of t={t}")
    if n_kv < t and t % n_kv != 0:
        raise ValueError(f"t={t} must be a multiple of n_kv={n_kv} to replicate key/value heads")


def query_heads(rank: int, t: int, n_heads: int) -> range:
    """Query heads of ``rank``: the contiguous block [rank*n_heads/t,
    (rank+1)*n_heads/t)."""
    if not 0 <= rank < t:
        raise ValueError(f"rank {rank} outside [0, {t})")
    q = n_heads // t
    return range(rank * q, (rank + 1) * q)


def kv_heads(rank: int, t: int, n_heads: int, n_kv: int) -> range:
    """Key/value heads ``rank`` holds: the groups of its query heads, i.e. the
    block [rank*n_kv/t, (rank+1)*n_kv/t) when n_kv >= t, and the single
    replicated head rank*n_kv//t otherwise."""
    check_heads(t, n_heads, n_kv)
    if n_kv >= t:
        k = n_kv // t
        return range(rank * k, (rank + 1) * k)
    j = rank * n_kv // t
    return range(j, j + 1)


def _cols(heads: range, d: int) -> np.ndarray:
    return np.concatenate([np.arange(j * d, (j + 1) * d) for j in heads]) if len(heads) else np.arange(0)


def attn_shard_weights(Wq, Wk, Wv, Wo, rank: int, t: int, n_heads: int, n_kv: int, d: int):
    """Rank ``rank``'s fused projection weight W_qkv_r [h, (q_r + 2 kv_r) d]
    and output-projection rows W_o_r [q_r d, h]."""
    check_heads(t, n_heads, n_kv)
    qc = _cols(query_heads(rank, t, n_heads), d)
    kc = _cols(kv_heads(rank, t, n_heads, n_kv), d)
    Wqkv = np.concatenate([np.asarray(Wq)[:, qc], np.asarray(Wk)[:, kc], np.asarray(Wv)[:, kc]], axis=1)
    return Wqkv, np.asarray(Wo)[qc, :]


def qkv_forward(X, Wqkv_i):
    """QKV_r = X @ W_qkv_r: this rank's query, key and value columns (no
    communication: X is replicated)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(Wqkv_i, dtype=np.float64)


def out_forward(O_i, Wo_i):
    """Y_r = O_r @ W_o_r: the full-shape partial sum of the output projection
    (to be added over ranks; no bias here)."""
    return np.asarray(O_i, dtype=np.float64) @ np.asarray(Wo_i, dtype=np.float64)


def out_backward(dY, O_i, Wo_i):
    """Backward of Y_r = O_r @ W_o_r for the output gradient dY (the same on
    every rank): dO_r = dY @ W_o_r^T, dW_o_r = O_r^T @ dY."""
    dY = np.asarray(dY, dtype=np.float64)
    return dY @ np.asarray(Wo_i, dtype=np.float64).T, np.asarray(O_i, dtype=np.float64).T @ dY


def qkv_backward(X, Wqkv_i, dQKV_i):
    """Backward of QKV_r = X @ W_qkv_r: the partial input gradient
    dX_r = dQKV_r @ W_qkv_r^T (summed over ranks) and dW_qkv_r = X^T @ dQKV_r."""
    dQKV_i = np.asarray(dQKV_i, dtype=np.float64)
    return dQKV_i @ np.asarray(Wqkv_i, dtype=np.float64).T, np.asarray(X, dtype=np.float64).T @ dQKV_i


def gather_qkv_weight_grads(dWqkv, t: int, n_heads: int, n_kv: int, d: int):
    """Full-model gradients (dW_q, dW_k, dW_v) from the ranks' fused
    dW_qkv_r: query columns are disjoint across ranks; a key/value head's
    gradient is the sum over the ranks that hold it (its replicas)."""
    check_heads(t, n_heads, n_kv)
    h = np.asarray(dWqkv[0]).shape[0]
    dWq = np.zeros((h, n_heads * d))
    dWk = np.zeros((h, n_kv * d))
    dWv = np.zeros((h, n_kv * d))
    for r in range(t):
        g = np.asarray(dWqkv[r], dtype=np.float64)
        qc = _cols(query_heads(r, t, n_heads), d)
        kc = _cols(kv_heads(r, t, n_heads, n_kv), d)
        nq, nk = len(qc), len(kc)
        dWq[:, qc] = g[:, :nq]
        dWk[:, kc] += g[:, nq:nq + nk]
        dWv[:, kc] += g[:, nq + nk:nq + 2 * nk]
    return dWq, dWk, dWv
