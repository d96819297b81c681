"""fp64 CPU oracle for one tensor-parallel rank of the Megatron paired MLP.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls it, and it shares no
code with the HIP path (no kernels, headers, helpers or constants).  The only
thing both sides consume is the seeded input generator, which holds none of
the method's arithmetic.

What it computes is the plain definition of the paired MLP block and of its
tensor-parallel split, in float64, with no intermediate rounding:

* column-parallel up-projection: each rank multiplies the replicated input by
  its own contiguous block of the first weight's output columns
  ("02 -- Tensor Parallelism", section "Column-parallel"; "Megatron-LM: Tensor
  Parallelism", section "MLP Block");
* an elementwise activation on the local hidden coordinates, which commutes
  with that split ("02 -- Tensor Parallelism", section "The MLP pairing";
  "Tensor Parallelism's Communication Boundary", section "Follow the
  coordinates");
* row-parallel down-projection to a full-shape partial sum, the partial sums
  added in rank order, and the output bias added once after that sum
  ("02 -- Tensor Parallelism", section "Row-parallel"; "Tensor Parallelism's
  Communication Boundary", the paragraph on bias handling before a reduction);
* the sharded backward: input gradient of the down-projection, activation
  derivative, local weight gradients, and a per-rank partial input gradient
  that must be summed over ranks ("Parallelism Strategies #1 - Tensor
  Parallelism", the sharded backward derivation and its code; "Tensor and
  sequence parallelism", the table of the f and g operators);
* the sequence-parallel boundary of that region: on leaving it, the partial
  sums are added and split back into contiguous sequence blocks (a
  reduce-scatter; the output bias once and the residual branch are added on
  the rank's block); on entering it, the blocks are concatenated in rank order
  (an all-gather) ("Tensor and sequence parallelism", section "Sequence
  parallelism").

Matrices are in math layout (input dim first): X [N, h], W1 [h, F],
W2 [F, h].  The pages that store weights PyTorch-style as (out, in) describe
the same partition transposed.

Readings taken where the pages are silent (each is pinned by a CPU test):

* GeLU is the exact erf form: GeLU(u) = u * Phi(u).
* SwiGLU: A = SiLU(X @ Wg) * (X @ Wu), SiLU(z) = z * sigmoid(z); gate and up
  are sharded on the same column indices; there is no bias inside the block.
* ReLU'(0) = 0.
* dY is an input; it is the same on every rank.
* Only the output bias b2 exists; db2 = column sums of dY, computed once.
* By default nothing is rounded.  The bf16_storage variant rounds, where the
  method stores them, exactly the tensors the pages keep in two bytes (the
  activations and their stashes, partial sums, activation gradients and
  partial input gradients, and the reduced sums); it is the reference for
  outputs whose exact values cancel so strongly that that storage alone
  exceeds the tolerance.

Every function here has a pin in ``tests/test_oracle_pins.py`` (worked example
from the pages, closed forms, brute force, finite differences, autograd of the
unsplit block and the split-equals-unsplit invariants).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

ACTS = ("relu", "gelu", "swiglu")


# --------------------------------------------------------------------------
# Input decoding
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly to float64.

    A bfloat16 value is the upper half of a float32, so placing the 16 bits in
    the high half of a 32-bit word and reinterpreting it is exact.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(a):
    """Nearest bfloat16 value of each float64 (ties to even): the 2-byte
    storage format of the activations, partial sums and gradients the pages
    price their messages and buffers in.  bfloat16 keeps 8 significant bits
    (7 stored) and float32's exponent range; values are finite and within
    that range here."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)              # a = m * 2^e, 0.5 <= |m| < 1
    scaled = m * 256.0               # 8 significant bits -> an integer part
    return np.ldexp(np.round(scaled), e - 8)   # np.round: half to even


# --------------------------------------------------------------------------
# Activations (elementwise on the local shard)
# --------------------------------------------------------------------------
def _phi_cdf(u):
    """Standard normal CDF, Phi(u) = (1 + erf(u / sqrt 2)) / 2."""
    return 0.5 * (1.0 + _erf(u / math.sqrt(2.0)))


def _phi_pdf(u):
    """Standard normal density, exp(-u^2/2) / sqrt(2 pi)."""
    return np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def _sigmoid(z):
    """Logistic function 1 / (1 + exp(-z)), written so exp never overflows."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def act_forward(act: str, U, G=None):
    """A = act(U) for ReLU / GeLU; A = SiLU(G) * U for SwiGLU (U is the up
    projection, G the gate projection).

    The activation acts coordinate by coordinate on the rank's own hidden
    columns ("02 -- Tensor Parallelism", section "The MLP pairing").
    """
    U = np.asarray(U, dtype=np.float64)
    if act == "relu":
        return np.maximum(U, 0.0)
    if act == "gelu":
        return U * _phi_cdf(U)
    if act == "swiglu":
        G = np.asarray(G, dtype=np.float64)
        return G * _sigmoid(G) * U
    raise ValueError(f"unknown activation {act!r}")


def act_backward(act: str, dA, U, G=None):
    """Gradient through the activation.

    ReLU / GeLU return dU = dA * act'(U), with ReLU'(u) = [u > 0] and
    GeLU'(u) = Phi(u) + u * phi(u).
    SwiGLU returns (dG, dU): with s = sigmoid(G),
    dG = dA * U * s * (1 + G * (1 - s)) and dU = dA * G * s.
    """
    dA = np.asarray(dA, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    if act == "relu":
        return dA * (U > 0.0)
    if act == "gelu":
        return dA * (_phi_cdf(U) + U * _phi_pdf(U))
    if act == "swiglu":
        G = np.asarray(G, dtype=np.float64)
        s = _sigmoid(G)
        dG = dA * U * s * (1.0 + G * (1.0 - s))
        dP = dA * G * s
        return dG, dP
    raise ValueError(f"unknown activation {act!r}")


# --------------------------------------------------------------------------
# One rank's shard
# --------------------------------------------------------------------------
def shard_forward(act: str, X, W1_i, W2_i, Wg_i=None, bf16_storage: bool = False):
    """Forward of one rank's shard.

    U_i = X @ W1_i (column-parallel, no communication), A_i = act(U_i)
    (SwiGLU: G_i = X @ Wg_i, A_i = SiLU(G_i) * U_i), and the full-shape partial
    sum Y_i = A_i @ W2_i (row-parallel, no bias)
    ("02 -- Tensor Parallelism", sections "Column-parallel", "Row-parallel",
    "The MLP pairing").

    bf16_storage: the same arithmetic with every tensor the method keeps in
    two bytes rounded to bfloat16 where it is stored: the pre-activations U_i
    (and G_i) as stored, A_i rounded after the activation (computed from the
    unrounded pre-activations) and used rounded by the down-projection, and
    Y_i rounded.  Nothing else is rounded (the products are exact).

    Returns a dict with U, G (None unless SwiGLU), A and Y.
    """
    X = np.asarray(X, dtype=np.float64)
    U = X @ np.asarray(W1_i, dtype=np.float64)
    G = X @ np.asarray(Wg_i, dtype=np.float64) if act == "swiglu" else None
    A = act_forward(act, U, G)
    if bf16_storage:
        U, A = round_bf16(U), round_bf16(A)
        G = round_bf16(G) if G is not None else None
    Y = A @ np.asarray(W2_i, dtype=np.float64)
    return {"U": U, "G": G, "A": A, "Y": round_bf16(Y) if bf16_storage else Y}


def shard_backward(act: str, X, W1_i, W2_i, dY, Wg_i=None, bf16_storage: bool = False):
    """Backward of one rank's shard for an output gradient dY that is the same
    on every rank.

    dA_i = dY @ W2_i^T; dU_i through the activation; dW2_i = A_i^T @ dY;
    dW1_i = X^T @ dU_i (SwiGLU: dWu_i = X^T @ dP_i, dWg_i = X^T @ dG_i); and the
    partial input gradient dX_i = dU_i @ W1_i^T (SwiGLU:
    dG_i @ Wg_i^T + dP_i @ Wu_i^T), which the ranks must sum
    ("Parallelism Strategies #1 - Tensor Parallelism", the sharded backward
    derivation, math layout; "02 -- Tensor Parallelism", section
    "Column-parallel", backward).

    The forward quantities are recomputed from X and the weights (with
    bf16_storage, as shard_forward stores them: the activation derivative is
    taken on the stored pre-activations and dW2 on the stored A_i; dU_i (dG_i,
    dP_i) and dX_i are rounded to bfloat16 where they are stored, dA_i and the
    weight gradients are not).
    Returns a dict with dA, dU (SwiGLU: the up gradient dP), dG (None unless
    SwiGLU), dW1 (SwiGLU: dW_up), dWg (None unless SwiGLU), dW2 and dX.
    """
    X = np.asarray(X, dtype=np.float64)
    W1_i = np.asarray(W1_i, dtype=np.float64)
    W2_i = np.asarray(W2_i, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    rnd = round_bf16 if bf16_storage else (lambda a: a)
    fwd = shard_forward(act, X, W1_i, W2_i, Wg_i, bf16_storage)
    dA = dY @ W2_i.T
    dW2 = fwd["A"].T @ dY
    if act == "swiglu":
        Wg_i = np.asarray(Wg_i, dtype=np.float64)
        dG, dU = act_backward(act, dA, fwd["U"], fwd["G"])
        dG, dU = rnd(dG), rnd(dU)
        dW1 = X.T @ dU
        dWg = X.T @ dG
        dX = dG @ Wg_i.T + dU @ W1_i.T
    else:
        dU = rnd(act_backward(act, dA, fwd["U"]))
        dG = None
        dW1 = X.T @ dU
        dWg = None
        dX = dU @ W1_i.T
    return {"dA": dA, "dU": dU, "dG": dG, "dW1": dW1, "dWg": dWg,
            "dW2": dW2, "dX": rnd(dX)}


# --------------------------------------------------------------------------
# The tensor-parallel group
# --------------------------------------------------------------------------
def column_block(rank: int, t: int, F: int) -> slice:
    """Hidden columns owned by ``rank``: the contiguous block
    [rank*F/t, (rank+1)*F/t), rank 0 lowest ("Tensor Parallelism's
    Communication Boundary", section "Follow the coordinates"; "Tensor and
    sequence parallelism", the check script's column slice).  F must divide
    by t."""
    if t < 1 or F % t != 0:
        raise ValueError(f"F={F} must be a multiple of t={t}")
    if not 0 <= rank < t:
        raise ValueError(f"rank {rank} outside [0, {t})")
    Fi = F // t
    return slice(rank * Fi, (rank + 1) * Fi)


def shard_weights(W1, W2, rank: int, t: int, Wg=None):
    """Rank ``rank``'s shards: W1[:, c] (and Wg[:, c]) column blocks, W2[c, :]
    row block, for c = column_block(rank, t, F)."""
    W1 = np.asarray(W1)
    c = column_block(rank, t, W1.shape[1])
    return (W1[:, c], np.asarray(W2)[c, :],
            None if Wg is None else np.asarray(Wg)[:, c])


def reduce_partials(partials, bias=None):
    """Sum of the ranks' full-shape partial sums in rank order, then the bias
    added once ("Tensor Parallelism's Communication Boundary": adding the same
    output bias on every worker before the reduction would count it t times).
    This is the arithmetic of the forward all-reduce of g and of the backward
    all-reduce of f ("Tensor and sequence parallelism", table of f and g)."""
    out = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        out = out + np.asarray(p, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def tp_forward(act: str, X, W1, W2, t: int, Wg=None, b2=None, bf16_storage: bool = False):
    """Every rank's shard forward, then the partial sums reduced and the bias
    added once (with bf16_storage, the shards as shard_forward stores them and
    the reduced sum rounded to bfloat16).  Returns (Y, per-rank list of
    shard_forward dicts)."""
    ranks = []
    for r in range(t):
        W1_i, W2_i, Wg_i = shard_weights(W1, W2, r, t, Wg)
        ranks.append(shard_forward(act, X, W1_i, W2_i, Wg_i, bf16_storage))
    Y = reduce_partials([f["Y"] for f in ranks], b2)
    return (round_bf16(Y) if bf16_storage else Y), ranks


def tp_backward(act: str, X, W1, W2, dY, t: int, Wg=None, bf16_storage: bool = False):
    """Every rank's shard backward; dX = sum of the partial input gradients in
    rank order; db2 = column sums of dY (once).  With bf16_storage, the shards
    as shard_backward stores them and the reduced dX rounded to bfloat16.
    Returns (dX, db2, per-rank list of shard_backward dicts)."""
    ranks = []
    for r in range(t):
        W1_i, W2_i, Wg_i = shard_weights(W1, W2, r, t, Wg)
        ranks.append(shard_backward(act, X, W1_i, W2_i, dY, Wg_i, bf16_storage))
    dX = reduce_partials([b["dX"] for b in ranks])
    if bf16_storage:
        dX = round_bf16(dX)
    db2 = np.asarray(dY, dtype=np.float64).sum(axis=0)
    return dX, db2, ranks


def column_sum(dY):
    """db2 = sum over token rows of dY (gradient of the once-added bias)."""
    return np.asarray(dY, dtype=np.float64).sum(axis=0)


# --------------------------------------------------------------------------
# Sequence-parallel boundary of the tensor-parallel region
# --------------------------------------------------------------------------
def sequence_block(rank: int, t: int, rows: int) -> slice:
    """Token rows handled by ``rank`` outside the tensor-parallel region under
    sequence parallelism: the contiguous block [rank*rows/t, (rank+1)*rows/t)
    ("Tensor and sequence parallelism", section "Sequence parallelism" and
    the rows slice of its check script).  rows must divide by t."""
    if t < 1 or rows % t != 0:
        raise ValueError(f"rows={rows} must be a multiple of t={t}")
    if not 0 <= rank < t:
        raise ValueError(f"rank {rank} outside [0, {t})")
    n = rows // t
    return slice(rank * n, (rank + 1) * n)


def reduce_scatter(partials, rank: int, bias=None, residual=None):
    """Leaving the tensor-parallel region under sequence parallelism: the t
    ranks' full-shape partial sums are added (rank order) and only rank
    ``rank``'s sequence block is kept; the output bias is added once and the
    residual branch (the rank's block, [rows/t, cols]) is added on it
    ("Tensor and sequence parallelism", section "Sequence parallelism": the
    partial sums are summed and split back into sequence shards; the residual
    additions are in the sequence-parallel region).  Returns the rank's block
    of reduce_partials(partials, bias), plus the residual."""
    t = len(partials)
    rows = np.asarray(partials[0]).shape[0]
    blk = sequence_block(rank, t, rows)
    out = reduce_partials([np.asarray(p)[blk] for p in partials], bias)
    if residual is not None:
        out = out + np.asarray(residual, dtype=np.float64)
    return out


def all_gather(shards):
    """Entering the tensor-parallel region under sequence parallelism: the t
    sequence blocks are concatenated along the token rows in rank order
    ("Tensor and sequence parallelism", section "Sequence parallelism")."""
    return np.concatenate([np.asarray(x, dtype=np.float64) for x in shards], axis=0)
