"""fp64 CPU oracle for the LayerNorm of the sequence-parallel region.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone; shares no code with
the HIP path).

Under sequence parallelism the LayerNorms, dropouts and residual additions
outside the tensor-parallel region work on the rank's own block of s/t token
rows; the block leaves through a reduce-scatter and enters through an
all-gather, and the LayerNorm weights, shared by every block, have their
gradients summed over the tensor-parallel group ("Tensor and sequence
parallelism", section "Sequence parallelism" and its check script, which
runs LayerNorm -> all-gather -> the MLP shard -> reduce-scatter and then
all-reduces the LayerNorm weight's gradient; "02 -- Tensor Parallelism",
the paragraph on LayerNorm and dropout between the two all-reduces).

What is computed is the plain definition, in float64 with no intermediate
rounding:

* LayerNorm of a row x of length h: mean mu = sum(x)/h, biased variance
  var = sum((x - mu)^2)/h, rstd = 1/sqrt(var + eps), xhat = (x - mu)*rstd,
  y = xhat*gamma + beta (beta optional; the pages' check uses the weight
  alone and torch's default eps = 1e-5);
* its backward by the chain rule through those steps, with the gradient
  arriving along the residual branch (dres) added to the input gradient;
* the all-reduce of a shared parameter's gradient: the ranks' contributions
  added in rank order;
* the pages' TP+SP block: LayerNorm on each rank's block, all-gather, the
  MLP shard of every rank, reduce-scatter (oracle/mlp.py), and its backward;
  optionally with the gathered activations rounded to bfloat16, the format
  in which they travel (round_bf16, the format's definition).
Dropout is not modelled (probability 0, as in the pages' check).

Every function here is pinned in ``tests/test_oracle_ln_pins.py``.
"""
from __future__ import annotations

import numpy as np

from . import mlp
from .mlp import round_bf16

EPS = 1e-5


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def layer_norm_forward(x, gamma, beta=None, eps: float = EPS):
    """Row-wise LayerNorm of x [rows, h].  Returns (y, mean, rstd) with
    mean and rstd of shape [rows] (the backward's stash)."""
    x = _f64(x)
    h = x.shape[-1]
    mean = x.sum(axis=-1) / h
    xc = x - mean[:, None]
    var = (xc * xc).sum(axis=-1) / h
    rstd = 1.0 / np.sqrt(var + eps)
    y = xc * rstd[:, None] * _f64(gamma)[None, :]
    if beta is not None:
        y = y + _f64(beta)[None, :]
    return y, mean, rstd


def layer_norm_backward(dy, x, gamma, eps: float = EPS, dres=None):
    """Gradients of the forward for the output gradient dy [rows, h]:
    (dx, dgamma, dbeta).  dx includes dres [rows, h] when given (the
    residual branch's gradient of the same rows).  dgamma and dbeta are the
    sums over this block's rows only.

    Chain rule, one step of the forward at a time (per row):
      y = xhat*gamma + beta      -> dxhat = dy*gamma, dgamma += dy*xhat,
                                    dbeta += dy
      xhat = xc*rstd             -> dxc = dxhat*rstd,
                                    drstd = sum(dxhat*xc)
      rstd = (var + eps)^(-1/2)  -> dvar = -1/2 * rstd^3 * drstd
      var = sum(xc^2)/h          -> dxc += 2*xc*dvar/h
      xc = x - mean              -> dx = dxc, dmean = -sum(dxc)
      mean = sum(x)/h            -> dx += dmean/h
    """
    x, dy, gamma = _f64(x), _f64(dy), _f64(gamma)
    h = x.shape[-1]
    mean = x.sum(axis=-1, keepdims=True) / h
    xc = x - mean
    var = (xc * xc).sum(axis=-1, keepdims=True) / h
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = xc * rstd
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    dxhat = dy * gamma[None, :]
    dxc = dxhat * rstd
    drstd = (dxhat * xc).sum(axis=-1, keepdims=True)
    dvar = -0.5 * rstd ** 3 * drstd
    dxc = dxc + 2.0 * xc * dvar / h
    dmean = -dxc.sum(axis=-1, keepdims=True)
    dx = dxc + dmean / h
    if dres is not None:
        dx = dx + _f64(dres)
    return dx, dgamma, dbeta


def sum_shared_grads(grads):
    """The all-reduce of a parameter shared by the sequence blocks (the
    LayerNorm weight and bias): the ranks' gradients added in rank order."""
    out = np.zeros_like(_f64(grads[0]))
    for g in grads:
        out = out + _f64(g)
    return out


def sp_block_forward(act, x, gamma, W1, W2, t, Wg=None, beta=None, b2=None, residual=None, eps: float = EPS,
                     payload_bf16: bool = False):
    """The pages' TP+SP block for the whole group: rank r normalises its
    block x[r*N/t:(r+1)*N/t] of x [N, h]; the blocks are all-gathered; every
    rank runs its MLP shard on the gathered rows; the partial sums are
    reduce-scattered, with the output bias added once and the rank's block of
    ``residual`` [N, h] added.  Returns (outs, ln), both lists of the ranks'
    [N/t, h] blocks (the block outputs and the LayerNorm outputs).

    payload_bf16: the LayerNorm outputs are rounded to bfloat16 before the
    all-gather, the format in which they travel; the default keeps them in
    float64 (no intermediate rounding).  With ReLU the backward's derivative
    is a decision (U > 0) taken on the gathered activations, so a comparison
    with a path that gathers bf16 activations takes it on the same values."""
    x = _f64(x)
    N, F = x.shape[0], _f64(W1).shape[1]
    blocks = [mlp.sequence_block(r, t, N) for r in range(t)]
    ln = [layer_norm_forward(x[b], gamma, beta, eps)[0] for b in blocks]
    X = mlp.all_gather([round_bf16(a) for a in ln] if payload_bf16 else ln)
    partials = []
    for r in range(t):
        c = mlp.column_block(r, t, F)
        Wg_r = _f64(Wg)[:, c] if Wg is not None else None
        partials.append(mlp.shard_forward(act, X, _f64(W1)[:, c], _f64(W2)[c, :], Wg_r)["Y"])
    outs = [mlp.reduce_scatter(partials, r, b2, None if residual is None else _f64(residual)[blocks[r]])
            for r in range(t)]
    return outs, ln


def sp_block_backward(act, x, gamma, W1, W2, douts, t, Wg=None, beta=None, eps: float = EPS, dres=None,
                      payload_bf16: bool = False):
    """Backward of sp_block_forward for the ranks' output-gradient blocks
    ``douts`` (list of t [N/t, h]).  The reduce-scatter's backward is an
    all-gather of douts (the MLP's dY, the same on every rank); each rank's
    shard backward gives its partial input gradient over all N rows; the
    all-gather's backward reduce-scatters those into the rank's rows; the
    LayerNorm backward of the rank's block follows (``dres``: list of t
    residual-branch gradients or None), and the LayerNorm weight's gradient is
    summed over the ranks.  payload_bf16 as for sp_block_forward.  Returns
    dict(dx=[t blocks], dgamma, dbeta, dgamma_r=[t], dbeta_r=[t],
    shard=[t shard_backward results])."""
    x = _f64(x)
    N, F = x.shape[0], _f64(W1).shape[1]
    blocks = [mlp.sequence_block(r, t, N) for r in range(t)]
    ln = [layer_norm_forward(x[b], gamma, beta, eps)[0] for b in blocks]
    X = mlp.all_gather([round_bf16(a) for a in ln] if payload_bf16 else ln)
    dY = mlp.all_gather(douts)
    shard = []
    for r in range(t):
        c = mlp.column_block(r, t, F)
        Wg_r = _f64(Wg)[:, c] if Wg is not None else None
        shard.append(mlp.shard_backward(act, X, _f64(W1)[:, c], _f64(W2)[c, :], dY, Wg_r))
    dx, dgs, dbs = [], [], []
    for r in range(t):
        dln = mlp.reduce_scatter([s["dX"] for s in shard], r)
        d, dg, db = layer_norm_backward(dln, x[blocks[r]], gamma, eps, None if dres is None else dres[r])
        dx.append(d)
        dgs.append(dg)
        dbs.append(db)
    return dict(dx=dx, dgamma=sum_shared_grads(dgs), dbeta=sum_shared_grads(dbs), dgamma_r=dgs, dbeta_r=dbs,
                shard=shard)
