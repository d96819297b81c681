"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same shapes, so the same tile choice).

The GPU runs rank 0's shard forward and backward on the whole workload.  The
oracle computes, on the same bf16 inputs:
  * every row-local output (U, G, A, Y_i, dU / dG / dP, dX_i) on a seeded
    sample of token rows -- a row of these depends only on that row of X and
    dY, so the oracle simply runs on the sampled rows;
  * the weight gradients dW1, dWg, dW2 on a seeded sample of hidden columns --
    the block decomposes over hidden columns, so the oracle runs on the
    column sub-shard W1[:, c], Wg[:, c], W2[c, :] over all tokens;
  * db2 in full; the reduction of t partials (with the bias for the
    prefill workload) on sampled rows.
The group test runs every rank's shard of each workload in turn at full
size, reduces the partial sums with the library's kernel and compares the
result with the oracle's unsplit block on sampled rows (and every rank's
weight gradients on sampled columns).
Tolerance: relative Frobenius error <= 5e-3 and max error <= 3e-2 * max|ref|
per tensor.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from megatron_tensor_transformer_rank_amd.configs import WORKLOADS
from tests.helpers import assert_close, bf16_dev, f64

pytestmark = pytest.mark.gpu

ROW_SAMPLE = 96
COL_SAMPLE = 24


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    w = WORKLOADS[name]
    N, h, Fi, t, act = w.N, w.h, w.Fi, w.t, w.act
    sw = act == "swiglu"
    say(f"[fullsize] {name}: N={N} h={h} F_i={Fi} t={t} act={act} backward={w.backward}")
    Xb = I.gen_x(w.wid, N, h)
    W1b = I.gen_w_up_shard(w.wid, h, Fi, 0)
    W2b = I.gen_w_down_shard(w.wid, h, Fi, 0)
    Wgb = I.gen_w_gate_shard(w.wid, h, Fi, 0) if sw else None
    dYb = I.gen_dy(w.wid, N, h) if w.backward else None

    shape = B.make_shape(N, h, w.F, t, 0, act)
    bf, f32 = torch.bfloat16, torch.float32
    X, W1, W2 = bf16_dev(Xb), bf16_dev(W1b), bf16_dev(W2b)
    Wg = bf16_dev(Wgb) if sw else None
    Y = torch.empty(N, h, dtype=bf, device="cuda")
    A = torch.empty(N, Fi, dtype=bf, device="cuda")
    U = torch.empty(N, Fi, dtype=bf, device="cuda")
    G = torch.empty(N, Fi, dtype=bf, device="cuda") if sw else None
    B.tp_mlp_fwd_shard(shape, X, W1, Wg, W2, Y, A, U, G, B.alloc_workspace(B.workspace_bytes(shape, False)))
    if w.backward:
        dY = bf16_dev(dYb)
        dU = torch.empty(N, w.g * Fi, dtype=bf, device="cuda")
        dW1 = torch.empty(h, Fi, dtype=f32, device="cuda")
        dWg = torch.empty(h, Fi, dtype=f32, device="cuda") if sw else None
        dW2 = torch.empty(Fi, h, dtype=f32, device="cuda")
        dX = torch.empty(N, h, dtype=bf, device="cuda")
        db2 = torch.empty(h, dtype=f32, device="cuda")
        B.tp_mlp_bwd_shard(shape, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX, db2,
                           B.alloc_workspace(B.workspace_bytes(shape, True)))
    torch.cuda.synchronize()
    say(f"[fullsize] {name}: GPU done")

    rng = np.random.default_rng(w.wid + 777)
    rows = np.sort(rng.choice(N, size=min(ROW_SAMPLE, N), replace=False))
    ridx = torch.from_numpy(rows).to("cuda")
    f = oracle.bf16_bits_to_f64
    W1f, W2f = f(W1b), f(W2b)
    Wgf = f(Wgb) if sw else None
    Xr = f(Xb[rows])
    fr = oracle.shard_forward(act, Xr, W1f, W2f, Wgf)
    assert_close("A rows", f64(A[ridx]), fr["A"])
    assert_close("U rows", f64(U[ridx]), fr["U"])
    if sw:
        assert_close("G rows", f64(G[ridx]), fr["G"])
    assert_close("Y_i rows", f64(Y[ridx]), fr["Y"])
    say(f"[fullsize] {name}: forward rows ok")
    if not w.backward:
        return

    br = oracle.shard_backward(act, Xr, W1f, W2f, f(dYb[rows]), Wgf)
    dUr = f64(dU[ridx])
    if sw:
        assert_close("dG rows", dUr[:, :Fi], br["dG"])
        assert_close("dP rows", dUr[:, Fi:], br["dU"])
    else:
        assert_close("dU rows", dUr, br["dU"])
    assert_close("dX_i rows", f64(dX[ridx]), br["dX"])
    say(f"[fullsize] {name}: backward rows ok")

    cols = np.sort(rng.choice(Fi, size=COL_SAMPLE, replace=False))
    cidx = torch.from_numpy(cols).to("cuda")
    Xall, dYall = f(Xb), f(dYb)
    bc = oracle.shard_backward(act, Xall, W1f[:, cols], W2f[cols, :], dYall,
                               Wgf[:, cols] if sw else None)
    assert_close("dW1 cols", f64(dW1[:, cidx]), bc["dW1"])
    assert_close("dW2 rows", f64(dW2[cidx, :]), bc["dW2"])
    if sw:
        assert_close("dWg cols", f64(dWg[:, cidx]), bc["dWg"])
    assert_close("db2", f64(db2), oracle.column_sum(dYall), rel_fro=1e-5, max_rel=1e-5)
    say(f"[fullsize] {name}: weight gradients ok")


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.N > 1])
def test_reduce_full_size(name):
    """The t-way reduction (bias once where the workload has one) at full
    output size, on seeded partials, checked on sampled rows."""
    w = WORKLOADS[name]
    N, h, t = w.N, w.h, w.t
    say(f"[fullsize-reduce] {name}: t={t} rows={N} cols={h} bias={w.bias}")
    parts = [I.normal_bf16([w.wid, 90, r], (N, h)) for r in range(t)]
    b2 = I.gen_b2(w.wid, h) if w.bias else None
    out = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([bf16_dev(p) for p in parts], out, bias=bf16_dev(b2) if w.bias else None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.wid + 99)
    rows = np.sort(rng.choice(N, size=min(256, N), replace=False))
    ref = oracle.reduce_partials([oracle.bf16_bits_to_f64(p[rows]) for p in parts],
                                 oracle.bf16_bits_to_f64(b2) if w.bias else None)
    got = f64(out[torch.from_numpy(rows).to("cuda")])
    assert_close("reduced rows", got, ref, rel_fro=5e-3, max_rel=1e-2)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_group_full_size_split_equals_unsplit(name):
    """The pages' invariant at every workload's full size: all t ranks' shards
    run in turn on the GPU (the whole workload, each rank's own weight
    block), their partial sums Y_r (and, for training, dX_r) are reduced by
    the library's reduction kernel (the output bias added once for the
    prefill workload), and the result is compared on sampled token rows with
    the oracle's unsplit block -- one MLP over the full weights, no shards
    ("Tensor Parallelism's Communication Boundary", "Follow the
    coordinates"; "Parallelism Strategies #1 - Tensor Parallelism", the
    sharded forward and backward checks).  Every rank's weight gradients are
    checked on sampled columns against the same columns of the unsplit
    block's gradients."""
    w = WORKLOADS[name]
    N, h, F, Fi, t, act = w.N, w.h, w.F, w.Fi, w.t, w.act
    sw = act == "swiglu"
    say(f"[group-fullsize] {name}: N={N} h={h} F={F} t={t} act={act} bias={w.bias} backward={w.backward}")
    bf, f32 = torch.bfloat16, torch.float32
    Xb = I.gen_x(w.wid, N, h)
    dYb = I.gen_dy(w.wid, N, h) if w.backward else None
    b2b = I.gen_b2(w.wid, h) if w.bias else None
    X = bf16_dev(Xb)
    dY = bf16_dev(dYb) if w.backward else None
    rng = np.random.default_rng(w.wid + 4242)
    rows = np.sort(rng.choice(N, size=min(ROW_SAMPLE, N), replace=False))
    ridx = torch.from_numpy(rows).to("cuda")
    shape0 = B.make_shape(N, h, F, t, 0, act)
    ws_f = B.alloc_workspace(B.workspace_bytes(shape0, False))
    A = torch.empty(N, Fi, dtype=bf, device="cuda")
    U = torch.empty(N, Fi, dtype=bf, device="cuda")
    G = torch.empty(N, Fi, dtype=bf, device="cuda") if sw else None
    if w.backward:
        dU = torch.empty(N, w.g * Fi, dtype=bf, device="cuda")
        dW1 = torch.empty(h, Fi, dtype=f32, device="cuda")
        dWg = torch.empty(h, Fi, dtype=f32, device="cuda") if sw else None
        dW2 = torch.empty(Fi, h, dtype=f32, device="cuda")
    Ys, dXs, wb, dw = [], [], [], []
    for r in range(t):
        shard = (I.gen_w_up_shard(w.wid, h, Fi, r), I.gen_w_down_shard(w.wid, h, Fi, r),
                 I.gen_w_gate_shard(w.wid, h, Fi, r) if sw else None)
        wb.append(shard)
        W1, W2 = bf16_dev(shard[0]), bf16_dev(shard[1])
        Wg = bf16_dev(shard[2]) if sw else None
        s = B.make_shape(N, h, F, t, r, act)
        Y = torch.empty(N, h, dtype=bf, device="cuda")
        B.tp_mlp_fwd_shard(s, X, W1, Wg, W2, Y, A, U, G, ws_f)
        Ys.append(Y)
        if w.backward:
            dX = torch.empty(N, h, dtype=bf, device="cuda")
            B.tp_mlp_bwd_shard(s, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX)
            dXs.append(dX)
            cols = np.sort(rng.choice(Fi, size=COL_SAMPLE, replace=False))
            cidx = torch.from_numpy(cols).to("cuda")
            torch.cuda.synchronize()
            dw.append((cols, f64(dW1[:, cidx]), f64(dW2[cidx, :]), f64(dWg[:, cidx]) if sw else None))
        del W1, W2, Wg
    Yred = torch.empty(N, h, dtype=bf, device="cuda")
    B.tp_mlp_reduce_partials_local(Ys, Yred, bias=bf16_dev(b2b) if w.bias else None)
    if w.backward:
        dXred = torch.empty(N, h, dtype=bf, device="cuda")
        B.tp_mlp_reduce_partials_local(dXs, dXred)
    torch.cuda.synchronize()
    say(f"[group-fullsize] {name}: GPU done")

    # the oracle's unsplit block: the full weights are the rank blocks side by side
    f = oracle.bf16_bits_to_f64
    W1f = np.concatenate([f(s[0]) for s in wb], axis=1)
    W2f = np.concatenate([f(s[1]) for s in wb], axis=0)
    Wgf = np.concatenate([f(s[2]) for s in wb], axis=1) if sw else None
    del wb
    Xr = f(Xb[rows])
    fr = oracle.shard_forward(act, Xr, W1f, W2f, Wgf)
    Yref = oracle.reduce_partials([fr["Y"]], f(b2b) if w.bias else None)
    e = assert_close("reduced Y rows vs unsplit", f64(Yred[ridx]), Yref)
    say(f"[group-fullsize] {name}: Y = unsplit on sampled rows (relFro {e[0]:.2e}, max {e[1]:.2e})")
    if not w.backward:
        return
    br = oracle.shard_backward(act, Xr, W1f, W2f, f(dYb[rows]), Wgf)
    e = assert_close("reduced dX rows vs unsplit", f64(dXred[ridx]), br["dX"])
    say(f"[group-fullsize] {name}: dX = unsplit on sampled rows (relFro {e[0]:.2e}, max {e[1]:.2e})")
    Xall, dYall = f(Xb), f(dYb)
    for r, (cols, g1, g2, gg) in enumerate(dw):
        gcol = r * Fi + cols                      # the rank's columns of the unsplit block
        bc = oracle.shard_backward(act, Xall, W1f[:, gcol], W2f[gcol, :], dYall, Wgf[:, gcol] if sw else None)
        assert_close(f"dW1[{r}] cols vs unsplit", g1, bc["dW1"])
        assert_close(f"dW2[{r}] rows vs unsplit", g2, bc["dW2"])
        if sw:
            assert_close(f"dWg[{r}] cols vs unsplit", gg, bc["dWg"])
    say(f"[group-fullsize] {name}: every rank's weight gradients = unsplit columns")
