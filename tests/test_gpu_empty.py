"""Empty batches through the C ABI on the GPU: N = 0 tokens (rows = 0).

A forward or a reduction over no rows computes nothing.  Every weight
gradient, db2, dgamma and dbeta is a sum over the batch's rows, so over an
empty batch it is zero; the oracle gives the same (its products over an
empty dimension are zero).  The output buffers are filled with NaN first,
so a gradient the library left unwritten fails the test.  Empty tensors
pass NULL storage, which the ABI accepts for buffers of zero bytes.  After
the empty calls, a non-empty call on the same buffers' shapes must still
match the oracle (nothing stale is kept)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import attn as OA
from oracle import ln as OL
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import assert_close, bf16_dev, f64, run_group

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


def nan_f32(*shape):
    return torch.full(shape, float("nan"), dtype=F32, device="cuda")


def empty_bf16(*shape):
    return torch.empty(*shape, dtype=BF, device="cuda")


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_empty_batch_forward_and_backward(act):
    print(f"[empty] mlp act={act}", file=sys.stderr, flush=True)
    h, F, t = 264, 2 * 136, 2
    sw = act == "swiglu"
    s = B.make_shape(0, h, F, t, 0, act)
    Fi, g = s.Fi, s.g
    W1b, W2b, Wgb = I.gen_full_weights(700, h, F, t, sw)
    c = oracle.column_block(0, t, F)
    W1, W2 = bf16_dev(np.ascontiguousarray(W1b[:, c])), bf16_dev(np.ascontiguousarray(W2b[c, :]))
    Wg = bf16_dev(np.ascontiguousarray(Wgb[:, c])) if sw else None
    X, Y, A, U = empty_bf16(0, h), empty_bf16(0, h), empty_bf16(0, Fi), empty_bf16(0, Fi)
    G = empty_bf16(0, Fi) if sw else None
    assert B.workspace_bytes(s, False) == 0 and B.workspace_bytes(s, True) == 0
    B.tp_mlp_fwd_shard(s, X, W1, Wg, W2, Y, A, U, G)
    dY, dU, dX = empty_bf16(0, h), empty_bf16(0, g * Fi), empty_bf16(0, h)
    dW1, dW2, db2 = nan_f32(h, Fi), nan_f32(Fi, h), nan_f32(h)
    dWg = nan_f32(h, Fi) if sw else None
    B.tp_mlp_bwd_shard(s, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX, db2)
    torch.cuda.synchronize()
    z = np.zeros((0, h))
    ref = oracle.shard_backward(act, z, oracle.bf16_bits_to_f64(W1b[:, c]), oracle.bf16_bits_to_f64(W2b[c, :]), z,
                                oracle.bf16_bits_to_f64(Wgb[:, c]) if sw else None)
    np.testing.assert_array_equal(f64(dW1), ref["dW1"])
    np.testing.assert_array_equal(f64(dW2), ref["dW2"])
    if sw:
        np.testing.assert_array_equal(f64(dWg), ref["dWg"])
    np.testing.assert_array_equal(f64(db2), oracle.column_sum(z))
    # the per-step entry points agree
    for buf in (dW1, dW2, dWg):
        if buf is not None:
            buf.fill_(float("nan"))
    B.tp_mlp_wgrad_shard(s, X, A, dY, dU, dW1, dW2, dWg)
    torch.cuda.synchronize()
    assert not torch.any(dW1) and not torch.any(dW2) and (dWg is None or not torch.any(dWg))
    dW2.fill_(float("nan"))
    B.tp_mlp_down_bwd_shard(s, dY, W2, U, G, A, dU, dW2)
    for buf in (dW1, dWg):
        if buf is not None:
            buf.fill_(float("nan"))
    B.tp_mlp_up_bwd_shard(s, X, dU, W1, Wg, dX, dW1, dWg)
    torch.cuda.synchronize()
    assert not torch.any(dW1) and not torch.any(dW2) and (dWg is None or not torch.any(dWg))
    dW2.fill_(float("nan"))
    B.tp_mlp_down_wgrad_shard(s, A, dY, dW2)
    dW1.fill_(float("nan"))
    B.tp_mlp_up_wgrad_shard(s, X, dU, dW1, dWg)
    db2.fill_(float("nan"))
    B.tp_mlp_bias_grad(dY, db2, None)
    torch.cuda.synchronize()
    assert not torch.any(dW1) and not torch.any(dW2) and not torch.any(db2)
    # reductions of empty partials
    out = empty_bf16(0, h)
    B.tp_mlp_reduce_partials_local([empty_bf16(0, h) for _ in range(t)], out, bias=bf16_dev(I.gen_b2(700, h)))
    B.tp_mlp_reduce_scatter_local([empty_bf16(0, h) for _ in range(t)], out, 1)
    B.tp_mlp_all_gather_local([empty_bf16(0, h) for _ in range(t)], out)
    torch.cuda.synchronize()
    # and a non-empty group afterwards still matches the oracle
    run_group(701, 40, h, F, t, act, sw)


def test_empty_batch_attention_projections():
    print("[empty] attention", file=sys.stderr, flush=True)
    h, nh, nkv, d, t = 256, 8, 4, 64, 2
    s = B.make_attn_shape(0, h, nh, nkv, d, t, 0)
    Wqkv = bf16_dev(I.normal_bf16([702, 1], (h, s.qkv_cols), 0.02))
    Wo = bf16_dev(I.normal_bf16([702, 2], (s.q_cols, h), 0.02))
    X, QKV, O, Y = empty_bf16(0, h), empty_bf16(0, s.qkv_cols), empty_bf16(0, s.q_cols), empty_bf16(0, h)
    assert B.attn_workspace_bytes(s) == 0
    B.tp_attn_qkv_shard(s, X, Wqkv, QKV)
    B.tp_attn_out_shard(s, O, Wo, Y)
    dWo, dWqkv = nan_f32(s.q_cols, h), nan_f32(h, s.qkv_cols)
    B.tp_attn_out_bwd_shard(s, Y, O, Wo, empty_bf16(0, s.q_cols), dWo)
    B.tp_attn_qkv_bwd_shard(s, X, Wqkv, QKV, dWqkv, empty_bf16(0, h))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(dWo), OA.out_backward(np.zeros((0, h)), np.zeros((0, s.q_cols)), f64(Wo))[1])
    np.testing.assert_array_equal(f64(dWqkv),
                                  OA.qkv_backward(np.zeros((0, h)), f64(Wqkv), np.zeros((0, s.qkv_cols)))[1])


def test_empty_block_layernorm():
    print("[empty] layernorm", file=sys.stderr, flush=True)
    cols, t = 1032, 2
    gm, bt = bf16_dev(I.gen_ln_weight(703, cols)), bf16_dev(I.gen_ln_bias(703, cols))
    x, y = empty_bf16(0, cols), empty_bf16(0, cols)
    mean, rstd = torch.empty(0, dtype=F32, device="cuda"), torch.empty(0, dtype=F32, device="cuda")
    B.tp_sp_layernorm_fwd(x, gm, y, beta=bt, mean=mean, rstd=rstd)
    B.tp_sp_reduce_scatter_layernorm_local([empty_bf16(0, cols) for _ in range(t)], 0, empty_bf16(0, cols), gm, y,
                                           beta=bt, mean=mean, rstd=rstd)
    assert B.layernorm_bwd_workspace_bytes(0, cols) == 0
    dg, db = nan_f32(cols), nan_f32(cols)
    B.tp_sp_layernorm_bwd(x, gm, mean, rstd, empty_bf16(0, cols), empty_bf16(0, cols), dg, dbeta=db)
    torch.cuda.synchronize()
    _, rdg, rdb = OL.layer_norm_backward(np.zeros((0, cols)), np.zeros((0, cols)), f64(gm))
    np.testing.assert_array_equal(f64(dg), rdg)
    np.testing.assert_array_equal(f64(db), rdb)
    # a non-empty block afterwards, against the oracle
    rows = 24
    xb = I.normal_bf16([703, 5], (rows, cols))
    dyb = I.normal_bf16([703, 6], (rows, cols))
    xd, dyd = bf16_dev(xb), bf16_dev(dyb)
    y, dx = empty_bf16(rows, cols), empty_bf16(rows, cols)
    mean, rstd = torch.empty(rows, dtype=F32, device="cuda"), torch.empty(rows, dtype=F32, device="cuda")
    B.tp_sp_layernorm_fwd(xd, gm, y, beta=bt, mean=mean, rstd=rstd)
    ws = B.alloc_workspace(B.layernorm_bwd_workspace_bytes(rows, cols))
    B.tp_sp_layernorm_bwd(xd, gm, mean, rstd, dyd, dx, dg, dbeta=db, workspace=ws)
    torch.cuda.synchronize()
    rx, rdg, rdb = OL.layer_norm_backward(oracle.bf16_bits_to_f64(dyb), oracle.bf16_bits_to_f64(xb), f64(gm))
    assert_close("dx", f64(dx), rx)
    assert_close("dgamma", f64(dg), rdg)
    assert_close("dbeta", f64(db), rdb)
