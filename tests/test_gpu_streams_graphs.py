"""Streams and HIP graphs.

Every entry point enqueues all of its work on the stream it is given.  The
test runs each path eagerly on a side stream, then captures the same calls
into a HIP graph on that stream: a launch on any other stream (the null
stream included) would break the capture.  The graph is replayed several
times, with eager work on the stream between replays (the outputs filled
with NaN by a fill kernel, then a full synchronisation), and every replay
must give the eager result bit for bit.  The library issues no memset and
allocates nothing, so its calls can be captured as they are.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import bf16_dev

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32
REPLAYS = 3


def capture_and_replay(run, outputs):
    """run() enqueues the calls on the current stream; outputs: the tensors
    they write."""
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    eager = [o.clone() for o in outputs]
    with torch.cuda.stream(s):
        for o in outputs:
            o.fill_(float("nan"))
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for k in range(REPLAYS):
        with torch.cuda.stream(s):
            for o in outputs:
                o.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, eager)):
            assert torch.equal(a, b), f"replay {k}: output {i} differs from the eager run"
    return eager


@pytest.mark.parametrize("N,act", [(1, "swiglu"), (16, "gelu"), (40, "swiglu"), (300, "relu")])
def test_mlp_shard_on_a_side_stream_and_in_a_graph(N, act):
    """Forward (one-token GEMVs, small-batch split-K products or wide
    tiles), backward with db2, and the reduction of both ranks' partials
    with the bias."""
    print(f"[graph] mlp N={N} act={act}", file=sys.stderr, flush=True)
    h, F, t = 520, 2 * 264, 2
    sw = act == "swiglu"
    wid = 1200 + N
    W1b, W2b, Wgb = I.gen_full_weights(wid, h, F, t, sw)
    s0 = B.make_shape(N, h, F, t, 0, act)
    s1 = B.make_shape(N, h, F, t, 1, act)
    Fi, g = s0.Fi, s0.g
    X, dY, b2 = bf16_dev(I.gen_x(wid, N, h)), bf16_dev(I.gen_dy(wid, N, h)), bf16_dev(I.gen_b2(wid, h))

    def shard(r):
        c = oracle.column_block(r, t, F)
        return (bf16_dev(np.ascontiguousarray(W1b[:, c])), bf16_dev(np.ascontiguousarray(W2b[c, :])),
                bf16_dev(np.ascontiguousarray(Wgb[:, c])) if sw else None)

    w0, w1 = shard(0), shard(1)
    e = dict(dtype=BF, device="cuda")
    Y0, Y1, Y = torch.empty(N, h, **e), torch.empty(N, h, **e), torch.empty(N, h, **e)
    A, U = torch.empty(N, Fi, **e), torch.empty(N, Fi, **e)
    G = torch.empty(N, Fi, **e) if sw else None
    A1 = torch.empty(N, Fi, **e)
    dU, dX = torch.empty(N, g * Fi, **e), torch.empty(N, h, **e)
    dW1, dW2 = torch.empty(h, Fi, dtype=F32, device="cuda"), torch.empty(Fi, h, dtype=F32, device="cuda")
    dWg = torch.empty(h, Fi, dtype=F32, device="cuda") if sw else None
    db2 = torch.empty(h, dtype=F32, device="cuda")
    ws_f = B.alloc_workspace(B.workspace_bytes(s0, False))
    ws_b = B.alloc_workspace(B.workspace_bytes(s0, True))

    def run():
        B.tp_mlp_fwd_shard(s0, X, w0[0], w0[2], w0[1], Y0, A, U, G, ws_f)
        B.tp_mlp_fwd_shard(s1, X, w1[0], w1[2], w1[1], Y1, A1, None, None, ws_f)
        B.tp_mlp_reduce_partials_local([Y0, Y1], Y, bias=b2)
        B.tp_mlp_bwd_shard(s0, X, w0[0], w0[2], w0[1], dY, A, U, G, dU, dW1, dWg, dW2, dX, db2, ws_b)

    outs = [o for o in (Y0, Y1, Y, A, U, G, A1, dU, dX, dW1, dWg, dW2, db2) if o is not None]
    eager = capture_and_replay(run, outs)
    # the eager result is the library's: checked against the oracle once here
    Xf, W1f, W2f = oracle.bf16_bits_to_f64(I.gen_x(wid, N, h)), oracle.bf16_bits_to_f64(W1b), \
        oracle.bf16_bits_to_f64(W2b)
    Yref, _ = oracle.tp_forward(act, Xf, W1f, W2f, t, Wg=oracle.bf16_bits_to_f64(Wgb) if sw else None,
                                b2=oracle.bf16_bits_to_f64(I.gen_b2(wid, h)))
    y = eager[2].float().cpu().numpy().astype(np.float64)
    assert np.linalg.norm(y - Yref) / np.linalg.norm(Yref) <= 5e-3


def test_layernorm_and_attention_on_a_side_stream_and_in_a_graph():
    """The fused reduce-scatter + LayerNorm, its backward (one-pass form at
    4096 rows), and the attention projections with both backwards
    (small-batch and wide)."""
    print("[graph] layernorm + attention", file=sys.stderr, flush=True)
    t, rows, cols = 2, 8192, 520
    n = rows // t
    e = dict(dtype=BF, device="cuda")
    parts = [bf16_dev(I.normal_bf16([1250, k], (rows, cols))) for k in range(t)]
    gm, bt = bf16_dev(I.gen_ln_weight(1250, cols)), bf16_dev(I.gen_ln_bias(1250, cols))
    res, dy = bf16_dev(I.normal_bf16([1250, 5], (n, cols))), bf16_dev(I.normal_bf16([1250, 6], (n, cols)))
    z, y, dx = torch.empty(n, cols, **e), torch.empty(n, cols, **e), torch.empty(n, cols, **e)
    mean, rstd = torch.empty(n, dtype=F32, device="cuda"), torch.empty(n, dtype=F32, device="cuda")
    dg, db = torch.empty(cols, dtype=F32, device="cuda"), torch.empty(cols, dtype=F32, device="cuda")
    ws_ln = B.alloc_workspace(B.layernorm_bwd_workspace_bytes(n, cols))
    h, nh, nkv, d = 512, 8, 4, 64
    # 8 tokens: split-K forward and backward; 96: split-K forward, wide backward
    shapes = [B.make_attn_shape(Na, h, nh, nkv, d, t, 1) for Na in (8, 96)]
    Wqkv = bf16_dev(I.normal_bf16([1251, 1], (h, shapes[0].qkv_cols), 0.02))
    Wo = bf16_dev(I.normal_bf16([1251, 2], (shapes[0].q_cols, h), 0.02))
    att = []
    for sa in shapes:
        Na = sa.n_tokens
        Xa = bf16_dev(I.normal_bf16([1251, 3, Na], (Na, h)))
        Oa = bf16_dev(I.normal_bf16([1251, 4, Na], (Na, sa.q_cols)))
        att.append((sa, Xa, Oa, torch.empty(Na, sa.qkv_cols, **e), torch.empty(Na, h, **e),
                    B.alloc_workspace(B.attn_workspace_bytes(sa))))
    # backward buffers: dY and dQKV in; dO, dW_o, dX, dW_qkv out
    bwd = []
    for sa in shapes:
        Na = sa.n_tokens
        bwd.append((bf16_dev(I.normal_bf16([1251, 5, Na], (Na, h))),
                    bf16_dev(I.normal_bf16([1251, 6, Na], (Na, sa.qkv_cols))),
                    torch.empty(Na, sa.q_cols, **e), torch.empty(sa.q_cols, h, dtype=F32, device="cuda"),
                    torch.empty(Na, h, **e), torch.empty(h, sa.qkv_cols, dtype=F32, device="cuda")))

    def run():
        B.tp_sp_reduce_scatter_layernorm_local(parts, 1, z, gm, y, residual=res, beta=bt, mean=mean, rstd=rstd)
        B.tp_sp_layernorm_bwd(z, gm, mean, rstd, dy, dx, dg, dbeta=db, workspace=ws_ln)
        for (sa, Xa, Oa, QKV, Ya, wsa), (dYa, dQa, dOa, dWoa, dXa, dWa) in zip(att, bwd):
            B.tp_attn_qkv_shard(sa, Xa, Wqkv, QKV, workspace=wsa)
            B.tp_attn_out_shard(sa, Oa, Wo, Ya, workspace=wsa)
            B.tp_attn_out_bwd_shard(sa, dYa, Oa, Wo, dOa, dWoa)
            B.tp_attn_qkv_bwd_shard(sa, Xa, Wqkv, dQa, dWa, dXa)

    outs = [z, y, mean, rstd, dx, dg, db] + [o for a in att for o in (a[3], a[4])] + \
        [o for b in bwd for o in b[2:]]
    capture_and_replay(run, outs)
