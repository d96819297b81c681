"""The library's maximum sizes on the GPU, against the oracle.

* t = 64 ranks (the most a call takes) for the reduction, the reduce-scatter,
  the all-gather and the gradient sum: bit for bit on sums that are exact in
  float32.
* A shard whose activations are as large as one GEMM operand may be: A_i,
  U_i and dU_i are [131056, 16384] bf16, 4,294,443,008 bytes, just under the
  4 GiB - 256 B a 32-bit buffer descriptor addresses.  Forward and backward
  run at that size (every GEMM layout reads or writes it: the up-projection
  writes it, the down-projection and the input gradient read it along k,
  the weight gradients read it along m or n), so the largest 32-bit offsets
  are exercised.  Rows from both ends of the batch and sampled weight-
  gradient columns are compared with the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import assert_close, bf16_dev, f64

pytestmark = pytest.mark.gpu
MAX_T = 64


def exact_parts(seed, t, shape):
    """bf16 bits of small multiples of 1/8: any sum of 64 of them is exact in
    float32 and rounds to bf16 the same way on both sides."""
    rng = np.random.default_rng(seed)
    return [I.f32_to_bf16_bits(rng.integers(-32, 32, size=shape).astype(np.float32) / 8) for _ in range(t)]


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_sixty_four_ranks():
    print("[limits] t = 64", file=sys.stderr, flush=True)
    t, rows, cols = MAX_T, 3 * MAX_T, 1032
    pb = exact_parts(1300, t, (rows, cols))
    bb = I.f32_to_bf16_bits(np.random.default_rng(1301).integers(-8, 8, size=cols).astype(np.float32) / 4)
    parts, bias = [bf16_dev(p) for p in pb], bf16_dev(bb)
    pf = [oracle.bf16_bits_to_f64(p) for p in pb]
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local(parts, out, bias=bias)
    rs = torch.empty(rows // t, cols, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_scatter_local(parts, rs, t - 1, bias=bias)
    shards = [bf16_dev(p[:5]) for p in pb]
    ag = torch.empty(5 * t, cols, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_all_gather_local(shards, ag)
    grads = [torch.from_numpy(np.random.default_rng([1302, k]).standard_normal(cols).astype(np.float32)).cuda()
             for k in range(t)]
    gsum = torch.empty(cols, dtype=torch.float32, device="cuda")
    B.tp_sp_sum_grads_local(grads, gsum)
    torch.cuda.synchronize()
    full = oracle.reduce_partials(pf, oracle.bf16_bits_to_f64(bb))
    assert np.array_equal(bits(out), I.f32_to_bf16_bits(full.astype(np.float32)))
    blk = oracle.sequence_block(t - 1, t, rows)
    assert np.array_equal(bits(rs), I.f32_to_bf16_bits(full[blk].astype(np.float32)))
    assert np.array_equal(bits(ag), np.concatenate([p[:5] for p in pb]))
    # the float32 sum in rank order, against the float64 sum of the same values
    g64 = np.sum([g.cpu().numpy().astype(np.float64) for g in grads], axis=0)
    np.testing.assert_allclose(gsum.cpu().numpy(), g64, rtol=1e-5, atol=1e-5)


def test_activations_at_the_buffer_descriptor_limit():
    N, h, Fi = 131056, 64, 16384
    assert N * Fi * 2 == 4_294_443_008 and N * Fi * 2 <= 0xFFFFFF00
    print(f"[limits] N={N} h={h} F_i={Fi}: A, U, dU of {N * Fi * 2} bytes", file=sys.stderr, flush=True)
    act, wid = "gelu", 1310
    s = B.make_shape(N, h, Fi, 1, 0, act)
    Xb, dYb = I.gen_x(wid, N, h), I.gen_dy(wid, N, h)
    W1b, W2b, _ = I.gen_full_weights(wid, h, Fi, 1, False)
    X, dY, W1, W2 = bf16_dev(Xb), bf16_dev(dYb), bf16_dev(W1b), bf16_dev(W2b)
    e = dict(dtype=torch.bfloat16, device="cuda")
    Y, A, U, dU, dX = (torch.empty(N, h, **e), torch.empty(N, Fi, **e), torch.empty(N, Fi, **e),
                       torch.empty(N, Fi, **e), torch.empty(N, h, **e))
    dW1 = torch.empty(h, Fi, dtype=torch.float32, device="cuda")
    dW2 = torch.empty(Fi, h, dtype=torch.float32, device="cuda")
    B.tp_mlp_fwd_shard(s, X, W1, None, W2, Y, A, U, None)
    B.tp_mlp_bwd_shard(s, X, W1, None, W2, dY, A, U, None, dU, dW1, None, dW2, dX)
    torch.cuda.synchronize()
    # rows at both ends (the largest offsets) and in between
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1],
                                     np.random.default_rng(wid).choice(N, size=27, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Xf, dYf = oracle.bf16_bits_to_f64(Xb), oracle.bf16_bits_to_f64(dYb)
    W1f, W2f = oracle.bf16_bits_to_f64(W1b), oracle.bf16_bits_to_f64(W2b)
    fr = oracle.shard_forward(act, Xf[rows], W1f, W2f)
    br = oracle.shard_backward(act, Xf[rows], W1f, W2f, dYf[rows])
    assert_close("A rows", f64(A[ridx]), fr["A"])
    assert_close("U rows", f64(U[ridx]), fr["U"])
    assert_close("Y rows", f64(Y[ridx]), fr["Y"])
    assert_close("dU rows", f64(dU[ridx]), br["dU"])
    assert_close("dX rows", f64(dX[ridx]), br["dX"])
    # weight gradients sum over every token: sampled columns of dW1 (rows of
    # dW2) from the oracle's full-batch products restricted to them
    cols = np.sort(np.random.default_rng(wid + 1).choice(Fi, size=24, replace=False))
    U_c = Xf @ W1f[:, cols]
    A_c = oracle.act_forward(act, U_c)
    dA_c = dYf @ W2f[cols, :].T
    dU_c = oracle.act_backward(act, dA_c, U_c)
    assert_close("dW1 columns", f64(dW1)[:, cols], Xf.T @ dU_c)
    assert_close("dW2 rows", f64(dW2)[cols, :], A_c.T @ dYf)
