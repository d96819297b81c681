"""GPU parity of the attention block's tensor-parallel projections against
the fp64 oracle (oracle/attn.py), through the C ABI.

Every rank of a group runs its QKV projection and output projection forward
and both backwards; the attention core's output O and its gradient dQKV are
seeded synthetic inputs (the core is not part of this path).  Checked per
rank: QKV_i, Y_i, dO_i, dWo_i, dX_i, dWqkv_i; summed over ranks: Y and dX
(through the library's reduce), the full dW_q, dW_k, dW_v (a replicated
key/value head's gradient summed over its replicas).  Shapes cover plain
multi-head, grouped-query with key/value heads split across ranks and
replicated on several ranks, ragged token counts, and the GPT-3-scale and
Llama-3-70B-scale per-rank widths with sampled rows and columns.  Input
gradients whose tile grid fills at most half the CUs run split along k
(float32 slice partials kept in the weight gradient's storage until it is
computed): the GPT-3-scale dO and a ragged two-slice case; one case takes
the unsplit fallback when that storage is too small.  With
1 <= N <= 128 tokens the forward projections take the small-batch path
(split-K products streaming each weight once), and so do the backward's
input gradients dO and dX (their partials kept in dW_o's and dW_qkv's
storage); those token counts are covered for several head layouts and at
the 70B per-rank widths, and the deferred pair stays bitwise equal to the
plain backward calls there too.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import attn
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import assert_close, bf16_dev, f64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gen_attn(wid, N, h, nh, nkv, d):
    """bf16 bit patterns: X, W_q, W_k, W_v, W_o, O (the core's output), dY and
    dQKV pieces (dQ for all query heads, dK and dV per rank: each replica of a
    key/value head gets its own gradient share)."""
    s = I.WEIGHT_SIGMA
    return dict(X=I.normal_bf16([wid, 50], (N, h)),
                Wq=I.normal_bf16([wid, 51], (h, nh * d), s), Wk=I.normal_bf16([wid, 52], (h, nkv * d), s),
                Wv=I.normal_bf16([wid, 53], (h, nkv * d), s), Wo=I.normal_bf16([wid, 54], (nh * d, h), s),
                O=I.normal_bf16([wid, 55], (N, nh * d)), dY=I.normal_bf16([wid, 56], (N, h)),
                dQ=I.normal_bf16([wid, 57], (N, nh * d)))


def run_attn_group(wid, N, h, nh, nkv, d, t, rows=None, ncols=None):
    say(f"[attn] wid={wid} N={N} h={h} heads={nh} kv={nkv} d={d} t={t}")
    g = gen_attn(wid, N, h, nh, nkv, d)
    f = oracle.bf16_bits_to_f64
    bf = dict(dtype=torch.bfloat16, device="cuda")
    Xd, dYd = bf16_dev(g["X"]), bf16_dev(g["dY"])
    Yparts, dXparts, dWqkv_gpu, ranks = [], [], [], []
    for r in range(t):
        s = B.make_attn_shape(N, h, nh, nkv, d, t, r)
        Wqkv_b, Wo_b = attn.attn_shard_weights(g["Wq"], g["Wk"], g["Wv"], g["Wo"], r, t, nh, nkv, d)
        qh, kh = attn.query_heads(r, t, nh), attn.kv_heads(r, t, nh, nkv)
        q0, q1 = qh[0] * d, (qh[-1] + 1) * d
        O_b = np.ascontiguousarray(g["O"][:, q0:q1])
        dK_b = I.normal_bf16([wid, 60, r], (N, len(kh) * d))
        dV_b = I.normal_bf16([wid, 61, r], (N, len(kh) * d))
        dQKV_b = np.ascontiguousarray(np.concatenate([g["dQ"][:, q0:q1], dK_b, dV_b], axis=1))
        assert Wqkv_b.shape == (h, s.qkv_cols) and Wo_b.shape == (s.q_cols, h)
        Wqkv, Wo = bf16_dev(np.ascontiguousarray(Wqkv_b)), bf16_dev(np.ascontiguousarray(Wo_b))
        QKV = torch.empty(N, s.qkv_cols, **bf)
        Y = torch.empty(N, h, **bf)
        dO = torch.empty(N, s.q_cols, **bf)
        dWo = torch.empty(s.q_cols, h, dtype=torch.float32, device="cuda")
        dWqkv = torch.empty(h, s.qkv_cols, dtype=torch.float32, device="cuda")
        dX = torch.empty(N, h, **bf)
        ws = B.alloc_workspace(B.attn_workspace_bytes(s))   # 1 <= N <= 128: small-batch path
        B.tp_attn_qkv_shard(s, Xd, Wqkv, QKV, workspace=ws)
        B.tp_attn_out_shard(s, bf16_dev(O_b), Wo, Y, workspace=ws)
        B.tp_attn_out_bwd_shard(s, dYd, bf16_dev(O_b), Wo, dO, dWo)
        B.tp_attn_qkv_bwd_shard(s, Xd, Wqkv, bf16_dev(dQKV_b), dWqkv, dX)
        Yparts.append(Y)
        dXparts.append(dX)
        dWqkv_gpu.append(dWqkv)
        ranks.append((Wqkv_b, Wo_b, O_b, dQKV_b, QKV, dO, dWo))
    Ysum, dXsum = torch.empty(N, h, **bf), torch.empty(N, h, **bf)
    B.tp_mlp_reduce_partials_local(Yparts, Ysum)
    B.tp_mlp_reduce_partials_local(dXparts, dXsum)
    torch.cuda.synchronize()

    ri = np.arange(N) if rows is None else rows
    Xr, dYr = f(g["X"][ri]), f(g["dY"][ri])
    Yref = np.zeros((len(ri), h))
    dXref = np.zeros((len(ri), h))
    dWqkv_ref = []
    for r, (Wqkv_b, Wo_b, O_b, dQKV_b, QKV, dO, dWo) in enumerate(ranks):
        Wqkv_f, Wo_f = f(Wqkv_b), f(Wo_b)
        assert_close(f"QKV[{r}]", f64(QKV)[ri], attn.qkv_forward(Xr, Wqkv_f))
        Y_r = attn.out_forward(f(O_b[ri]), Wo_f)
        assert_close(f"Y_i[{r}]", f64(Yparts[r])[ri], Y_r)
        Yref += Y_r
        dO_r, _ = attn.out_backward(dYr, f(O_b[ri]), Wo_f)
        assert_close(f"dO[{r}]", f64(dO)[ri], dO_r)
        dX_r, _ = attn.qkv_backward(Xr, Wqkv_f, f(dQKV_b[ri]))
        assert_close(f"dX_i[{r}]", f64(dXparts[r])[ri], dX_r)
        dXref += dX_r
        # weight gradients need every token: full reference, or sampled columns
        rng = np.random.default_rng(wid + r)
        cq = np.arange(h) if ncols is None else np.sort(rng.choice(h, size=ncols, replace=False))
        _, dWo_ref = attn.out_backward(f(g["dY"][:, cq]), f(O_b), Wo_f[:, cq])
        assert_close(f"dWo[{r}]", f64(dWo)[:, cq], dWo_ref)
        w = Wqkv_b.shape[1]
        cw = np.arange(w) if ncols is None else np.sort(rng.choice(w, size=ncols, replace=False))
        dW_ref = f(g["X"]).T @ f(dQKV_b[:, cw])
        assert_close(f"dWqkv[{r}]", f64(dWqkv_gpu[r])[:, cw], dW_ref)
        if ncols is None:
            dWqkv_ref.append(f64(dWqkv_gpu[r]))
    assert_close("Y", f64(Ysum)[ri], Yref)
    assert_close("dX", f64(dXsum)[ri], dXref)
    if ncols is None:
        # the full-model gradients: replicas of a key/value head summed
        full = [f(g["X"]).T @ f(rk[3]) for rk in ranks]
        want = attn.gather_qkv_weight_grads(full, t, nh, nkv, d)
        got = attn.gather_qkv_weight_grads(dWqkv_ref, t, nh, nkv, d)
        for name, a, b in zip(("dWq", "dWk", "dWv"), got, want):
            assert_close(name, a, b)


# (wid, N, h, n_heads, n_kv, head_dim, t)
GROUPS = [
    (701, 128, 512, 8, 8, 64, 2),      # multi-head, t = 2
    (702, 200, 264, 8, 2, 64, 4),      # 2 key/value heads over 4 ranks: each replicated on 2
    (703, 77, 384, 16, 8, 32, 4),      # grouped-query, key/value heads split 2 per rank
    (704, 300, 1032, 16, 4, 128, 8),   # 4 key/value heads over 8 ranks
    (705, 33, 136, 4, 1, 64, 1),       # multi-query
    # dO = dY @ W_o^T has few tiles here and runs split along k: 2 slices of
    # 1088, the last ending mid k-tile (2056 = 32 k-tiles + 8)
    (706, 333, 2056, 8, 8, 64, 4),
    # a k-split would be chosen but dW_o (the partials' scratch) is too small
    # for 2 x 4096 x 128 floats: one unsplit pass
    (707, 4096, 2048, 8, 2, 64, 4),
    # unsplit, 96 output tiles per forward projection, ragged in h
    (708, 2000, 2824, 16, 4, 128, 1),
]


@pytest.mark.parametrize("case", GROUPS, ids=[f"N{c[1]}_h{c[2]}_H{c[3]}_kv{c[4]}_d{c[5]}_t{c[6]}" for c in GROUPS])
def test_attn_projections_match_oracle(case):
    run_attn_group(*case)


@pytest.mark.parametrize("name,N,h,nh,nkv,d,t", [
    ("gpt3_attn_t8", 2048, 12288, 96, 96, 128, 8),        # the GPT-3-scale shape of "The Communication Pattern"
    ("llama3_70b_attn_t4", 4096, 8192, 64, 8, 128, 4),     # Llama-3-70B heads, t = 4
])
def test_attn_projections_full_size_sampled(name, N, h, nh, nkv, d, t):
    """Every rank at the per-rank widths of the named model; 32 sampled token
    rows for the row-local outputs and 48 sampled columns for the weight
    gradients are compared with the oracle."""
    rng = np.random.default_rng(len(name))
    rows = np.sort(rng.choice(N, size=32, replace=False))
    run_attn_group(800 + t, N, h, nh, nkv, d, t, rows=rows, ncols=48)


# small batches: the forward projections on the split-K path, the backward on
# the wide tiles; (wid, N, h, n_heads, n_kv, head_dim, t)
SMALL = [
    (711, 1, 1032, 8, 8, 64, 2),       # one token
    (712, 2, 264, 8, 2, 64, 4),        # replicated key/value heads
    (713, 16, 520, 16, 8, 32, 4),
    (714, 33, 1544, 16, 4, 128, 8),    # ragged: 33 rows, h tail past 256-column strips
    (715, 64, 136, 4, 1, 64, 1),       # multi-query, the 64-row tile's largest N
    (717, 100, 520, 8, 4, 64, 2),      # the 128-row tile, ragged rows
    (718, 128, 264, 8, 8, 64, 2),      # the path's largest N
    (716, 129, 264, 8, 8, 64, 2),      # just past it: wide tiles
]


def _small_sweep(seed=20261204, n=8):
    """Seeded few-token head layouts, h large enough (1032-4104) that the
    backward's input gradients take the split-K kernel at most of them."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        t = int(rng.choice([1, 2, 4]))
        nkv = int(rng.choice([1, 2, 4, 8]))
        nh = nkv * int(rng.choice([1, 2, 4]))
        if nh % t or (nkv % t and t % nkv):
            continue
        d = 8 * int(rng.integers(4, 17))
        h = 8 * int(rng.integers(129, 514))
        N = int(rng.integers(1, 65))
        out.append((740 + len(out), N, h, nh, nkv, d, t))
    return out


SMALL += _small_sweep()


@pytest.mark.parametrize("case", SMALL, ids=[f"N{c[1]}_h{c[2]}_H{c[3]}_kv{c[4]}_t{c[6]}" for c in SMALL])
def test_attn_small_batch_matches_oracle(case):
    run_attn_group(*case)


@pytest.mark.parametrize("N", [8, 32, 128])
def test_attn_small_batch_llama3_70b_widths(N):
    """Every rank of the 70B attention block (t = 4: 16 query heads and 2
    key/value heads of 128 per rank) at a decode batch of N tokens; all rows,
    48 sampled weight-gradient columns."""
    run_attn_group(820 + N, N, 8192, 64, 8, 128, 4, ncols=48)



@pytest.mark.parametrize("N,h,nh,nkv,d,t", [(2048, 12288, 96, 96, 128, 8), (333, 2056, 8, 8, 64, 4),
                                            (8, 8192, 64, 8, 128, 4), (100, 1032, 8, 4, 64, 2),
                                            (1, 520, 8, 8, 64, 2)])
def test_deferred_out_wgrad_equals_the_separate_calls(N, h, nh, nkv, d, t):
    """tp_attn_out_dgrad_shard (dO alone, k-split partials in a workspace)
    and tp_attn_qkv_bwd_out_wgrad_shard (dX, dWqkv and the deferred dWo in
    one call: one mixed launch at the GPT-3 per-rank shape, three at the
    333-token one; with up to 128 tokens the split-K dX and both weight
    gradients in one launch) give bitwise what tp_attn_out_bwd_shard and
    tp_attn_qkv_bwd_shard give; those are checked against the oracle
    above."""
    say(f"[attn deferred] N={N} h={h} heads={nh} kv={nkv} d={d} t={t}")
    s = B.make_attn_shape(N, h, nh, nkv, d, t, t - 1)
    qc, wc = s.q_cols, s.qkv_cols
    sig = I.WEIGHT_SIGMA
    X, dY = bf16_dev(I.normal_bf16([730, 0], (N, h))), bf16_dev(I.normal_bf16([730, 1], (N, h)))
    Wqkv, Wo = bf16_dev(I.normal_bf16([730, 2], (h, wc), sig)), bf16_dev(I.normal_bf16([730, 3], (qc, h), sig))
    O, dQKV = bf16_dev(I.normal_bf16([730, 4], (N, qc))), bf16_dev(I.normal_bf16([730, 5], (N, wc)))
    bf, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")
    dO_a, dO_b = torch.empty(N, qc, **bf), torch.empty(N, qc, **bf)
    dWo_a, dWo_b = torch.empty(qc, h, **f32), torch.empty(qc, h, **f32)
    dW_a, dW_b = torch.empty(h, wc, **f32), torch.empty(h, wc, **f32)
    dX_a, dX_b = torch.empty(N, h, **bf), torch.empty(N, h, **bf)
    B.tp_attn_out_bwd_shard(s, dY, O, Wo, dO_a, dWo_a)
    B.tp_attn_qkv_bwd_shard(s, X, Wqkv, dQKV, dW_a, dX_a)
    ws = B.alloc_workspace(B.attn_out_dgrad_workspace_bytes(s))
    B.tp_attn_out_dgrad_shard(s, dY, Wo, dO_b, workspace=ws)
    B.tp_attn_qkv_bwd_out_wgrad_shard(s, X, Wqkv, dQKV, dY, O, dW_b, dX_b, dWo_b)
    torch.cuda.synchronize()
    for name, a, b in (("dO", dO_a, dO_b), ("dWo", dWo_a, dWo_b), ("dWqkv", dW_a, dW_b), ("dX", dX_a, dX_b)):
        assert torch.equal(a, b), f"{name} differs"
