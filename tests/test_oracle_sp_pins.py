"""Pins of the oracle's sequence-parallel boundary functions.

The reduce-scatter and all-gather that replace the tensor-parallel region's
all-reduce under sequence parallelism ("Tensor and sequence parallelism",
section "Sequence parallelism") are tied to brute force on tiny inputs, to the
decomposition of an all-reduce into a reduce-scatter followed by an
all-gather that the page's section relies on, and to an independent float64 torch computation of the unsplit block at the shape of
that page's TP=4 + sequence-parallel check (S=8, H=16, FFN=64): LayerNorm on
each rank's rows, all-gather, the sharded MLP, reduce-scatter with the output
bias once and the residual, against the unsplit x + MLP(LayerNorm(x)) + b2.
"""
import math

import numpy as np
import pytest

import oracle


def test_sequence_block_matches_check_script_rows():
    S, t = 8, 4
    # contiguous row blocks of S / t rows each, rank 0 lowest (the sequence
    # split of the TP=4 check, "Tensor and sequence parallelism", "The
    # implementation")
    for r in range(t):
        assert oracle.sequence_block(r, t, S) == slice(r * S // t, (r + 1) * S // t)
    with pytest.raises(ValueError):
        oracle.sequence_block(0, 3, 8)
    with pytest.raises(ValueError):
        oracle.sequence_block(4, 4, 8)


@pytest.mark.parametrize("rank", [0, 1, 2])
def test_reduce_scatter_brute_force(rank):
    rng = np.random.default_rng(7 + rank)
    t, rows, cols = 3, 6, 4
    P = [rng.standard_normal((rows, cols)) for _ in range(t)]
    b = rng.standard_normal(cols)
    n = rows // t
    res = rng.standard_normal((n, cols))
    want = [[0.0] * cols for _ in range(n)]
    for i in range(n):
        for c in range(cols):
            acc = 0.0
            for k in range(t):
                acc += P[k][rank * n + i][c]
            want[i][c] = acc + b[c] + res[i][c]
    got = oracle.reduce_scatter(P, rank, bias=b, residual=res)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-15, atol=1e-15)
    # without bias or residual: the plain partial sum of the rank's rows
    got0 = oracle.reduce_scatter(P, rank)
    np.testing.assert_allclose(got0, sum(p[rank * n:(rank + 1) * n] for p in P), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("t", [2, 4, 8])
def test_all_reduce_is_reduce_scatter_then_all_gather(t):
    """Summing every rank's partials and keeping one row block per rank,
    then concatenating the blocks, gives the full all-reduce result ("Tensor
    and sequence parallelism", section "Sequence parallelism": the two
    collectives together move what the one all-reduce moves)."""
    rng = np.random.default_rng(t)
    rows, cols = 4 * t, 16
    P = [rng.standard_normal((rows, cols)) for _ in range(t)]
    b = rng.standard_normal(cols)
    full = oracle.reduce_partials(P, b)
    pieces = [oracle.reduce_scatter(P, r, bias=b) for r in range(t)]
    assert np.array_equal(oracle.all_gather(pieces), full)


def test_all_gather_inverts_the_sequence_split():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((12, 5))
    t = 3
    shards = [X[oracle.sequence_block(r, t, 12)] for r in range(t)]
    assert np.array_equal(oracle.all_gather(shards), X)
    # rank order matters: a rotated gather is a different matrix
    assert not np.array_equal(oracle.all_gather(shards[1:] + shards[:1]), X)


def test_bias_per_rank_before_reduce_scatter_fails():
    """Adding the output bias on every rank's partial before the reduction
    counts it t times ("Tensor Parallelism's Communication Boundary")."""
    rng = np.random.default_rng(11)
    t, rows, cols = 4, 8, 8
    P = [rng.standard_normal((rows, cols)) for _ in range(t)]
    b = rng.standard_normal(cols)
    once = oracle.reduce_scatter(P, 1, bias=b)
    wrong = oracle.reduce_scatter([p + b[None, :] for p in P], 1)
    np.testing.assert_allclose(wrong - once, np.tile((t - 1) * b, (rows // t, 1)), rtol=1e-12, atol=1e-12)
    assert not np.allclose(wrong, once)


def _layer_norm_torch(x, w):
    import torch
    import torch.nn.functional as F
    return F.layer_norm(torch.from_numpy(x), (x.shape[1],), weight=torch.from_numpy(w)).numpy()


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_sequence_parallel_block_matches_unsplit_on_check_shape(act):
    """S=8, H=16, FFN=64, t=4 (the page's check): per rank, LayerNorm of its
    S/t rows; all-gather; each rank's shard of the MLP; reduce-scatter with
    the output bias once and the residual x added on the rank's rows.  Equals
    the rows of the unsplit x + MLP(LayerNorm(x)) + b2 computed by torch in
    float64.  The backward mirror: the output gradient's sequence blocks are
    all-gathered, each rank's partial input gradient of the MLP is
    reduce-scattered, and each rank's block equals the unsplit block's input
    gradient rows (torch autograd)."""
    import torch
    rng = np.random.default_rng(2024)
    S, H, FFN, t = 8, 16, 64, 4
    x = rng.standard_normal((S, H))
    lw = 1.0 + 0.1 * rng.standard_normal(H)
    W1 = rng.standard_normal((H, FFN)) / math.sqrt(H)
    W2 = rng.standard_normal((FFN, H)) / math.sqrt(FFN)
    Wg = rng.standard_normal((H, FFN)) / math.sqrt(H) if act == "swiglu" else None
    b2 = 0.1 * rng.standard_normal(H)

    # unsplit reference, float64 torch
    xt = torch.from_numpy(x)
    ht = torch.nn.functional.layer_norm(xt, (H,), weight=torch.from_numpy(lw)).requires_grad_(True)
    W1t, W2t = torch.from_numpy(W1), torch.from_numpy(W2)
    if act == "gelu":
        At = torch.nn.functional.gelu(ht @ W1t)
    else:
        At = torch.nn.functional.silu(ht @ torch.from_numpy(Wg)) * (ht @ W1t)
    yt = xt + At @ W2t + torch.from_numpy(b2)
    dy = rng.standard_normal((S, H))
    (yt * torch.from_numpy(dy)).sum().backward()
    y_ref, dh_ref = yt.detach().numpy(), ht.grad.numpy()

    # sequence-parallel composition through the oracle
    blocks = [oracle.sequence_block(r, t, S) for r in range(t)]
    h_full = oracle.all_gather([_layer_norm_torch(x[b], lw) for b in blocks])
    partials = []
    for r in range(t):
        W1_i, W2_i, Wg_i = oracle.shard_weights(W1, W2, r, t, Wg)
        partials.append(oracle.shard_forward(act, h_full, W1_i, W2_i, Wg_i)["Y"])
    for r in range(t):
        y_r = oracle.reduce_scatter(partials, r, bias=b2, residual=x[blocks[r]])
        np.testing.assert_allclose(y_r, y_ref[blocks[r]], rtol=1e-12, atol=1e-12)

    dy_full = oracle.all_gather([dy[b] for b in blocks])
    dX_parts = []
    for r in range(t):
        W1_i, W2_i, Wg_i = oracle.shard_weights(W1, W2, r, t, Wg)
        dX_parts.append(oracle.shard_backward(act, h_full, W1_i, W2_i, dy_full, Wg_i)["dX"])
    for r in range(t):
        np.testing.assert_allclose(oracle.reduce_scatter(dX_parts, r), dh_ref[blocks[r]], rtol=1e-11, atol=1e-12)
