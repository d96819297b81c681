"""Pins of the attention-projection oracle (oracle/attn.py).

Tied to: the head-to-rank assignments the pages describe (query heads in
blocks, key/value heads by group, replicated when there are fewer of them
than ranks: the closing exercise of "Tensor and sequence parallelism", 8
key/value heads at t = 16), brute force on a tiny shape, the split-equals-
unsplit invariants of "02 -- Tensor Parallelism" ("The attention pairing":
the partial outputs add up to the unsplit output projection), and torch
float64 autograd of the unsplit projections for every gradient, with a
replicated key/value head's gradient summed over its replicas.
"""
import numpy as np
import pytest

from oracle import attn


def test_heads_llama3_70b_t4_and_replication_at_t16():
    n_heads, n_kv = 64, 8
    # t = 4: 16 query heads and 2 key/value heads per rank
    for r in range(4):
        assert list(attn.query_heads(r, 4, n_heads)) == list(range(16 * r, 16 * r + 16))
        assert list(attn.kv_heads(r, 4, n_heads, n_kv)) == [2 * r, 2 * r + 1]
    # t = 16 > 8 key/value heads: each is replicated on t / n_kv = 2 ranks
    holders = {}
    for r in range(16):
        kv = list(attn.kv_heads(r, 16, n_heads, n_kv))
        assert len(kv) == 1
        holders.setdefault(kv[0], []).append(r)
    assert sorted(holders) == list(range(8)) and all(len(v) == 2 for v in holders.values())


@pytest.mark.parametrize("t,n_heads,n_kv", [(1, 8, 8), (2, 8, 2), (4, 64, 8), (8, 64, 8), (16, 64, 8),
                                            (4, 8, 1), (8, 32, 4)])
def test_each_rank_holds_the_groups_of_its_query_heads(t, n_heads, n_kv):
    """Query head j belongs to key/value group j // (n_heads / n_kv); every
    rank must hold exactly the groups of its own query heads."""
    per_group = n_heads // n_kv
    for r in range(t):
        groups = sorted({j // per_group for j in attn.query_heads(r, t, n_heads)})
        assert list(attn.kv_heads(r, t, n_heads, n_kv)) == groups


def test_invalid_head_splits():
    with pytest.raises(ValueError):
        attn.check_heads(3, 64, 8)       # 64 % 3
    with pytest.raises(ValueError):
        attn.check_heads(4, 12, 6)       # 6 key/value heads over 4 ranks: neither blocks nor replicas
    with pytest.raises(ValueError):
        attn.check_heads(2, 10, 4)       # 10 % 4
    with pytest.raises(ValueError):
        attn.query_heads(4, 4, 64)


def _model(rng, N, h, n_heads, n_kv, d):
    X = rng.standard_normal((N, h))
    Wq = rng.standard_normal((h, n_heads * d)) / np.sqrt(h)
    Wk = rng.standard_normal((h, n_kv * d)) / np.sqrt(h)
    Wv = rng.standard_normal((h, n_kv * d)) / np.sqrt(h)
    Wo = rng.standard_normal((n_heads * d, h)) / np.sqrt(n_heads * d)
    return X, Wq, Wk, Wv, Wo


def test_qkv_brute_force_tiny():
    rng = np.random.default_rng(1)
    N, h, n_heads, n_kv, d, t = 3, 4, 4, 2, 2, 2
    X, Wq, Wk, Wv, Wo = _model(rng, N, h, n_heads, n_kv, d)
    for r in range(t):
        Wqkv, Wo_r = attn.attn_shard_weights(Wq, Wk, Wv, Wo, r, t, n_heads, n_kv, d)
        got = attn.qkv_forward(X, Wqkv)
        # columns by hand: query heads 2r, 2r+1; key/value head r
        cols = [Wq[:, 2 * d * r + c] for c in range(2 * d)] + [Wk[:, d * r + c] for c in range(d)] + \
               [Wv[:, d * r + c] for c in range(d)]
        for i in range(N):
            for j, wcol in enumerate(cols):
                acc = 0.0
                for k in range(h):
                    acc += X[i, k] * wcol[k]
                assert abs(got[i, j] - acc) <= 1e-14
        assert np.array_equal(Wo_r, Wo[2 * d * r:2 * d * (r + 1), :])


@pytest.mark.parametrize("t,n_heads,n_kv", [(2, 8, 2), (4, 16, 8), (4, 8, 2), (8, 16, 2)])
def test_split_equals_unsplit(t, n_heads, n_kv):
    rng = np.random.default_rng(10 + t + n_kv)
    N, h, d = 6, 24, 4
    X, Wq, Wk, Wv, Wo = _model(rng, N, h, n_heads, n_kv, d)
    O = rng.standard_normal((N, n_heads * d))
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    Y = np.zeros((N, h))
    for r in range(t):
        Wqkv, Wo_r = attn.attn_shard_weights(Wq, Wk, Wv, Wo, r, t, n_heads, n_kv, d)
        qkv = attn.qkv_forward(X, Wqkv)
        qh, kh = attn.query_heads(r, t, n_heads), attn.kv_heads(r, t, n_heads, n_kv)
        nq, nk = len(qh) * d, len(kh) * d
        np.testing.assert_allclose(qkv[:, :nq], Q[:, qh[0] * d:(qh[-1] + 1) * d], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(qkv[:, nq:nq + nk], K[:, kh[0] * d:(kh[-1] + 1) * d], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(qkv[:, nq + nk:], V[:, kh[0] * d:(kh[-1] + 1) * d], rtol=1e-13, atol=1e-13)
        Y = Y + attn.out_forward(O[:, qh[0] * d:(qh[-1] + 1) * d], Wo_r)
    np.testing.assert_allclose(Y, O @ Wo, rtol=1e-12, atol=1e-12)


def test_wrong_rows_of_the_output_projection_fail():
    """Taking the output projection's rows of another rank's heads (or
    splitting it along its output dimension) does not add up to O @ W_o."""
    rng = np.random.default_rng(5)
    N, h, n_heads, n_kv, d, t = 5, 16, 8, 8, 2, 2
    X, Wq, Wk, Wv, Wo = _model(rng, N, h, n_heads, n_kv, d)
    O = rng.standard_normal((N, n_heads * d))
    half = n_heads * d // t
    wrong = O[:, :half] @ Wo[half:, :] + O[:, half:] @ Wo[:half, :]
    assert not np.allclose(wrong, O @ Wo)


@pytest.mark.parametrize("t,n_heads,n_kv", [(2, 8, 4), (4, 8, 2), (8, 16, 4)])
def test_backward_against_autograd(t, n_heads, n_kv):
    """Loss <dY, O W_o> + <GQ, X W_q> + <GK, X W_k> + <GV, X W_v> (the G's
    stand for the attention core's gradients).  A replicated key/value head's
    gradient GK is split between its replicas (any split that adds up to it);
    summed over ranks, the oracle's pieces equal autograd of the unsplit
    projections."""
    import torch
    rng = np.random.default_rng(20 + t)
    N, h, d = 5, 16, 4
    X, Wq, Wk, Wv, Wo = _model(rng, N, h, n_heads, n_kv, d)
    O = rng.standard_normal((N, n_heads * d))
    dY = rng.standard_normal((N, h))
    GQ, GK, GV = (rng.standard_normal((N, c)) for c in (n_heads * d, n_kv * d, n_kv * d))
    T = {k: torch.tensor(v, requires_grad=True) for k, v in dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, O=O).items()}
    L = (torch.from_numpy(dY) * (T["O"] @ T["Wo"])).sum() + (torch.from_numpy(GQ) * (T["X"] @ T["Wq"])).sum() + \
        (torch.from_numpy(GK) * (T["X"] @ T["Wk"])).sum() + (torch.from_numpy(GV) * (T["X"] @ T["Wv"])).sum()
    L.backward()
    g = {k: v.grad.numpy() for k, v in T.items()}

    # each replica of a key/value head receives a random share of its gradient
    holders = {}
    for r in range(t):
        for j in attn.kv_heads(r, t, n_heads, n_kv):
            holders.setdefault(j, []).append(r)
    share = {}
    for j, rs in holders.items():
        w = rng.random(len(rs))
        w /= w.sum()
        for r, wr in zip(rs, w):
            share[(j, r)] = wr
    dX = np.zeros_like(X)
    dO, dWo, dWqkv = [], [], []
    for r in range(t):
        Wqkv, Wo_r = attn.attn_shard_weights(Wq, Wk, Wv, Wo, r, t, n_heads, n_kv, d)
        qh, kh = attn.query_heads(r, t, n_heads), attn.kv_heads(r, t, n_heads, n_kv)
        q0, q1 = qh[0] * d, (qh[-1] + 1) * d
        dO_r, dWo_r = attn.out_backward(dY, O[:, q0:q1], Wo_r)
        dO.append(dO_r)
        dWo.append(dWo_r)
        dK = np.concatenate([GK[:, j * d:(j + 1) * d] * share[(j, r)] for j in kh], axis=1)
        dV = np.concatenate([GV[:, j * d:(j + 1) * d] * share[(j, r)] for j in kh], axis=1)
        dX_r, dW_r = attn.qkv_backward(X, Wqkv, np.concatenate([GQ[:, q0:q1], dK, dV], axis=1))
        dX = dX + dX_r
        dWqkv.append(dW_r)
    np.testing.assert_allclose(np.hstack(dO), g["O"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.vstack(dWo), g["Wo"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dX, g["X"], rtol=1e-11, atol=1e-12)
    dWq, dWk, dWv = attn.gather_qkv_weight_grads(dWqkv, t, n_heads, n_kv, d)
    np.testing.assert_allclose(dWq, g["Wq"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dWk, g["Wk"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dWv, g["Wv"], rtol=1e-11, atol=1e-12)
