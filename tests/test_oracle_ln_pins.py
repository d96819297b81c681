"""Pins of the sequence-parallel LayerNorm oracle (oracle/ln.py).

Tied to things other than the oracle itself:

* torch's float64 ``layer_norm`` and autograd (a library implementation of
  the same definition) for the forward and every gradient;
* brute force on tiny inputs: pure-Python mean / variance loops, and central
  finite differences of a scalar loss for dx, dgamma and dbeta;
* closed forms and invariants: with gamma = 1, beta = 0 and eps = 0 every
  row has mean 0 and variance 1; the output does not change when a constant
  is added to a row, nor (eps = 0) when a row is scaled by a > 0, so dx sums
  to zero along every row and (eps = 0) is orthogonal to xhat; a constant
  row maps to beta; h = 1 always gives beta;
* the check of "Tensor and sequence parallelism" ("The implementation"): the
  LayerNorm on each rank's s/t rows, all-gather, the MLP shard, reduce-scatter
  give the single-process block's output rows, input gradient rows and
  weight-shard gradients, and the LayerNorm weight's gradient only after it
  is summed over the ranks (closing question 4 of that page).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ln

torch = pytest.importorskip("torch")


def _rand(seed, rows, h, shift=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, h)) * rng.uniform(0.5, 3.0, size=(rows, 1)) + shift
    gamma = 1.0 + 0.3 * rng.standard_normal(h)
    beta = 0.2 * rng.standard_normal(h)
    dy = rng.standard_normal((rows, h))
    return x, gamma, beta, dy


@pytest.mark.parametrize("rows,h,eps,with_beta", [(5, 16, 1e-5, True), (3, 1, 1e-5, True), (7, 33, 0.1, False),
                                                  (4, 64, 1e-12, True)])
def test_forward_and_backward_match_torch_float64(rows, h, eps, with_beta):
    x, gamma, beta, dy = _rand(rows * h, rows, h, shift=2.0)
    b = beta if with_beta else None
    y, mean, rstd = ln.layer_norm_forward(x, gamma, b, eps)
    T = {k: torch.tensor(v, requires_grad=True) for k, v in dict(x=x, g=gamma, b=beta).items()}
    yt = torch.nn.functional.layer_norm(T["x"], (h,), weight=T["g"], bias=T["b"] if with_beta else None, eps=eps)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(x.var(axis=1) + eps), rtol=1e-12)
    (yt * torch.from_numpy(dy)).sum().backward()
    dx, dg, db = ln.layer_norm_backward(dy, x, gamma, eps)
    np.testing.assert_allclose(dx, T["x"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dg, T["g"].grad.numpy(), rtol=1e-11, atol=1e-11)
    if with_beta:
        np.testing.assert_allclose(db, T["b"].grad.numpy(), rtol=1e-12, atol=1e-12)


def test_forward_brute_force_tiny():
    x, gamma, beta, _ = _rand(3, 2, 5)
    y, mean, rstd = ln.layer_norm_forward(x, gamma, beta, 1e-5)
    for i in range(2):
        row = [float(v) for v in x[i]]
        m = sum(row) / len(row)
        var = sum((v - m) ** 2 for v in row) / len(row)   # biased (1/h)
        r = 1.0 / math.sqrt(var + 1e-5)
        assert abs(mean[i] - m) < 1e-14 and abs(rstd[i] - r) < 1e-12 * r
        for j in range(5):
            assert abs(y[i, j] - ((row[j] - m) * r * gamma[j] + beta[j])) < 1e-12


def test_backward_finite_differences_tiny():
    rows, h, eps = 2, 6, 1e-3
    x, gamma, beta, dy = _rand(11, rows, h)
    dres = np.random.default_rng(12).standard_normal((rows, h))

    def loss(x_, g_, b_):
        # <dy, LN(x)> + <dres, x>: dres is the residual branch's gradient
        return float((dy * ln.layer_norm_forward(x_, g_, b_, eps)[0]).sum() + (dres * x_).sum())

    dx, dg, db = ln.layer_norm_backward(dy, x, gamma, eps, dres=dres)
    step = 1e-6
    for arr, grad, which in ((x, dx, 0), (gamma, dg, 1), (beta, db, 2)):
        for idx in np.ndindex(arr.shape):
            args = [x.copy(), gamma.copy(), beta.copy()]
            args[which][idx] += step
            up = loss(*args)
            args[which][idx] -= 2 * step
            dn = loss(*args)
            fd = (up - dn) / (2 * step)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def test_normalised_rows_have_mean_zero_and_unit_variance():
    x, _, _, _ = _rand(21, 9, 40, shift=-5.0)
    y, _, _ = ln.layer_norm_forward(x, np.ones(40), None, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-12)


def test_shift_and_scale_invariance():
    x, gamma, beta, dy = _rand(31, 6, 24)
    c = np.random.default_rng(32).standard_normal((6, 1)) * 10
    y0 = ln.layer_norm_forward(x, gamma, beta, 1e-5)[0]
    np.testing.assert_allclose(ln.layer_norm_forward(x + c, gamma, beta, 1e-5)[0], y0, rtol=1e-10, atol=1e-10)
    z0 = ln.layer_norm_forward(x, gamma, beta, 0.0)[0]
    np.testing.assert_allclose(ln.layer_norm_forward(3.5 * x, gamma, beta, 0.0)[0], z0, rtol=1e-12, atol=1e-12)
    # their consequences for the gradient: dx sums to 0 along a row (any eps);
    # with eps = 0, dx is orthogonal to xhat
    dx = ln.layer_norm_backward(dy, x, gamma, 1e-5)[0]
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-11)
    dx0 = ln.layer_norm_backward(dy, x, gamma, 0.0)[0]
    xhat = (x - x.mean(axis=1, keepdims=True)) / x.std(axis=1, keepdims=True)
    np.testing.assert_allclose((dx0 * xhat).sum(axis=1), 0.0, atol=1e-10)


def test_constant_rows_and_single_column():
    gamma = np.array([2.0, -1.0, 0.5])
    beta = np.array([0.25, 0.0, -3.0])
    x = np.array([[4.0, 4.0, 4.0], [-1.5, -1.5, -1.5]])
    y, mean, rstd = ln.layer_norm_forward(x, gamma, beta, 1e-5)
    np.testing.assert_array_equal(y, np.tile(beta, (2, 1)))
    np.testing.assert_allclose(rstd, 1.0 / math.sqrt(1e-5), rtol=1e-15)
    # constant row: xhat = 0, so dx = rstd * (dy*gamma - mean(dy*gamma))
    dy = np.array([[1.0, 2.0, 3.0], [0.5, -0.5, 1.0]])
    dx, dg, db = ln.layer_norm_backward(dy, x, gamma, 1e-5)
    g = dy * gamma
    np.testing.assert_allclose(dx, (g - g.mean(axis=1, keepdims=True)) / math.sqrt(1e-5), rtol=1e-12)
    np.testing.assert_array_equal(dg, np.zeros(3))
    np.testing.assert_array_equal(db, dy.sum(axis=0))
    # h = 1: the output is beta and nothing flows back to x
    y1 = ln.layer_norm_forward(np.array([[3.0], [-7.0]]), np.array([5.0]), np.array([0.5]), 1e-5)[0]
    np.testing.assert_array_equal(y1, [[0.5], [0.5]])
    dx1 = ln.layer_norm_backward(np.array([[1.0], [2.0]]), np.array([[3.0], [-7.0]]), np.array([5.0]))[0]
    np.testing.assert_array_equal(dx1, np.zeros((2, 1)))


def test_sum_shared_grads_rank_order_and_plain_sum():
    g = [np.array([1.0, 2.0]), np.array([0.5, -4.0]), np.array([1e-3, 0.0])]
    np.testing.assert_array_equal(ln.sum_shared_grads(g), np.array([1.501, -2.0]))


def _torch_block(act, x, gamma, beta, W1, W2, Wg, b2, res, dout, eps):
    """The single-process block of the pages' check in torch float64:
    LayerNorm, up-projection, activation, down-projection (+ bias, residual),
    loss <dout, out>."""
    T = {k: torch.tensor(v, requires_grad=True) for k, v in dict(x=x, g=gamma, b=beta, W1=W1, W2=W2).items()}
    if Wg is not None:
        T["Wg"] = torch.tensor(Wg, requires_grad=True)
    h = torch.nn.functional.layer_norm(T["x"], (x.shape[1],), weight=T["g"], bias=T["b"], eps=eps)
    u = h @ T["W1"]
    if act == "gelu":
        a = torch.nn.functional.gelu(u)
    elif act == "relu":
        a = torch.relu(u)
    else:
        a = torch.nn.functional.silu(h @ T["Wg"]) * u
    out = a @ T["W2"]
    if b2 is not None:
        out = out + torch.from_numpy(b2)
    if res is not None:
        out = out + torch.from_numpy(res)
    (out * torch.from_numpy(dout)).sum().backward()
    return out.detach().numpy(), {k: v.grad.numpy() for k, v in T.items()}


@pytest.mark.parametrize("act,t,with_extras", [("gelu", 4, False), ("swiglu", 2, True), ("relu", 8, True)])
def test_sp_block_equals_single_process_block(act, t, with_extras):
    """The pages' TP+SP check: output rows, input-gradient rows, the MLP
    weight shards' gradients and the summed LayerNorm weight gradient all
    equal the unsplit block's."""
    rng = np.random.default_rng(40 + t)
    N, h, F = 8 * t, 16, 64
    x = rng.standard_normal((N, h))
    gamma = rng.standard_normal(h)
    beta = 0.1 * rng.standard_normal(h) if with_extras else None
    W1 = rng.standard_normal((h, F)) / h ** 0.5
    W2 = rng.standard_normal((F, h)) / F ** 0.5
    Wg = rng.standard_normal((h, F)) / h ** 0.5 if act == "swiglu" else None
    b2 = 0.1 * rng.standard_normal(h) if with_extras else None
    res = rng.standard_normal((N, h)) if with_extras else None
    dout = rng.standard_normal((N, h))
    ref_out, g = _torch_block(act, x, gamma, beta if beta is not None else np.zeros(h), W1, W2, Wg, b2, res, dout,
                              ln.EPS)

    outs, _ = ln.sp_block_forward(act, x, gamma, W1, W2, t, Wg=Wg, beta=beta, b2=b2, residual=res)
    blocks = [oracle.sequence_block(r, t, N) for r in range(t)]
    for r in range(t):
        np.testing.assert_allclose(outs[r], ref_out[blocks[r]], rtol=1e-11, atol=1e-12)
    bw = ln.sp_block_backward(act, x, gamma, W1, W2, [dout[b] for b in blocks], t, Wg=Wg, beta=beta)
    np.testing.assert_allclose(np.vstack(bw["dx"]), g["x"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(bw["dgamma"], g["g"], rtol=1e-10, atol=1e-11)
    if with_extras:
        np.testing.assert_allclose(bw["dbeta"], g["b"], rtol=1e-10, atol=1e-11)
    for r in range(t):
        c = oracle.column_block(r, t, F)
        np.testing.assert_allclose(bw["shard"][r]["dW1"], g["W1"][:, c], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(bw["shard"][r]["dW2"], g["W2"][c, :], rtol=1e-10, atol=1e-11)
        if act == "swiglu":
            np.testing.assert_allclose(bw["shard"][r]["dWg"], g["Wg"][:, c], rtol=1e-10, atol=1e-11)
    # one rank's LayerNorm weight gradient is only its block's contribution
    assert not np.allclose(bw["dgamma_r"][0], g["g"])


def test_residual_gradient_adds_to_dx():
    rng = np.random.default_rng(50)
    t, N, h, F = 2, 6, 8, 16
    x, gamma = rng.standard_normal((N, h)), rng.standard_normal(h)
    W1, W2 = rng.standard_normal((h, F)) / 3, rng.standard_normal((F, h)) / 4
    douts = [rng.standard_normal((N // t, h)) for _ in range(t)]
    dres = [rng.standard_normal((N // t, h)) for _ in range(t)]
    a = ln.sp_block_backward("gelu", x, gamma, W1, W2, douts, t)
    b = ln.sp_block_backward("gelu", x, gamma, W1, W2, douts, t, dres=dres)
    for r in range(t):
        np.testing.assert_allclose(b["dx"][r] - a["dx"][r], dres[r], rtol=1e-12, atol=1e-12)


def test_round_bf16_matches_torch_and_ties_to_even():
    """Against torch's float32 -> bfloat16 conversion (round to nearest even)
    on float32 values (exact in float64, so no double rounding), and on
    hand-made ties."""
    rng = np.random.default_rng(60)
    v = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ln.round_bf16(v.astype(np.float64)), want)
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even 1;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6;
    # 1028 = 2^10 (1 + 2^-8) lies halfway between 1024 and 1032: goes to 1024
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1028.0, 0.0])
    np.testing.assert_array_equal(ln.round_bf16(ties), [1.0, 1 + 2.0 ** -6, -1.0, 1024.0, 0.0])
    # a value just above a tie rounds up
    assert ln.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


def test_sp_block_bf16_payload_is_the_rounded_gather():
    """With payload_bf16 the MLP sees the bf16-rounded LayerNorm outputs: the
    block output equals the plain MLP of the rounded gathered rows."""
    rng = np.random.default_rng(70)
    t, N, h, F = 2, 6, 16, 32
    x, gamma = rng.standard_normal((N, h)), rng.standard_normal(h)
    W1, W2 = rng.standard_normal((h, F)) / 4, rng.standard_normal((F, h)) / 6
    outs, lnb = ln.sp_block_forward("relu", x, gamma, W1, W2, t, payload_bf16=True)
    Xr = ln.round_bf16(np.vstack(lnb))
    assert not np.array_equal(Xr, np.vstack(lnb))
    full = np.maximum(Xr @ W1, 0.0) @ W2
    np.testing.assert_allclose(np.vstack(outs), full, rtol=1e-12, atol=1e-12)
    douts = [rng.standard_normal((N // t, h)) for _ in range(t)]
    bw = ln.sp_block_backward("relu", x, gamma, W1, W2, douts, t, payload_bf16=True)
    dA = np.vstack(douts) @ W2.T
    dXfull = (dA * (Xr @ W1 > 0)) @ W1.T
    for r in range(t):
        blk = oracle.sequence_block(r, t, N)
        np.testing.assert_allclose(bw["dx"][r], ln.layer_norm_backward(dXfull[blk], x[blk], gamma)[0],
                                   rtol=1e-10, atol=1e-12)

