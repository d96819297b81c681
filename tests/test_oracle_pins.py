"""Pins of the fp64 oracle to things other than itself.

Each test ties an oracle function to something the pages or the mathematics
fix: the worked example the pages print, hand-derived values of its backward,
closed forms of the activations, brute force on tiny inputs, finite
differences, autograd of the unsplit block (torch on the CPU, an independent
library) and the split-equals-unsplit invariants the pages assert.  The
constructions the pages warn against are planted here, on the CPU, and must
fail.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from megatron_tensor_transformer_rank_amd.configs import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# The worked example ("Tensor Parallelism's Communication Boundary")
# ---------------------------------------------------------------------------
def _worked():
    g = _load("worked_example.json")
    X = np.array([g["x"]], dtype=np.float64)
    W1 = np.array(g["w1"], dtype=np.float64)
    W2 = np.array(g["w2"], dtype=np.float64)
    return g, X, W1, W2


def test_worked_example_forward_exact():
    g, X, W1, W2 = _worked()
    Y, ranks = oracle.tp_forward("relu", X, W1, W2, g["t"])
    # pre-activation of the unsplit block, local hidden vectors, partials
    _, dense = oracle.tp_forward("relu", X, W1, W2, 1)
    assert dense[0]["U"][0].tolist() == g["pre_activation"]
    for r in range(g["t"]):
        assert ranks[r]["A"][0].tolist() == g["local_hidden"][r]
        assert ranks[r]["Y"][0].tolist() == g["partials"][r]
    assert Y[0].tolist() == g["output"]
    assert oracle.tp_forward("relu", X, W1, W2, 1)[0][0].tolist() == g["output"]


def test_worked_example_byte_sizes_match_first_workload():
    g = _load("worked_example.json")["bytes"]
    w = WORKLOADS["mlp128_h1024_gelu_t2"]
    assert (w.N, w.h, w.F) == (g["tokens"], g["width"], g["expanded"])
    assert w.N * w.F * g["element_bytes"] == g["expanded_tensor_bytes"]
    assert w.N * w.h * g["element_bytes"] == g["output_reduction_tensor_bytes"]
    # one rank holds half of the expanded tensor
    assert w.N * w.Fi * 2 == g["expanded_tensor_bytes"] // 2


def test_worked_example_backward_hand_derived():
    g, X, W1, W2 = _worked()
    bw = _load("worked_example_backward.json")
    for case in bw["cases"]:
        dY = np.array([case["dY"]], dtype=np.float64)
        dX, db2, ranks = oracle.tp_backward("relu", X, W1, W2, dY, g["t"])
        assert dX[0].tolist() == case["dX"]
        assert db2.tolist() == case["dY"]
        if "dX_partials" in case:
            assert [r["dX"][0].tolist() for r in ranks] == case["dX_partials"]
        if "dA" in case:
            full = oracle.shard_backward("relu", X, W1, W2, dY)
            assert full["dA"][0].tolist() == case["dA"]
            assert full["dU"][0].tolist() == case["dU"]
            assert full["dW1"].tolist() == case["dW1"]
            assert full["dW2"].tolist() == case["dW2"]
            # the sharded weight gradients stack to the unsplit ones
            assert np.hstack([r["dW1"] for r in ranks]).tolist() == case["dW1"]
            assert np.vstack([r["dW2"] for r in ranks]).tolist() == case["dW2"]
            # ReLU'(0) = 0 is a real choice here: the third pre-activation is 0
            assert dX[0].tolist() != case["dX_if_relu_grad_at_zero_were_one"]


def test_relu_gradient_at_zero_choice_is_visible():
    """Planting ReLU'(0) = 1 in a copy of the derivative changes dX of the
    worked example to the hand-derived alternative."""
    g, X, W1, W2 = _worked()
    case = _load("worked_example_backward.json")["cases"][0]
    dY = np.array([case["dY"]], dtype=np.float64)
    U = X @ W1
    dA = dY @ W2.T
    planted = dA * (U >= 0.0)
    assert (planted @ W1.T)[0].tolist() == case["dX_if_relu_grad_at_zero_were_one"]
    assert (oracle.act_backward("relu", dA, U) @ W1.T)[0].tolist() == case["dX"]


def test_wrong_split_along_input_dim_fails():
    """Splitting W1 on its input dimension and applying ReLU to the partial
    pre-activations gives a different answer."""
    g, X, W1, W2 = _worked()
    wrong = _load("worked_example_backward.json")["wrong_split"]
    out = np.zeros(2)
    for k in range(2):
        pre = X[0, k] * W1[k, :]
        assert pre.tolist() == wrong["worker_preacts"][k]
        out += oracle.act_forward("relu", pre) @ W2
    assert out.tolist() == wrong["output"]
    assert out.tolist() != g["output"]
    # the scalar counterexample: ReLU(1 + (-1)) != ReLU(1) + ReLU(-1)
    assert oracle.act_forward("relu", np.array([0.0]))[0] != (
        oracle.act_forward("relu", np.array([1.0]))[0]
        + oracle.act_forward("relu", np.array([-1.0]))[0])


def test_bias_added_once():
    rng = np.random.default_rng(7)
    X, W1, W2 = rng.standard_normal((5, 8)), rng.standard_normal((8, 12)), rng.standard_normal((12, 8))
    b = rng.standard_normal(8)
    t = 4
    Yb, ranks = oracle.tp_forward("gelu", X, W1, W2, t, b2=b)
    Y0, _ = oracle.tp_forward("gelu", X, W1, W2, t)
    np.testing.assert_allclose(Yb - Y0, np.broadcast_to(b, Y0.shape), rtol=0, atol=1e-12)
    # a bias added to every partial before the sum counts it t times
    per_partial = oracle.reduce_partials([r["Y"] + b for r in ranks])
    assert np.abs(per_partial - Yb).max() > 1.0
    np.testing.assert_allclose(per_partial - Yb, np.broadcast_to((t - 1) * b, Y0.shape), atol=1e-12)


def test_swapped_f_and_g_fails():
    """g at the start and f at the end: the input is summed over t replicas
    and the output is left as one rank's partial sum."""
    rng = np.random.default_rng(11)
    X, W1, W2 = rng.standard_normal((6, 16)), rng.standard_normal((16, 32)) / 4, rng.standard_normal((32, 16)) / 6
    t = 4
    Y, ranks = oracle.tp_forward("gelu", X, W1, W2, t)
    assert np.abs(ranks[0]["Y"] - Y).max() > 1e-3          # unsummed partial
    Yt, _ = oracle.tp_forward("gelu", t * X, W1, W2, t)   # replicated input summed
    assert np.abs(Yt - Y).max() > 1e-3


# ---------------------------------------------------------------------------
# Activation closed forms (standard normal CDF / logistic values)
# ---------------------------------------------------------------------------
# Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208,
# phi(1) = 0.24197072451914337, sigmoid(1) = 0.7310585786300049.
@pytest.mark.parametrize("u,gelu", [
    (1.0, 0.8413447460685429),
    (-1.0, -0.15865525393145707),
    (2.0, 1.9544997361036416),
    (0.0, 0.0),
    (-2.0, -0.04550026389635842),
])
def test_gelu_values(u, gelu):
    assert oracle.act_forward("gelu", np.array([u]))[0] == pytest.approx(gelu, rel=1e-14, abs=1e-16)


@pytest.mark.parametrize("u,d", [(0.0, 0.5), (1.0, 1.0833154705876864), (-1.0, -0.0833154705876864)])
def test_gelu_derivative_values(u, d):
    assert oracle.act_backward("gelu", np.array([1.0]), np.array([u]))[0] == pytest.approx(d, rel=1e-14, abs=1e-16)


@pytest.mark.parametrize("g,silu", [(1.0, 0.7310585786300049), (-1.0, -0.2689414213699951),
                                    (0.0, 0.0), (-40.0, -40.0 / (1.0 + math.exp(40.0)))])
def test_silu_values(g, silu):
    # SwiGLU with up projection 1 reduces to SiLU(gate)
    a = oracle.act_forward("swiglu", np.array([1.0]), np.array([g]))[0]
    assert a == pytest.approx(silu, rel=1e-14, abs=1e-300)


def test_gelu_cdf_matches_integral_of_density():
    """Phi(u) by numerical quadrature of the Gaussian density, independent of
    erf."""
    from scipy.integrate import quad
    for u in (-3.0, -0.7, 0.3, 1.9):
        phi_int = quad(lambda s: math.exp(-0.5 * s * s) / math.sqrt(2 * math.pi), -np.inf, u)[0]
        assert oracle.act_forward("gelu", np.array([u]))[0] == pytest.approx(u * phi_int, rel=1e-10)


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_activation_derivative_by_central_difference(act):
    rng = np.random.default_rng(3)
    U = rng.standard_normal(400) * 3
    U = U[np.abs(U) > 1e-3]                       # keep ReLU away from its kink
    G = rng.standard_normal(U.size) * 3
    eps = 1e-6
    if act == "swiglu":
        dG, dP = oracle.act_backward(act, np.ones_like(U), U, G)
        numG = (oracle.act_forward(act, U, G + eps) - oracle.act_forward(act, U, G - eps)) / (2 * eps)
        numP = (oracle.act_forward(act, U + eps, G) - oracle.act_forward(act, U - eps, G)) / (2 * eps)
        np.testing.assert_allclose(dG, numG, rtol=1e-7, atol=1e-8)
        np.testing.assert_allclose(dP, numP, rtol=1e-7, atol=1e-8)
    else:
        d = oracle.act_backward(act, np.ones_like(U), U)
        num = (oracle.act_forward(act, U + eps) - oracle.act_forward(act, U - eps)) / (2 * eps)
        np.testing.assert_allclose(d, num, rtol=1e-7, atol=1e-8)


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (pure Python, scalar math module)
# ---------------------------------------------------------------------------
def _bf_act(act, u, g=None):
    if act == "relu":
        return u if u > 0 else 0.0
    if act == "gelu":
        return u * 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))
    return g / (1.0 + math.exp(-g)) * u


def _bf_forward(act, X, W1, W2, Wg):
    N, h = len(X), len(X[0])
    F = len(W1[0])
    Y = [[0.0] * h for _ in range(N)]
    for n in range(N):
        for f in range(F):
            u = sum(X[n][k] * W1[k][f] for k in range(h))
            gg = sum(X[n][k] * Wg[k][f] for k in range(h)) if act == "swiglu" else None
            a = _bf_act(act, u, gg)
            for j in range(h):
                Y[n][j] += a * W2[f][j]
    return Y


def _loss(act, X, W1, W2, Wg, dY):
    Y = _bf_forward(act, X, W1, W2, Wg)
    return sum(Y[n][j] * dY[n][j] for n in range(len(Y)) for j in range(len(Y[0])))


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_forward_brute_force(act):
    rng = np.random.default_rng(5)
    N, h, F, t = 3, 4, 6, 3
    X, W1, W2, Wg = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F)])
    Y, _ = oracle.tp_forward(act, X, W1, W2, t, Wg=Wg if act == "swiglu" else None)
    ref = _bf_forward(act, X.tolist(), W1.tolist(), W2.tolist(), Wg.tolist())
    np.testing.assert_allclose(Y, np.array(ref), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_backward_by_finite_differences(act):
    """Central differences of L = <dY, Y> in fp64 against every gradient the
    oracle returns (dW1, dWg, dW2, dX, db2), on a tiny shape, t = 2."""
    rng = np.random.default_rng(17)
    N, h, F, t = 3, 4, 6, 2
    X, W1, W2, Wg, dY = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F), (N, h)])
    if act == "relu":                       # push pre-activations off the kink
        U = X @ W1
        assert np.abs(U).min() > 1e-3
    sw = act == "swiglu"
    dX, db2, ranks = oracle.tp_backward(act, X, W1, W2, dY, t, Wg=Wg if sw else None)
    dW1 = np.hstack([r["dW1"] for r in ranks])
    dW2 = np.vstack([r["dW2"] for r in ranks])
    dWg = np.hstack([r["dWg"] for r in ranks]) if sw else None
    eps = 1e-6
    args = {"X": X, "W1": W1, "W2": W2, "Wg": Wg}

    def L(a):
        return _loss(act, a["X"].tolist(), a["W1"].tolist(), a["W2"].tolist(), a["Wg"].tolist(), dY.tolist())

    checks = [("X", dX), ("W1", dW1), ("W2", dW2)] + ([("Wg", dWg)] if sw else [])
    for name, grad in checks:
        num = np.zeros_like(args[name])
        for idx in np.ndindex(*args[name].shape):
            p = {k: v.copy() for k, v in args.items()}
            m = {k: v.copy() for k, v in args.items()}
            p[name][idx] += eps
            m[name][idx] -= eps
            num[idx] = (L(p) - L(m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)
    # the output bias: dL/db2 = column sums of dY
    np.testing.assert_allclose(db2, dY.sum(axis=0), rtol=1e-15)


# ---------------------------------------------------------------------------
# Autograd of the unsplit block (torch, CPU, float64) and the invariants
# ---------------------------------------------------------------------------
def _torch_block(act, X, W1, W2, Wg, loss):
    import torch
    import torch.nn.functional as Fn
    ts = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
          for k, v in dict(X=X, W1=W1, W2=W2, Wg=Wg if Wg is not None else np.zeros(1)).items()}
    U = ts["X"] @ ts["W1"]
    if act == "relu":
        A = Fn.relu(U)
    elif act == "gelu":
        A = Fn.gelu(U)                      # exact erf form
    else:
        A = Fn.silu(ts["X"] @ ts["Wg"]) * U
    Y = A @ ts["W2"]
    L = loss(Y)
    L.backward()
    Ynp = Y.detach().numpy()
    return Ynp, {k: v.grad.numpy() for k, v in ts.items() if v.grad is not None}


@pytest.mark.parametrize("act", ["gelu", "swiglu", "relu"])
def test_tensor_sequence_check_shape_against_autograd(act):
    """The shape of the TP=4 check script in 'Tensor and sequence
    parallelism' (S=8, H=16, FFN=64, loss = sum of Y^2 so dY = 2Y): the
    sharded oracle matches autograd of the unsplit block."""
    import torch
    rng = np.random.default_rng(0)
    S, H, FFN, t = 8, 16, 64, 4
    X = rng.standard_normal((S, H))
    W1 = rng.standard_normal((H, FFN)) / math.sqrt(H)
    W2 = rng.standard_normal((FFN, H)) / math.sqrt(FFN)
    Wg = rng.standard_normal((H, FFN)) / math.sqrt(H) if act == "swiglu" else None
    Yt, grads = _torch_block(act, X, W1, W2, Wg, lambda Y: Y.square().sum())
    Y, _ = oracle.tp_forward(act, X, W1, W2, t, Wg=Wg)
    np.testing.assert_allclose(Y, Yt, rtol=1e-12, atol=1e-12)
    dY = 2 * Y
    dX, _, ranks = oracle.tp_backward(act, X, W1, W2, dY, t, Wg=Wg)
    np.testing.assert_allclose(dX, grads["X"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.hstack([r["dW1"] for r in ranks]), grads["W1"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.vstack([r["dW2"] for r in ranks]), grads["W2"], rtol=1e-11, atol=1e-12)
    if act == "swiglu":
        np.testing.assert_allclose(np.hstack([r["dWg"] for r in ranks]), grads["Wg"], rtol=1e-11, atol=1e-12)
    del torch


def test_two_device_script_shape_linear_case():
    """The 3x3 / hidden 2 / t = 2 example of 'Parallelism Strategies #1 -
    Tensor Parallelism' has no activation; with non-negative inputs ReLU is the
    identity, so the block is the matmul chain X @ W1 @ W2 and, for the mean
    loss (dY = 1/9), its gradients are those of that chain."""
    rng = np.random.default_rng(42)
    X, W1, W2 = rng.random((3, 3)), rng.random((3, 2)), rng.random((2, 3))
    Y, ranks = oracle.tp_forward("relu", X, W1, W2, 2)
    np.testing.assert_allclose(Y, X @ W1 @ W2, rtol=1e-14)
    dY = np.full((3, 3), 1.0 / 9.0)
    dX, _, ranks = oracle.tp_backward("relu", X, W1, W2, dY, 2)
    np.testing.assert_allclose(dX, dY @ W2.T @ W1.T, rtol=1e-14)
    np.testing.assert_allclose(np.hstack([r["dW1"] for r in ranks]), X.T @ (dY @ W2.T), rtol=1e-14)
    np.testing.assert_allclose(np.vstack([r["dW2"] for r in ranks]), (X @ W1).T @ dY, rtol=1e-14)
    _, grads = _torch_block("relu", X, W1, W2, None, lambda Y: Y.mean())
    np.testing.assert_allclose(dX, grads["X"], rtol=1e-13)


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
@pytest.mark.parametrize("t", [2, 3, 8])
def test_split_equals_unsplit(act, t):
    rng = np.random.default_rng(100 + t)
    N, h, F = 7, 24, 48
    X, W1, W2, Wg, dY = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F), (N, h)])
    Wg = Wg if act == "swiglu" else None
    Y1, r1 = oracle.tp_forward(act, X, W1, W2, 1, Wg=Wg)
    Yt, rt = oracle.tp_forward(act, X, W1, W2, t, Wg=Wg)
    scale = np.abs(Y1).max()
    np.testing.assert_allclose(Yt, Y1, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(np.hstack([r["U"] for r in rt]), r1[0]["U"], rtol=1e-13, atol=1e-13)
    dX1, _, b1 = oracle.tp_backward(act, X, W1, W2, dY, 1, Wg=Wg)
    dXt, _, bt = oracle.tp_backward(act, X, W1, W2, dY, t, Wg=Wg)
    np.testing.assert_allclose(dXt, dX1, rtol=0, atol=1e-12 * np.abs(dX1).max())
    np.testing.assert_allclose(np.hstack([r["dW1"] for r in bt]), b1[0]["dW1"], rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(np.vstack([r["dW2"] for r in bt]), b1[0]["dW2"], rtol=1e-13, atol=1e-12)
    if Wg is not None:
        np.testing.assert_allclose(np.hstack([r["dWg"] for r in bt]), b1[0]["dWg"], rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_weight_gradients_add_over_row_blocks_and_vanish_on_none(act):
    """The block treats tokens independently, so the weight gradients over a
    batch (dW1_i = X^T dU_i, dW2_i = A_i^T dY, db2 = the column sum of dY, as
    derived in "Parallelism Strategies #1 - Tensor Parallelism") are sums
    over its token rows: they add over any split of the rows, and the empty
    block, the identity of that sum, gives zero.  A mean over rows instead
    of a sum, or a forward / input gradient that mixed rows, fails here."""
    rng = np.random.default_rng(77)
    N, h, F = 9, 16, 24
    X, W1, W2, Wg, dY = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F), (N, h)])
    Wg = Wg if act == "swiglu" else None
    full = oracle.shard_backward(act, X, W1, W2, dY, Wg)
    blocks = [slice(0, 0), slice(0, 4), slice(4, 4), slice(4, N)]
    parts = [oracle.shard_backward(act, X[b], W1, W2, dY[b], Wg) for b in blocks]
    for k in ("dW1", "dW2") + (("dWg",) if Wg is not None else ()):
        np.testing.assert_allclose(sum(p[k] for p in parts), full[k], rtol=1e-13, atol=1e-13)
        assert parts[0][k].shape == full[k].shape and not np.any(parts[0][k]), k
    np.testing.assert_allclose(np.vstack([p["dX"] for p in parts]), full["dX"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sum(oracle.column_sum(dY[b]) for b in blocks), oracle.column_sum(dY), rtol=1e-13)
    assert not np.any(oracle.column_sum(dY[:0])) and oracle.column_sum(dY[:0]).shape == (h,)
    f0 = oracle.shard_forward(act, X[:0], W1, W2, Wg)
    assert f0["Y"].shape == (0, h) and f0["A"].shape == (0, F)


def test_column_block_contiguous_rank_order():
    F, t = 4096, 2
    assert oracle.column_block(0, t, F) == slice(0, 2048)      # W1[:, :2048]
    assert oracle.column_block(1, t, F) == slice(2048, 4096)
    with pytest.raises(ValueError):
        oracle.column_block(0, 3, 4096)
    with pytest.raises(ValueError):
        oracle.column_block(2, 2, 4096)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3F81, 0x8000, 0x4049], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and math.isinf(vals[2])
    assert vals[3] == 2.0 ** -133
    assert vals[4] == 1.0 + 2.0 ** -7
    assert vals[5] == 0.0 and math.copysign(1, vals[5]) < 0
    assert vals[6] == 3.140625


# ---------------------------------------------------------------------------
# The bfloat16-storage variant: the same arithmetic, with the tensors the
# method keeps in two bytes rounded where they are stored
# ---------------------------------------------------------------------------
def test_bf16_storage_equals_exact_on_the_worked_example():
    """Every value of the worked example is a small integer, exact in
    bfloat16: the storage variant gives the same results as the exact
    oracle, forward and backward, split and unsplit."""
    g, X, W1, W2 = _worked()
    for t in (1, g["t"]):
        Y, ranks = oracle.tp_forward("relu", X, W1, W2, t)
        Ys, ranks_s = oracle.tp_forward("relu", X, W1, W2, t, bf16_storage=True)
        assert np.array_equal(Y, Ys) and Ys[0].tolist() == g["output"]
        for a, b in zip(ranks, ranks_s):
            for k in ("U", "A", "Y"):
                assert np.array_equal(a[k], b[k])
        for dy in ([[1.0, 0.0]], [[0.0, 1.0]], [[1.0, 1.0]]):
            dY = np.array(dy)
            dX, _, br = oracle.tp_backward("relu", X, W1, W2, dY, t)
            dXs, _, brs = oracle.tp_backward("relu", X, W1, W2, dY, t, bf16_storage=True)
            assert np.array_equal(dX, dXs)
            for a, b in zip(br, brs):
                for k in ("dA", "dU", "dW1", "dW2", "dX"):
                    assert np.array_equal(a[k], b[k])


def _torch_bf16(v):
    """bfloat16 rounding through torch's float64 -> bfloat16 conversion (not
    the oracle's round_bf16), for the brute-force storage check."""
    import torch
    return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64))


def _bf_storage_shard(act, X, W1, W2, Wg, dY):
    """Pure-Python loops with the method's stores rounded: U (and G) stashed,
    A from the unrounded pre-activations then rounded, Y rounded; the
    activation derivative on the stashes, dU (dG, dP) rounded, dW2 from the
    stored A, dX rounded."""
    N, h, F = len(X), len(X[0]), len(W1[0])
    U = [[sum(X[n][k] * W1[k][f] for k in range(h)) for f in range(F)] for n in range(N)]
    G = [[sum(X[n][k] * Wg[k][f] for k in range(h)) for f in range(F)] for n in range(N)] if act == "swiglu" else None
    A = [[_torch_bf16(_bf_act(act, U[n][f], G[n][f] if G else None)) for f in range(F)] for n in range(N)]
    Us = [[_torch_bf16(U[n][f]) for f in range(F)] for n in range(N)]
    Gs = [[_torch_bf16(G[n][f]) for f in range(F)] for n in range(N)] if G else None
    Y = [[_torch_bf16(sum(A[n][f] * W2[f][j] for f in range(F))) for j in range(h)] for n in range(N)]
    dA = [[sum(dY[n][j] * W2[f][j] for j in range(h)) for f in range(F)] for n in range(N)]
    dP = [[0.0] * F for _ in range(N)]
    dG = [[0.0] * F for _ in range(N)]
    for n in range(N):
        for f in range(F):
            u = Us[n][f]
            if act == "relu":
                dP[n][f] = _torch_bf16(dA[n][f] * (1.0 if u > 0 else 0.0))
            elif act == "gelu":
                d = 0.5 * (1.0 + math.erf(u / math.sqrt(2.0))) + u * math.exp(-0.5 * u * u) / math.sqrt(2 * math.pi)
                dP[n][f] = _torch_bf16(dA[n][f] * d)
            else:
                gg = Gs[n][f]
                s = 1.0 / (1.0 + math.exp(-gg))
                dG[n][f] = _torch_bf16(dA[n][f] * u * s * (1.0 + gg * (1.0 - s)))
                dP[n][f] = _torch_bf16(dA[n][f] * gg * s)
    dX = [[_torch_bf16(sum(dP[n][f] * W1[k][f] + (dG[n][f] * Wg[k][f] if act == "swiglu" else 0.0)
                           for f in range(F))) for k in range(h)] for n in range(N)]
    dW2 = [[sum(A[n][f] * dY[n][j] for n in range(N)) for j in range(h)] for f in range(F)]
    dW1 = [[sum(X[n][k] * dP[n][f] for n in range(N)) for f in range(F)] for k in range(h)]
    return {"U": Us, "G": Gs, "A": A, "Y": Y, "dU": dP, "dG": dG, "dX": dX, "dW1": dW1, "dW2": dW2}


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_bf16_storage_brute_force(act):
    """The storage variant of one shard against pure-Python loops that round
    through torch's conversion: the same stores, the same values."""
    rng = np.random.default_rng(11)
    N, h, F = 3, 5, 4
    X, W1, W2, Wg, dY = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F), (N, h)])
    Wg = Wg if act == "swiglu" else None
    f = oracle.shard_forward(act, X, W1, W2, Wg, bf16_storage=True)
    b = oracle.shard_backward(act, X, W1, W2, dY, Wg, bf16_storage=True)
    ref = _bf_storage_shard(act, X.tolist(), W1.tolist(), W2.tolist(), Wg.tolist() if Wg is not None else None,
                            dY.tolist())
    for k, got in (("U", f["U"]), ("A", f["A"]), ("Y", f["Y"]), ("dU", b["dU"]), ("dX", b["dX"]),
                   ("dW1", b["dW1"]), ("dW2", b["dW2"])):
        np.testing.assert_allclose(got, np.array(ref[k]), rtol=1e-12, atol=1e-14, err_msg=k)
    if act == "swiglu":
        np.testing.assert_allclose(f["G"], np.array(ref["G"]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(b["dG"], np.array(ref["dG"]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_bf16_storage_rounding_bounds(act):
    """Each stored tensor is the exact one computed from the stored inputs,
    rounded once: within half a bfloat16 unit (2^-8 relative) of it; the
    reduced sums likewise over the stored partials."""
    rng = np.random.default_rng(12)
    N, h, F, t = 7, 16, 24, 3
    X, W1, W2, Wg, dY = (rng.standard_normal(s) for s in [(N, h), (h, F), (F, h), (h, F), (N, h)])
    Wg = Wg if act == "swiglu" else None
    Y, ranks = oracle.tp_forward(act, X, W1, W2, t, Wg=Wg, bf16_storage=True)
    dX, _, branks = oracle.tp_backward(act, X, W1, W2, dY, t, Wg=Wg, bf16_storage=True)
    half_ulp = lambda v: 2.0 ** -8 * np.abs(v) * (1 + 1e-12)   # 8 significant bits: unit roundoff 2^-8
    for r, (fr, br) in enumerate(zip(ranks, branks)):
        W1_i, W2_i, Wg_i = oracle.shard_weights(W1, W2, r, t, Wg)
        exact_A = oracle.act_forward(act, X @ W1_i, X @ Wg_i if Wg is not None else None)
        assert np.all(np.abs(fr["A"] - exact_A) <= half_ulp(exact_A))
        assert np.all(np.abs(fr["Y"] - fr["A"] @ W2_i) <= half_ulp(fr["A"] @ W2_i))
        dXe = br["dU"] @ W1_i.T + (br["dG"] @ Wg_i.T if Wg is not None else 0.0)
        assert np.all(np.abs(br["dX"] - dXe) <= half_ulp(dXe))
    Ye = sum(f["Y"] for f in ranks)
    assert np.all(np.abs(Y - Ye) <= half_ulp(Ye))
    dXe = sum(b["dX"] for b in branks)
    assert np.all(np.abs(dX - dXe) <= half_ulp(dXe))
