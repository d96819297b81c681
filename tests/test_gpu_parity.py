"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small and ragged shapes that span several tiles and leave tails in every
dimension; every rank of the tensor-parallel group is run, the partials are
reduced by the library's reduction kernel, and every output (U, G, A, Y_i, Y,
dU, dW1, dWg, dW2, dX_i, dX, db2) is compared elementwise with the oracle on
the same bf16 inputs: relative Frobenius error <= 5e-3 and max error <=
3e-2 * max|ref| (bf16 inputs, float32 accumulation).  Integer work is
bit-exact: the zero-padded worked example and the reduction of exactly
representable sums.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import Shard, assert_close, bf16_dev, f64, run_group

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (wid, N, h, F, t, act, bias): several 256-wide tiles plus ragged tails in
# N (tokens), h (a K tail for the up-projection) and F_i
CASES = [
    (101, 128, 1024, 4096, 2, "gelu", False),    # the pages' 128 x 1024 x 4096 example, t = 2
    (102, 300, 520, 2328, 3, "relu", True),      # ragged everywhere, F_i = 776
    (103, 257, 264, 784, 2, "swiglu", True),     # F_i = 392, SwiGLU
    (104, 77, 136, 512, 4, "gelu", False),       # small N, t = 4
    (105, 530, 384, 1536, 1, "swiglu", False),   # unsplit block
    (106, 8, 64, 128, 2, "relu", False),         # a single partial tile
    (107, 2, 1032, 2080, 2, "gelu", False),      # two tokens (MFMA path, 1 row tile)
    # the smallest shards the ABI takes: h = 8 and F_i = 8, over 8 and 16 ranks,
    # and a whole block of 8 x 8 (the one-token path and wide tiles)
    (108, 40, 8, 64, 8, "swiglu", True),
    (109, 200, 8, 128, 16, "gelu", False),
    (111, 1, 8, 8, 1, "gelu", True),
    (112, 70, 8, 8, 1, "swiglu", False),
    # ReLU with one pre-activation of |U| = 9.3e-8 on rank 1, inside float32
    # accumulation error of zero: the GPU's decision there differs from the
    # exact sign, and both are valid (the comparison follows the GPU's)
    (5087, 2049, 1008, 3864, 3, "relu", False),
    # one token, ReLU, an ambiguous pre-activation whose dA is small: the
    # GPU's decision must be followed into dW1 = x^T dU column by column
    (8080, 1, 1720, 3136, 7, "relu", False),
    # unsplit blocks of 88 to 100 output tiles per product, ragged in every
    # dimension (N, h and F_i a few rows or columns past a 256-tile edge,
    # and k past a 64-deep k-tile)
    (120, 2000, 2824, 2760, 1, "gelu", True),
    (121, 1000, 5400, 2824, 1, "swiglu", False),
    (122, 2310, 2312, 2312, 1, "relu", False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[1]}_h{c[2]}_F{c[3]}_t{c[4]}_{c[5]}" for c in CASES])
def test_group_matches_oracle(case):
    run_group(*case)


@pytest.mark.parametrize("act", ["gelu", "swiglu", "relu"])
def test_decode_one_token(act):
    """N = 1 routes the forward to the split-K GEMV path and the backward's
    input gradients to the small-batch split-K MFMA kernel."""
    run_group(200 + len(act), 1, 1024, 3 * 1024, 2, act, False)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_decode_ragged_splits(act):
    """h = 4104, F_i = 1544: the last k-split of both GEMVs is short, the last
    column strip of the down-projection holds 8 columns, and the final reduce
    ends in a partial block."""
    run_group(220 + len(act), 1, 4104, 2 * 1544, 2, act, False)


def test_decode_without_stash():
    """Inference: forward only, no stash buffers."""
    sw = True
    N, h, F, t = 1, 520, 1040, 2
    Xb = I.gen_x(211, N, h)
    W1b, W2b, Wgb = I.gen_full_weights(211, h, F, t, sw)
    Yref, _ = oracle.tp_forward("swiglu", oracle.bf16_bits_to_f64(Xb), oracle.bf16_bits_to_f64(W1b),
                                oracle.bf16_bits_to_f64(W2b), t, Wg=oracle.bf16_bits_to_f64(Wgb))
    parts = []
    for r in range(t):
        c = oracle.column_block(r, t, F)
        s = Shard(N, h, F, t, r, "swiglu", bf16_dev(Xb), bf16_dev(np.ascontiguousarray(W1b[:, c])),
                  bf16_dev(np.ascontiguousarray(W2b[c, :])), bf16_dev(np.ascontiguousarray(Wgb[:, c])),
                  stash=False)
        s.forward()
        parts.append(s.Y)
    Y = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local(parts, Y)
    assert_close("Y", f64(Y), Yref)


def test_split_sum_equals_unsplit_on_gpu():
    """The pages' invariant on the GPU: the reduced partials of t = 4 match
    the GPU's own unsplit (t = 1) run."""
    N, h, F, act = 192, 512, 2048, "gelu"
    Xb = I.gen_x(300, N, h)
    W1b, W2b, _ = I.gen_full_weights(300, h, F, 4, False)
    Xd = bf16_dev(Xb)
    one = Shard(N, h, F, 1, 0, act, Xd, bf16_dev(W1b), bf16_dev(W2b))
    one.forward()
    parts = []
    for r in range(4):
        c = oracle.column_block(r, 4, F)
        s = Shard(N, h, F, 4, r, act, Xd, bf16_dev(np.ascontiguousarray(W1b[:, c])),
                  bf16_dev(np.ascontiguousarray(W2b[c, :])))
        s.forward()
        parts.append(s)
        # the concatenated activation shards equal the unsplit activation exactly
        assert torch.equal(s.A, one.A[:, c])
    Y = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([p.Y for p in parts], Y)
    assert_close("sum of partials vs unsplit", f64(Y), f64(one.Y))


def _pad(a, shape):
    out = np.zeros(shape, dtype=np.float32)
    out[tuple(slice(0, s) for s in a.shape)] = a
    return I.f32_to_bf16_bits(out)


@pytest.mark.parametrize("N_pad", [1, 16])
def test_worked_example_exact(N_pad):
    """The pages' worked example, zero-padded to the ABI's multiples of 8
    (exact: act(0) = 0 and padded weights are 0), bit-exact on the GPU on the
    decode path (one row) and on the MFMA path (16 rows, the real one first)."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    bw = json.load(open(os.path.join(GOLDEN, "worked_example_backward.json")))["cases"][0]
    x = np.array([g["x"]], np.float32)
    w1, w2 = np.array(g["w1"], np.float32), np.array(g["w2"], np.float32)
    h, Fi, t = 8, 8, 2
    Xb = _pad(x, (N_pad, h))
    dYb = _pad(np.array([bw["dY"]], np.float32), (N_pad, h))
    shards, parts, dparts = [], [], []
    for r in range(t):
        cols = slice(2 * r, 2 * r + 2)
        W1b = _pad(w1[:, cols], (h, Fi))
        W2b = _pad(w2[cols, :], (Fi, h))
        s = Shard(N_pad, h, Fi * t, t, r, "relu", bf16_dev(Xb), bf16_dev(W1b), bf16_dev(W2b))
        s.forward()
        s.backward(bf16_dev(dYb))
        shards.append(s)
        parts.append(s.Y)
        dparts.append(s.dX)
    Y = torch.empty(N_pad, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local(parts, Y)
    dX = torch.empty(N_pad, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local(dparts, dX)
    torch.cuda.synchronize()
    for r in range(t):
        assert f64(shards[r].A)[0, :2].tolist() == g["local_hidden"][r]
        assert f64(shards[r].Y)[0, :2].tolist() == g["partials"][r]
        assert f64(shards[r].dX)[0, :2].tolist() == bw["dX_partials"][r]
        assert np.all(f64(shards[r].Y)[1:] == 0) and np.all(f64(shards[r].Y)[0, 2:] == 0)
    assert f64(Y)[0, :2].tolist() == g["output"]
    assert f64(dX)[0, :2].tolist() == bw["dX"]
    dW1 = np.hstack([f64(s.dW1)[:2, :2] for s in shards])
    dW2 = np.vstack([f64(s.dW2)[:2, :2] for s in shards])
    assert dW1.tolist() == bw["dW1"]
    assert dW2.tolist() == bw["dW2"]


def test_reduce_bitexact_on_representable_sums():
    """Partials that are small multiples of 1/8 sum exactly in float32, so the
    reduction (+ bias) must equal the oracle's sum bit for bit."""
    rng = np.random.default_rng(5)
    t, rows, cols = 5, 333, 1032
    parts = [rng.integers(-64, 64, size=(rows, cols)).astype(np.float32) / 8 for _ in range(t)]
    bias = rng.integers(-16, 16, size=cols).astype(np.float32) / 4
    pb = [I.f32_to_bf16_bits(p) for p in parts]
    bb = I.f32_to_bf16_bits(bias)
    ref = oracle.reduce_partials([oracle.bf16_bits_to_f64(p) for p in pb], oracle.bf16_bits_to_f64(bb))
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([bf16_dev(p) for p in pb], out, bias=bf16_dev(bb))
    ref_bits = I.f32_to_bf16_bits(ref.astype(np.float32))
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref_bits)


def test_reduce_in_place_and_random():
    rng = np.random.default_rng(6)
    t, rows, cols = 8, 1000, 2048
    pb = [I.normal_bf16([7, i], (rows, cols)) for i in range(t)]
    ref = oracle.reduce_partials([oracle.bf16_bits_to_f64(p) for p in pb])
    ds = [bf16_dev(p) for p in pb]
    B.tp_mlp_reduce_partials_local(ds, ds[0])        # out aliases partials[0]
    torch.cuda.synchronize()
    assert_close("reduce in place", f64(ds[0]), ref, rel_fro=5e-3, max_rel=1e-2)
    del rng


def test_deterministic_and_guard_bands():
    """Every output is bitwise identical across two runs, and nothing is
    written outside the output buffers (canary bytes around each)."""
    N, h, F, t, act = 300, 520, 2 * 776, 2, "swiglu"
    Xb, dYb = I.gen_x(400, N, h), I.gen_dy(400, N, h)
    W1b, W2b, Wgb = I.gen_full_weights(400, h, F, t, True)
    c = oracle.column_block(0, t, F)
    Fi = F // t
    s = Shard(N, h, F, t, 0, act, bf16_dev(Xb), bf16_dev(np.ascontiguousarray(W1b[:, c])),
              bf16_dev(np.ascontiguousarray(W2b[c, :])), bf16_dev(np.ascontiguousarray(Wgb[:, c])))
    # replace outputs with views into canary-padded buffers
    PAD = 4096
    guards = {}
    for name, shape, dt in [("Y", (N, h), torch.bfloat16), ("A", (N, Fi), torch.bfloat16),
                            ("U", (N, Fi), torch.bfloat16), ("G", (N, Fi), torch.bfloat16),
                            ("dU", (N, 2 * Fi), torch.bfloat16), ("dW1", (h, Fi), torch.float32),
                            ("dWg", (h, Fi), torch.float32), ("dW2", (Fi, h), torch.float32),
                            ("dX", (N, h), torch.bfloat16)]:
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * PAD,), 7.0, dtype=dt, device="cuda")
        guards[name] = buf
        setattr(s, name, buf[PAD:PAD + n].view(*shape))
    dYd = bf16_dev(dYb)
    s.forward()
    s.backward(dYd)
    first = {k: getattr(s, k).clone() for k in guards}
    s.forward()
    s.backward(dYd)
    torch.cuda.synchronize()
    for k, buf in guards.items():
        assert torch.equal(getattr(s, k), first[k]), f"{k} differs between runs"
        assert torch.all(buf[:PAD] == 7.0) and torch.all(buf[-PAD:] == 7.0), f"{k}: write outside buffer"


def test_step_entry_points_match_composite():
    """The one-kernel step entry points give bitwise the composite results."""
    N, h, F, t, act = 260, 392, 2 * 520, 2, "gelu"
    Xb, dYb = I.gen_x(500, N, h), I.gen_dy(500, N, h)
    W1b, W2b, _ = I.gen_full_weights(500, h, F, t, False)
    c = oracle.column_block(1, t, F)
    s = Shard(N, h, F, t, 1, act, bf16_dev(Xb), bf16_dev(np.ascontiguousarray(W1b[:, c])),
              bf16_dev(np.ascontiguousarray(W2b[c, :])))
    dYd = bf16_dev(dYb)
    s.forward()
    s.backward(dYd, db2=True)
    sh = s.shape
    A = torch.empty_like(s.A); U = torch.empty_like(s.U); Y = torch.empty_like(s.Y)
    dU = torch.empty_like(s.dU); dW1 = torch.empty_like(s.dW1); dW2 = torch.empty_like(s.dW2)
    dX = torch.empty_like(s.dX); db2 = torch.empty_like(s.db2)
    B.tp_mlp_up_act_shard(sh, s.X, s.W1, None, A, U, None)
    B.tp_mlp_down_shard(sh, A, s.W2, Y)
    B.tp_mlp_down_dgrad_act_shard(sh, dYd, s.W2, U, None, dU)
    B.tp_mlp_down_wgrad_shard(sh, A, dYd, dW2)
    B.tp_mlp_up_wgrad_shard(sh, s.X, dU, dW1)
    B.tp_mlp_up_dgrad_shard(sh, dU, s.W1, None, dX)
    ws = B.alloc_workspace(B.bias_grad_workspace_bytes(N, h))
    B.tp_mlp_bias_grad(dYd, db2, ws)
    # both weight gradients in one launch (what the composite runs)
    dW1g, dW2g = torch.empty_like(s.dW1), torch.empty_like(s.dW2)
    B.tp_mlp_wgrad_shard(sh, s.X, A, dYd, dU, dW1g, dW2g)
    torch.cuda.synchronize()
    for a, b, n in [(A, s.A, "A"), (U, s.U, "U"), (Y, s.Y, "Y"), (dU, s.dU, "dU"), (dW1, s.dW1, "dW1"),
                    (dW2, s.dW2, "dW2"), (dX, s.dX, "dX"), (db2, s.db2, "db2"), (dW1g, s.dW1, "dW1 grouped"),
                    (dW2g, s.dW2, "dW2 grouped")]:
        assert torch.equal(a, b), n


@pytest.mark.parametrize("N,h,F,t", [(4096, 4096, 11008, 2), (300, 1032, 2 * 2056, 2)])
def test_grouped_weight_gradients_bitwise_separate(N, h, F, t):
    """SwiGLU: the one-launch weight gradients (dW2, dWg, dW_up) equal the two
    separate launches bitwise (those are checked against the oracle in the
    group tests), at the 7B shard's shape (the two gradients have 1.4 and 2.7
    waves of tiles alone) and at a ragged one."""
    Fi = F // t
    s = B.make_shape(N, h, F, t, 0, "swiglu")
    X, dY = bf16_dev(I.gen_x(510, N, h)), bf16_dev(I.gen_dy(510, N, h))
    A = bf16_dev(I.normal_bf16([510, 7], (N, Fi)))
    dU = bf16_dev(I.normal_bf16([510, 8], (N, 2 * Fi)))
    f32 = dict(dtype=torch.float32, device="cuda")
    out = []
    for grouped in (False, True):
        dW1, dWg, dW2 = torch.empty(h, Fi, **f32), torch.empty(h, Fi, **f32), torch.empty(Fi, h, **f32)
        if grouped:
            B.tp_mlp_wgrad_shard(s, X, A, dY, dU, dW1, dW2, dWg)
        else:
            B.tp_mlp_down_wgrad_shard(s, A, dY, dW2)
            B.tp_mlp_up_wgrad_shard(s, X, dU, dW1, dWg)
        torch.cuda.synchronize()
        out.append((dW1, dWg, dW2))
    for a, b in zip(*out):
        assert torch.equal(a, b)


def _t256(m, n):
    return ((m + 255) // 256) * ((n + 255) // 256)


def _mixed_sweep(seed=20261203, n=8):
    """Seeded shapes whose two backward pairs both take the mixed grid on 256
    CUs (at least 256 tiles of 256 x 256 per pair), with tile counts that do
    not divide evenly over the 8 XCDs."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N = int(rng.integers(1200, 3201))
        h, Fi = 8 * int(rng.integers(200, 601)), 8 * int(rng.integers(200, 601))
        act = ["relu", "gelu", "swiglu"][int(rng.integers(0, 3))]
        g = 2 if act == "swiglu" else 1
        down = _t256(N, Fi) + _t256(Fi, h)           # dU, dW2
        up = _t256(N, h) + _t256(h, g * Fi)          # dX, dW1 (dWg | dWu)
        if down >= 256 and up >= 256 and (down % 8 or up % 8):
            out.append((N, h, Fi, 1, act))
    return out


# Shapes whose backward pairs take the mixed grid (at least 256 tiles of
# 256 x 256 per pair): GeLU with whole tiles, SwiGLU and ReLU ragged in every
# dimension, and a seeded sweep.
@pytest.mark.parametrize("N,h,F,t,act", [(2048, 4096, 8192, 2, "gelu"), (1500, 4104, 6000, 2, "swiglu"),
                                         (2100, 3000, 3504, 1, "relu")] + _mixed_sweep())
def test_mixed_backward_bitwise_separate(N, h, F, t, act):
    """tp_mlp_down_bwd_shard and tp_mlp_up_bwd_shard (one launch each here)
    equal the one-product calls bitwise, and the composite backward equals
    the two of them bitwise; the one-product calls are checked against the
    oracle in the group tests."""
    say(f"[mixed backward] N={N} h={h} F={F} t={t} {act}")
    Fi, sw = F // t, act == "swiglu"
    g = 2 if sw else 1
    s = B.make_shape(N, h, F, t, 0, act)
    X, dY = bf16_dev(I.gen_x(520, N, h)), bf16_dev(I.gen_dy(520, N, h))
    W1 = bf16_dev(I.normal_bf16([520, 1], (h, Fi), I.WEIGHT_SIGMA))
    Wg = bf16_dev(I.normal_bf16([520, 2], (h, Fi), I.WEIGHT_SIGMA)) if sw else None
    W2 = bf16_dev(I.normal_bf16([520, 3], (Fi, h), I.WEIGHT_SIGMA))
    A, U = bf16_dev(I.normal_bf16([520, 4], (N, Fi))), bf16_dev(I.normal_bf16([520, 5], (N, Fi)))
    G = bf16_dev(I.normal_bf16([520, 6], (N, Fi))) if sw else None
    bf, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")

    def outs():
        return (torch.empty(N, g * Fi, **bf), torch.empty(Fi, h, **f32), torch.empty(N, h, **bf),
                torch.empty(h, Fi, **f32), torch.empty(h, Fi, **f32) if sw else None)
    sep, mix, comp = outs(), outs(), outs()
    B.tp_mlp_down_dgrad_act_shard(s, dY, W2, U, G, sep[0])
    B.tp_mlp_down_wgrad_shard(s, A, dY, sep[1])
    B.tp_mlp_up_dgrad_shard(s, sep[0], W1, Wg, sep[2])
    B.tp_mlp_up_wgrad_shard(s, X, sep[0], sep[3], sep[4])
    B.tp_mlp_down_bwd_shard(s, dY, W2, U, G, A, mix[0], mix[1])
    B.tp_mlp_up_bwd_shard(s, X, mix[0], W1, Wg, mix[2], mix[3], mix[4])
    B.tp_mlp_bwd_shard(s, X, W1, Wg, W2, dY, A, U, G, comp[0], comp[3], comp[4], comp[1], comp[2])
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dU", "dW2", "dX", "dW1", "dWg"), sep, mix, comp):
        if a is None:
            continue
        assert torch.equal(a, b), f"{name}: mixed launch differs from the separate calls"
        assert torch.equal(b, c), f"{name}: composite differs from the step calls"
