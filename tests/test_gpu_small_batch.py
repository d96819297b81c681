"""GPU parity of the small-batch path (up to 128 tokens) against the fp64
oracle, through the C ABI.

tp_mlp_fwd_shard routes 2 <= N <= 128 to split-K MFMA products that stream
each weight once.  In the backward (1 <= N <= 128) the two input gradients
(dU through W2 and the activation, dX_partial through W1) run as split-K
products too, their float32 partials kept in the weight gradient's storage
before the weight gradient (k = N) runs on the wide tiles; a shape whose
weight-gradient storage cannot hold one split (h < N for dU, F_i < g*N for
dX) keeps the wide tiles.  Checked:

* whole tensor-parallel groups (forward on this path, backward on the GEMMs,
  the partials reduced) at token counts on both sides of every row-tile
  boundary (16, 32, 64) and at the path's edges (2 and 128; 129 goes to the
  GEMMs), with ragged h and F_i (k-split and column-strip tails), all
  activations, with and without the stash.  Small weights split the rows
  into two to four 32-row tiles; larger ones keep one 64- or 128-row tile,
  or take two 64-row tiles;
* the Llama-3-70B-shaped decode shard at full size (h = 8192, F_i = 7168,
  SwiGLU) for batches of 2, 8, 32, 64 and 128 tokens: A_i, the stashes and Y_i of
  rank 0 against the oracle;
* the result does not depend on which buffer held the workspace before
  (two calls, the second on a dirtied workspace, bitwise equal);
* the backward step calls (tp_mlp_down_bwd_shard, tp_mlp_up_bwd_shard) equal
  the composite backward bitwise, their weight gradients equal the
  one-product calls bitwise, and their input gradients agree with the
  one-product calls (the wide tiles, a different summation order) to the
  parity bound;
* the 70B shard's backward at full size for 8 and 128 tokens against the
  oracle (dU, dX_i, and sampled weight-gradient columns).
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
from tests.helpers import Shard, assert_close, bf16_dev, f64, run_group

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (wid, N, h, F, t, act, bias)
GROUPS = [
    (301, 2, 1032, 2080, 2, "gelu", False),
    (302, 3, 520, 2 * 776, 2, "swiglu", True),     # F_i = 776: the last 256-column strip is 8 wide
    (303, 16, 4104, 3 * 1544, 3, "relu", False),   # h = 4104: a 8-deep k tail
    (304, 17, 264, 4 * 392, 4, "swiglu", False),
    (305, 32, 1024, 4096, 2, "gelu", True),
    (306, 33, 136, 512, 1, "relu", False),
    (307, 64, 392, 2 * 520, 2, "swiglu", True),
    (308, 65, 392, 2 * 520, 2, "swiglu", True),    # first count past 64 rows: three 32-row tiles
    (330, 96, 4104, 2 * 776, 2, "gelu", False),    # k tail and an 8-wide strip
    (331, 127, 264, 3 * 392, 3, "relu", True),
    (332, 128, 1032, 2 * 1040, 2, "swiglu", False),
    (333, 129, 392, 2 * 520, 2, "swiglu", True),   # just past the path: wide-tile GEMMs
    (334, 96, 64, 2 * 80, 2, "swiglu", False),     # h < N and F_i < 2N: the backward keeps the wide tiles
    (335, 40, 520, 2 * 56, 2, "gelu", True),       # F_i = 56: one k-split fits dX's partials
    (336, 1, 2056, 2 * 1544, 2, "relu", False),    # one token: split-K backward
    # Smaller weights than these split the rows into 32-row tiles; these keep
    # the 64- and 128-row tiles: one 64-row tile; 128-row tiles for the gate/up
    # product and dX with two 64-row tiles for the down product and dU (k
    # tail, 8-wide last strip)
    (337, 48, 4104, 2 * 4104, 2, "gelu", False),
    (338, 100, 2056, 2 * 2056, 2, "swiglu", True),
    (339, 72, 3080, 2 * 1544, 2, "swiglu", False),
]


@pytest.mark.parametrize("case", GROUPS, ids=[f"N{c[1]}_h{c[2]}_F{c[3]}_t{c[4]}_{c[5]}" for c in GROUPS])
def test_small_batch_group_matches_oracle(case):
    run_group(*case)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_small_batch_without_stash(act):
    """Inference: forward only, no stash buffers; both ranks' partials reduced."""
    sw = act == "swiglu"
    N, h, F, t = 8, 520, 2 * 1040, 2
    say(f"[small batch no stash] N={N} h={h} F={F} t={t} act={act}")
    wid = 310 + len(act)
    Xb = I.gen_x(wid, N, h)
    W1b, W2b, Wgb = I.gen_full_weights(wid, h, F, t, sw)
    f = oracle.bf16_bits_to_f64
    Yref, fr = oracle.tp_forward(act, f(Xb), f(W1b), f(W2b), t, Wg=f(Wgb) if sw else None)
    parts = []
    for r in range(t):
        c = oracle.column_block(r, t, F)
        s = Shard(N, h, F, t, r, act, bf16_dev(Xb), bf16_dev(np.ascontiguousarray(W1b[:, c])),
                  bf16_dev(np.ascontiguousarray(W2b[c, :])),
                  bf16_dev(np.ascontiguousarray(Wgb[:, c])) if sw else None, stash=False)
        s.forward()
        parts.append(s)
    Y = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([s.Y for s in parts], Y)
    torch.cuda.synchronize()
    for r, s in enumerate(parts):
        assert_close(f"A[{r}]", f64(s.A), fr[r]["A"])
    assert_close("Y", f64(Y), Yref)


@pytest.mark.parametrize("N", [2, 8, 32, 64, 128])
def test_small_batch_llama3_70b_shard_full_size(N):
    w = WORKLOADS["llama3_70b_decode_t4"]
    h, Fi = w.h, w.Fi
    say(f"[small batch full size] N={N} h={h} F_i={Fi} swiglu")
    Xb = I.normal_bf16([w.wid, 40, N], (N, h))
    W1b = I.gen_w_up_shard(w.wid, h, Fi, 0)
    Wgb = I.gen_w_gate_shard(w.wid, h, Fi, 0)
    W2b = I.gen_w_down_shard(w.wid, h, Fi, 0)
    f = oracle.bf16_bits_to_f64
    ref = oracle.shard_forward("swiglu", f(Xb), f(W1b), f(W2b), f(Wgb))
    shape = B.make_shape(N, h, w.F, w.t, 0, "swiglu")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    Y, A = torch.empty(N, h, **bf), torch.empty(N, Fi, **bf)
    U, G = torch.empty(N, Fi, **bf), torch.empty(N, Fi, **bf)
    ws = B.alloc_workspace(B.workspace_bytes(shape, False))
    assert ws is not None
    B.tp_mlp_fwd_shard(shape, bf16_dev(Xb), bf16_dev(W1b), bf16_dev(Wgb), bf16_dev(W2b), Y, A, U, G, ws)
    torch.cuda.synchronize()
    assert_close("G", f64(G), ref["G"])
    assert_close("U", f64(U), ref["U"])
    assert_close("A", f64(A), ref["A"])
    assert_close("Y_i", f64(Y), ref["Y"])


def test_small_batch_deterministic_and_workspace_contents_irrelevant():
    N, h, F, t, act = 24, 1032, 2 * 1544, 2, "gelu"
    Xb = I.gen_x(320, N, h)
    W1b, W2b, _ = I.gen_full_weights(320, h, F, t, False)
    c = oracle.column_block(0, t, F)
    shape = B.make_shape(N, h, F, t, 0, act)
    Fi = F // t
    X, W1, W2 = bf16_dev(Xb), bf16_dev(np.ascontiguousarray(W1b[:, c])), bf16_dev(np.ascontiguousarray(W2b[c, :]))
    ws = B.alloc_workspace(B.workspace_bytes(shape, False))
    outs = []
    for fill in (0, 0x7f):
        ws.fill_(fill)
        Y = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
        A = torch.empty(N, Fi, dtype=torch.bfloat16, device="cuda")
        B.tp_mlp_fwd_shard(shape, X, W1, None, W2, Y, A, None, None, ws)
        torch.cuda.synchronize()
        outs.append((Y.clone(), A.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# (wid, N, h, F, t, act)
BWD_STEPS = [(340, 1, 1032, 2 * 776, 2, "swiglu"), (341, 8, 4104, 2 * 1544, 2, "gelu"),
             (342, 77, 1544, 3 * 1032, 3, "relu"), (343, 128, 1024, 4096, 2, "gelu"),
             (344, 128, 2056, 2 * 2064, 2, "swiglu")]


@pytest.mark.parametrize("case", BWD_STEPS, ids=[f"N{c[1]}_h{c[2]}_F{c[3]}_{c[5]}" for c in BWD_STEPS])
def test_small_batch_backward_step_calls(case):
    wid, N, h, F, t, act = case
    say(f"[small batch backward steps] N={N} h={h} F={F} t={t} {act}")
    Fi, sw = F // t, act == "swiglu"
    g = 2 if sw else 1
    s = B.make_shape(N, h, F, t, 0, act)
    X, dY = bf16_dev(I.gen_x(wid, N, h)), bf16_dev(I.gen_dy(wid, N, h))
    W1 = bf16_dev(I.normal_bf16([wid, 1], (h, Fi), I.WEIGHT_SIGMA))
    Wg = bf16_dev(I.normal_bf16([wid, 2], (h, Fi), I.WEIGHT_SIGMA)) if sw else None
    W2 = bf16_dev(I.normal_bf16([wid, 3], (Fi, h), I.WEIGHT_SIGMA))
    A, U = bf16_dev(I.normal_bf16([wid, 4], (N, Fi))), bf16_dev(I.normal_bf16([wid, 5], (N, Fi)))
    G = bf16_dev(I.normal_bf16([wid, 6], (N, Fi))) if sw else None
    bf, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")

    def outs():
        return (torch.empty(N, g * Fi, **bf), torch.empty(Fi, h, **f32), torch.empty(N, h, **bf),
                torch.empty(h, Fi, **f32), torch.empty(h, Fi, **f32) if sw else None)
    sep, steps, comp = outs(), outs(), outs()
    B.tp_mlp_down_dgrad_act_shard(s, dY, W2, U, G, sep[0])
    B.tp_mlp_down_wgrad_shard(s, A, dY, sep[1])
    B.tp_mlp_down_bwd_shard(s, dY, W2, U, G, A, steps[0], steps[1])
    # the up-projection's calls on the same dU
    B.tp_mlp_up_dgrad_shard(s, steps[0], W1, Wg, sep[2])
    B.tp_mlp_up_wgrad_shard(s, X, steps[0], sep[3], sep[4])
    B.tp_mlp_up_bwd_shard(s, X, steps[0], W1, Wg, steps[2], steps[3], steps[4])
    B.tp_mlp_bwd_shard(s, X, W1, Wg, W2, dY, A, U, G, comp[0], comp[3], comp[4], comp[1], comp[2])
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dU", "dW2", "dX", "dW1", "dWg"), sep, steps, comp):
        if a is None:
            continue
        assert torch.equal(b, c), f"{name}: composite differs from the step calls"
        if name.startswith("dW"):
            assert torch.equal(a, b), f"{name}: differs from the one-product call"
        else:
            assert_close(name, f64(b), f64(a))


@pytest.mark.parametrize("N", [8, 128])
def test_small_batch_backward_llama3_70b_shard_full_size(N):
    """Rank 0 of the 70B shard (h = 8192, F_i = 7168, SwiGLU): forward, then
    the backward through the composite call; dU and dX_i whole, 64 sampled
    columns of each weight gradient."""
    w = WORKLOADS["llama3_70b_decode_t4"]
    h, Fi = w.h, w.Fi
    say(f"[small batch backward full size] N={N} h={h} F_i={Fi} swiglu")
    Xb, dYb = I.normal_bf16([w.wid, 41, N], (N, h)), I.normal_bf16([w.wid, 42, N], (N, h))
    W1b = I.gen_w_up_shard(w.wid, h, Fi, 0)
    Wgb = I.gen_w_gate_shard(w.wid, h, Fi, 0)
    W2b = I.gen_w_down_shard(w.wid, h, Fi, 0)
    f = oracle.bf16_bits_to_f64
    ref = oracle.shard_backward("swiglu", f(Xb), f(W1b), f(W2b), f(dYb), f(Wgb))
    shape = B.make_shape(N, h, w.F, w.t, 0, "swiglu")
    bf, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    W1, Wg, W2 = bf16_dev(W1b), bf16_dev(Wgb), bf16_dev(W2b)
    Y, A = torch.empty(N, h, **bf), torch.empty(N, Fi, **bf)
    U, G = torch.empty(N, Fi, **bf), torch.empty(N, Fi, **bf)
    ws = B.alloc_workspace(B.workspace_bytes(shape, False))
    B.tp_mlp_fwd_shard(shape, X, W1, Wg, W2, Y, A, U, G, ws)
    dU, dX = torch.empty(N, 2 * Fi, **bf), torch.empty(N, h, **bf)
    dW1, dWg, dW2 = torch.empty(h, Fi, **f32), torch.empty(h, Fi, **f32), torch.empty(Fi, h, **f32)
    B.tp_mlp_bwd_shard(shape, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX)
    torch.cuda.synchronize()
    du = f64(dU)
    assert_close("dG", du[:, :Fi], ref["dG"])
    assert_close("dP", du[:, Fi:], ref["dU"])
    assert_close("dX_i", f64(dX), ref["dX"])
    rng = np.random.default_rng(N)
    cf, ch = np.sort(rng.choice(Fi, 64, replace=False)), np.sort(rng.choice(h, 64, replace=False))
    assert_close("dW1 cols", dW1[:, cf].cpu().double().numpy(), ref["dW1"][:, cf])
    assert_close("dWg cols", dWg[:, cf].cpu().double().numpy(), ref["dWg"][:, cf])
    assert_close("dW2 cols", dW2[:, ch].cpu().double().numpy(), ref["dW2"][:, ch])
