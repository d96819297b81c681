"""Shared test utilities: moving the generator's bf16 bit patterns to the
device, reading device results back as float64, the tolerance metrics,
running one rank's shard through the C ABI, and running a whole
tensor-parallel group against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I

# Tolerances for bf16 inputs with float32 accumulation (stated with the
# method's target): relative Frobenius error and max elementwise error as a
# fraction of max |ref|.
REL_FRO = 5e-3
MAX_REL = 3e-2


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    d = gpu - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mref = np.abs(ref).max() if ref.size else 0.0
    mx = np.abs(d).max() / mref if mref > 0 else (np.abs(d).max() if d.size else 0.0)
    return rel, mx


def assert_close(name: str, gpu, ref, rel_fro=REL_FRO, max_rel=MAX_REL):
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    rel, mx = errors(gpu, ref)
    assert rel <= rel_fro and mx <= max_rel, f"{name}: relFro {rel:.3e} (<= {rel_fro}), maxabs/max {mx:.3e} (<= {max_rel})"
    return rel, mx


def assert_relu_grad(name: str, gpu_dU, ref_dU, ref_dA, X, W1, rel_fro=REL_FRO, max_rel=MAX_REL):
    """dU = dA * [U > 0] through ReLU, whose derivative is a decision on the
    sign of U (ReLU'(0) = 0).  The GPU takes it on U accumulated in float32;
    where the exact |U| is within the worst-case float32 accumulation bound
    h * 2^-24 * sum_k |x_k w_k|, either decision is correct.  The GPU's
    epilogue writes exactly 0 or its rounded dA there, so such an element
    must be exactly 0, or within dA's own elementwise tolerance of dA.  The
    reference takes the GPU's decision at those elements (0 or dA) and the
    GPU values are left as they are, so the dA decisions still count in the
    error.  Returns that reference: the one the gradients computed from dU
    are compared against."""
    gpu = np.array(gpu_dU, dtype=np.float64)
    X, W1 = np.asarray(X, np.float64), np.asarray(W1, np.float64)
    U = X @ W1
    amb = np.abs(U) <= X.shape[1] * 2.0 ** -24 * (np.abs(X) @ np.abs(W1))
    if np.any(amb):
        dA = np.asarray(ref_dA, np.float64)
        tol = max_rel * np.abs(dA).max()
        g, a = gpu[amb], dA[amb]
        zero, kept = g == 0.0, np.abs(g - a) <= tol
        ok = zero | kept
        assert np.all(ok), f"{name}: {int((~ok).sum())} of {int(amb.sum())} sign-ambiguous elements are neither 0 nor dA"
        ref_dU = np.array(ref_dU, dtype=np.float64)
        ref_dU[amb] = np.where(zero, 0.0, a)   # the GPU's decision
    assert_close(name, gpu, ref_dU, rel_fro, max_rel)
    return ref_dU


class Shard:
    """Device buffers of one rank's shard and its forward / backward through
    the composite C entry points."""

    def __init__(self, N, h, F, t, rank, act, X, W1_i, W2_i, Wg_i=None, stash=True):
        self.shape = B.make_shape(N, h, F, t, rank, act)
        Fi, g = self.shape.Fi, self.shape.g
        dev = "cuda"
        self.X, self.W1, self.W2 = X, W1_i, W2_i
        self.Wg = Wg_i
        bf = torch.bfloat16
        self.Y = torch.empty(N, h, dtype=bf, device=dev)
        self.A = torch.empty(N, Fi, dtype=bf, device=dev)
        self.U = torch.empty(N, Fi, dtype=bf, device=dev) if stash else None
        self.G = torch.empty(N, Fi, dtype=bf, device=dev) if (stash and act == "swiglu") else None
        self.dU = torch.empty(N, g * Fi, dtype=bf, device=dev)
        self.dW1 = torch.empty(h, Fi, dtype=torch.float32, device=dev)
        self.dWg = torch.empty(h, Fi, dtype=torch.float32, device=dev) if act == "swiglu" else None
        self.dW2 = torch.empty(Fi, h, dtype=torch.float32, device=dev)
        self.dX = torch.empty(N, h, dtype=bf, device=dev)
        self.db2 = torch.empty(h, dtype=torch.float32, device=dev)
        self.ws_f = B.alloc_workspace(B.workspace_bytes(self.shape, False))
        self.ws_b = B.alloc_workspace(B.workspace_bytes(self.shape, True))

    def forward(self):
        B.tp_mlp_fwd_shard(self.shape, self.X, self.W1, self.Wg, self.W2, self.Y, self.A,
                           self.U, self.G, self.ws_f)

    def backward(self, dY, db2=False):
        B.tp_mlp_bwd_shard(self.shape, self.X, self.W1, self.Wg, self.W2, dY, self.A, self.U,
                           self.G, self.dU, self.dW1, self.dWg, self.dW2, self.dX,
                           self.db2 if db2 else None, self.ws_b)


def run_group(wid, N, h, F, t, act, bias, stash=True):
    """Run all t shards fwd+bwd on the GPU and the oracle on the same bf16
    inputs; compare everything."""
    print(f"[group] wid={wid} N={N} h={h} F={F} t={t} act={act} bias={bias}", file=sys.stderr, flush=True)
    sw = act == "swiglu"
    Fi = F // t
    Xb, dYb = I.gen_x(wid, N, h), I.gen_dy(wid, N, h)
    W1b, W2b, Wgb = I.gen_full_weights(wid, h, F, t, sw)
    b2b = I.gen_b2(wid, h) if bias else None
    X, dY = oracle.bf16_bits_to_f64(Xb), oracle.bf16_bits_to_f64(dYb)
    W1, W2 = oracle.bf16_bits_to_f64(W1b), oracle.bf16_bits_to_f64(W2b)
    Wg = oracle.bf16_bits_to_f64(Wgb) if sw else None
    b2 = oracle.bf16_bits_to_f64(b2b) if bias else None
    Yref, fr = oracle.tp_forward(act, X, W1, W2, t, Wg=Wg, b2=b2)
    _, db2ref, br = oracle.tp_backward(act, X, W1, W2, dY, t, Wg=Wg)

    Xd, dYd = bf16_dev(Xb), bf16_dev(dYb)
    shards = []
    for r in range(t):
        c = oracle.column_block(r, t, F)
        s = Shard(N, h, F, t, r, act, Xd, bf16_dev(np.ascontiguousarray(W1b[:, c])),
                  bf16_dev(np.ascontiguousarray(W2b[c, :])),
                  bf16_dev(np.ascontiguousarray(Wgb[:, c])) if sw else None, stash=stash)
        s.forward()
        s.backward(dYd, db2=(r == 0))
        shards.append(s)
    Y = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([s.Y for s in shards], Y, bias=bf16_dev(b2b) if bias else None)
    dX = torch.empty(N, h, dtype=torch.bfloat16, device="cuda")
    B.tp_mlp_reduce_partials_local([s.dX for s in shards], dX)
    torch.cuda.synchronize()

    dX_parts = []
    for r, s in enumerate(shards):
        f, b = fr[r], br[r]
        dW1_ref, dX_ref = b["dW1"], b["dX"]
        assert_close(f"A[{r}]", f64(s.A), f["A"])
        if stash:
            assert_close(f"U[{r}]", f64(s.U), f["U"])
            if sw:
                assert_close(f"G[{r}]", f64(s.G), f["G"])
        assert_close(f"Y_i[{r}]", f64(s.Y), f["Y"])
        dU = f64(s.dU)
        if sw:
            assert_close(f"dG[{r}]", dU[:, :Fi], b["dG"])
            assert_close(f"dP[{r}]", dU[:, Fi:], b["dU"])
            assert_close(f"dWg[{r}]", f64(s.dWg), b["dWg"])
        elif act == "relu":
            # the GPU's ReLU decisions at sign-ambiguous pre-activations are
            # valid; the gradients computed from dU follow them
            c = oracle.column_block(r, t, F)
            dU_ref = assert_relu_grad(f"dU[{r}]", dU, b["dU"], b["dA"], X, W1[:, c])
            if not np.array_equal(dU_ref, b["dU"]):
                dW1_ref, dX_ref = X.T @ dU_ref, dU_ref @ W1[:, c].T
        else:
            assert_close(f"dU[{r}]", dU, b["dU"])
        assert_close(f"dW1[{r}]", f64(s.dW1), dW1_ref)
        assert_close(f"dW2[{r}]", f64(s.dW2), b["dW2"])
        assert_close(f"dX_i[{r}]", f64(s.dX), dX_ref)
        dX_parts.append(dX_ref)
    assert_close("Y", f64(Y), Yref)
    assert_close("dX", f64(dX), oracle.reduce_partials(dX_parts))
    assert_close("db2", f64(shards[0].db2), db2ref, rel_fro=1e-5, max_rel=1e-5)
    return shards, Y, dX


