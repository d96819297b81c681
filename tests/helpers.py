"""Shared test utilities: moving the generator's bf16 bit patterns to the
device, reading device results back as float64, the tolerance metrics, and
running one rank's shard through the C ABI."""
from __future__ import annotations

import numpy as np
import torch

from megatron_tensor_transformer_rank_amd import binding as B

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
