"""The forward entry point that allocates nothing (tp_mlp_fwd_shard_noalloc),
through the C ABI: its k-split partials live in the library's fixed per-GPU
scratch instead of a caller's workspace.  It runs the same kernels as
tp_mlp_fwd_shard, so its outputs must equal that call's bitwise.  Four calls
in a row, each smaller than the one before, share the scratch: the 70B shard
at 128 and at 32 tokens (small-batch path, 60 and 15 MiB of partials), a
7B-shaped shard at one token (the decode GEMVs, under 1 MiB), and a ragged
SwiGLU shard at 5 tokens.
A shape beyond the scratch is refused before any launch (host test in
test_abi_host.py)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from megatron_tensor_transformer_rank_amd import binding as B
from megatron_tensor_transformer_rank_amd import inputs as I
from tests.helpers import bf16_dev

pytestmark = pytest.mark.gpu

# (wid, N, h, F, t, act)
CALLS = [(933, 128, 8192, 28672, 4, "swiglu"), (930, 32, 8192, 28672, 4, "swiglu"), (931, 1, 4096, 11008, 2, "gelu"), (932, 5, 1032, 2 * 776, 2, "swiglu")]


def test_noalloc_forward_equals_workspace_forward():
    bf = dict(dtype=torch.bfloat16, device="cuda")
    for wid, N, h, F, t, act in CALLS:
        print(f"[noalloc] N={N} h={h} F={F} t={t} {act}", file=sys.stderr, flush=True)
        s = B.make_shape(N, h, F, t, 1, act)
        Fi, sw = s.Fi, act == "swiglu"
        need = B.workspace_bytes(s, False)
        assert 0 < need <= 64 << 20
        X = bf16_dev(I.gen_x(wid, N, h))
        W1 = bf16_dev(I.normal_bf16([wid, 1], (h, Fi), I.WEIGHT_SIGMA))
        Wg = bf16_dev(I.normal_bf16([wid, 2], (h, Fi), I.WEIGHT_SIGMA)) if sw else None
        W2 = bf16_dev(I.normal_bf16([wid, 3], (Fi, h), I.WEIGHT_SIGMA))
        outs = []
        for noalloc in (False, True):
            Y, A, U = torch.full((N, h), float("nan"), **bf), torch.full((N, Fi), float("nan"), **bf), \
                torch.full((N, Fi), float("nan"), **bf)
            G = torch.full((N, Fi), float("nan"), **bf) if sw else None
            if noalloc:
                B.tp_mlp_fwd_shard_noalloc(s, X, W1, Wg, W2, Y, A, U, G)
            else:
                ws = B.alloc_workspace(need)
                ws.fill_(0xFF)                  # every float of it a NaN
                B.tp_mlp_fwd_shard(s, X, W1, Wg, W2, Y, A, U, G, ws)
            torch.cuda.synchronize()
            outs.append((Y, A, U, G))
        for name, a, b in zip(("Y_i", "A_i", "U_i", "G_i"), *outs):
            if a is None:
                continue
            assert torch.isfinite(a.float()).all(), f"{name}: not written"
            assert torch.equal(a, b), f"{name}: N={N} h={h}: the no-allocation call differs from the workspace call"
