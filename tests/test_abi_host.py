"""Host-only checks of the C ABI: the library loads, exports every function
the header declares, and rejects invalid arguments before touching the GPU
(no compute calls are made here)."""
import ctypes
import os
import re

import pytest

from megatron_tensor_transformer_rank_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced by validation


def P(k):
    """The k-th fake device buffer: 1 GiB apart, so distinct buffers never
    overlap and each check below fails for the reason it names."""
    return FAKE + k * (1 << 30)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tp_(?:mlp|attn|sp)_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    for required in ("tp_mlp_fwd_shard", "tp_mlp_bwd_shard", "tp_mlp_reduce_partials_local",
                     "tp_attn_qkv_shard", "tp_attn_out_shard", "tp_attn_out_bwd_shard", "tp_attn_qkv_bwd_shard",
                     "tp_sp_layernorm_fwd", "tp_sp_reduce_scatter_layernorm_local", "tp_sp_layernorm_bwd",
                     "tp_sp_layernorm_bwd_workspace_bytes", "tp_sp_sum_grads_local"):
        assert required in names


def test_status_strings():
    for s in range(5):
        assert B.status_string(s)
    assert B.status_string(99) == "unknown status"


def test_workspace_sizes():
    assert B.workspace_bytes(B.make_shape(129, 1024, 4096, 2, 0, "gelu"), False) == 0
    dec = B.workspace_bytes(B.make_shape(1, 8192, 28672, 4, 0, "swiglu"), False)
    assert dec > 0 and dec % 256 == 0
    # bias-gradient scratch: at most 64 row slabs of float32 columns
    assert 0 < B.workspace_bytes(B.make_shape(16384, 8192, 28672, 4, 0, "swiglu"), True) <= 64 * 8192 * 4
    assert B.workspace_bytes(B.make_shape(4, 8, 12, 5, 0, "gelu"), False) == 0  # invalid: F % t
    assert B.bias_grad_workspace_bytes(1, 8) == 8 * 4


def _fwd(shape, **over):
    a = dict(X=P(0), W1=P(1), Wg=None, W2=P(3), Y=P(4), A=P(5), U=None, G=None, ws=None, wsb=0)
    a.update(over)
    return B.lib().tp_mlp_fwd_shard(ctypes.byref(shape), a["X"], a["W1"], a["Wg"], a["W2"], a["Y"],
                                    a["A"], a["U"], a["G"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("shape,expect", [
    (B.make_shape(-1, 64, 128, 1, 0, "gelu"), INVALID),        # N < 0
    (B.make_shape(4, 60, 128, 1, 0, "gelu"), INVALID),         # h % 8
    (B.make_shape(4, 64, 100, 2, 0, "gelu"), INVALID),         # F_i = 50, not a multiple of 8
    (B.make_shape(4, 64, 130, 4, 0, "gelu"), INVALID),         # F % t
    (B.make_shape(4, 64, 128, 2, 2, "gelu"), INVALID),         # rank >= t
    (B.make_shape(4, 64, 128, 2, -1, "gelu"), INVALID),        # rank < 0
    (B.make_shape(4, 64, 128, 2, 0, 7), INVALID),              # unknown activation
    (B.make_shape(4, 64, 128 * 80, 80, 0, "gelu"), UNSUPPORTED),  # t > 64
])
def test_fwd_rejects_bad_shapes(shape, expect):
    assert _fwd(shape) == expect


@pytest.mark.parametrize("shape", [
    B.make_shape(1 << 18, 8192, 16, 2, 0, "gelu"),           # X: 2^31 elements, past one buffer resource
    B.make_shape(16, 65536, 2 * 65536, 2, 0, "relu"),        # W1_i: 2^32 elements
    B.make_shape(1 << 16, 64, 2 * (1 << 15), 2, 0, "swiglu"),  # [dG | dP]: N * 2F_i = 2^32 elements
], ids=["X", "W1", "dU"])
def test_operands_past_the_buffer_limit_are_unsupported(shape):
    """Every bf16 operand a GEMM reads is addressed through one buffer
    resource (< 4 GiB): larger shapes are UNSUPPORTED for every entry point,
    before any launch."""
    L = B.lib()
    r = ctypes.byref(shape)
    assert _fwd(shape) == UNSUPPORTED
    assert L.tp_mlp_bwd_shard(r, *([P(k) for k in range(13)] + [None, None, 0, None])) == UNSUPPORTED
    assert L.tp_mlp_up_act_shard(r, P(0), P(1), P(2), P(3), P(4), P(5), None) == UNSUPPORTED
    assert L.tp_mlp_wgrad_shard(r, P(0), P(1), P(2), P(3), P(4), P(5), P(6), None) == UNSUPPORTED


def test_attn_operands_past_the_buffer_limit_are_unsupported():
    s = B.make_attn_shape(1 << 18, 8192, 64, 8, 128, 4, 0)    # X: 2^31 elements
    r = ctypes.byref(s)
    assert B.lib().tp_attn_qkv_shard(r, P(0), P(1), P(2), None, 0, None) == UNSUPPORTED
    assert B.lib().tp_attn_qkv_bwd_shard(r, P(0), P(1), P(2), P(3), P(4), None) == UNSUPPORTED
    assert B.attn_workspace_bytes(s) == 0


def test_fwd_rejects_bad_pointers():
    s = B.make_shape(4, 64, 128, 2, 0, "gelu")
    assert _fwd(s, X=None) == INVALID
    assert _fwd(s, W2=None) == INVALID
    assert _fwd(s, Y=P(4) + 2) == INVALID                       # misaligned
    assert _fwd(s, Wg=P(2)) == INVALID                          # gate weight given without SwiGLU
    assert _fwd(s, G=P(7)) == INVALID                           # gate stash without SwiGLU
    sw = B.make_shape(4, 64, 128, 2, 0, "swiglu")
    assert _fwd(sw) == INVALID                                  # SwiGLU needs the gate shard
    assert _fwd(sw, Wg=P(2), U=P(6)) == INVALID                 # U and G stashes come together
    dec = B.make_shape(1, 64, 128, 2, 0, "gelu")
    assert _fwd(dec) == WORKSPACE                               # decode path needs workspace
    assert _fwd(dec, ws=P(8), wsb=16) == WORKSPACE


def test_fwd_rejects_overlaps():
    """Outputs may not overlap each other, an input or the workspace in use
    (N = 4, h = 64, F_i = 64: Y and X 512 B, A 512 B, weights 8 KiB)."""
    s = B.make_shape(4, 64, 128, 2, 0, "gelu")
    assert _fwd(s, Y=P(0)) == INVALID                           # Y on X
    assert _fwd(s, A=P(4) + 256) == INVALID                     # A inside Y
    assert _fwd(s, Y=P(1) + 4096) == INVALID                    # Y inside W1
    assert _fwd(s, U=P(5)) == INVALID                           # the stash on A
    dec = B.make_shape(1, 64, 128, 2, 0, "gelu")
    need = B.workspace_bytes(dec, False)
    assert _fwd(dec, ws=P(3), wsb=need) == INVALID              # workspace on W2
    assert _fwd(dec, ws=P(4), wsb=need) == INVALID              # workspace on Y


def test_bwd_rejects_bad_arguments():
    s = B.make_shape(4, 64, 128, 2, 0, "gelu")
    args = [P(k) for k in range(13)] + [None, None, 0, None]
    base = dict(zip(["X", "W1", "Wg", "W2", "dY", "A", "U", "G", "dU", "dW1", "dWg", "dW2", "dX",
                     "db2", "ws", "wsb", "st"], args))
    base.update(Wg=None, G=None, dWg=None)

    def call(**o):
        a = dict(base)
        a.update(o)
        return B.lib().tp_mlp_bwd_shard(ctypes.byref(s), *a.values())

    assert call(U=None) == INVALID
    assert call(dW2=P(11) + 4) == INVALID
    assert call(dWg=P(10)) == INVALID
    assert call(db2=P(13)) == WORKSPACE
    # overlaps: outputs against inputs and each other, the workspace in use
    assert call(dX=P(4)) == INVALID                             # dX on dY
    assert call(dU=P(5)) == INVALID                             # dU on A
    assert call(dW1=P(11) + 1024) == INVALID                    # dW1 inside dW2
    assert call(db2=P(13), ws=P(12), wsb=1 << 20) == INVALID    # workspace on dX


def test_reduce_rejects_bad_arguments():
    L = B.lib()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.tp_mlp_reduce_partials_local(0, ptrs, 4, 8, None, FAKE, None) == INVALID
    assert L.tp_mlp_reduce_partials_local(2, None, 4, 8, None, FAKE, None) == INVALID
    assert L.tp_mlp_reduce_partials_local(2, ptrs, 4, 12, None, FAKE, None) == INVALID
    assert L.tp_mlp_reduce_partials_local(2, ptrs, -1, 8, None, FAKE, None) == INVALID
    assert L.tp_mlp_reduce_partials_local(2, ptrs, 4, 8, FAKE + 8, FAKE, None) == INVALID
    bad = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.tp_mlp_reduce_partials_local(2, bad, 4, 8, None, FAKE, None) == INVALID
    big = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert L.tp_mlp_reduce_partials_local(65, big, 4, 8, None, FAKE, None) == UNSUPPORTED


def test_step_entry_points_validate():
    L = B.lib()
    s = B.make_shape(4, 64, 128, 2, 0, "swiglu")
    r = ctypes.byref(s)
    assert L.tp_mlp_up_act_shard(r, P(0), P(1), None, P(2), None, None, None) == INVALID    # SwiGLU: no gate
    assert L.tp_mlp_down_shard(r, P(0), None, P(2), None) == INVALID
    assert L.tp_mlp_down_dgrad_act_shard(r, P(0), P(1), P(2), None, P(3), None) == INVALID  # no gate stash
    assert L.tp_mlp_down_wgrad_shard(r, P(0), P(1), P(2) + 1, None) == INVALID
    assert L.tp_mlp_up_wgrad_shard(r, P(0), P(1), P(2), None, None) == INVALID             # no dWg
    assert L.tp_mlp_up_dgrad_shard(r, P(0), P(1), None, P(2), None) == INVALID             # no Wg
    assert L.tp_mlp_bias_grad(P(0), 4, 12, P(1), P(2), 1 << 20, None) == INVALID
    assert L.tp_mlp_bias_grad(P(0), 4, 8, P(1), None, 0, None) == WORKSPACE
    # overlaps of each step's output with its inputs
    assert L.tp_mlp_up_act_shard(r, P(0), P(1), P(2), P(0), P(4), P(5), None) == INVALID   # A on X
    assert L.tp_mlp_down_shard(r, P(0), P(1), P(1), None) == INVALID                       # Y on W2
    assert L.tp_mlp_down_dgrad_act_shard(r, P(0), P(1), P(2), P(3), P(3), None) == INVALID  # dU on G
    assert L.tp_mlp_down_wgrad_shard(r, P(0), P(1), P(0), None) == INVALID                 # dW2 on A
    assert L.tp_mlp_up_wgrad_shard(r, P(0), P(1), P(2), P(2) + 64, None) == INVALID        # dWg inside dW1
    assert L.tp_mlp_up_dgrad_shard(r, P(0), P(1), P(2), P(2), None) == INVALID             # dX on Wg
    assert L.tp_mlp_bias_grad(P(0), 4, 8, P(1), P(0), 1 << 20, None) == INVALID            # workspace on dY
    wg = L.tp_mlp_wgrad_shard                     # (s, X, A, dY, dU, dW1, dWg, dW2)
    assert wg(r, P(0), P(1), P(2), P(3), P(4), None, P(6), None) == INVALID               # SwiGLU: dWg needed
    assert wg(r, P(0), P(1), P(2), P(3), P(4), P(5), P(3), None) == INVALID               # dW2 on dU
    assert wg(r, P(0), P(1), P(2), P(3), P(4), P(4) + 1024, P(6), None) == INVALID        # dWg inside dW1
    assert wg(r, P(0), None, P(2), P(3), P(4), P(5), P(6), None) == INVALID
    db = L.tp_mlp_down_bwd_shard                  # (s, dY, W2, U, G, A, dU, dW2)
    assert db(r, P(0), P(1), P(2), None, P(4), P(5), P(6), None) == INVALID               # SwiGLU: gate stash needed
    assert db(r, P(0), P(1), P(2), P(3), None, P(5), P(6), None) == INVALID               # no A
    assert db(r, P(0), P(1), P(2), P(3), P(4), P(5), None, None) == INVALID               # no dW2
    assert db(r, P(0), P(1), P(2), P(3), P(4), P(4), P(6), None) == INVALID               # dU on A
    assert db(r, P(0), P(1), P(2), P(3), P(4), P(5), P(5) + 256, None) == INVALID         # dW2 inside dU
    assert db(r, P(0), P(1), P(2), P(3), P(4) + 8, P(5), P(6), None) == INVALID           # misaligned A
    ub = L.tp_mlp_up_bwd_shard                    # (s, X, dU, W1, Wg, dX, dW1, dWg)
    assert ub(r, P(0), P(1), P(2), None, P(4), P(5), P(6), None) == INVALID               # SwiGLU: Wg needed
    assert ub(r, P(0), P(1), P(2), P(3), P(4), P(5), None, None) == INVALID               # SwiGLU: dWg needed
    assert ub(r, P(0), P(1), P(2), P(3), P(0), P(5), P(6), None) == INVALID               # dX on X
    assert ub(r, P(0), P(1), P(2), P(3), P(4), P(5), P(5) + 1024, None) == INVALID        # dWg inside dW1
    sg = B.make_shape(4, 64, 128, 2, 0, "gelu")
    assert L.tp_mlp_up_bwd_shard(ctypes.byref(sg), P(0), P(1), P(2), P(3), P(4), P(5), None, None) == INVALID
    assert L.tp_mlp_down_bwd_shard(ctypes.byref(sg), P(0), P(1), P(2), P(3), P(4), P(5), P(6), None) == INVALID


def test_streaming_extents_past_the_limits_are_unsupported():
    """The streaming kernels index a row by cols / 8 in an int and count a
    block's bytes in 64 bits: cols above 2^33 or rows * cols above 2^50 are
    refused before any launch (a [1, 2^34] bf16 block would fit in HBM)."""
    L = B.lib()
    ptrs = (ctypes.c_void_p * 2)(P(0), P(1))
    wide, tall = 1 << 34, (1 << 30, 1 << 21)      # cols over 2^33; rows * cols = 2^51
    assert L.tp_mlp_reduce_partials_local(2, ptrs, 1, wide, None, P(2), None) == UNSUPPORTED
    assert L.tp_mlp_reduce_partials_local(2, ptrs, *tall, None, P(2), None) == UNSUPPORTED
    assert L.tp_mlp_reduce_scatter_local(2, ptrs, 2, wide, 0, None, None, P(2), None) == UNSUPPORTED
    assert L.tp_mlp_all_gather_local(2, ptrs, 1, wide, P(2), None) == UNSUPPORTED
    assert L.tp_mlp_all_gather_local(2, ptrs, *tall, P(2), None) == UNSUPPORTED
    assert L.tp_mlp_bias_grad(P(0), 1, wide, P(1), P(2), 1 << 40, None) == UNSUPPORTED
    assert L.tp_mlp_bias_grad(P(0), *tall, P(1), P(2), 1 << 40, None) == UNSUPPORTED
    assert B.bias_grad_workspace_bytes(1, wide) == 0
    assert B.bias_grad_workspace_bytes(1, 12) == 0                # cols % 8
    # the limits themselves are accepted by the checks
    assert B.bias_grad_workspace_bytes(1, 1 << 33) == (1 << 33) * 4
    assert B.bias_grad_workspace_bytes(1 << 17, 1 << 33) > 0


def test_empty_batch_calls_that_launch_nothing():
    """N = 0 tokens (rows = 0) is valid: forwards and reductions return OK
    without launching anything (so this runs without a GPU), and buffers of
    zero bytes may be NULL, as an empty tensor's storage is.  The weights and
    the gradient outputs stay required; negative sizes stay invalid.  The
    backward calls, which write zero weight gradients, are checked on the
    GPU."""
    L = B.lib()
    for act, Wg in (("gelu", None), ("swiglu", P(2))):
        s = B.make_shape(0, 64, 128, 2, 0, act)
        r = ctypes.byref(s)
        assert B.workspace_bytes(s, False) == 0 and B.workspace_bytes(s, True) == 0
        # (s, X, W1, Wg, W2, Y, A, U, G, ws, wsb, stream)
        assert L.tp_mlp_fwd_shard(r, None, P(1), Wg, P(3), None, None, None, None, None, 0, None) == OK
        assert L.tp_mlp_fwd_shard(r, None, None, Wg, P(3), None, None, None, None, None, 0, None) == INVALID
        assert L.tp_mlp_fwd_shard(r, FAKE + 8, P(1), Wg, P(3), None, None, None, None, None, 0, None) == INVALID
        assert L.tp_mlp_up_act_shard(r, None, P(1), Wg, None, None, None, None) == OK
        assert L.tp_mlp_down_shard(r, None, P(3), None, None) == OK
        assert L.tp_mlp_down_dgrad_act_shard(r, None, P(3), None, None, None, None) == OK
        assert L.tp_mlp_up_dgrad_shard(r, None, P(1), Wg, None, None) == OK
        # the pairs write zero weight gradients (on the GPU); here: what stays required
        assert L.tp_mlp_down_bwd_shard(r, None, P(3), None, P(5) if Wg else None, None, None, None, None) == INVALID
        assert L.tp_mlp_up_bwd_shard(r, None, None, None, Wg, None, P(6), P(7) if Wg else None, None) == INVALID
        # the weight-gradient outputs are still required
        assert L.tp_mlp_down_wgrad_shard(r, None, None, None, None) == INVALID
    # reductions, reduce-scatter and all-gather of empty blocks
    nulls = (ctypes.c_void_p * 2)(None, None)
    assert L.tp_mlp_reduce_partials_local(2, nulls, 0, 8, None, None, None) == OK
    assert L.tp_mlp_reduce_partials_local(2, nulls, 0, 8, P(0), None, None) == OK     # bias given
    assert L.tp_mlp_reduce_partials_local(2, None, 0, 8, None, None, None) == INVALID  # no host array
    assert L.tp_mlp_reduce_scatter_local(2, nulls, 0, 8, 1, None, None, None, None) == OK
    assert L.tp_mlp_all_gather_local(2, nulls, 0, 8, None, None) == OK
    assert B.bias_grad_workspace_bytes(0, 64) == 0
    # attention projections
    a = B.make_attn_shape(0, 64, 8, 8, 64, 2, 0)
    assert B.attn_workspace_bytes(a) == 0
    assert L.tp_attn_qkv_shard(ctypes.byref(a), None, P(1), None, None, 0, None) == OK
    assert L.tp_attn_out_shard(ctypes.byref(a), None, P(1), None, None, 0, None) == OK
    # LayerNorm forward, fused reduce-scatter + LayerNorm, gradient sum
    assert L.tp_sp_layernorm_fwd(0, 16, ctypes.c_float(1e-5), None, P(1), None, None, None, None, None) == OK
    assert L.tp_sp_layernorm_fwd(0, 16, ctypes.c_float(1e-5), None, None, None, None, None, None, None) == INVALID
    assert L.tp_sp_reduce_scatter_layernorm_local(2, nulls, 0, 16, 0, None, None, None, ctypes.c_float(1e-5), P(1),
                                                  None, None, None, None, None) == OK
    assert B.layernorm_bwd_workspace_bytes(0, 16) == 0
    assert L.tp_sp_sum_grads_local(2, nulls, 0, None, None) == OK


def test_reduce_rejects_partial_overlap():
    L = B.lib()
    p0, p1 = FAKE, FAKE + (1 << 20)
    ptrs = (ctypes.c_void_p * 2)(p0, p1)
    # rows 4, cols 8: each partial is 64 bytes; out exactly on a partial is allowed (checked on the GPU),
    # out straddling one is not
    assert L.tp_mlp_reduce_partials_local(2, ptrs, 4, 8, None, p1 + 16, None) == INVALID
    assert L.tp_mlp_reduce_partials_local(2, ptrs, 4, 8, None, p0 - 16, None) == INVALID


def test_reduce_scatter_rejects_bad_arguments():
    L = B.lib()
    p0, p1 = FAKE, FAKE + (1 << 20)
    out = FAKE + (2 << 20)
    ptrs = (ctypes.c_void_p * 2)(p0, p1)
    rs = L.tp_mlp_reduce_scatter_local
    assert rs(2, ptrs, 5, 8, 0, None, None, out, None) == INVALID         # rows % t
    assert rs(2, ptrs, 4, 8, 2, None, None, out, None) == INVALID         # rank >= t
    assert rs(2, ptrs, 4, 8, -1, None, None, out, None) == INVALID        # rank < 0
    assert rs(2, ptrs, 4, 12, 0, None, None, out, None) == INVALID        # cols % 8
    assert rs(2, None, 4, 8, 0, None, None, out, None) == INVALID
    assert rs(2, ptrs, 4, 8, 0, FAKE + 8, None, out, None) == INVALID     # misaligned bias
    assert rs(2, ptrs, 4, 8, 0, None, FAKE + 8, out, None) == INVALID     # misaligned residual
    assert rs(2, ptrs, 4, 8, 0, None, None, out + 4, None) == INVALID     # misaligned out
    # rows 4, cols 8, t 2: rank 1's block of each partial is bytes [32, 64); out is 32 bytes
    assert rs(2, ptrs, 4, 8, 1, None, None, p1 + 16, None) == INVALID     # straddles rank 1's block
    assert rs(2, ptrs, 4, 8, 1, None, None, p0, None) == INVALID          # on rank 0's block of a partial
    assert rs(2, ptrs, 4, 8, 1, None, out + 16, out, None) == INVALID     # straddles the residual
    big = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert rs(65, big, 65, 8, 0, None, None, out, None) == UNSUPPORTED


def test_all_gather_rejects_bad_arguments():
    L = B.lib()
    s0, s1 = FAKE, FAKE + (1 << 20)
    ptrs = (ctypes.c_void_p * 2)(s0, s1)
    ag = L.tp_mlp_all_gather_local
    assert ag(2, ptrs, 4, 12, FAKE + (2 << 20), None) == INVALID          # cols % 8
    assert ag(2, ptrs, -1, 8, FAKE + (2 << 20), None) == INVALID          # negative rows
    assert ag(0, ptrs, 4, 8, FAKE + (2 << 20), None) == INVALID
    assert ag(2, ptrs, 4, 8, None, None) == INVALID
    assert ag(2, ptrs, 4, 8, s1 - 64, None) == INVALID                    # out (128 B) runs into shard 1
    assert ag(2, ptrs, 4, 8, s0, None) == INVALID                         # out on shard 0
    bad = (ctypes.c_void_p * 2)(s0, s1 + 8)
    assert ag(2, bad, 4, 8, FAKE + (2 << 20), None) == INVALID            # misaligned shard
    big = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert ag(65, big, 4, 8, FAKE + (2 << 20), None) == UNSUPPORTED


def test_small_batch_workspace_sizes():
    """2 <= N <= 128 uses the split-K small-batch path, which needs float32
    partials; N == 129 goes to the wide-tile GEMMs, which need none."""
    prev = 0
    for N in (2, 16, 17, 32, 33, 64, 65, 96, 128):
        ws = B.workspace_bytes(B.make_shape(N, 8192, 28672, 4, 0, "swiglu"), False)
        assert ws > 0 and ws % 256 == 0
        assert ws >= prev
        prev = ws
    assert B.workspace_bytes(B.make_shape(129, 8192, 28672, 4, 0, "swiglu"), False) == 0
    s = B.make_shape(8, 64, 128, 2, 0, "gelu")
    assert _fwd(s) == WORKSPACE                                  # small batch needs workspace
    assert _fwd(s, ws=P(8), wsb=B.workspace_bytes(s, False) - 1) == WORKSPACE


@pytest.mark.parametrize("shape,expect", [
    (B.make_attn_shape(-1, 64, 8, 8, 64, 2, 0), INVALID),       # negative token count
    (B.make_attn_shape(4, 60, 8, 8, 64, 2, 0), INVALID),        # h % 8
    (B.make_attn_shape(4, 64, 8, 8, 60, 2, 0), INVALID),        # head_dim % 8
    (B.make_attn_shape(4, 64, 6, 4, 64, 2, 0), INVALID),        # n_heads % n_kv
    (B.make_attn_shape(4, 64, 12, 6, 64, 4, 0), INVALID),       # 6 kv heads over 4 ranks: neither split nor replicas
    (B.make_attn_shape(4, 64, 8, 8, 64, 3, 0), INVALID),        # n_heads % t
    (B.make_attn_shape(4, 64, 8, 8, 64, 2, 2), INVALID),        # rank >= t
    (B.make_attn_shape(4, 64, 128, 1, 64, 128, 0), UNSUPPORTED),  # t > 64
])
def test_attn_rejects_bad_shapes(shape, expect):
    L = B.lib()
    r = ctypes.byref(shape)
    assert L.tp_attn_qkv_shard(r, P(0), P(1), P(2), None, 0, None) == expect
    assert L.tp_attn_out_shard(r, P(0), P(1), P(2), None, 0, None) == expect
    assert B.attn_workspace_bytes(shape) == 0
    assert L.tp_attn_out_bwd_shard(r, P(0), P(1), P(2), P(3), P(4), None) == expect
    assert L.tp_attn_qkv_bwd_shard(r, P(0), P(1), P(2), P(3), P(4), None) == expect


def test_attn_rejects_bad_pointers_and_reports_widths():
    L = B.lib()
    s = B.make_attn_shape(4, 64, 8, 2, 64, 4, 1)     # 2 kv heads over 4 ranks: replicated
    assert (s.q_cols, s.kv_cols, s.qkv_cols) == (128, 64, 256)
    r = ctypes.byref(s)
    assert L.tp_attn_qkv_shard(r, None, P(1), P(2), None, 0, None) == INVALID
    assert L.tp_attn_out_shard(r, P(0), P(1) + 2, P(2), None, 0, None) == INVALID
    assert L.tp_attn_out_bwd_shard(r, P(0), P(1), P(2), P(3), None, None) == INVALID
    assert L.tp_attn_qkv_bwd_shard(r, P(0), P(1), P(2), P(3) + 4, P(4), None) == INVALID
    # overlaps (N = 129 here: the wide-tile path, no workspace)
    s129 = B.make_attn_shape(129, 64, 8, 2, 64, 4, 1)
    r129 = ctypes.byref(s129)
    assert L.tp_attn_qkv_shard(r129, P(0), P(1), P(0), None, 0, None) == INVALID        # QKV on X
    assert L.tp_attn_out_shard(r129, P(0), P(1), P(1), None, 0, None) == INVALID        # Y on Wo
    assert L.tp_attn_out_bwd_shard(r129, P(0), P(1), P(2), P(0), P(4), None) == INVALID  # dO on dY
    assert L.tp_attn_qkv_bwd_shard(r129, P(0), P(1), P(2), P(3), P(3), None) == INVALID  # dX on dWqkv


def test_attn_small_batch_workspace():
    """1 <= N <= 128 tokens take the small-batch path, which needs float32
    k-split partials; N = 129 goes to the wide tiles, which need none."""
    L = B.lib()
    for N in (1, 2, 17, 64, 65, 128):
        s = B.make_attn_shape(N, 8192, 64, 8, 128, 4, 0)     # 70B heads, t = 4
        need = B.attn_workspace_bytes(s)
        assert need > 0 and need % 256 == 0
        # the larger of the two projections' partials: ks * N * cols floats
        assert need >= N * max(s.qkv_cols, 8192) * 4
        r = ctypes.byref(s)
        assert L.tp_attn_qkv_shard(r, P(0), P(1), P(2), None, 0, None) == WORKSPACE
        assert L.tp_attn_out_shard(r, P(0), P(1), P(2), P(3), need - 1, None) == WORKSPACE
        assert L.tp_attn_out_shard(r, P(0), P(1), P(2), P(3) + 8, need, None) == WORKSPACE  # alignment
        assert L.tp_attn_qkv_shard(r, P(0), P(1), P(2), P(2), need, None) == INVALID      # workspace on the output
        assert L.tp_attn_qkv_shard(r, P(0), P(1), P(2), P(1), need, None) == INVALID      # workspace on the weight
    assert B.attn_workspace_bytes(B.make_attn_shape(129, 8192, 64, 8, 128, 4, 0)) == 0


# ------------------------------------------- sequence-parallel LayerNorm
MB = 1 << 20


def test_layernorm_fwd_rejects_bad_arguments():
    f = B.lib().tp_sp_layernorm_fwd
    x, g, y, m, r = FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB, FAKE + 4 * MB
    assert f(-1, 16, 1e-5, x, g, None, y, m, r, None) == INVALID           # negative rows
    assert f(4, 12, 1e-5, x, g, None, y, m, r, None) == INVALID            # cols % 8
    assert f(4, 16, 0.0, x, g, None, y, m, r, None) == INVALID             # eps must be > 0
    assert f(4, 16, -1.0, x, g, None, y, m, r, None) == INVALID
    assert f(4, 16, float("nan"), x, g, None, y, m, r, None) == INVALID
    assert f(4, 16, float("inf"), x, g, None, y, m, r, None) == INVALID
    assert f(4, 16, 1e-5, None, g, None, y, m, r, None) == INVALID
    assert f(4, 16, 1e-5, x, None, None, y, m, r, None) == INVALID         # gamma required
    assert f(4, 16, 1e-5, x, g, FAKE + 8, y, m, r, None) == INVALID        # misaligned beta
    assert f(4, 16, 1e-5, x, g, None, y, m, None, None) == INVALID         # mean without rstd
    assert f(4, 16, 1e-5, x, g, None, y, None, r, None) == INVALID
    assert f(4, 16, 1e-5, x, g, None, x + 16, m, r, None) == INVALID       # y straddles x
    assert f(4, 16, 1e-5, x, g, None, g, m, r, None) == INVALID            # y on gamma
    assert f(4, 16, 1e-5, x, g, None, y, y, r, None) == INVALID            # stash on y
    assert f(4, 16, 1e-5, x, g, None, y, m, m, None) == INVALID            # mean == rstd
    assert f(4, 16400, 1e-5, x, g, None, y, m, r, None) == UNSUPPORTED     # more than 16384 columns


def test_layernorm_fused_rejects_bad_arguments():
    f = B.lib().tp_sp_reduce_scatter_layernorm_local
    p0, p1 = FAKE, FAKE + MB
    z, g, y, m, r = FAKE + 2 * MB, FAKE + 3 * MB, FAKE + 4 * MB, FAKE + 5 * MB, FAKE + 6 * MB
    ptrs = (ctypes.c_void_p * 2)(p0, p1)

    def call(**o):
        a = dict(t=2, ptrs=ptrs, rows=4, cols=16, rank=0, bias=None, res=None, z=z, eps=1e-5, g=g, beta=None,
                 y=y, m=m, r=r)
        a.update(o)
        return f(a["t"], a["ptrs"], a["rows"], a["cols"], a["rank"], a["bias"], a["res"], a["z"], a["eps"],
                 a["g"], a["beta"], a["y"], a["m"], a["r"], None)

    assert call(rows=5) == INVALID                    # rows % t
    assert call(rank=2) == INVALID
    assert call(eps=0.0) == INVALID
    assert call(g=None) == INVALID
    assert call(y=p0) == INVALID                      # y on a partial
    assert call(y=z) == INVALID                       # y on z
    assert call(res=FAKE + 7 * MB, y=FAKE + 7 * MB) == INVALID   # y on the residual
    assert call(z=p1 + 16) == INVALID                 # z straddles rank 0's block of a partial
    assert call(m=z) == INVALID                       # stash on z
    assert call(z=g) == INVALID                       # z on gamma
    assert call(beta=FAKE + 7 * MB, z=FAKE + 7 * MB) == INVALID   # z on beta
    assert call(cols=16400) == UNSUPPORTED
    big = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert call(t=65, ptrs=big, rows=65) == UNSUPPORTED


def test_layernorm_bwd_workspace_and_arguments():
    ws = B.layernorm_bwd_workspace_bytes
    # row slabs of at least 8 rows; dgamma and dbeta partials.  Below 4096
    # rows at most 64 slabs (the column kernel); from 4096 rows one block per
    # slab in the one-pass kernel, at most 1024 of 256 threads up to 4096
    # columns and 256 of 512 threads over that
    assert ws(1, 8) == 2 * 1 * 8 * 4
    assert ws(17, 8) == 2 * 3 * 8 * 4                # 3 slabs of 6 rows
    assert ws(256, 12288) == 2 * 32 * 12288 * 4
    assert ws(1000, 16) == 2 * 63 * 16 * 4           # 64 slabs of 16 rows cover 1000 in 63
    assert ws(4095, 16) == 2 * 64 * 16 * 4
    assert ws(4096, 8192) == 2 * 256 * 8192 * 4      # 512 threads per row: 256 slabs of 16 rows
    assert ws(4100, 16) == 2 * 513 * 16 * 4          # every 513th row: 513 slabs of 7 or 8 rows
    assert ws(4096, 4096) == 2 * 512 * 4096 * 4      # 256 threads per row, 8 rows per slab
    assert ws(16384, 4096) == 2 * 1024 * 4096 * 4
    assert ws(4096, 4104) == 2 * 256 * 4104 * 4
    assert ws(5000, 16384) == 2 * 256 * 16384 * 4
    assert ws(0, 16) == 0 and ws(4, 12) == 0 and ws(4, 16392) == 0
    f = B.lib().tp_sp_layernorm_bwd
    x, g, m, r, dy, dx, dg, db, w = (FAKE + i * MB for i in range(9))
    need = ws(4, 16)

    def call(**o):
        a = dict(rows=4, cols=16, x=x, g=g, m=m, r=r, dy=dy, dres=None, dx=dx, dg=dg, db=db, w=w, wb=need)
        a.update(o)
        return f(a["rows"], a["cols"], a["x"], a["g"], a["m"], a["r"], a["dy"], a["dres"], a["dx"], a["dg"],
                 a["db"], a["w"], a["wb"], None)

    assert call(w=None) == WORKSPACE
    assert call(wb=need - 1) == WORKSPACE
    assert call(w=w + 8) == WORKSPACE                 # misaligned workspace
    assert call(m=None) == INVALID                    # the stash is required
    assert call(dg=None) == INVALID
    assert call(dx=x) == INVALID                      # dx on the forward input
    assert call(dx=dy + 16) == INVALID                # dx straddles dy
    assert call(dres=dx + 16) == INVALID              # dx straddles dres
    assert call(db=dg) == INVALID                     # dbeta on dgamma
    assert call(w=dx) == INVALID                      # workspace on dx
    assert call(w=g) == INVALID                       # workspace on gamma
    assert call(dg=x) == INVALID                      # dgamma on x
    assert call(dg=dy + 16) == INVALID                # dgamma inside dy
    assert call(db=m) == INVALID                      # dbeta on the stash
    assert call(dres=FAKE + 10 * MB, dg=FAKE + 10 * MB) == INVALID   # dgamma on dres
    assert call(cols=12) == INVALID
    assert call(rows=-1) == INVALID
    assert call(cols=16400, wb=1 << 30) == UNSUPPORTED


def test_sum_grads_rejects_bad_arguments():
    f = B.lib().tp_sp_sum_grads_local
    g0, g1, out = FAKE, FAKE + MB, FAKE + 2 * MB
    ptrs = (ctypes.c_void_p * 2)(g0, g1)
    assert f(2, ptrs, 6, out, None) == INVALID        # n % 4
    assert f(2, ptrs, -4, out, None) == INVALID
    assert f(0, ptrs, 8, out, None) == INVALID
    assert f(2, None, 8, out, None) == INVALID
    assert f(2, ptrs, 8, None, None) == INVALID
    assert f(2, ptrs, 8, g1, None) == INVALID         # out on a later rank's gradient
    assert f(2, ptrs, 8, g0 + 16, None) == INVALID    # out straddles rank 0's
    bad = (ctypes.c_void_p * 2)(g0, g1 + 4)
    assert f(2, bad, 8, out, None) == INVALID
    big = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert f(65, big, 8, out, None) == UNSUPPORTED



def test_noalloc_forward_validates_and_refuses_shapes_beyond_its_scratch():
    """tp_mlp_fwd_shard_noalloc checks its arguments as tp_mlp_fwd_shard does
    and refuses a shape whose k-split partials exceed its fixed 64 MiB
    scratch, before any launch (so this runs without a GPU)."""
    L = B.lib()
    fn = L.tp_mlp_fwd_shard_noalloc               # (s, X, W1, Wg, W2, Y, A, U, G, stream)
    s = B.make_shape(128, 16384, 98304, 1, 0, "gelu")        # 80 MiB of partials, operands within limits
    assert B.workspace_bytes(s, False) > 64 << 20
    # (the 3 GiB weights need fake buffers further apart)
    assert fn(ctypes.byref(s), P(0), P(4), None, P(8), P(12), P(13), P(14), None, None) == WORKSPACE
    s = B.make_shape(8, 64, 128, 2, 0, "swiglu")
    r = ctypes.byref(s)
    assert fn(r, P(0), P(1), None, P(3), P(4), P(5), P(6), P(7), None) == INVALID           # SwiGLU: no gate
    assert fn(r, P(0), P(1), P(2), P(3), P(0), P(5), P(6), P(7), None) == INVALID           # Y on X
    assert fn(r, P(0) + 8, P(1), P(2), P(3), P(4), P(5), P(6), P(7), None) == INVALID       # misaligned X
    s0 = B.make_shape(0, 64, 128, 2, 0, "gelu")                                              # no tokens: nothing to do
    assert fn(ctypes.byref(s0), None, P(1), None, P(3), None, None, None, None, None) == OK


def test_attn_deferred_wgrad_entry_points_validate():
    """tp_attn_out_dgrad_shard and tp_attn_qkv_bwd_out_wgrad_shard check their
    arguments before any launch; the dO workspace is sized for its k-split."""
    L = B.lib()
    s = B.make_attn_shape(2048, 12288, 96, 96, 128, 8, 7)
    r = ctypes.byref(s)
    need = B.attn_out_dgrad_workspace_bytes(s)
    assert need >= 4 * 2048 * 1536 * 4                 # dO = dY Wo^T splits along k at this shape
    od = L.tp_attn_out_dgrad_shard                     # (s, dY, Wo, dO, ws, wsb)
    assert od(r, P(0), P(1), P(2), None, 0, None) == WORKSPACE
    assert od(r, P(0), P(1), P(2), P(3), need - 256, None) == WORKSPACE
    assert od(r, P(0), P(1), P(0), P(3), need, None) == INVALID        # dO on dY
    assert od(r, P(0), P(1), P(2), P(2), need, None) == INVALID        # workspace on dO
    assert od(r, P(0), None, P(2), P(3), need, None) == INVALID
    small = B.make_attn_shape(4096, 512, 8, 8, 64, 1, 0)               # a full grid: no split, no workspace
    assert B.attn_out_dgrad_workspace_bytes(small) == 0
    # few tokens at the 70B widths: the split-K kernel's partials (as many
    # splits as dW_o would hold, h / N, and at least one)
    for N in (1, 8, 32):
        few = B.make_attn_shape(N, 8192, 64, 8, 128, 4, 0)
        need_few = B.attn_out_dgrad_workspace_bytes(few)
        assert need_few % 256 == 0 and N * few.q_cols * 4 <= need_few <= (8192 // N) * N * few.q_cols * 4 + 255
        fr = ctypes.byref(few)
        assert od(fr, P(0), P(1), P(2), P(3), need_few - 256, None) == WORKSPACE
    qw = L.tp_attn_qkv_bwd_out_wgrad_shard             # (s, X, Wqkv, dQKV, dY, O, dWqkv, dX, dWo)
    assert qw(r, P(0), P(1), P(2), P(3), P(4), P(5), P(6), None, None) == INVALID   # no dWo
    assert qw(r, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(5), None) == INVALID   # dWo on dWqkv
    assert qw(r, P(0), P(1), P(2), P(3), P(4), P(5), P(3), P(7), None) == INVALID   # dX on dY
    assert qw(r, P(0), P(1), P(2), None, P(4), P(5), P(6), P(7), None) == INVALID   # no dY
