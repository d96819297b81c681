"""ctypes binding of libtpmlp.so (declared in include/tp_mlp.h).

Argument marshalling only: every function here checks that the torch tensors
it is handed are device-resident, contiguous, of the dtype and at least the
size the C entry point will touch, passes their device pointers and the
current HIP stream, and raises ``TpMlpError`` on a non-OK status.  All
arithmetic runs in the library's HIP kernels; there is no fallback.  The
library is loaded on the first call and its absence is an error.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

# TPMLP_LIB selects another build of the library (e.g. the host-sanitized one
# of build.py --host-sanitize); by default the in-tree libtpmlp.so.
LIB_PATH = os.environ.get("TPMLP_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

ACTS = {"relu": 0, "gelu": 1, "swiglu": 2}
STATUS = {0: "TP_MLP_OK", 1: "TP_MLP_ERR_INVALID_ARG", 2: "TP_MLP_ERR_UNSUPPORTED",
          3: "TP_MLP_ERR_WORKSPACE", 4: "TP_MLP_ERR_HIP"}


class TpMlpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {status_string(status)}")


class Shape(ctypes.Structure):
    """Mirror of tp_mlp_shape."""
    _fields_ = [("n_tokens", c_int64), ("hidden", c_int64), ("ffn", c_int64),
                ("t", c_int32), ("rank", c_int32), ("act", c_int32)]

    @property
    def Fi(self) -> int:
        return self.ffn // self.t

    @property
    def g(self) -> int:
        return 2 if self.act == ACTS["swiglu"] else 1


def make_shape(N: int, h: int, F: int, t: int = 1, rank: int = 0, act: str | int = "gelu") -> Shape:
    return Shape(N, h, F, t, rank, ACTS[act] if isinstance(act, str) else act)


class AttnShape(ctypes.Structure):
    """Mirror of tp_attn_shape."""
    _fields_ = [("n_tokens", c_int64), ("hidden", c_int64), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("t", c_int32), ("rank", c_int32)]

    @property
    def q_cols(self) -> int:
        return self.n_heads // self.t * self.head_dim

    @property
    def kv_cols(self) -> int:
        return (self.n_kv_heads // self.t if self.n_kv_heads >= self.t else 1) * self.head_dim

    @property
    def qkv_cols(self) -> int:
        return self.q_cols + 2 * self.kv_cols


def make_attn_shape(N: int, h: int, n_heads: int, n_kv_heads: int, head_dim: int, t: int = 1,
                    rank: int = 0) -> AttnShape:
    return AttnShape(N, h, n_heads, n_kv_heads, head_dim, t, rank)


_lib = None

_SIGS = {
    "tp_mlp_fwd_shard": [POINTER(Shape)] + [c_void_p] * 9 + [c_size_t, c_void_p],
    "tp_mlp_fwd_shard_noalloc": [POINTER(Shape)] + [c_void_p] * 8 + [c_void_p],
    "tp_mlp_bwd_shard": [POINTER(Shape)] + [c_void_p] * 15 + [c_size_t, c_void_p],
    "tp_mlp_reduce_partials_local": [c_int32, POINTER(c_void_p), c_int64, c_int64, c_void_p, c_void_p, c_void_p],
    "tp_mlp_reduce_scatter_local": [c_int32, POINTER(c_void_p), c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                    c_void_p, c_void_p],
    "tp_mlp_all_gather_local": [c_int32, POINTER(c_void_p), c_int64, c_int64, c_void_p, c_void_p],
    "tp_mlp_up_act_shard": [POINTER(Shape)] + [c_void_p] * 6 + [c_void_p],
    "tp_mlp_down_shard": [POINTER(Shape)] + [c_void_p] * 3 + [c_void_p],
    "tp_mlp_down_dgrad_act_shard": [POINTER(Shape)] + [c_void_p] * 5 + [c_void_p],
    "tp_mlp_down_wgrad_shard": [POINTER(Shape)] + [c_void_p] * 3 + [c_void_p],
    "tp_mlp_up_wgrad_shard": [POINTER(Shape)] + [c_void_p] * 4 + [c_void_p],
    "tp_mlp_up_dgrad_shard": [POINTER(Shape)] + [c_void_p] * 4 + [c_void_p],
    "tp_mlp_wgrad_shard": [POINTER(Shape)] + [c_void_p] * 7 + [c_void_p],
    "tp_mlp_down_bwd_shard": [POINTER(Shape)] + [c_void_p] * 7 + [c_void_p],
    "tp_mlp_up_bwd_shard": [POINTER(Shape)] + [c_void_p] * 7 + [c_void_p],
    "tp_mlp_bias_grad": [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_size_t, c_void_p],
    "tp_attn_qkv_shard": [POINTER(AttnShape)] + [c_void_p] * 4 + [c_size_t, c_void_p],
    "tp_attn_out_shard": [POINTER(AttnShape)] + [c_void_p] * 4 + [c_size_t, c_void_p],
    "tp_attn_out_bwd_shard": [POINTER(AttnShape)] + [c_void_p] * 5 + [c_void_p],
    "tp_attn_qkv_bwd_shard": [POINTER(AttnShape)] + [c_void_p] * 5 + [c_void_p],
    "tp_attn_out_dgrad_shard": [POINTER(AttnShape)] + [c_void_p] * 4 + [c_size_t, c_void_p],
    "tp_attn_qkv_bwd_out_wgrad_shard": [POINTER(AttnShape)] + [c_void_p] * 8 + [c_void_p],
    "tp_sp_layernorm_fwd": [c_int64, c_int64, c_float] + [c_void_p] * 6 + [c_void_p],
    "tp_sp_reduce_scatter_layernorm_local": [c_int32, POINTER(c_void_p), c_int64, c_int64, c_int32, c_void_p,
                                             c_void_p, c_void_p, c_float] + [c_void_p] * 5 + [c_void_p],
    "tp_sp_layernorm_bwd": [c_int64, c_int64] + [c_void_p] * 10 + [c_size_t, c_void_p],
    "tp_sp_sum_grads_local": [c_int32, POINTER(c_void_p), c_int64, c_void_p, c_void_p],
}


def lib() -> ctypes.CDLL:
    """Load libtpmlp.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m megatron_tensor_transformer_rank_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = c_int32
        L.tp_mlp_workspace_bytes.argtypes = [POINTER(Shape), c_int32]
        L.tp_mlp_workspace_bytes.restype = c_size_t
        L.tp_mlp_bias_grad_workspace_bytes.argtypes = [c_int64, c_int64]
        L.tp_mlp_bias_grad_workspace_bytes.restype = c_size_t
        L.tp_attn_workspace_bytes.argtypes = [POINTER(AttnShape)]
        L.tp_attn_workspace_bytes.restype = c_size_t
        L.tp_attn_out_dgrad_workspace_bytes.argtypes = [POINTER(AttnShape)]
        L.tp_attn_out_dgrad_workspace_bytes.restype = c_size_t
        L.tp_sp_layernorm_bwd_workspace_bytes.argtypes = [c_int64, c_int64]
        L.tp_sp_layernorm_bwd_workspace_bytes.restype = c_size_t
        L.tp_mlp_status_string.argtypes = [c_int32]
        L.tp_mlp_status_string.restype = c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tp_mlp_status_string(status).decode()


def workspace_bytes(shape: Shape, backward: bool) -> int:
    return int(lib().tp_mlp_workspace_bytes(ctypes.byref(shape), 1 if backward else 0))


def bias_grad_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().tp_mlp_bias_grad_workspace_bytes(rows, cols))


def attn_workspace_bytes(shape: AttnShape) -> int:
    return int(lib().tp_attn_workspace_bytes(ctypes.byref(shape)))


def attn_out_dgrad_workspace_bytes(shape: AttnShape) -> int:
    return int(lib().tp_attn_out_dgrad_workspace_bytes(ctypes.byref(shape)))


def layernorm_bwd_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().tp_sp_layernorm_bwd_workspace_bytes(rows, cols))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    """Device workspace of nbytes (zero-filled; no entry point needs particular
    initial contents), or None when no workspace is needed."""
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- marshalling
def _p(t, dtype, numel, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _ws(ws, need):
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _stream(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, st):
    if st != 0:
        raise TpMlpError(fn, st)


BF16, F32 = torch.bfloat16, torch.float32


def tp_mlp_fwd_shard(shape: Shape, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i=None, G_i=None,
                     workspace=None, stream=None):
    N, h, Fi = shape.n_tokens, shape.hidden, shape.Fi
    args = [_p(X, BF16, N * h, "X"), _p(W1_i, BF16, h * Fi, "W1_i"),
            _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True), _p(W2_i, BF16, Fi * h, "W2_i"),
            _p(Y_i, BF16, N * h, "Y_i"), _p(A_i, BF16, N * Fi, "A_i"),
            _p(U_i, BF16, N * Fi, "U_i", optional=True), _p(G_i, BF16, N * Fi, "G_i", optional=True)]
    wp, wb = _ws(workspace, 0)
    _check("tp_mlp_fwd_shard", lib().tp_mlp_fwd_shard(ctypes.byref(shape), *args, wp, wb, _stream(stream)))


def tp_mlp_fwd_shard_noalloc(shape: Shape, X, W1_i, Wg_i, W2_i, Y_i, A_i, U_i=None, G_i=None, stream=None):
    """tp_mlp_fwd_shard without a workspace: the library's fixed per-GPU
    scratch holds the small-batch partials (calls on one GPU must not
    overlap in time)."""
    N, h, Fi = shape.n_tokens, shape.hidden, shape.Fi
    args = [_p(X, BF16, N * h, "X"), _p(W1_i, BF16, h * Fi, "W1_i"),
            _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True), _p(W2_i, BF16, Fi * h, "W2_i"),
            _p(Y_i, BF16, N * h, "Y_i"), _p(A_i, BF16, N * Fi, "A_i"),
            _p(U_i, BF16, N * Fi, "U_i", optional=True), _p(G_i, BF16, N * Fi, "G_i", optional=True)]
    _check("tp_mlp_fwd_shard_noalloc", lib().tp_mlp_fwd_shard_noalloc(ctypes.byref(shape), *args, _stream(stream)))


def tp_mlp_bwd_shard(shape: Shape, X, W1_i, Wg_i, W2_i, dY, A_i, U_i, G_i, dU_i, dW1_i, dWg_i,
                     dW2_i, dX_partial, db2=None, workspace=None, stream=None):
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    args = [_p(X, BF16, N * h, "X"), _p(W1_i, BF16, h * Fi, "W1_i"),
            _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True), _p(W2_i, BF16, Fi * h, "W2_i"),
            _p(dY, BF16, N * h, "dY"), _p(A_i, BF16, N * Fi, "A_i"), _p(U_i, BF16, N * Fi, "U_i"),
            _p(G_i, BF16, N * Fi, "G_i", optional=True), _p(dU_i, BF16, N * g * Fi, "dU_i"),
            _p(dW1_i, F32, h * Fi, "dW1_i"), _p(dWg_i, F32, h * Fi, "dWg_i", optional=True),
            _p(dW2_i, F32, Fi * h, "dW2_i"), _p(dX_partial, BF16, N * h, "dX_partial"),
            _p(db2, F32, h, "db2", optional=True)]
    wp, wb = _ws(workspace, 0)
    _check("tp_mlp_bwd_shard", lib().tp_mlp_bwd_shard(ctypes.byref(shape), *args, wp, wb, _stream(stream)))


def tp_mlp_reduce_partials_local(partials, out, bias=None, stream=None):
    """out = sum(partials) (+ bias once); partials: list of equal-shape bf16
    [rows, cols] device tensors."""
    t = len(partials)
    if t == 0:
        raise ValueError("need at least one partial")
    rows, cols = partials[0].shape
    ptrs = (c_void_p * t)(*[_p(p, BF16, rows * cols, f"partials[{i}]") for i, p in enumerate(partials)])
    for p in partials:
        if tuple(p.shape) != (rows, cols):
            raise ValueError("partials must share one shape")
    _check("tp_mlp_reduce_partials_local",
           lib().tp_mlp_reduce_partials_local(t, ptrs, rows, cols, _p(bias, BF16, cols, "bias", optional=True),
                                              _p(out, BF16, rows * cols, "out"), _stream(stream)))


def _ptr_list(tensors, name):
    t = len(tensors)
    if t == 0:
        raise ValueError(f"need at least one of {name}")
    rows, cols = tensors[0].shape
    for x in tensors:
        if tuple(x.shape) != (rows, cols):
            raise ValueError(f"{name} must share one shape")
    ptrs = (c_void_p * t)(*[_p(x, BF16, rows * cols, f"{name}[{i}]") for i, x in enumerate(tensors)])
    return t, rows, cols, ptrs


def tp_mlp_reduce_scatter_local(partials, out, rank, bias=None, residual=None, stream=None):
    """out = rank's block of rows of sum(partials) (+ bias once, + residual);
    partials: list of t equal-shape bf16 [rows, cols] device tensors, rows
    divisible by t; out and residual are [rows / t, cols]."""
    t, rows, cols, ptrs = _ptr_list(partials, "partials")
    n = rows // t
    _check("tp_mlp_reduce_scatter_local", lib().tp_mlp_reduce_scatter_local(
        t, ptrs, rows, cols, rank, _p(bias, BF16, cols, "bias", optional=True),
        _p(residual, BF16, n * cols, "residual", optional=True), _p(out, BF16, n * cols, "out"),
        _stream(stream)))


def tp_mlp_all_gather_local(shards, out, stream=None):
    """out = the t bf16 [shard_rows, cols] shards stacked along rows in order."""
    t, rows, cols, ptrs = _ptr_list(shards, "shards")
    _check("tp_mlp_all_gather_local", lib().tp_mlp_all_gather_local(
        t, ptrs, rows, cols, _p(out, BF16, t * rows * cols, "out"), _stream(stream)))


def tp_mlp_up_act_shard(shape: Shape, X, W1_i, Wg_i, A_i, U_i=None, G_i=None, stream=None):
    N, h, Fi = shape.n_tokens, shape.hidden, shape.Fi
    _check("tp_mlp_up_act_shard", lib().tp_mlp_up_act_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(W1_i, BF16, h * Fi, "W1_i"),
        _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True), _p(A_i, BF16, N * Fi, "A_i"),
        _p(U_i, BF16, N * Fi, "U_i", optional=True), _p(G_i, BF16, N * Fi, "G_i", optional=True),
        _stream(stream)))


def tp_mlp_down_shard(shape: Shape, A_i, W2_i, Y_i, stream=None):
    N, h, Fi = shape.n_tokens, shape.hidden, shape.Fi
    _check("tp_mlp_down_shard", lib().tp_mlp_down_shard(
        ctypes.byref(shape), _p(A_i, BF16, N * Fi, "A_i"), _p(W2_i, BF16, Fi * h, "W2_i"),
        _p(Y_i, BF16, N * h, "Y_i"), _stream(stream)))


def tp_mlp_down_dgrad_act_shard(shape: Shape, dY, W2_i, U_i, G_i, dU_i, stream=None):
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_down_dgrad_act_shard", lib().tp_mlp_down_dgrad_act_shard(
        ctypes.byref(shape), _p(dY, BF16, N * h, "dY"), _p(W2_i, BF16, Fi * h, "W2_i"),
        _p(U_i, BF16, N * Fi, "U_i"), _p(G_i, BF16, N * Fi, "G_i", optional=True),
        _p(dU_i, BF16, N * g * Fi, "dU_i"), _stream(stream)))


def tp_mlp_down_wgrad_shard(shape: Shape, A_i, dY, dW2_i, stream=None):
    N, h, Fi = shape.n_tokens, shape.hidden, shape.Fi
    _check("tp_mlp_down_wgrad_shard", lib().tp_mlp_down_wgrad_shard(
        ctypes.byref(shape), _p(A_i, BF16, N * Fi, "A_i"), _p(dY, BF16, N * h, "dY"),
        _p(dW2_i, F32, Fi * h, "dW2_i"), _stream(stream)))


def tp_mlp_up_wgrad_shard(shape: Shape, X, dU_i, dW1_i, dWg_i=None, stream=None):
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_up_wgrad_shard", lib().tp_mlp_up_wgrad_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(dU_i, BF16, N * g * Fi, "dU_i"),
        _p(dW1_i, F32, h * Fi, "dW1_i"), _p(dWg_i, F32, h * Fi, "dWg_i", optional=True), _stream(stream)))


def tp_mlp_wgrad_shard(shape: Shape, X, A_i, dY, dU_i, dW1_i, dW2_i, dWg_i=None, stream=None):
    """dW2_i = A_i^T dY and dW1_i (dWg_i) = X^T dU_i in one launch."""
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_wgrad_shard", lib().tp_mlp_wgrad_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(A_i, BF16, N * Fi, "A_i"), _p(dY, BF16, N * h, "dY"),
        _p(dU_i, BF16, N * g * Fi, "dU_i"), _p(dW1_i, F32, h * Fi, "dW1_i"),
        _p(dWg_i, F32, h * Fi, "dWg_i", optional=True), _p(dW2_i, F32, Fi * h, "dW2_i"), _stream(stream)))


def tp_mlp_up_dgrad_shard(shape: Shape, dU_i, W1_i, Wg_i, dX_partial, stream=None):
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_up_dgrad_shard", lib().tp_mlp_up_dgrad_shard(
        ctypes.byref(shape), _p(dU_i, BF16, N * g * Fi, "dU_i"), _p(W1_i, BF16, h * Fi, "W1_i"),
        _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True), _p(dX_partial, BF16, N * h, "dX_partial"),
        _stream(stream)))


def tp_mlp_down_bwd_shard(shape: Shape, dY, W2_i, U_i, G_i, A_i, dU_i, dW2_i, stream=None):
    """dU_i (dgrad through W2 with the activation derivative) and dW2_i =
    A_i^T dY: the first half of the composite backward."""
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_down_bwd_shard", lib().tp_mlp_down_bwd_shard(
        ctypes.byref(shape), _p(dY, BF16, N * h, "dY"), _p(W2_i, BF16, Fi * h, "W2_i"),
        _p(U_i, BF16, N * Fi, "U_i"), _p(G_i, BF16, N * Fi, "G_i", optional=True), _p(A_i, BF16, N * Fi, "A_i"),
        _p(dU_i, BF16, N * g * Fi, "dU_i"), _p(dW2_i, F32, Fi * h, "dW2_i"), _stream(stream)))


def tp_mlp_up_bwd_shard(shape: Shape, X, dU_i, W1_i, Wg_i, dX_partial, dW1_i, dWg_i=None, stream=None):
    """dX_partial = dU_i W1_i^T and dW1_i (dWg_i) = X^T dU_i: the second half
    of the composite backward."""
    N, h, Fi, g = shape.n_tokens, shape.hidden, shape.Fi, shape.g
    _check("tp_mlp_up_bwd_shard", lib().tp_mlp_up_bwd_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(dU_i, BF16, N * g * Fi, "dU_i"),
        _p(W1_i, BF16, h * Fi, "W1_i"), _p(Wg_i, BF16, h * Fi, "Wg_i", optional=True),
        _p(dX_partial, BF16, N * h, "dX_partial"), _p(dW1_i, F32, h * Fi, "dW1_i"),
        _p(dWg_i, F32, h * Fi, "dWg_i", optional=True), _stream(stream)))


def tp_mlp_bias_grad(dY, db2, workspace, stream=None):
    rows, cols = dY.shape
    wp, wb = _ws(workspace, 0)
    _check("tp_mlp_bias_grad", lib().tp_mlp_bias_grad(
        _p(dY, BF16, rows * cols, "dY"), rows, cols, _p(db2, F32, cols, "db2"), wp, wb, _stream(stream)))


# ------------------------------------------------------ attention projections
def tp_attn_qkv_shard(shape: AttnShape, X, Wqkv_i, QKV_i, workspace=None, stream=None):
    """QKV_i = X @ Wqkv_i; workspace: attn_workspace_bytes(shape) bytes (needed
    only for 1 <= N <= 128)."""
    N, h, w = shape.n_tokens, shape.hidden, shape.qkv_cols
    wp, wb = _ws(workspace, 0)
    _check("tp_attn_qkv_shard", lib().tp_attn_qkv_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(Wqkv_i, BF16, h * w, "Wqkv_i"),
        _p(QKV_i, BF16, N * w, "QKV_i"), wp, wb, _stream(stream)))


def tp_attn_out_shard(shape: AttnShape, O_i, Wo_i, Y_i, workspace=None, stream=None):
    """Y_i = O_i @ Wo_i (partial sum); workspace as for tp_attn_qkv_shard."""
    N, h, q = shape.n_tokens, shape.hidden, shape.q_cols
    wp, wb = _ws(workspace, 0)
    _check("tp_attn_out_shard", lib().tp_attn_out_shard(
        ctypes.byref(shape), _p(O_i, BF16, N * q, "O_i"), _p(Wo_i, BF16, q * h, "Wo_i"),
        _p(Y_i, BF16, N * h, "Y_i"), wp, wb, _stream(stream)))


def tp_attn_out_bwd_shard(shape: AttnShape, dY, O_i, Wo_i, dO_i, dWo_i, stream=None):
    N, h, q = shape.n_tokens, shape.hidden, shape.q_cols
    _check("tp_attn_out_bwd_shard", lib().tp_attn_out_bwd_shard(
        ctypes.byref(shape), _p(dY, BF16, N * h, "dY"), _p(O_i, BF16, N * q, "O_i"),
        _p(Wo_i, BF16, q * h, "Wo_i"), _p(dO_i, BF16, N * q, "dO_i"), _p(dWo_i, F32, q * h, "dWo_i"),
        _stream(stream)))


def tp_attn_qkv_bwd_shard(shape: AttnShape, X, Wqkv_i, dQKV_i, dWqkv_i, dX_partial, stream=None):
    N, h, w = shape.n_tokens, shape.hidden, shape.qkv_cols
    _check("tp_attn_qkv_bwd_shard", lib().tp_attn_qkv_bwd_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(Wqkv_i, BF16, h * w, "Wqkv_i"),
        _p(dQKV_i, BF16, N * w, "dQKV_i"), _p(dWqkv_i, F32, h * w, "dWqkv_i"),
        _p(dX_partial, BF16, N * h, "dX_partial"), _stream(stream)))


def tp_attn_out_dgrad_shard(shape: AttnShape, dY, Wo_i, dO_i, workspace=None, stream=None):
    """dO_i = dY Wo_i^T alone (k-split partials in the workspace)."""
    N, h, qc = shape.n_tokens, shape.hidden, shape.q_cols
    wp, wb = _ws(workspace, 0)
    _check("tp_attn_out_dgrad_shard", lib().tp_attn_out_dgrad_shard(
        ctypes.byref(shape), _p(dY, BF16, N * h, "dY"), _p(Wo_i, BF16, qc * h, "Wo_i"),
        _p(dO_i, BF16, N * qc, "dO_i"), wp, wb, _stream(stream)))


def tp_attn_qkv_bwd_out_wgrad_shard(shape: AttnShape, X, Wqkv_i, dQKV_i, dY, O_i, dWqkv_i, dX_partial, dWo_i,
                                    stream=None):
    """dX_partial, dWqkv_i and the deferred dWo_i = O_i^T dY in one call."""
    N, h, qc, wc = shape.n_tokens, shape.hidden, shape.q_cols, shape.qkv_cols
    _check("tp_attn_qkv_bwd_out_wgrad_shard", lib().tp_attn_qkv_bwd_out_wgrad_shard(
        ctypes.byref(shape), _p(X, BF16, N * h, "X"), _p(Wqkv_i, BF16, h * wc, "Wqkv_i"),
        _p(dQKV_i, BF16, N * wc, "dQKV_i"), _p(dY, BF16, N * h, "dY"), _p(O_i, BF16, N * qc, "O_i"),
        _p(dWqkv_i, F32, h * wc, "dWqkv_i"), _p(dX_partial, BF16, N * h, "dX_partial"),
        _p(dWo_i, F32, qc * h, "dWo_i"), _stream(stream)))


# ------------------------------------------- sequence-parallel LayerNorm
LN_EPS = 1e-5


def tp_sp_layernorm_fwd(x, gamma, y, beta=None, mean=None, rstd=None, eps=LN_EPS, stream=None):
    """y = LayerNorm(x) over the rank's bf16 [rows, cols] block; mean / rstd
    float32 [rows] (both or neither) receive the backward's stash."""
    rows, cols = x.shape
    _check("tp_sp_layernorm_fwd", lib().tp_sp_layernorm_fwd(
        rows, cols, eps, _p(x, BF16, rows * cols, "x"), _p(gamma, BF16, cols, "gamma"),
        _p(beta, BF16, cols, "beta", optional=True), _p(y, BF16, rows * cols, "y"),
        _p(mean, F32, rows, "mean", optional=True), _p(rstd, F32, rows, "rstd", optional=True), _stream(stream)))


def tp_sp_reduce_scatter_layernorm_local(partials, rank, z, gamma, y, bias=None, residual=None, beta=None,
                                         mean=None, rstd=None, eps=LN_EPS, stream=None):
    """z = rank's block of sum(partials) + bias + residual (bf16), then
    y = LayerNorm(z); z, y, residual are [rows / t, cols]."""
    t, rows, cols, ptrs = _ptr_list(partials, "partials")
    n = rows // t
    _check("tp_sp_reduce_scatter_layernorm_local", lib().tp_sp_reduce_scatter_layernorm_local(
        t, ptrs, rows, cols, rank, _p(bias, BF16, cols, "bias", optional=True),
        _p(residual, BF16, n * cols, "residual", optional=True), _p(z, BF16, n * cols, "z"), eps,
        _p(gamma, BF16, cols, "gamma"), _p(beta, BF16, cols, "beta", optional=True), _p(y, BF16, n * cols, "y"),
        _p(mean, F32, n, "mean", optional=True), _p(rstd, F32, n, "rstd", optional=True), _stream(stream)))


def tp_sp_layernorm_bwd(x, gamma, mean, rstd, dy, dx, dgamma, dbeta=None, dres=None, workspace=None, stream=None):
    """dx = LayerNorm backward of dy (+ dres); dgamma / dbeta: float32 [cols]
    sums over this block's rows."""
    rows, cols = x.shape
    wp, wb = _ws(workspace, 0)
    _check("tp_sp_layernorm_bwd", lib().tp_sp_layernorm_bwd(
        rows, cols, _p(x, BF16, rows * cols, "x"), _p(gamma, BF16, cols, "gamma"), _p(mean, F32, rows, "mean"),
        _p(rstd, F32, rows, "rstd"), _p(dy, BF16, rows * cols, "dy"),
        _p(dres, BF16, rows * cols, "dres", optional=True), _p(dx, BF16, rows * cols, "dx"),
        _p(dgamma, F32, cols, "dgamma"), _p(dbeta, F32, cols, "dbeta", optional=True), wp, wb, _stream(stream)))


def tp_sp_sum_grads_local(grads, out, stream=None):
    """out = sum of the ranks' float32 gradients of a shared parameter, in
    rank order (the all-reduce's arithmetic)."""
    t = len(grads)
    if t == 0:
        raise ValueError("need at least one gradient")
    n = grads[0].numel()
    for g in grads:
        if g.numel() != n:
            raise ValueError("grads must share one size")
    ptrs = (c_void_p * t)(*[_p(g, F32, n, f"grads[{i}]") for i, g in enumerate(grads)])
    _check("tp_sp_sum_grads_local", lib().tp_sp_sum_grads_local(t, ptrs, n, _p(out, F32, n, "out"),
                                                                 _stream(stream)))
