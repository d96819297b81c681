"""One tensor-parallel rank of the Megatron paired MLP, native on MI355X.

The compute lives in ``libtpmlp.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/tp_mlp.h``).  ``binding`` marshals torch
tensors to that ABI and nothing else; importing this package does not load the
library, the first call does, and it raises if the library is missing.
"""
from .configs import WORKLOADS, Workload  # noqa: F401
