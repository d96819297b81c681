"""The five synthetic workloads: one tensor-parallel rank's MLP shard at
the shapes the pages discuss.

* ``mlp128_h1024_gelu_t2``: 128 token rows, hidden 1024, expanded 4096, two
  ranks, GeLU ("Tensor Parallelism's Communication Boundary", section "Count
  the object, then the collective").
* ``llama3_70b_decode_t4``: one decode token, hidden 8192, SwiGLU with
  intermediate 28672 over four ranks ("02 -- Tensor Parallelism", section
  "Concrete numbers for Llama-3-70B, TP=4, decode batch 1, bf16").
* ``llama_7b_train_t2``: hidden 4096, SwiGLU intermediate 11008 over two
  ranks, 2 x 2048 tokens ("Parallelism Strategies #1 - Tensor Parallelism",
  the 7B model on two devices).
* ``gpt3_train_t8``: 2048 tokens, d = 12288, 4d = 49152 over eight ranks,
  GeLU ("Megatron-LM: Tensor Parallelism", section "The Communication
  Pattern").
* ``llama3_70b_prefill_t4``: 4 x 4096 tokens, hidden 8192, SwiGLU
  intermediate 28672 over four ranks, output bias added once after the sum of
  the partials.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int          # seed namespace for inputs.py
    N: int            # tokens b*s
    h: int            # hidden
    F: int            # full intermediate width
    t: int            # tensor-parallel degree
    act: str          # "relu" | "gelu" | "swiglu"
    backward: bool    # forward + backward (training) or forward only
    bias: bool        # output bias b2 added once after the reduction

    @property
    def Fi(self) -> int:
        return self.F // self.t

    @property
    def g(self) -> int:
        """Number of up-projection matrices (2 for SwiGLU: gate and up)."""
        return 2 if self.act == "swiglu" else 1

    def flops_forward(self) -> int:
        """Algorithmic FLOPs of one rank's forward: 2*N*h*Fi*(g+1)."""
        return 2 * self.N * self.h * self.Fi * (self.g + 1)

    def flops_train(self) -> int:
        """Forward + backward: the backward costs twice the forward."""
        return 3 * self.flops_forward()

    def weight_bytes(self) -> int:
        """bf16 bytes of one rank's weight shards, (g+1)*h*Fi*2."""
        return (self.g + 1) * self.h * self.Fi * 2


WORKLOADS = {
    w.name: w for w in (
        Workload("mlp128_h1024_gelu_t2", 1, 128, 1024, 4096, 2, "gelu", True, False),
        Workload("llama3_70b_decode_t4", 2, 1, 8192, 28672, 4, "swiglu", False, False),
        Workload("llama_7b_train_t2", 3, 4096, 4096, 11008, 2, "swiglu", True, False),
        Workload("gpt3_train_t8", 4, 2048, 12288, 49152, 8, "gelu", True, False),
        Workload("llama3_70b_prefill_t4", 5, 16384, 8192, 28672, 4, "swiglu", True, True),
    )
}
