"""fp64 CPU oracle for one tensor-parallel rank of the Megatron paired MLP.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the GPU library or its
binding.  See ``oracle/mlp.py`` (the MLP shard and its sequence-parallel
boundary), ``oracle/attn.py`` (the attention block's projections) and
``oracle/ln.py`` (the LayerNorm of the sequence-parallel region) for what it
computes and which passages it follows.
"""
from . import attn, ln
from .mlp import (ACTS, act_backward, act_forward, all_gather,
                  bf16_bits_to_f64, column_block, column_sum, reduce_partials,
                  reduce_scatter, round_bf16, sequence_block, shard_backward,
                  shard_forward, shard_weights, tp_backward, tp_forward)

__all__ = ["attn", "ln", "ACTS", "act_backward", "act_forward", "all_gather",
           "bf16_bits_to_f64", "column_block", "column_sum", "reduce_partials",
           "reduce_scatter", "round_bf16", "sequence_block", "shard_backward",
           "shard_forward", "shard_weights", "tp_backward", "tp_forward"]
