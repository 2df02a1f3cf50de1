"""Seeded synthetic decode workloads (shapes and random inputs only)."""
from .configs import ALL, BY_NAME, EXTRA, LONG, PREFILL, TINY, V2_MULTI, V3, VARLEN, Workload
from .inputs import (Batch, OutputInputs, ProducerInputs, bf16_bits, bf16_round, make_inputs,
                     make_output_inputs, make_producer_inputs)

__all__ = ["ALL", "BY_NAME", "EXTRA", "LONG", "PREFILL", "TINY", "V2_MULTI", "V3", "VARLEN", "Workload",
           "Batch", "ProducerInputs", "bf16_bits", "bf16_round", "make_inputs",
           "make_producer_inputs", "OutputInputs", "make_output_inputs"]
