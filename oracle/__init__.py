"""CPU oracle for absorbed MLA decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library or its binding.
"""
from . import cache_sizes
from .mla_oracle import (absorb_q_ref, absorbed_without_rope_ref, append_ref, attend_ref,
                         brute_force_ref, decode_ref, fold_uv_o_ref, gather_rows_ref,
                         kv_produce_ref, lse_combine_ref, naive_ref,
                         naive_rope_on_rebuilt_keys_ref, o_proj_folded_ref, o_proj_ref,
                         out_proj_ref, partial_attend_ref, produce_append_ref, rope_ref,
                         split_decode_ref, step_ref, visible_count)

__all__ = ["cache_sizes", "absorb_q_ref", "absorbed_without_rope_ref", "append_ref",
           "attend_ref", "brute_force_ref", "decode_ref", "fold_uv_o_ref", "gather_rows_ref",
           "kv_produce_ref", "o_proj_folded_ref", "o_proj_ref",
           "lse_combine_ref", "naive_ref", "naive_rope_on_rebuilt_keys_ref", "out_proj_ref",
           "partial_attend_ref", "produce_append_ref", "rope_ref", "split_decode_ref", "step_ref", "visible_count"]
