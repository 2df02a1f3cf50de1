"""MI355X-native absorbed multi-head latent attention (MLA) decode.

The computation lives in ``libmla.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/mla.h``); ``binding`` exposes its calls
to Python under the same names, and ``step`` chains them into one decode step.
"""
from .binding import (MLA_BF16, MLA_F32, MlaConfig, load, make_config, mla_abi_version,
                      mla_absorb_q, mla_cache_append, mla_decode, mla_decode_num_splits,
                      mla_decode_workspace_size, mla_gather_rows, mla_out_proj,
                      mla_status_string, mla_validate_block_table)

__all__ = ["MLA_BF16", "MLA_F32", "MlaConfig", "load", "make_config", "mla_abi_version",
           "mla_absorb_q", "mla_cache_append", "mla_decode", "mla_decode_num_splits",
           "mla_decode_workspace_size", "mla_gather_rows", "mla_out_proj", "mla_status_string",
           "mla_validate_block_table"]
