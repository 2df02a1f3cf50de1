"""One MLA decode step as the four library calls, on device buffers.

``DecodeStep`` owns the outputs and the workspace of one step and runs
absorb -> append -> decode -> out-projection on the current stream (the step
as two calls: absorb with append, decode with out-projection).  It is
plumbing around the C ABI (allocation through torch, then the library calls); all of
the arithmetic happens in libmla's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as mla


class DecodeStep:
    def __init__(self, cfg: mla.MlaConfig, *, q_nope: torch.Tensor, q_rope: torch.Tensor,
                 w_uk: torch.Tensor, w_uv: torch.Tensor, pool: torch.Tensor,
                 block_table: torch.Tensor, lengths: torch.Tensor, new_rows: torch.Tensor,
                 max_len_after: int, causal: bool = True, num_splits: int = 0,
                 total_tokens: int = 0):
        self.cfg = cfg
        self.B, self.T, self.H = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
        self.M = self.B * self.T
        dev = q_nope.device
        W = cfg.d_c + cfg.d_rope
        dt = q_nope.dtype
        self.q_nope = q_nope.reshape(self.M, self.H, cfg.d_nope)
        self.q_rope = q_rope.reshape(self.M, self.H, cfg.d_rope)
        self.w_uk, self.w_uv = w_uk, w_uv
        self.pool, self.block_table = pool, block_table
        self.lengths = lengths                                  # rows before the step
        self.seq_lens = (lengths + self.T).to(torch.int32)      # rows after the append
        self.new_rows = new_rows
        self.max_len_after = int(max_len_after)
        self.causal = causal
        self.total_tokens = int(total_tokens)
        self.num_splits = int(num_splits)
        self.q_abs = torch.empty(self.B, self.T, self.H, W, dtype=dt, device=dev)
        self.o_lat = torch.empty(self.B, self.T, self.H, cfg.d_c, dtype=torch.float32, device=dev)
        self.lse = torch.empty(self.B, self.T, self.H, dtype=torch.float32, device=dev)
        self.out = torch.empty(self.M, self.H, cfg.d_v, dtype=dt, device=dev)
        nbytes = mla.mla_decode_workspace_size(cfg, self.B, self.T, self.max_len_after,
                                               self.total_tokens, self.num_splits)
        self.workspace: Optional[torch.Tensor] = (
            torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else None)

    def absorb(self, stream=None):
        mla.mla_absorb_q(self.cfg, self.q_nope, self.q_rope, self.w_uk,
                         self.q_abs.view(self.M, self.H, -1), stream)

    def append(self, stream=None):
        mla.mla_cache_append(self.cfg, self.pool, self.block_table, self.lengths, self.new_rows,
                             self.max_len_after, stream)

    def absorb_append(self, stream=None):
        """absorb and append in one call (one launch where the MFMA absorb
        kernel applies)."""
        mla.mla_absorb_q_append(self.cfg, self.q_nope, self.q_rope, self.w_uk,
                                self.q_abs.view(self.M, self.H, -1), self.pool, self.block_table,
                                self.lengths, self.new_rows, self.max_len_after, stream)

    def decode(self, stream=None):
        mla.mla_decode(self.cfg, self.q_abs, self.pool, self.block_table, self.seq_lens,
                       self.max_len_after, self.o_lat, self.lse, causal=self.causal,
                       num_splits=self.num_splits, total_tokens_host=self.total_tokens,
                       workspace=self.workspace, stream=stream)

    def decode_fused(self, stream=None):
        """decode in one launch (mla_decode_fused) into the same outputs; its
        workspace is allocated zeroed on first use and left zeroed by every
        call."""
        if getattr(self, "fused_workspace", None) is None:
            nbytes = mla.mla_decode_fused_workspace_size(self.cfg, self.B, self.T,
                                                         self.max_len_after, self.total_tokens,
                                                         self.num_splits)
            self.fused_workspace = torch.zeros(nbytes, dtype=torch.uint8,
                                               device=self.q_abs.device)
        mla.mla_decode_fused(self.cfg, self.q_abs, self.pool, self.block_table, self.seq_lens,
                             self.max_len_after, self.o_lat, self.lse,
                             workspace=self.fused_workspace, causal=self.causal,
                             num_splits=self.num_splits, total_tokens_host=self.total_tokens,
                             stream=stream)

    def out_proj(self, stream=None):
        mla.mla_out_proj(self.cfg, self.o_lat.view(self.M, self.H, -1), self.w_uv, self.out,
                         stream)

    def decode_out_proj(self, stream=None):
        """decode and out_proj in one call (the merge and the projection share
        a launch where they can)."""
        mla.mla_decode_out_proj(self.cfg, self.q_abs, self.pool, self.block_table, self.seq_lens,
                                self.max_len_after, self.w_uv, self.o_lat, self.out, self.lse,
                                causal=self.causal, num_splits=self.num_splits,
                                total_tokens_host=self.total_tokens, workspace=self.workspace,
                                stream=stream)

    def run(self, stream=None):
        self.absorb_append(stream)
        self.decode_out_proj(stream)
