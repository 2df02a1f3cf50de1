"""Closed forms for how much each attention variant caches per token.

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

* Plain multi-head attention keeps one key and one value per head per layer:
  2 * n_h * d_h numbers per token per layer ("Multi-head latent attention
  (MLA)", section 1; in bytes 2 * L * H * d_h * b, "Attention, Part 2: MQA,
  GQA and MLA", section "How big is it?").
* Grouped-query attention keeps 2 * n_kv * d_h ("Multi-head latent attention
  (MLA)", section 2; "Attention, Part 2", section "Grouped-query attention").
* MLA keeps the latent plus the decoupled rotary key: d_c + d^R_h numbers
  ("Multi-head latent attention (MLA)", sections 2 and 3; "Attention, Part 2",
  section "The MLA equations").
"""
from __future__ import annotations


def mha_numbers(n_heads: int, d_head: int) -> int:
    return 2 * n_heads * d_head


def gqa_numbers(n_kv: int, d_head: int) -> int:
    return 2 * n_kv * d_head


def mla_numbers(d_c: int, d_rope: int) -> int:
    return d_c + d_rope


def mha_bytes_per_token(layers: int, kv_heads: int, d_head: int, bytes_per: int) -> int:
    """2 * L * H * d_h * b: one key and one value per head per layer."""
    return 2 * layers * kv_heads * d_head * bytes_per


def mha_bytes_split_widths(layers: int, heads: int, d_key: int, d_value: int,
                           bytes_per: int) -> int:
    """Plain attention whose keys and values have different widths
    (DeepSeek-V3 keys carry 128 content + 64 rotary dims, values 128)."""
    return layers * heads * (d_key + d_value) * bytes_per


def mla_bytes_per_token(layers: int, d_c: int, d_rope: int, bytes_per: int) -> int:
    """L * (d_c + d_r) * b."""
    return layers * (d_c + d_rope) * bytes_per


def gqa_equivalent_groups(d_head: float, latent_mult: float = 4.0,
                          rope_frac: float = 0.5) -> float:
    """Groups n_g at which GQA caches as much as MLA with d_c = latent_mult*d_h
    and d^R_h = rope_frac*d_h: solve 2 * n_g * d_h = d_c + d^R_h ("Attention,
    Part 2", section "How big is the difference?")."""
    return (latent_mult * d_head + rope_frac * d_head) / (2.0 * d_head)
