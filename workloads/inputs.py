"""Seeded synthetic inputs for one decode step, shared by the oracle tests and
the GPU path.

This module draws random numbers and lays them out; it performs none of the
attention arithmetic.  Every draw comes from ``numpy.random.default_rng(seed)``
in a fixed order (documented in ``make_inputs``), as float32 standard normals,
rounded to the nearest bfloat16 (ties to even) when the workload is bf16.  The
rounded values are returned as float32 arrays whose every element is exactly a
bfloat16 value, so the oracle can upcast them to float64 without loss and the
GPU path can convert them to bfloat16 without loss.

Cache layout: a page pool ``[num_blocks, block_size, W]`` and a block table
``[B, max_blocks]`` of int32 page ids.  Row j of sequence b lives at
``pool[block_table[b, j // block_size], j % block_size]``.  Every pool slot that
holds no row is filled with NaN ("poison"), so a kernel that reads past a
sequence's end produces NaN instead of a plausible wrong number.  One extra
all-poison page is appended to the pool; unused block-table entries point to it
so that they are valid page ids that hold no data.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from .configs import Workload


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; return float32.

    Works on the IEEE-754 bit pattern: adding 0x7FFF plus the lowest kept bit
    and truncating the low 16 bits rounds to nearest with ties to even.  NaN
    stays NaN (quiet), infinities stay infinite, finite values past the largest
    bfloat16 round to infinity.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        r = r.copy()
        r[nan] = np.float32(np.nan)
    return r


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are exact bfloat16 values."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Batch:
    workload: Workload
    lengths: np.ndarray        # int32 [B]: rows cached before the step
    seq_lens: np.ndarray       # int32 [B]: rows after the T new ones are appended
    rows: List[np.ndarray]     # per sequence float32 [lengths[b], W], logical order
    new_rows: np.ndarray       # float32 [B, T, W]
    q_nope: np.ndarray         # float32 [B, T, H, d_n]
    q_rope: np.ndarray         # float32 [B, T, H, d_r]
    w_uk: np.ndarray           # float32 [H, d_n, d_c]
    w_uv: np.ndarray           # float32 [H, d_v, d_c]
    q_abs: np.ndarray          # float32 [B, T, H, W]: a directly drawn absorbed query
    pool: np.ndarray           # float32 [num_blocks, block_size, W] (poisoned empties)
    block_table: np.ndarray    # int32 [B, max_blocks]
    poison_block: int          # id of the all-poison page

    @property
    def num_blocks(self) -> int:
        return int(self.pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0


def _pages(n: int, bs: int) -> int:
    return (n + bs - 1) // bs


def make_inputs(w: Workload, seed: int | None = None, *, with_rows: bool = True) -> Batch:
    """Draw one decode step's inputs for workload ``w``.

    Draw order (all from one ``default_rng(seed)``, seed defaults to ``w.seed``):
      1. lengths: ``integers(1, N, endpoint=True, size=B)`` if ``var_len`` else N;
      2. for each sequence b in order: its cached rows ``standard_normal((L_b, W))``,
         then, if ``outlier_frac > 0``, ``choice(L_b, int(L_b*outlier_frac),
         replace=False)`` row indices whose whole row is multiplied by
         ``outlier_scale``;
      3. the new rows ``standard_normal((B, T, W))``;
      4. ``q_nope (B,T,H,d_n)``, then ``q_rope (B,T,H,d_r)``;
      5. ``W^UK (H,d_n,d_c)`` and ``W^UV (H,d_v,d_c)``, each times 1/sqrt(d_c)
         (standard deviation 1/sqrt(d_c));
      6. a directly drawn absorbed query ``q_abs (B,T,H,W)``;
      7. if the table is permuted: ``permutation(total_pages)``, assigned to the
         logical pages in order (sequence-major).
    All draws are float32, rounded to bfloat16 afterwards when ``dtype == "bf16"``.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, T, H, W, bs = w.B, w.T, w.H, w.W, w.block_size
    if w.var_len:
        lengths = rng.integers(1, w.N, endpoint=True, size=B).astype(np.int32)
    else:
        lengths = np.full(B, w.N, dtype=np.int32)
    rnd = bf16_round if w.dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))

    rows = []
    for b in range(B):
        r = rng.standard_normal((int(lengths[b]), W), dtype=np.float32)
        if w.outlier_frac > 0.0:
            k = int(int(lengths[b]) * w.outlier_frac)
            idx = rng.choice(int(lengths[b]), k, replace=False)
            r[idx] *= np.float32(w.outlier_scale)
        rows.append(rnd(r))
    new_rows = rnd(rng.standard_normal((B, T, W), dtype=np.float32))
    q_nope = rnd(rng.standard_normal((B, T, H, w.d_n), dtype=np.float32))
    q_rope = rnd(rng.standard_normal((B, T, H, w.d_r), dtype=np.float32))
    s = np.float32(1.0 / np.sqrt(w.d_c))
    w_uk = rnd(rng.standard_normal((H, w.d_n, w.d_c), dtype=np.float32) * s)
    w_uv = rnd(rng.standard_normal((H, w.d_v, w.d_c), dtype=np.float32) * s)
    q_abs = rnd(rng.standard_normal((B, T, H, W), dtype=np.float32))

    seq_lens = (lengths + T).astype(np.int32)
    n_pages = [_pages(int(n), bs) for n in seq_lens]
    total = int(sum(n_pages))
    if w.table == "permuted":
        ids = rng.permutation(total).astype(np.int32)
    elif w.table == "sequential":
        ids = np.arange(total, dtype=np.int32)
    else:
        raise ValueError(f"unknown table kind {w.table!r}")
    max_blocks = max(n_pages) if n_pages else 1
    poison = total
    table = np.full((B, max_blocks), poison, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, : n_pages[b]] = ids[off: off + n_pages[b]]
        off += n_pages[b]

    pool = np.full((total + 1, bs, W), np.nan, dtype=np.float32)
    if with_rows:
        for b in range(B):
            L = int(lengths[b])
            full = L // bs
            if full:
                pool[table[b, :full]] = rows[b][: full * bs].reshape(full, bs, W)
            rem = L - full * bs
            if rem:
                pool[table[b, full], :rem] = rows[b][full * bs:]
    return Batch(workload=w, lengths=lengths, seq_lens=seq_lens, rows=rows,
                 new_rows=new_rows, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv,
                 q_abs=q_abs, pool=pool, block_table=table, poison_block=poison)


@dataclass
class ProducerInputs:
    """Inputs of the producer step of one batch: the new tokens' hidden vectors
    and the two down-projections.  Positions come from the batch's lengths."""
    hidden: np.ndarray   # [B, T, d]
    w_dkv: np.ndarray    # [d_c, d]
    w_kr: np.ndarray     # [d_r, d]


def make_producer_inputs(w: Workload, seed: int | None = None) -> ProducerInputs:
    """Draws for the producer step, from their own ``default_rng`` stream
    (seed 1000 + the workload's seed by default, so the decode inputs of
    ``make_inputs`` are unchanged).  Order: hidden ``[B, T, d]`` ~ N(0, 1);
    ``W^DKV [d_c, d]`` and ``W^KR [d_r, d]`` ~ N(0, 1) times 1/sqrt(d)
    (standard deviation 1/sqrt(fan-in), the rule used for W^UK and W^UV).
    Rounded to bf16 like the rest when the workload is bf16."""
    if w.d_model <= 0:
        raise ValueError(f"workload {w.name} has no model width for the producer step")
    rng = np.random.default_rng(1000 + w.seed if seed is None else seed)
    rnd = bf16_round if w.dtype == "bf16" else (lambda a: a.astype(np.float32))
    d = w.d_model
    hidden = rnd(rng.standard_normal((w.B, w.T, d), dtype=np.float32))
    s = np.float32(1.0 / np.sqrt(d))
    w_dkv = rnd(rng.standard_normal((w.d_c, d), dtype=np.float32) * s)
    w_kr = rnd(rng.standard_normal((w.d_r, d), dtype=np.float32) * s)
    return ProducerInputs(hidden=hidden, w_dkv=w_dkv, w_kr=w_kr)


@dataclass
class OutputInputs:
    """Inputs of the output side of one batch (M = B * T tokens): per-head
    outputs, latent outputs, W^UV and the output projection W^O."""
    attn: np.ndarray     # [M, H, d_v]  (what the W^UV up-projection hands on)
    o_lat: np.ndarray    # [M, H, d_c]  float32 (what decode hands on)
    w_uv: np.ndarray     # [H, d_v, d_c]
    w_o: np.ndarray      # [d, H * d_v]


def make_output_inputs(w: Workload, seed: int | None = None) -> OutputInputs:
    """Draws for the output side, from their own ``default_rng`` stream (seed
    2000 + the workload's seed by default).  Order: ``attn [M, H, d_v]`` ~ N(0, 1);
    ``o_lat [M, H, d_c]`` ~ N(0, 1) in float32; ``W^UV [H, d_v, d_c]`` ~ N(0, 1)
    times 1/sqrt(d_c); ``W^O [d, H*d_v]`` ~ N(0, 1) times 1/sqrt(H*d_v) (standard
    deviation 1/sqrt(fan-in)).  Rounded to bf16 like the rest when the workload
    is bf16 (o_lat stays float32)."""
    if w.d_model <= 0:
        raise ValueError(f"workload {w.name} has no model width for the output side")
    rng = np.random.default_rng(2000 + w.seed if seed is None else seed)
    rnd = bf16_round if w.dtype == "bf16" else (lambda a: a.astype(np.float32))
    M, H = w.B * w.T, w.H
    attn = rnd(rng.standard_normal((M, H, w.d_v), dtype=np.float32))
    o_lat = rng.standard_normal((M, H, w.d_c), dtype=np.float32)
    w_uv = rnd(rng.standard_normal((H, w.d_v, w.d_c), dtype=np.float32)
               * np.float32(1.0 / np.sqrt(w.d_c)))
    w_o = rnd(rng.standard_normal((w.d_model, H * w.d_v), dtype=np.float32)
              * np.float32(1.0 / np.sqrt(H * w.d_v)))
    return OutputInputs(attn=attn, o_lat=o_lat, w_uv=w_uv, w_o=w_o)
