"""CPU oracle for absorbed multi-head latent attention (MLA) decode.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
GPU library.  Only the test suite, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import or call it; the product path
never does, and it shares no code with the HIP kernels or their binding.

Everything here is plain float64 numpy (float32 when asked, for timing only),
written as the definitions read, with no blocking or fusion beyond them.

What is computed (the pages' statement of the method):

* The cache holds, per token, only the latent ``c`` (width d_c) followed by the
  decoupled rotary key ``k^R`` (width d^R_h): "Multi-head latent attention
  (MLA)", section 2 (the latent is the only thing cached) and section 3 (the
  cache also holds the small rotary key); "Attention, Part 2: MQA, GQA and
  MLA", section "The MLA equations" (cache per token is d_c + d_r numbers).
* Query-side absorption: each head's content query is multiplied once by the
  transpose of that head's W^UK block, giving a d_c-wide latent query
  ("Attention, Part 2", section "The trick that makes it fast: never rebuild
  at all"; "Multi-head latent attention (MLA)", section 2 and Exercise 3).
* The score adds a content term (latent query . latent) and a positional term
  (rotary query . rotary key) and divides by sqrt(d_n + d_r) (same section of
  "Attention, Part 2", and its section "Why position needs its own key").
* A causal mask, a softmax over the visible cached tokens, a weighted sum of
  the cached latents (the values are the first d_c columns of the row: "How
  DeepSeek Rewrote the Transformer", section "Absorbed projections: the
  mathematician's shortcut", point 3), then one up-projection per head through
  W^UV ("Attention, Part 2", the value side of absorption).

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):

* Layouts: ``W^UK`` is ``[H, d_n, d_c]`` and ``W^UV`` is ``[H, d_v, d_c]``, the
  per-head views of linear weights of shape ``(H*d, d_c)``, as the page-3 code
  reshapes them; a cached row is ``[c | k^R]``; an absorbed query is
  ``[q_lat | q_rope]``.
* Decode with T new tokens: the T new rows are appended first; query t of a
  sequence with N rows after the append sees rows ``0 .. N - T + t``.
* Paging (fixed pages plus a block table) and split-KV with a log-sum-exp merge
  are not on the pages; they are the data layout and work split of the GPU
  path, defined here by their plain meaning.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# paged cache: plain definitions of where a logical row lives
# --------------------------------------------------------------------------

def gather_rows_ref(pool: np.ndarray, block_table: np.ndarray, b: int, n: int,
                    block_size: int) -> np.ndarray:
    """Logical rows 0..n-1 of sequence b: row j is slot j % block_size of page
    block_table[b, j // block_size].  Returns a copy, shape [n, W]."""
    out = np.empty((n, pool.shape[2]), dtype=pool.dtype)
    for j in range(n):
        out[j] = pool[block_table[b, j // block_size], j % block_size]
    return out


def append_ref(pool: np.ndarray, block_table: np.ndarray, seq_lens_before: np.ndarray,
               new_rows: np.ndarray, block_size: int) -> np.ndarray:
    """Write new_rows[b, i] to logical position seq_lens_before[b] + i of
    sequence b.  Returns a new pool; the input pool is not modified."""
    out = pool.copy()
    B, T = new_rows.shape[:2]
    for b in range(B):
        for i in range(T):
            pos = int(seq_lens_before[b]) + i
            out[block_table[b, pos // block_size], pos % block_size] = new_rows[b, i]
    return out


# --------------------------------------------------------------------------
# the absorbed decode path
# --------------------------------------------------------------------------

def absorb_q_ref(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray,
                 dtype=F64) -> np.ndarray:
    """q_abs[..., h, :] = [ W^UK[h]^T q_nope[..., h, :]  |  q_rope[..., h, :] ].

    q_nope [..., H, d_n], q_rope [..., H, d_r], w_uk [H, d_n, d_c]
    -> [..., H, d_c + d_r].
    """
    qn = np.asarray(q_nope, dtype=dtype)
    wk = np.asarray(w_uk, dtype=dtype)
    q_lat = np.einsum("...hd,hdc->...hc", qn, wk)
    return np.concatenate([q_lat, np.asarray(q_rope, dtype=dtype)], axis=-1)


def visible_count(n_rows: int, T: int, t: int, causal: bool) -> int:
    """Number of cached rows query t (0-based among T new tokens) may attend to."""
    return n_rows - T + t + 1 if causal else n_rows


def attend_ref(q_abs_b: np.ndarray, rows: np.ndarray, d_c: int, scale: float,
               causal: bool, dtype=F64, return_probs: bool = False):
    """Latent-space attention for one sequence.

    q_abs_b [T, H, W], rows [N, W] (logical order, N counts the T new rows).
    Returns o_lat [T, H, d_c], lse [T, H] (natural log of the softmax
    denominator, including the max), and optionally the probabilities
    [T, H, N] (zero where masked).  A query that sees no row gets o_lat = 0 and
    lse = -inf.
    """
    q = np.asarray(q_abs_b, dtype=dtype)
    R = np.asarray(rows, dtype=dtype)
    T, H, W = q.shape
    N = R.shape[0]
    o = np.zeros((T, H, d_c), dtype=dtype)
    lse = np.full((T, H), -np.inf, dtype=dtype)
    probs = np.zeros((T, H, N), dtype=dtype) if return_probs else None
    for t in range(T):
        n = max(0, min(N, visible_count(N, T, t, causal)))
        if n == 0:
            continue
        s = (q[t] @ R[:n].T) * dtype(scale)          # [H, n]: content + rotary terms
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        o[t] = p @ R[:n, :d_c]                        # values are the latents
        lse[t] = (m + np.log(l))[:, 0]
        if return_probs:
            probs[t, :, :n] = p
    if return_probs:
        return o, lse, probs
    return o, lse


def decode_ref(q_abs: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
               seq_lens: np.ndarray, d_c: int, scale: float, causal: bool,
               block_size: int, dtype=F64) -> Tuple[np.ndarray, np.ndarray]:
    """Absorbed decode over a paged cache: o_lat [B, T, H, d_c], lse [B, T, H]."""
    B, T, H, _ = q_abs.shape
    o = np.zeros((B, T, H, d_c), dtype=dtype)
    lse = np.full((B, T, H), -np.inf, dtype=dtype)
    for b in range(B):
        R = gather_rows_ref(pool, block_table, b, int(seq_lens[b]), block_size)
        o[b], lse[b] = attend_ref(q_abs[b], R, d_c, scale, causal, dtype=dtype)
    return o, lse


def out_proj_ref(o_lat: np.ndarray, w_uv: np.ndarray, dtype=F64) -> np.ndarray:
    """o[..., h, v] = sum_c W^UV[h, v, c] o_lat[..., h, c]  (up-project once per head)."""
    return np.einsum("...hc,hvc->...hv", np.asarray(o_lat, dtype=dtype),
                     np.asarray(w_uv, dtype=dtype))


# --------------------------------------------------------------------------
# the output side: W^O over the heads, and W^UV folded into it
# --------------------------------------------------------------------------

def o_proj_ref(attn: np.ndarray, w_o: np.ndarray, dtype=F64) -> np.ndarray:
    """y[m, :] = W^O x_m, where x_m lists the per-head outputs attn[m, h, :]
    head after head ("Attention, Part 2: MQA, GQA and MLA", section "The trick
    that makes it fast": its inference code reshapes the per-head outputs of a
    token into one vector and applies the output projection W_o).
    attn [M, H, d_v], w_o [d, H * d_v] (the weight of a linear layer
    H * d_v -> d) -> y [M, d]."""
    a = np.asarray(attn, dtype=dtype)
    return a.reshape(a.shape[0], -1) @ np.asarray(w_o, dtype=dtype).T


def fold_uv_o_ref(w_uv: np.ndarray, w_o: np.ndarray, dtype=F64) -> np.ndarray:
    """The output-side absorption: W^UV and W^O merged into one matrix ("How
    DeepSeek Rewrote the Transformer", section "Absorbed projections: the
    mathematician's shortcut", point 2; "Multi-head latent attention (MLA)",
    section 2: the up-projections fold into the output projection).  The block
    of head h is W^O's block of head h times W^UV[h]:
    W_fold[:, h*d_c + c] = sum_v W^O[:, h*d_v + v] W^UV[h, v, c].
    w_uv [H, d_v, d_c], w_o [d, H * d_v] -> w_fold [d, H * d_c]."""
    wv = np.asarray(w_uv, dtype=dtype)
    H, d_v, d_c = wv.shape
    wo = np.asarray(w_o, dtype=dtype)
    d = wo.shape[0]
    out = np.empty((d, H * d_c), dtype=dtype)
    for h in range(H):
        out[:, h * d_c:(h + 1) * d_c] = wo[:, h * d_v:(h + 1) * d_v] @ wv[h]
    return out


def o_proj_folded_ref(o_lat: np.ndarray, w_fold: np.ndarray, dtype=F64) -> np.ndarray:
    """y[m, :] = W_fold z_m, where z_m lists the latent outputs o_lat[m, h, :]
    head after head: the folded matrix applied straight to the latent-space
    sums.  o_lat [M, H, d_c], w_fold [d, H * d_c] -> y [M, d]."""
    z = np.asarray(o_lat, dtype=dtype)
    return z.reshape(z.shape[0], -1) @ np.asarray(w_fold, dtype=dtype).T


# --------------------------------------------------------------------------
# split-KV: partial attention over a contiguous row range, merged by log-sum-exp
# --------------------------------------------------------------------------

def partial_attend_ref(q_abs_b: np.ndarray, rows: np.ndarray, lo: int, hi: int,
                       d_c: int, scale: float, causal: bool, dtype=F64):
    """Attention of every query restricted to rows [lo, hi) (intersected with
    what each query may see).  Returns the normalised partial output
    [T, H, d_c] and its log-sum-exp [T, H]; an empty range gives 0 and -inf."""
    q = np.asarray(q_abs_b, dtype=dtype)
    R = np.asarray(rows, dtype=dtype)
    T, H, _ = q.shape
    N = R.shape[0]
    o = np.zeros((T, H, d_c), dtype=dtype)
    lse = np.full((T, H), -np.inf, dtype=dtype)
    for t in range(T):
        end = min(hi, max(0, min(N, visible_count(N, T, t, causal))))
        if end <= lo:
            continue
        s = (q[t] @ R[lo:end].T) * dtype(scale)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        o[t] = (e / l) @ R[lo:end, :d_c]
        lse[t] = (m + np.log(l))[:, 0]
    return o, lse


def lse_combine_ref(parts_o: List[np.ndarray], parts_lse: List[np.ndarray]):
    """Merge normalised partials: with M = max_s lse_s and w_s = exp(lse_s - M),
    O = sum_s w_s O_s / sum_s w_s and lse = M + log sum_s w_s.  Partials whose
    lse is -inf carry no weight; if all are -inf the result is 0 and -inf."""
    L = np.stack(parts_lse)                    # [S, ...]
    O = np.stack(parts_o)                      # [S, ..., d_c]
    M = L.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - Ms), 0.0)
    den = w.sum(axis=0)
    safe = np.where(den > 0, den, 1.0)
    out = (w[..., None] * O).sum(axis=0) / safe[..., None]
    out = np.where(finite[..., None], out, 0.0)
    lse = np.where(finite, Ms + np.log(safe), -np.inf)
    return out, lse


def split_decode_ref(q_abs: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                     seq_lens: np.ndarray, d_c: int, scale: float, causal: bool,
                     block_size: int, pages_per_split: int, dtype=F64):
    """Decode computed as contiguous page ranges of ``pages_per_split`` pages
    each, merged by log-sum-exp.  Equal to ``decode_ref`` in exact arithmetic."""
    B, T, H, _ = q_abs.shape
    o = np.zeros((B, T, H, d_c), dtype=dtype)
    lse = np.full((B, T, H), -np.inf, dtype=dtype)
    span = pages_per_split * block_size
    for b in range(B):
        n = int(seq_lens[b])
        R = gather_rows_ref(pool, block_table, b, n, block_size)
        n_splits = max(1, -(-n // span))
        po, pl = [], []
        for s in range(n_splits):
            a, c = partial_attend_ref(q_abs[b], R, s * span, (s + 1) * span, d_c, scale,
                                      causal, dtype=dtype)
            po.append(a)
            pl.append(c)
        o[b], lse[b] = lse_combine_ref(po, pl)
    return o, lse


# --------------------------------------------------------------------------
# the naive path: rebuild every head's keys and values, then plain attention
# --------------------------------------------------------------------------

def naive_ref(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
              rows: np.ndarray, d_c: int, scale: float, causal: bool) -> np.ndarray:
    """Per head h: K_h[j] = [W^UK[h] c_j | k^R_j], V_h[j] = W^UV[h] c_j, query
    [q_nope | q_rope]; textbook softmax attention.  One sequence:
    q_nope [T, H, d_n], q_rope [T, H, d_r], rows [N, W] -> o [T, H, d_v]."""
    qn = np.asarray(q_nope, F64)
    qr = np.asarray(q_rope, F64)
    wk = np.asarray(w_uk, F64)
    wv = np.asarray(w_uv, F64)
    R = np.asarray(rows, F64)
    T, H, _ = qn.shape
    N = R.shape[0]
    C, KR = R[:, :d_c], R[:, d_c:]
    o = np.zeros((T, H, wv.shape[1]))
    for h in range(H):
        K = np.concatenate([C @ wk[h].T, KR], axis=1)        # [N, d_n + d_r]
        V = C @ wv[h].T                                       # [N, d_v]
        for t in range(T):
            n = max(0, min(N, visible_count(N, T, t, causal)))
            if n == 0:
                continue
            q = np.concatenate([qn[t, h], qr[t, h]])
            s = (K[:n] @ q) * scale
            e = np.exp(s - s.max())
            o[t, h] = (e / e.sum()) @ V[:n]
    return o


def brute_force_ref(q_nope, q_rope, w_uk, w_uv, rows, d_c: int, scale: float,
                    causal: bool):
    """The naive path in pure-Python loops (no numpy arithmetic), for tiny
    inputs.  Returns o as nested lists [T][H][d_v]."""
    qn, qr = np.asarray(q_nope).tolist(), np.asarray(q_rope).tolist()
    wk, wv, R = np.asarray(w_uk).tolist(), np.asarray(w_uv).tolist(), np.asarray(rows).tolist()
    T, H, d_n = len(qn), len(qn[0]), len(qn[0][0])
    d_r = len(qr[0][0])
    d_v = len(wv[0])
    N = len(R)
    out = [[[0.0] * d_v for _ in range(H)] for _ in range(T)]
    for t in range(T):
        n = max(0, min(N, visible_count(N, T, t, causal)))
        for h in range(H):
            if n == 0:
                continue
            scores = []
            for j in range(n):
                s = 0.0
                for d in range(d_n):                      # content key W^UK[h] c_j
                    k = 0.0
                    for c in range(d_c):
                        k += wk[h][d][c] * R[j][c]
                    s += qn[t][h][d] * k
                for r in range(d_r):                      # rotary key
                    s += qr[t][h][r] * R[j][d_c + r]
                scores.append(s * scale)
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            tot = sum(ex)
            for v in range(d_v):
                acc = 0.0
                for j in range(n):
                    val = 0.0                             # value W^UV[h] c_j
                    for c in range(d_c):
                        val += wv[h][v][c] * R[j][c]
                    acc += ex[j] / tot * val
                out[t][h][v] = acc
    return out


# --------------------------------------------------------------------------
# the whole step, and RoPE (used only to show why it must stay out of the latent)
# --------------------------------------------------------------------------

def step_ref(q_nope, q_rope, w_uk, w_uv, pool, block_table, lengths, new_rows,
             d_c: int, scale: float, causal: bool, block_size: int, dtype=F64):
    """One decode step: absorb the queries, append the new rows, attend, and
    up-project.  Returns (pool_after, q_abs, o_lat, lse, o)."""
    pool_after = append_ref(pool, block_table, lengths, new_rows, block_size)
    q_abs = absorb_q_ref(q_nope, q_rope, w_uk, dtype=dtype)
    seq_lens = np.asarray(lengths) + new_rows.shape[1]
    o_lat, lse = decode_ref(q_abs, pool_after, block_table, seq_lens, d_c, scale,
                            causal, block_size, dtype=dtype)
    return pool_after, q_abs, o_lat, lse, out_proj_ref(o_lat, w_uv, dtype=dtype)


def rope_ref(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate consecutive pairs (x[2i], x[2i+1]) of the last axis by the angle
    pos * theta_i with theta_i = base^(-2i/d), as RoFormer defines it (the
    rotation of one pair at position m by m*theta in "Attention, Part 2",
    section "Why position needs its own key").  x [..., n, d], pos [n]."""
    x = np.asarray(x, F64)
    d = x.shape[-1]
    theta = base ** (-np.arange(0, d, 2, dtype=F64) / d)
    ang = np.asarray(pos, F64)[:, None] * theta[None, :]     # [n, d/2]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x1 * sin + x2 * cos
    return out


def kv_produce_ref(hidden: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray,
                   pos: np.ndarray, base: float = 10000.0, dtype=F64) -> np.ndarray:
    """The cached row of each new token, from its hidden vector h (width d):
    the latent c = W^DKV h ("Multi-head latent attention (MLA)", section 2: the
    down-projection is the only thing cached) and the decoupled rotary key
    k^R = RoPE(W^KR h) at the token's position (same page, section 3: the key
    has its own projection and is rotated directly; "Attention, Part 2",
    section "The MLA equations" and its inference code, which computes the two
    and nothing else for the cache).  The latent is never rotated.
    hidden [n, d], w_dkv [d_c, d], w_kr [d_r, d], pos [n] -> [n, d_c + d_r]."""
    h = np.asarray(hidden, dtype)
    c = h @ np.asarray(w_dkv, dtype).T
    kr = h @ np.asarray(w_kr, dtype).T
    return np.concatenate([c, rope_ref(kr, pos, base)], axis=-1)


def produce_append_ref(pool, block_table, seq_lens_before, hidden, w_dkv, w_kr,
                       block_size: int, base: float = 10000.0) -> np.ndarray:
    """The producer step of a batch: token i of sequence b (hidden [B, T, d])
    sits at position seq_lens_before[b] + i; its row is produced and appended
    there.  Returns the pool after (float64)."""
    B, T, _ = hidden.shape
    rows = np.stack([kv_produce_ref(hidden[b], w_dkv, w_kr,
                                    int(seq_lens_before[b]) + np.arange(T), base)
                     for b in range(B)])
    return append_ref(pool, block_table, seq_lens_before, rows, block_size)


def naive_rope_on_rebuilt_keys_ref(q_nope, w_uk, w_uv, rows, d_c: int, scale: float,
                                   q_pos: np.ndarray, k_pos: Optional[np.ndarray] = None,
                                   base: float = 10000.0):
    """The mistake the page-3 author tested: rotate the rebuilt content keys and
    the content queries by position (no decoupled rotary part).  One sequence,
    causal over its rows: q_nope [T, H, d_n], rows [N, W] -> o [T, H, d_v].
    Key positions default to 0..N-1."""
    qn = np.asarray(q_nope, F64)
    wk, wv, R = np.asarray(w_uk, F64), np.asarray(w_uv, F64), np.asarray(rows, F64)
    T, H, _ = qn.shape
    N = R.shape[0]
    C = R[:, :d_c]
    o = np.zeros((T, H, wv.shape[1]))
    kpos = np.arange(N) if k_pos is None else np.asarray(k_pos)
    for h in range(H):
        K = rope_ref(C @ wk[h].T, kpos, base)
        V = C @ wv[h].T
        Q = rope_ref(qn[:, h, :], q_pos, base)
        for t in range(T):
            n = N - T + t + 1
            s = (K[:n] @ Q[t]) * scale
            e = np.exp(s - s.max())
            o[t, h] = (e / e.sum()) @ V[:n]
    return o


def absorbed_without_rope_ref(q_nope, w_uk, w_uv, rows, d_c: int, scale: float):
    """The absorbed path with the content term only (what absorption can still
    compute when the rotation sat on the rebuilt keys).  One sequence, causal."""
    q_lat = absorb_q_ref(q_nope, np.zeros(q_nope.shape[:-1] + (0,)), w_uk)
    R = np.asarray(rows, F64)[:, :d_c]
    o_lat, _ = attend_ref(q_lat, R, d_c, scale, True)
    return out_proj_ref(o_lat, w_uv)
