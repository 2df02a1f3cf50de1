"""Planted mistakes: copies of the oracle's attention with one plausible bug
each must be rejected by the independent pins (the torch SDPA library routine
and the naive rebuild-every-key path).  This shows the pins are sharp enough
to catch a dropped term, a wrong sign or index, a transposed operand."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import V2_MULTI, make_inputs


def _attend_variant(q, R, d_c, scale, causal, bug):
    T, H, W = q.shape
    N = R.shape[0]
    o = np.zeros((T, H, d_c))
    for t in range(T):
        n = N - T + t + 1 if causal else N
        if bug == "mask_off_by_one":
            n -= 1
        if bug == "scale_squared":
            sc = scale * scale
        else:
            sc = scale
        if bug == "drop_rope_term":
            s = (q[t, :, :d_c] @ R[:n, :d_c].T) * sc
        elif bug == "rope_sign":
            s = (q[t, :, :d_c] @ R[:n, :d_c].T - q[t, :, d_c:] @ R[:n, d_c:].T) * sc
        else:
            s = (q[t] @ R[:n].T) * sc
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        V = R[:n, W - d_c:] if bug == "values_from_tail" else R[:n, :d_c]
        o[t] = p @ V
    return o


def _absorb_variant(q_nope, q_rope, w_uk, bug):
    if bug == "heads_shifted":
        w_uk = np.roll(w_uk, 1, axis=0)
    if bug == "transposed_head_block":
        # reads W^UK[h] as if it were stored [d_c, d_n]
        H, d_n, d_c = w_uk.shape
        w_uk = w_uk.reshape(H, d_c, d_n).transpose(0, 2, 1)
    return np.concatenate([np.einsum("...hd,hdc->...hc", q_nope, w_uk), q_rope], axis=-1)


def _sdpa(q_abs_b, rows, d_c, scale):
    T, H, W = q_abs_b.shape
    N = rows.shape[0]
    q = torch.from_numpy(np.ascontiguousarray(q_abs_b.transpose(1, 0, 2)))[None]
    k = torch.from_numpy(rows)[None, None].expand(1, H, N, W)
    v = torch.from_numpy(np.ascontiguousarray(rows[:, :d_c]))[None, None].expand(1, H, N, d_c)
    mask = torch.arange(N)[None, :] <= (N - T + torch.arange(T)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.fixture(scope="module")
def case():
    w = V2_MULTI.scaled(B=1, H=4, N=96, d_c=64, d_n=32, d_v=16)
    bt = make_inputs(w)
    rows = np.concatenate([bt.rows[0], bt.new_rows[0]]).astype(np.float64)
    return w, bt, rows


def _attend_pin(w, bt, rows, attend):
    q = bt.q_abs[0].astype(np.float64)
    got = attend(q, rows, w.d_c, w.scale, True)
    ref = _sdpa(q, rows, w.d_c, w.scale)
    return np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def _absorb_pin(w, bt, rows, absorb):
    q_abs = absorb(bt.q_nope[0].astype(np.float64), bt.q_rope[0].astype(np.float64),
                   bt.w_uk.astype(np.float64))
    o_lat, _ = oracle.attend_ref(q_abs, rows, w.d_c, w.scale, True)
    o = oracle.out_proj_ref(o_lat, bt.w_uv)
    ref = oracle.naive_ref(bt.q_nope[0], bt.q_rope[0], bt.w_uk, bt.w_uv, rows, w.d_c,
                           w.scale, True)
    return np.max(np.abs(o - ref)) <= 1e-10 * max(1.0, np.max(np.abs(ref)))


def test_true_oracle_passes_pins(case):
    w, bt, rows = case
    assert _attend_pin(w, bt, rows, lambda *a: oracle.attend_ref(*a)[0])
    assert _attend_pin(w, bt, rows, lambda *a: _attend_variant(*a, bug=None))
    assert _absorb_pin(w, bt, rows, lambda qn, qr, wk: oracle.absorb_q_ref(qn, qr, wk))


@pytest.mark.parametrize("bug", ["mask_off_by_one", "scale_squared", "drop_rope_term",
                                 "rope_sign", "values_from_tail"])
def test_attend_mutant_rejected(case, bug):
    w, bt, rows = case
    assert not _attend_pin(w, bt, rows, lambda *a: _attend_variant(*a, bug=bug))


@pytest.mark.parametrize("bug", ["heads_shifted", "transposed_head_block"])
def test_absorb_mutant_rejected(case, bug):
    w, bt, rows = case
    assert not _absorb_pin(w, bt, rows, lambda qn, qr, wk: _absorb_variant(qn, qr, wk, bug))


# ------------------------------------------------------------------ producer step

def _rope_variant(x, pos, bug, base=10000.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    k = np.arange(0, d, 2, dtype=np.float64)
    if bug == "angle_exponent_shifted":
        k = k + 2
    theta = base ** (-k / d)
    ang = np.asarray(pos, np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    if bug == "half_split_pairs":     # pairs (x[i], x[i + d/2]) instead of (x[2i], x[2i+1])
        x1, x2 = x[..., : d // 2], x[..., d // 2:]
        out = np.empty_like(x)
        out[..., : d // 2] = x1 * c - x2 * s
        out[..., d // 2:] = x1 * s + x2 * c
        return out
    sgn = -1.0 if bug == "rotation_sign" else 1.0
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - sgn * x2 * s
    out[..., 1::2] = sgn * x1 * s + x2 * c
    return out


def _produce_variant(bug):
    def produce(h, w_dkv, w_kr, pos):
        h = np.asarray(h, np.float64)
        if bug == "transposed_down_projection":
            w = np.asarray(w_dkv, np.float64)
            c = h @ w.reshape(w.shape[1], w.shape[0])
        else:
            c = h @ np.asarray(w_dkv, np.float64).T
        kr = h @ np.asarray(w_kr, np.float64).T
        if bug == "latent_rotated":
            c = oracle.rope_ref(c, pos)
        return np.concatenate([c, _rope_variant(kr, pos, bug)], axis=-1)
    return produce


@pytest.mark.parametrize("bug", ["transposed_down_projection", "latent_rotated",
                                 "half_split_pairs", "angle_exponent_shifted", "rotation_sign"])
def test_producer_pins_reject_planted_bug(bug):
    from test_oracle import producer_one_hot_pin, producer_position_pin, rope_angle_pin
    produce = _produce_variant(bug)
    rope = lambda x, pos: _rope_variant(x, pos, bug)
    assert not (producer_one_hot_pin(produce) and producer_position_pin(produce)
                and rope_angle_pin(rope))


def _produce_append_variant(bug):
    """produce_append_ref with one planted mistake: "step_local_positions"
    rotates token i of every step at position i instead of
    seq_lens_before[b] + i."""
    def produce_append(pool, block_table, seq_lens_before, hidden, w_dkv, w_kr, block_size):
        B, T, _ = hidden.shape
        rows = []
        for b in range(B):
            first = 0 if bug == "step_local_positions" else int(seq_lens_before[b])
            rows.append(oracle.kv_produce_ref(hidden[b], w_dkv, w_kr, first + np.arange(T)))
        return oracle.append_ref(pool, block_table, seq_lens_before, np.stack(rows), block_size)
    return produce_append


def test_producer_append_pins_reject_step_local_positions():
    from test_oracle import producer_chunking_pin, producer_self_score_pin
    bad = _produce_append_variant("step_local_positions")
    assert not producer_chunking_pin(bad)
    assert not producer_self_score_pin(bad)


def test_producer_append_pins_accept_the_unmutated_variant():
    from test_oracle import producer_chunking_pin, producer_self_score_pin
    good = _produce_append_variant("none")
    assert producer_chunking_pin(good) and producer_self_score_pin(good)


def test_producer_pins_accept_the_unmutated_variant():
    from test_oracle import producer_one_hot_pin, producer_position_pin, rope_angle_pin
    produce = _produce_variant("none")
    rope = lambda x, pos: _rope_variant(x, pos, "none")
    assert producer_one_hot_pin(produce) and producer_position_pin(produce) and rope_angle_pin(rope)


# ------------------------------------------------------------------ output side

def _o_proj_variant(bug):
    def o_proj(attn, w_o):
        a = np.asarray(attn, np.float64)
        M, H, d_v = a.shape
        if bug == "value_major_concat":   # heads interleaved: x[v*H + h]
            x = a.transpose(0, 2, 1).reshape(M, -1)
        else:
            x = a.reshape(M, -1)
        w = np.asarray(w_o, np.float64)
        if bug == "transposed_weight":    # W^O read as stored [H*d_v, d]
            return x @ w.reshape(w.shape[1], w.shape[0])
        return x @ w.T
    return o_proj


def _fold_variant(bug):
    def fold(w_uv, w_o):
        wv = np.asarray(w_uv, np.float64)
        H, d_v, d_c = wv.shape
        wo = np.asarray(w_o, np.float64)
        d = wo.shape[0]
        if bug == "heads_reversed":
            wv = wv[::-1]
        if bug == "value_major_blocks":   # W^O's columns read as v*H + h
            wo = wo.reshape(d, d_v, H).transpose(0, 2, 1).reshape(d, H * d_v)
        if bug == "uv_block_transposed":  # W^UV[h] read as if stored [d_c, d_v]
            wv = wv.reshape(H, d_c, d_v).transpose(0, 2, 1)
        out = np.empty((d, H * d_c))
        for h in range(H):
            out[:, h * d_c:(h + 1) * d_c] = wo[:, h * d_v:(h + 1) * d_v] @ wv[h]
        return out
    return fold


def _o_proj_folded_variant(bug):
    def folded(o_lat, w_fold):
        z = np.asarray(o_lat, np.float64)
        M, H, d_c = z.shape
        x = z.transpose(0, 2, 1).reshape(M, -1) if bug == "latent_value_major" else z.reshape(M, -1)
        return x @ np.asarray(w_fold, np.float64).T
    return folded


@pytest.mark.parametrize("bug", ["value_major_concat", "transposed_weight"])
def test_o_proj_pin_rejects_planted_bug(bug):
    from test_oracle import o_proj_linear_pin
    assert not o_proj_linear_pin(_o_proj_variant(bug))


@pytest.mark.parametrize("bug", ["heads_reversed", "value_major_blocks", "uv_block_transposed",
                                 "latent_value_major"])
def test_fold_pins_reject_planted_bug(bug):
    from test_oracle import fold_equals_full_path_pin, fold_one_hot_pin
    fold, folded = _fold_variant(bug), _o_proj_folded_variant(bug)
    assert not (fold_one_hot_pin(fold) and fold_equals_full_path_pin(fold, folded))


def test_output_side_pins_accept_the_unmutated_variants():
    from test_oracle import fold_equals_full_path_pin, fold_one_hot_pin, o_proj_linear_pin
    assert o_proj_linear_pin(_o_proj_variant("none"))
    fold, folded = _fold_variant("none"), _o_proj_folded_variant("none")
    assert fold_one_hot_pin(fold) and fold_equals_full_path_pin(fold, folded)
