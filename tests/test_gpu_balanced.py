"""The balanced split plan of mla_decode (the library's choice for the MFMA
kernel when the sequence lengths may differ).

Work item k of each 64-row group takes one contiguous range of one sequence;
each sequence gets splits in proportion to its length, so that no item holds
more than C units of 32 rows, C as small as the K = 256 / G items allow (and
at least 8).  The plan is computed on the device from seq_lens and written to
the workspace as a per-sequence table (first item, split count, units per
split) for the merge kernel.

* the table equals the plan re-derived here from the lengths (integers:
  bit-exact), and no item holds more than C units;
* outputs match the fp64 oracle for length mixes with empty, one-row,
  page-edge and long sequences, causal multi-token queries, and more
  sequences than one split each;
* the plain plan (an explicit split count) on the same inputs agrees.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_36_amd import binding as mla
from workloads import V2_MULTI, V3, make_inputs
from workloads.device import to_dev, torch_dtype

from gpu_util import cfg_of, max_err_ratio, note, oracle_decode, oracle_pool_after

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def _r256(x: int) -> int:
    return -(-x // 256) * 256


def plan_ref(n_rows, K, min_units=8):
    """The balanced plan from the rows each sequence's last token sees."""
    U = [(int(n) + 31) // 32 for n in n_rows]
    cnt = lambda C: sum(0 if u == 0 else -(-u // C) for u in U)
    lo = max(min_units, -(-sum(U) // K))
    hi = max(lo, max(U))
    while lo < hi:
        mid = (lo + hi) // 2
        if cnt(mid) <= K:
            hi = mid
        else:
            lo = mid + 1
    C = lo
    S = [0 if u == 0 else -(-u // C) for u in U]
    ch = [0 if s == 0 else -(-u // s) for u, s in zip(U, S)]
    P = list(np.concatenate([[0], np.cumsum(S)[:-1]]).astype(int))
    return C, P, S, ch


def _run(w, bt, pool_after, seq_lens, total_tokens_host=0, num_splits=0):
    cfg = cfg_of(w)
    dt = torch_dtype(bt)
    B, T = bt.q_abs.shape[:2]
    cap = int(seq_lens.max())
    pool = to_dev(pool_after, dt, "cuda")
    tbl = torch.from_numpy(bt.block_table).cuda()
    sl = torch.from_numpy(seq_lens.astype(np.int32)).cuda()
    q = to_dev(bt.q_abs, dt, "cuda")
    o = torch.full((B, T, w.H, w.d_c), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, T, w.H), float("nan"), dtype=torch.float32, device="cuda")
    n = mla.mla_decode_workspace_size(cfg, B, T, cap, total_tokens_host, num_splits)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    mla.mla_decode(cfg, q, pool, tbl, sl, cap, o, lse, causal=w.causal, num_splits=num_splits,
                   total_tokens_host=total_tokens_host, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), ws


def _check(bt, pool_after, seq_lens, o, lse):
    bt.seq_lens = seq_lens
    o_ref, lse_ref = oracle_decode(bt, pool_after, bt.q_abs)
    assert max_err_ratio(o, o_ref) <= 2e-2
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    if fin.any():
        assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= 1e-3
    empty = seq_lens == 0
    if empty.any():
        assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))


CASES = {
    # empty, one row, page and unit edges, and long sequences in one batch
    "edges": (V3.scaled(name="bal_edges", seed=9100, B=12, N=2000, var_len=True, table="permuted"),
              [0, 1, 31, 32, 33, 64, 65, 700, 2001, 1500, 3, 1999]),
    # drawn lengths, permuted pages
    "drawn": (V3.scaled(name="bal_drawn", seed=9101, B=20, N=3000, var_len=True,
                        table="permuted"), None),
    # causal multi-token queries (G = 8 groups, K = 32 items per group)
    "multi_token": (V2_MULTI.scaled(name="bal_multi", seed=9102, B=6, N=900, var_len=True), None),
    # 80 heads and 3 causal tokens: each token's second 64-row group is
    # partial (G = 6 groups, K = 42 items per group)
    "partial_groups": (V3.scaled(name="bal_h80", seed=9103, B=7, T=3, H=80, N=1100,
                                 var_len=True, causal=True, table="permuted"), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_balanced_plan_matches_oracle_and_table(name):
    w, lens = CASES[name]
    bt = make_inputs(w)
    pool_after = oracle_pool_after(bt)
    seq_lens = bt.seq_lens.copy()
    if lens is not None:
        seq_lens = np.minimum(np.array(lens, dtype=np.int32), seq_lens)
    note(f"balanced {name}: seq_lens={seq_lens.tolist()}")
    cfg = cfg_of(w)
    B, T = bt.q_abs.shape[:2]
    cap = int(seq_lens.max())
    K = 256 // (T * -(-w.H // 64))  # 64-row groups: ceil(H / 64) per new token
    assert K > B and mla.mla_decode_num_splits(cfg, B, T, cap, 0) == K
    o, lse, ws = _run(w, bt, pool_after, seq_lens)
    # the table in the workspace tail, after the bf16 partial outputs and the
    # fp32 partial log-sum-exps: (P_b, S_b, ch_b) per sequence
    rows = K * T * w.H
    off = _r256(rows * w.d_c * 2) + _r256(rows * 4)
    table = ws[off:off + 16 * B].cpu().numpy().view(np.int32).reshape(B, 4)[:, :3]
    C, P, S, ch = plan_ref(np.minimum(seq_lens, cap), K)
    assert table[:, 0].tolist() == P
    assert table[:, 1].tolist() == S
    assert table[:, 2].tolist() == ch
    assert sum(S) <= K and max(ch) <= C
    _check(bt, pool_after, seq_lens, o, lse)


def test_many_short_sequences():
    """More sequences than the plain plan would split: 100 sequences of 1 .. 64
    rows, K = 128 items, one split each."""
    w = V3.scaled(name="bal_short", seed=9103, B=100, N=64, var_len=True)
    bt = make_inputs(w)
    pool_after = oracle_pool_after(bt)
    note("balanced: 100 short sequences")
    o, lse, _ = _run(w, bt, pool_after, bt.seq_lens.copy())
    _check(bt, pool_after, bt.seq_lens.copy(), o, lse)


def test_balanced_and_plain_plans_agree():
    """The same varlen batch through the balanced plan and a plain plan of 6
    splits: both within the bf16 bound of the oracle and of each other."""
    w = V3.scaled(name="bal_vs_plain", seed=9104, B=10, N=2500, var_len=True, table="permuted")
    bt = make_inputs(w)
    pool_after = oracle_pool_after(bt)
    note("balanced vs plain")
    o_b, lse_b, _ = _run(w, bt, pool_after, bt.seq_lens.copy())
    o_p, lse_p, _ = _run(w, bt, pool_after, bt.seq_lens.copy(), num_splits=6)
    _check(bt, pool_after, bt.seq_lens.copy(), o_b, lse_b)
    _check(bt, pool_after, bt.seq_lens.copy(), o_p, lse_p)
    assert max_err_ratio(o_b, o_p) <= 2e-2
