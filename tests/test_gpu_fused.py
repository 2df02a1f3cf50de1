"""mla_decode_fused: split-KV decode and its log-sum-exp merge in one launch
(persistent workgroups, an on-device work queue, and merges handed out by the
last split to arrive in each 64-row group).

* Under a plain plan with more than one split, the fused call computes the
  same bf16 partials as mla_decode and merges them with the same arithmetic
  in the same split order: o_lat and lse equal mla_decode's bit for bit.
* Every case matches the fp64 oracle within the bf16 bound (balanced plans,
  whose one-split sequences are written directly, included).
* More work items than workgroups (the queue hands out several per
  workgroup), more than 8 splits per sequence (the merge's long form), empty
  sequences, multi-token causal queries and partial head groups.
* The counter region is zero after every call, and the error word stays 0;
  one workspace serves calls of different shapes in a row.
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


def _inputs(w, lens=None):
    bt = make_inputs(w)
    pool_after = oracle_pool_after(bt)
    seq_lens = bt.seq_lens.copy()
    if lens is not None:
        seq_lens = np.minimum(np.array(lens, dtype=np.int32), seq_lens)
    bt.seq_lens = seq_lens
    return bt, pool_after


def _dev_args(bt, pool_after):
    dt = torch_dtype(bt)
    return (to_dev(bt.q_abs, dt, "cuda"), to_dev(pool_after, dt, "cuda"),
            torch.from_numpy(bt.block_table).cuda(),
            torch.from_numpy(bt.seq_lens.astype(np.int32)).cuda())


def _outs(w, B, T):
    o = torch.full((B, T, w.H, w.d_c), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, T, w.H), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def _fused(w, bt, args, ws, num_splits=0, total=None):
    cfg = cfg_of(w)
    B, T = bt.q_abs.shape[:2]
    cap = int(bt.seq_lens.max())
    total = int(bt.seq_lens.sum()) if total is None else total
    need = mla.mla_decode_fused_workspace_size(cfg, B, T, cap, total, num_splits)
    assert ws.numel() >= need
    o, lse = _outs(w, B, T)
    q, pool, tbl, sl = args
    mla.mla_decode_fused(cfg, q, pool, tbl, sl, cap, o, lse, workspace=ws, causal=w.causal,
                         num_splits=num_splits, total_tokens_host=total)
    torch.cuda.synchronize()
    counters = ws[:mla.mla_decode_fused_counter_bytes()]
    assert int(torch.count_nonzero(counters)) == 0, "counters not left zero"
    return o.cpu().numpy(), lse.cpu().numpy()


def _two_kernel(w, bt, args, num_splits, total=None):
    cfg = cfg_of(w)
    B, T = bt.q_abs.shape[:2]
    cap = int(bt.seq_lens.max())
    total = int(bt.seq_lens.sum()) if total is None else total
    n = mla.mla_decode_workspace_size(cfg, B, T, cap, total, num_splits)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    o, lse = _outs(w, B, T)
    q, pool, tbl, sl = args
    mla.mla_decode(cfg, q, pool, tbl, sl, cap, o, lse, causal=w.causal, num_splits=num_splits,
                   total_tokens_host=total, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _workspace(nbytes):
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")


def _r256(x: int) -> int:
    return -(-x // 256) * 256


def plan_ref_min_one(n_rows, K, min_units=8):
    """The balanced plan of the one-launch call: as mla_decode's, except that a
    sequence with no visible row gets one (empty) split, which writes its
    zero output."""
    U = [(int(n) + 31) // 32 for n in n_rows]
    cnt = lambda C: sum(1 if u == 0 else -(-u // C) for u in U)
    lo = max(min_units, -(-sum(U) // K))
    hi = max(lo, max(U))
    while lo < hi:
        mid = (lo + hi) // 2
        if cnt(mid) <= K:
            hi = mid
        else:
            lo = mid + 1
    C = lo
    S = [1 if u == 0 else -(-u // C) for u in U]
    ch = [-(-u // s) for u, s in zip(U, S)]
    P = list(np.concatenate([[0], np.cumsum(S)[:-1]]).astype(int))
    return C, P, S, ch


def _check_oracle(bt, pool_after, o, lse):
    o_ref, lse_ref = oracle_decode(bt, pool_after, bt.q_abs)
    assert max_err_ratio(o, o_ref) <= 2e-2
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    if fin.any():
        assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= 1e-3
    empty = bt.seq_lens == 0
    if empty.any():
        assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))


# (workload, lengths or None, num_splits, total_tokens_host or None = the sum)
CASES = {
    # equal lengths: the plain plan, 8 splits, one item per workgroup
    "plain_equal": (V3.scaled(name="fz_eq", seed=9200, B=4, N=2048), None, 0, None),
    # 32 splits of 4 units: 512 items over at most 256 workgroups (the queue
    # hands out the rest) and merges of more than 8 splits
    "queue_32_splits": (V3.scaled(name="fz_q", seed=9201, B=8, N=4096, table="permuted"),
                        None, 40, None),
    # balanced plan: empty, one-row, page-edge and long sequences
    "balanced_edges": (V3.scaled(name="fz_edges", seed=9202, B=12, N=2000, var_len=True,
                                 table="permuted"),
                       [0, 1, 31, 32, 33, 64, 65, 700, 2001, 1500, 3, 1999], 0, 0),
    # causal 4-token queries (G = 8 groups per sequence), balanced
    "multi_token": (V2_MULTI.scaled(name="fz_multi", seed=9203, B=6, N=900, var_len=True),
                    None, 0, 0),
    # 80 heads, 3 causal tokens: partial head groups, plain plan of 5 splits
    "partial_groups": (V3.scaled(name="fz_h80", seed=9204, B=5, T=3, H=80, N=1100,
                                 causal=True, table="permuted"), None, 5, None),
    # one split: every item writes its output directly
    "one_split": (V3.scaled(name="fz_one", seed=9205, B=6, N=600), None, 1, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_oracle(name):
    w, lens, ns, total = CASES[name]
    bt, pool_after = _inputs(w, lens)
    note(f"fused {name}: seq_lens={bt.seq_lens.tolist()} num_splits={ns}")
    cfg = cfg_of(w)
    B, T = bt.q_abs.shape[:2]
    cap = int(bt.seq_lens.max())
    tot = int(bt.seq_lens.sum()) if total is None else total
    ws = _workspace(mla.mla_decode_fused_workspace_size(cfg, B, T, cap, tot, ns))
    args = _dev_args(bt, pool_after)
    o, lse = _fused(w, bt, args, ws, ns, tot)
    _check_oracle(bt, pool_after, o, lse)
    err = ws[512:516].cpu().numpy().view(np.uint32)[0]
    assert err == 0
    K = mla.mla_decode_num_splits(cfg, B, T, cap, tot)
    if ns == 0 and tot < B * cap and K > B:
        # balanced: the per-sequence table after the counter region and the
        # per-group records, (P_b, S_b, ch_b) per sequence
        G = T * -(-w.H // 64)
        off = mla.mla_decode_fused_counter_bytes() + _r256(8 * B * G)
        table = ws[off:off + 16 * B].cpu().numpy().view(np.int32).reshape(B, 4)[:, :3]
        C, P, S, ch = plan_ref_min_one(np.minimum(bt.seq_lens, cap), K)
        assert table[:, 0].tolist() == P
        assert table[:, 1].tolist() == S
        assert table[:, 2].tolist() == ch
        assert sum(S) <= K and max(ch) <= C


@pytest.mark.parametrize("name", ["plain_equal", "queue_32_splits", "partial_groups"])
def test_fused_equals_two_kernel_bitwise(name):
    """A plain plan with several splits: the same partials, merged the same
    way, so the two calls agree bit for bit."""
    w, lens, ns, total = CASES[name]
    bt, pool_after = _inputs(w, lens)
    note(f"fused vs two-kernel {name}")
    cfg = cfg_of(w)
    B, T = bt.q_abs.shape[:2]
    cap = int(bt.seq_lens.max())
    tot = int(bt.seq_lens.sum())
    splits = ns if ns > 0 else mla.mla_decode_num_splits(cfg, B, T, cap, tot)
    assert splits > 1
    args = _dev_args(bt, pool_after)
    ws = _workspace(mla.mla_decode_fused_workspace_size(cfg, B, T, cap, tot, splits))
    o_f, lse_f = _fused(w, bt, args, ws, splits, tot)
    o_t, lse_t = _two_kernel(w, bt, args, splits, tot)
    assert np.array_equal(o_f.view(np.uint32), o_t.view(np.uint32))
    assert np.array_equal(lse_f.view(np.uint32), lse_t.view(np.uint32))


def test_fused_workspace_reused_across_shapes():
    """One zeroed workspace, three calls in a row: a large plain plan, a
    smaller balanced batch, then the first again (bit-identical to its first
    run)."""
    w1, _, ns1, _ = CASES["queue_32_splits"]
    w2, lens2, _, _ = CASES["balanced_edges"]
    bt1, pa1 = _inputs(w1)
    bt2, pa2 = _inputs(w2, lens2)
    cfg1, cfg2 = cfg_of(w1), cfg_of(w2)
    n1 = mla.mla_decode_fused_workspace_size(cfg1, bt1.q_abs.shape[0], 1, int(bt1.seq_lens.max()),
                                             int(bt1.seq_lens.sum()), ns1)
    n2 = mla.mla_decode_fused_workspace_size(cfg2, bt2.q_abs.shape[0], 1, int(bt2.seq_lens.max()),
                                             0, 0)
    ws = _workspace(max(n1, n2))
    note("fused reuse: large plain plan")
    a1 = _dev_args(bt1, pa1)
    o1, lse1 = _fused(w1, bt1, a1, ws, ns1)
    note("fused reuse: smaller balanced batch")
    o2, lse2 = _fused(w2, bt2, _dev_args(bt2, pa2), ws, 0, 0)
    _check_oracle(bt2, pa2, o2, lse2)
    note("fused reuse: the first again")
    o3, lse3 = _fused(w1, bt1, a1, ws, ns1)
    assert np.array_equal(o1.view(np.uint32), o3.view(np.uint32))
    assert np.array_equal(lse1.view(np.uint32), lse3.view(np.uint32))
    _check_oracle(bt1, pa1, o1, lse1)


def test_fused_all_empty():
    """Every sequence empty under a balanced plan: one (empty) item each,
    o = 0 and lse = -inf everywhere."""
    w = V3.scaled(name="fz_empty", seed=9206, B=5, N=300, var_len=True)
    bt, pool_after = _inputs(w, [0, 0, 0, 0, 0])
    note("fused all empty")
    cfg = cfg_of(w)
    cap = bt.block_table.shape[1] * w.block_size  # what the table could hold
    ws = _workspace(mla.mla_decode_fused_workspace_size(cfg, 5, 1, cap, 0, 0))
    q, pool, tbl, sl = _dev_args(bt, pool_after)
    o, lse = _outs(w, 5, 1)
    mla.mla_decode_fused(cfg, q, pool, tbl, sl, cap, o, lse, workspace=ws, causal=w.causal,
                         num_splits=0, total_tokens_host=0)
    torch.cuda.synchronize()
    assert torch.all(o == 0.0) and torch.all(torch.isneginf(lse))
    assert int(torch.count_nonzero(ws[:mla.mla_decode_fused_counter_bytes()])) == 0
