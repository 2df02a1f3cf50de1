"""mla_decode_noalloc (the decode call for callers that cannot allocate)
against mla_decode, through the C ABI.

Two calls in a row on the shared scratch array, the second with a smaller
batch, each compared with mla_decode on the same inputs at the same split
choice: bit-exact (same kernels, same plan) and within the bf16 tolerance of
the oracle.  Then an explicit split count and a balanced plan (lengths that
differ), likewise.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_36_amd import binding as mla
from workloads import V3, VARLEN, make_inputs
from workloads.device import to_dev, torch_dtype

from gpu_util import cfg_of, max_err_ratio, note, oracle_decode, oracle_pool_after

pytestmark = pytest.mark.gpu
BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def _inputs(w):
    bt = make_inputs(w)
    pool_after = oracle_pool_after(bt)
    dt = torch_dtype(bt)
    dev = dict(pool=to_dev(pool_after, dt, "cuda"), q=to_dev(bt.q_abs, dt, "cuda"),
               tbl=torch.from_numpy(bt.block_table).cuda(),
               sl=torch.from_numpy(np.ascontiguousarray(bt.seq_lens, np.int32)).cuda())
    return bt, pool_after, dev


def _outs(w, B):
    o = torch.full((B, w.T, w.H, w.d_c), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, w.T, w.H), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def _pair(w, num_splits=0):
    bt, pool_after, dev = _inputs(w)
    cfg = cfg_of(w)
    cap, total = bt.max_seq_len, int(bt.seq_lens.sum())
    o_ref, lse_ref = _outs(w, w.B)
    nbytes = mla.mla_decode_workspace_size(cfg, w.B, w.T, cap, total, num_splits)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    mla.mla_decode(cfg, dev["q"], dev["pool"], dev["tbl"], dev["sl"], cap, o_ref, lse_ref,
                   causal=w.causal, num_splits=num_splits, total_tokens_host=total, workspace=ws)
    o, lse = _outs(w, w.B)
    mla.mla_decode_noalloc(cfg, dev["q"], dev["pool"], dev["tbl"], dev["sl"], cap, o, lse,
                           causal=w.causal, num_splits=num_splits, total_tokens_host=total)
    torch.cuda.synchronize()
    return bt, pool_after, o.cpu().numpy(), lse.cpu().numpy(), o_ref.cpu().numpy(), \
        lse_ref.cpu().numpy(), nbytes


def _check_oracle(bt, pool_after, o, lse):
    o_r, lse_r = oracle_decode(bt, pool_after, bt.q_abs)
    assert max_err_ratio(o, o_r) <= BF16
    assert np.max(np.abs(lse - lse_r)) <= 1e-3


def test_noalloc_matches_decode_twice_second_smaller():
    scratch = mla.mla_decode_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    for w in (V3.scaled(B=4, N=1500), V3.scaled(B=2, N=300)):
        note(f"noalloc B={w.B} N={w.N}")
        bt, pool_after, o, lse, o_ref, lse_ref, nbytes = _pair(w)
        assert 0 < nbytes <= scratch          # the plan merges splits
        assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
        _check_oracle(bt, pool_after, o, lse)


def test_noalloc_explicit_splits_and_balanced_plan():
    # an explicit split count, then a balanced plan (lengths that differ)
    note("noalloc explicit splits")
    w = V3.scaled(B=3, N=700)
    bt, pool_after, o, lse, o_ref, lse_ref, _ = _pair(w, num_splits=5)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    _check_oracle(bt, pool_after, o, lse)
    note("noalloc balanced plan")
    w = VARLEN.scaled(B=5, N=900)
    bt, pool_after, o, lse, o_ref, lse_ref, _ = _pair(w)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    _check_oracle(bt, pool_after, o, lse)
