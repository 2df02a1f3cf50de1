"""mla_absorb_q_append (the absorb and the cache append of one step in one
call) against the two separate calls on the same inputs: q_abs and the whole
pool bit for bit (both are exact copies of the same kernels' arithmetic or
pure data movement), on the fused MFMA launch (bf16) and on the fallback
(fp32), with row counts that leave the last append workgroup partly idle, and
with pages that are out of the table's range (skipped by both)."""
import numpy as np
import pytest
import torch

from mla_latent_kv_36_amd import binding as mla
from workloads import TINY, V3, make_inputs
from workloads.device import upload

from gpu_util import cfg_of, dev_bits, note

pytestmark = pytest.mark.gpu

CASES = {
    "v3_fused": V3.scaled(B=3, N=200, table="permuted"),      # 3 rows: one partly idle workgroup
    "v3_fused_multi": V3.scaled(B=5, T=3, N=130),               # 15 rows, T_new = 3
    "tiny_f32_fallback": TINY.scaled(B=2, T=2),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def _run(w, fused):
    bt = make_inputs(w)
    dev = upload(bt)
    cfg = cfg_of(w)
    M = w.B * w.T
    q_abs = torch.zeros((M, w.H, w.d_c + w.d_r), dtype=dev["q_nope"].dtype, device="cuda")
    lengths = torch.from_numpy(bt.lengths.astype(np.int32)).cuda()
    cap = int(bt.seq_lens.max())
    qn = dev["q_nope"].view(M, w.H, -1)
    qr = dev["q_rope"].view(M, w.H, -1)
    if fused:
        mla.mla_absorb_q_append(cfg, qn, qr, dev["w_uk"], q_abs, dev["pool"], dev["block_table"],
                                lengths, dev["new_rows"], cap)
    else:
        mla.mla_absorb_q(cfg, qn, qr, dev["w_uk"], q_abs)
        mla.mla_cache_append(cfg, dev["pool"], dev["block_table"], lengths, dev["new_rows"], cap)
    torch.cuda.synchronize()
    return dev_bits(q_abs), dev_bits(dev["pool"])


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_separate_calls(name):
    w = CASES[name]
    note(f"absorb_q_append {name}")
    qa_f, pool_f = _run(w, True)
    qa_s, pool_s = _run(w, False)
    assert np.array_equal(qa_f, qa_s)
    assert np.array_equal(pool_f, pool_s)


def test_fused_skips_rows_outside_the_table():
    """Sequence 1's new row falls on a page the table does not have (its length
    reaches the table's end): both paths skip it and write everything else."""
    w = V3.scaled(B=3, N=128)
    bt = make_inputs(w)
    dev = upload(bt)
    cfg = cfg_of(w)
    lengths = torch.from_numpy(bt.lengths.astype(np.int32)).cuda()
    lengths[1] = bt.block_table.shape[1] * w.block_size   # position past the last page
    note("absorb_q_append: row outside the table")
    pools = []
    for fused in (True, False):
        pool = dev["pool"].clone()
        q_abs = torch.zeros((w.B, w.H, w.d_c + w.d_r), dtype=pool.dtype, device="cuda")
        qn, qr = dev["q_nope"].view(w.B, w.H, -1), dev["q_rope"].view(w.B, w.H, -1)
        cap = bt.block_table.shape[1] * w.block_size
        if fused:
            mla.mla_absorb_q_append(cfg, qn, qr, dev["w_uk"], q_abs, pool, dev["block_table"],
                                    lengths, dev["new_rows"], cap)
        else:
            mla.mla_absorb_q(cfg, qn, qr, dev["w_uk"], q_abs)
            mla.mla_cache_append(cfg, pool, dev["block_table"], lengths, dev["new_rows"], cap)
        torch.cuda.synchronize()
        pools.append(dev_bits(pool))
    assert np.array_equal(pools[0], pools[1])
    assert not np.array_equal(pools[0], dev_bits(dev["pool"]))   # the other rows were written
