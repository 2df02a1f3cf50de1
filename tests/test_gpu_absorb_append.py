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


@pytest.mark.parametrize("M", [70, 200])
def test_projections_two_tiles_per_workgroup(M):
    """65 .. 256 query rows: each workgroup of mla_absorb_q and mla_out_proj
    takes two 16-row tiles (the second ragged or absent in the last
    workgroup).  Against the fp64 oracle: q_abs within bf16 rounding of each
    element plus an fp32-accumulation floor, out within 2e-2 of max|out|."""
    import oracle
    from workloads import V2_MULTI
    from workloads.device import to_dev
    w = V2_MULTI.scaled(B=M, T=1, N=64)
    bt = make_inputs(w)
    cfg = cfg_of(w)
    note(f"projections with {M} query rows")
    qn = to_dev(bt.q_nope.reshape(M, w.H, -1), torch.bfloat16, "cuda")
    qr = to_dev(bt.q_rope.reshape(M, w.H, -1), torch.bfloat16, "cuda")
    q_abs = torch.empty((M, w.H, w.d_c + w.d_r), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(cfg, qn, qr, to_dev(bt.w_uk, torch.bfloat16, "cuda"), q_abs)
    o_lat = np.random.default_rng(5).standard_normal((M, w.H, w.d_c)).astype(np.float32)
    out = torch.empty((M, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
    mla.mla_out_proj(cfg, torch.from_numpy(o_lat).cuda(), to_dev(bt.w_uv, torch.bfloat16, "cuda"), out)
    torch.cuda.synchronize()
    want = oracle.absorb_q_ref(bt.q_nope.reshape(M, w.H, -1), bt.q_rope.reshape(M, w.H, -1), bt.w_uk)
    got = q_abs.float().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(want) + 1e-4 * np.max(np.abs(want))
    assert np.all(np.abs(got - want) <= bound)
    want_o = oracle.out_proj_ref(o_lat, bt.w_uv)
    got_o = out.float().cpu().numpy()
    assert np.max(np.abs(got_o - want_o)) <= 2e-2 * np.max(np.abs(want_o))
