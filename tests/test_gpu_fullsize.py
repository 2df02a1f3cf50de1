"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the library's own split plan, one whole decode step), checked
on outputs the oracle can compute one by one: every sequence where that is
cheap, else a sample of sequences or heads chosen up front."""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_36_amd import binding as mla
from workloads import LONG, PREFILL, V2_MULTI, V3, VARLEN, make_inputs
from workloads.device import upload

from gpu_util import (dev_bits, make_step, max_err_ratio, note, oracle_pool_after,
                      pool_bits, tol_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def _check_step(w, seqs, heads=None, num_splits=0):
    bt = make_inputs(w)
    note(f"full-size step {w.name} splits={num_splits}")
    dev = upload(bt)
    step = make_step(bt, dev, num_splits=num_splits)
    step.run()
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else heads
    o_lat = step.o_lat.cpu().numpy()
    lse = step.lse.cpu().numpy()
    out = step.out.float().cpu().numpy().reshape(w.B, w.T, w.H, w.d_v)
    q_abs = step.q_abs.float().cpu().numpy()
    pool_after = oracle_pool_after(bt)
    tol = tol_of(w)
    for b in seqs:
        rows = oracle.gather_rows_ref(pool_after, bt.block_table, b, int(bt.seq_lens[b]),
                                      w.block_size)
        qa = oracle.absorb_q_ref(bt.q_nope[b][:, hs], bt.q_rope[b][:, hs], bt.w_uk[hs])
        o_ref, lse_ref = oracle.attend_ref(qa, rows, w.d_c, w.scale, w.causal)
        out_ref = oracle.out_proj_ref(o_ref, bt.w_uv[hs])
        assert max_err_ratio(q_abs[b][:, hs], qa) <= tol, f"q_abs seq {b}"
        assert max_err_ratio(o_lat[b][:, hs], o_ref) <= tol, f"o_lat seq {b}"
        assert max_err_ratio(out[b][:, hs], out_ref) <= tol, f"out seq {b}"
        assert np.max(np.abs(lse[b][:, hs] - lse_ref)) <= 5e-2, f"lse seq {b}"
    # the appended rows landed bit-exactly, nothing else moved
    assert np.array_equal(dev_bits(dev["pool"]), pool_bits(pool_after, w.dtype))
    return step


def test_v3_decode_full():
    """16 sequences x 4,096 cached rows (+1 appended): every output checked."""
    _check_step(V3, seqs=range(V3.B))


def test_varlen_serving_full():
    """64 sequences of 1..32,768 rows, permuted pages: the shortest, the longest
    and three more sequences drawn with a fixed seed, every head."""
    bt = make_inputs(VARLEN, with_rows=False)
    order = np.argsort(bt.lengths)
    pick = np.random.default_rng(123).choice(VARLEN.B, 3, replace=False)
    seqs = sorted({int(order[0]), int(order[-1]), *map(int, pick)})
    _check_step(VARLEN, seqs=seqs)


@pytest.mark.parametrize("num_splits", [0, 64])
def test_long_context_full(num_splits):
    """4 sequences x 131,072 rows with 1% of rows x8; 64 splits per sequence is
    256 partitions in all.  Eight heads per sequence, chosen up front."""
    heads = [0, 17, 38, 63, 64, 90, 101, 127]
    _check_step(LONG, seqs=range(LONG.B), heads=heads, num_splits=num_splits)


def test_v2_multi_token_full():
    """32 sequences x (8,192 + 4) rows, 4 causal queries each: four sequences."""
    _check_step(V2_MULTI, seqs=[0, 9, 22, 31])


def test_prefill_chunk_full():
    """4 sequences x (3,584 + 512) rows, 512 causal queries each (a prefill
    chunk through the absorbed path): every sequence, six heads chosen up front,
    all 512 queries."""
    heads = [0, 31, 64, 77, 100, 127]
    _check_step(PREFILL, seqs=range(PREFILL.B), heads=heads)

