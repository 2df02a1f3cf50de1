"""The C ABI on the host: the library loads without a GPU, exports every call
the header declares, and rejects bad arguments before launching anything.

No test here reaches a kernel launch: every call either fails validation or
has nothing to launch, so these run on a machine without a GPU.  Device
pointers are stand-in addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import mla_latent_kv_36_amd as mla
from mla_latent_kv_36_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, DIM, DTYPE, CAP, WS, HIP, ALIGN = range(8)
FAKE = 0x10000          # aligned stand-in device address (never dereferenced)
FAKE_MIS = 0x10008      # misaligned stand-in


@pytest.fixture(scope="module")
def lib():
    from mla_latent_kv_36_amd import build
    if not build.built():
        build.build()
    return mla.load()


def v3_cfg(**kw):
    d = dict(n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128, block_size=64,
             softmax_scale=0.0, dtype="bf16")
    d.update(kw)
    return mla.make_config(**d)


def test_header_symbols_are_exported(lib):
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    names = set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text))
    assert {"mla_absorb_q", "mla_cache_append", "mla_decode", "mla_out_proj"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/mla.h but not exported"
    # the binding wraps every declared call under the same name
    for n in names:
        assert hasattr(binding, n), f"binding lacks {n}"


def test_status_strings(lib):
    for code in range(8):
        s = mla.mla_status_string(code)
        assert s.startswith("MLA_")
    assert "unknown" in mla.mla_status_string(99)
    assert mla.mla_abi_version() == 2


def _decode(lib, cfg, q=FAKE, pool=FAKE, nb=10, bt=FAKE, mb=4, sl=FAKE, cap=256, B=2, T=1,
            causal=1, ns=0, tot=0, ws=None, wsb=0, o=FAKE, lse=None):
    return lib.mla_decode(ctypes.byref(cfg) if cfg is not None else None, q, pool, nb, bt, mb,
                          sl, cap, B, T, causal, ns, tot, ws, wsb, o, lse, None)


def test_decode_validation(lib):
    cfg = v3_cfg()
    assert _decode(lib, None) == NULL
    assert _decode(lib, v3_cfg(dtype=7)) == DTYPE
    assert _decode(lib, v3_cfg(n_heads=0)) == DIM
    assert _decode(lib, v3_cfg(block_size=0)) == DIM
    assert _decode(lib, v3_cfg(softmax_scale=-1.0)) == DIM
    assert _decode(lib, v3_cfg(softmax_scale=float("nan"))) == DIM
    assert _decode(lib, cfg, T=0) == DIM
    assert _decode(lib, cfg, causal=2) == DIM
    assert _decode(lib, cfg, ns=-1) == DIM
    assert _decode(lib, cfg, nb=0) == DIM
    assert _decode(lib, cfg, cap=4 * 64 + 1) == CAP          # longer than the table holds
    assert _decode(lib, cfg, q=None) == NULL
    assert _decode(lib, cfg, o=None) == NULL
    assert _decode(lib, cfg, sl=None) == NULL
    assert _decode(lib, cfg, q=FAKE_MIS) == ALIGN
    assert _decode(lib, cfg, lse=FAKE_MIS) == ALIGN
    # a split plan needs a workspace; too small or missing is refused
    need = mla.mla_decode_workspace_size(cfg, 2, 1, 256, 0, 4)
    assert need > 0
    assert _decode(lib, cfg, ns=4) == WS
    assert _decode(lib, cfg, ns=4, ws=FAKE, wsb=need - 1) == WS
    # nothing to do: no launch, success
    assert _decode(lib, cfg, B=0) == OK


def _decode_noalloc(lib, cfg, q=FAKE, pool=FAKE, nb=10, bt=FAKE, mb=4, sl=FAKE, cap=256, B=2,
                    T=1, causal=1, ns=0, tot=0, o=FAKE, lse=None):
    return lib.mla_decode_noalloc(ctypes.byref(cfg) if cfg is not None else None, q, pool, nb,
                                  bt, mb, sl, cap, B, T, causal, ns, tot, o, lse, None)


def test_decode_noalloc_validation(lib):
    cfg = v3_cfg()
    assert binding.mla_decode_noalloc_scratch_bytes() == 64 << 20
    # the same argument checks as mla_decode, before anything else
    assert _decode_noalloc(lib, None) == NULL
    assert _decode_noalloc(lib, v3_cfg(dtype=7)) == DTYPE
    assert _decode_noalloc(lib, cfg, T=0) == DIM
    assert _decode_noalloc(lib, cfg, causal=2) == DIM
    assert _decode_noalloc(lib, cfg, cap=4 * 64 + 1) == CAP
    assert _decode_noalloc(lib, cfg, q=None) == NULL
    assert _decode_noalloc(lib, cfg, q=FAKE_MIS) == ALIGN
    assert _decode_noalloc(lib, cfg, B=0) == OK
    # an explicit split count whose partials exceed the scratch array is
    # refused with nothing launched
    B, T, cap = 40, 2, 32768
    assert mla.mla_decode_workspace_size(cfg, B, T, cap, B * cap, 64) > 64 << 20
    assert _decode_noalloc(lib, cfg, B=B, T=T, mb=512, cap=cap, ns=64, tot=B * cap) == WS


def _decode_out_proj(lib, cfg, q=FAKE, pool=FAKE, nb=10, bt=FAKE, mb=4, sl=FAKE, cap=256, B=2,
                     T=1, causal=1, ns=0, tot=0, w_uv=FAKE, ws=None, wsb=0, o=FAKE, lse=None,
                     out=FAKE):
    return lib.mla_decode_out_proj(ctypes.byref(cfg) if cfg is not None else None, q, pool, nb,
                                   bt, mb, sl, cap, B, T, causal, ns, tot, w_uv, ws, wsb, o, lse,
                                   out, None)


def test_decode_out_proj_validation(lib):
    cfg = v3_cfg()
    # mla_decode's checks
    assert _decode_out_proj(lib, None) == NULL
    assert _decode_out_proj(lib, v3_cfg(dtype=7)) == DTYPE
    assert _decode_out_proj(lib, cfg, T=0) == DIM
    assert _decode_out_proj(lib, cfg, cap=4 * 64 + 1) == CAP
    assert _decode_out_proj(lib, cfg, q=None) == NULL
    assert _decode_out_proj(lib, cfg, o=None) == NULL
    # mla_out_proj's
    assert _decode_out_proj(lib, v3_cfg(d_v=0)) == DIM
    assert _decode_out_proj(lib, cfg, w_uv=None) == NULL
    assert _decode_out_proj(lib, cfg, out=None) == NULL
    assert _decode_out_proj(lib, cfg, out=FAKE_MIS) == ALIGN
    assert _decode_out_proj(lib, cfg, w_uv=FAKE_MIS) == ALIGN
    # mla_decode's workspace
    need = mla.mla_decode_workspace_size(cfg, 2, 1, 256, 0, 4)
    assert _decode_out_proj(lib, cfg, ns=4) == WS
    assert _decode_out_proj(lib, cfg, ns=4, ws=FAKE, wsb=need - 1) == WS
    assert _decode_out_proj(lib, cfg, B=0) == OK


def _decode_fused(lib, cfg, q=FAKE, pool=FAKE, nb=10, bt=FAKE, mb=4, sl=FAKE, cap=256, B=2,
                  T=1, causal=1, ns=0, tot=0, ws=None, wsb=0, o=FAKE, lse=None):
    return lib.mla_decode_fused(ctypes.byref(cfg) if cfg is not None else None, q, pool, nb, bt,
                                mb, sl, cap, B, T, causal, ns, tot, ws, wsb, o, lse, None)


def test_decode_fused_validation(lib):
    cfg = v3_cfg()
    ctr = binding.mla_decode_fused_counter_bytes()
    assert ctr == 256 << 10
    # the same argument checks as mla_decode
    assert _decode_fused(lib, None) == NULL
    assert _decode_fused(lib, v3_cfg(dtype=7)) == DTYPE
    assert _decode_fused(lib, cfg, T=0) == DIM
    assert _decode_fused(lib, cfg, causal=2) == DIM
    assert _decode_fused(lib, cfg, cap=4 * 64 + 1) == CAP
    assert _decode_fused(lib, cfg, q=None) == NULL
    assert _decode_fused(lib, cfg, q=FAKE_MIS) == ALIGN
    # only the bf16 MFMA shape (d_c 512, d_rope 64, 64-row pages)
    for bad in (v3_cfg(dtype="f32"), v3_cfg(d_c=256), v3_cfg(d_rope=32), v3_cfg(block_size=16)):
        assert _decode_fused(lib, bad, cap=64) == DIM
        with pytest.raises(RuntimeError):
            binding.mla_decode_fused_workspace_size(bad, 2, 1, 256, 0, 0)
    # the workspace always holds the counter region, then the partials
    need = binding.mla_decode_fused_workspace_size(cfg, 2, 1, 256, 0, 1)
    assert need >= ctr
    need4 = binding.mla_decode_fused_workspace_size(cfg, 2, 1, 256, 0, 4)
    assert need4 == need + mla.mla_decode_workspace_size(cfg, 2, 1, 256, 0, 4)
    assert _decode_fused(lib, cfg, ns=4) == WS
    assert _decode_fused(lib, cfg, ns=4, ws=FAKE, wsb=need4 - 1) == WS
    assert _decode_fused(lib, cfg, ns=4, ws=FAKE_MIS, wsb=need4) == ALIGN
    # (sequence, 64-row group) pairs beyond what the counter region holds
    B_big = 4000
    with pytest.raises(RuntimeError):
        binding.mla_decode_fused_workspace_size(cfg, B_big, 1, 256, 0, 1)
    assert _decode_fused(lib, cfg, B=B_big, ws=FAKE, wsb=1 << 40) == DIM
    assert _decode_fused(lib, cfg, B=0) == OK


def test_workspace_and_split_plan(lib):
    cfg = v3_cfg()
    # one split needs no workspace
    assert mla.mla_decode_workspace_size(cfg, 16, 1, 4097, 0, 1) == 0
    # S splits of B x T x H rows: d_c bf16 values (the MFMA kernel's partials)
    # + one fp32 lse each, both rounded up to 256 B.  The MFMA kernel splits the longest sequence into ranges of whole
    # 32-row units, so S is first reduced to the number of ranges that cover it.
    for B, T, cap, S in [(16, 1, 4097, 8), (4, 1, 131073, 64), (32, 4, 8196, 3)]:
        units = -(-cap // 32)
        chunk = -(-units // S)
        s_eff = -(-units // chunk)
        rows = B * s_eff * T * 128
        r256 = lambda x: -(-x // 256) * 256
        want = r256(rows * 512 * 2) + r256(rows * 4)
        assert mla.mla_decode_workspace_size(cfg, B, T, cap, 0, S) == want
    # equal lengths (total = B x longest): the library's choice is a plain
    # plan, a valid split count, sized like that count given explicitly
    s = mla.mla_decode_num_splits(cfg, 16, 1, 4097, 16 * 4097)
    assert 1 <= s <= 129
    assert mla.mla_decode_workspace_size(cfg, 16, 1, 4097, 16 * 4097, 0) == \
        mla.mla_decode_workspace_size(cfg, 16, 1, 4097, 16 * 4097, s)
    # lengths that may differ (total unknown, or below B x longest): a balanced
    # plan of 256 / G work items per 64-row group (G = T*H/64), partials indexed
    # by work item, plus a 16-byte table entry per sequence
    r256 = lambda x: -(-x // 256) * 256
    for B, T, total in [(16, 1, 0), (64, 1, 64 * 1000), (8, 4, 0)]:
        K = 256 // (T * 128 // 64)
        assert mla.mla_decode_num_splits(cfg, B, T, 4097, total) == K
        rows = K * T * 128
        want = r256(rows * 512 * 2) + r256(rows * 4) + r256(B * 16)
        assert mla.mla_decode_workspace_size(cfg, B, T, 4097, total, 0) == want
    # no more work items than sequences: the plain plan
    assert mla.mla_decode_num_splits(cfg, 200, 1, 4097, 0) <= 129
    # more splits than 32-row units collapse to one split per unit
    assert mla.mla_decode_workspace_size(cfg, 1, 1, 32, 0, 8) == 0
    with pytest.raises(RuntimeError):
        mla.mla_decode_workspace_size(v3_cfg(d_c=0), 1, 1, 64)


def test_append_validation(lib):
    cfg = v3_cfg()
    f = lib.mla_cache_append
    c = ctypes.byref(cfg)
    assert f(c, FAKE, 10, FAKE, 4, FAKE, FAKE, 2, 1, 4 * 64 + 1, None) == CAP
    assert f(c, None, 10, FAKE, 4, FAKE, FAKE, 2, 1, 10, None) == NULL
    assert f(c, FAKE, 0, FAKE, 4, FAKE, FAKE, 2, 1, 10, None) == DIM
    assert f(c, FAKE, 10, FAKE, 4, FAKE, FAKE_MIS, 2, 1, 10, None) == ALIGN
    assert f(c, FAKE, 10, FAKE, 4, FAKE, FAKE, 2, 0, 10, None) == OK     # no new rows
    assert f(c, FAKE, 10, FAKE, 4, FAKE, FAKE, -1, 1, 10, None) == DIM


def test_absorb_and_out_proj_validation(lib):
    cfg = v3_cfg()
    c = ctypes.byref(cfg)
    assert lib.mla_absorb_q(c, None, FAKE, FAKE, FAKE, 4, None) == NULL
    assert lib.mla_absorb_q(c, FAKE, None, FAKE, FAKE, 4, None) == NULL   # d_rope > 0
    assert lib.mla_absorb_q(ctypes.byref(v3_cfg(d_nope=0)), FAKE, FAKE, FAKE, FAKE, 4,
                            None) == DIM
    assert lib.mla_absorb_q(c, FAKE, FAKE, FAKE_MIS, FAKE, 4, None) == ALIGN
    assert lib.mla_absorb_q(c, FAKE, FAKE, FAKE, FAKE, 0, None) == OK
    assert lib.mla_absorb_q(c, FAKE, FAKE, FAKE, FAKE, -1, None) == DIM
    assert lib.mla_out_proj(c, None, FAKE, FAKE, 4, None) == NULL
    assert lib.mla_out_proj(ctypes.byref(v3_cfg(d_v=0)), FAKE, FAKE, FAKE, 4, None) == DIM
    assert lib.mla_out_proj(c, FAKE, FAKE, FAKE_MIS, 4, None) == ALIGN
    assert lib.mla_out_proj(c, FAKE, FAKE, FAKE, 0, None) == OK


def test_absorb_append_validation(lib):
    """mla_absorb_q_append reports the checks of mla_absorb_q, then those of
    mla_cache_append, and launches nothing on an error."""
    c = ctypes.byref(v3_cfg())
    f = lib.mla_absorb_q_append
    args = lambda **k: [c, k.get("qn", FAKE), FAKE, FAKE, FAKE, k.get("M", 4), k.get("pool", FAKE),
                        10, FAKE, 4, FAKE, FAKE, k.get("B", 2), k.get("T", 2), k.get("cap", 10),
                        None]
    assert f(*args(qn=None)) == NULL
    assert f(*args(M=-1)) == DIM
    assert f(*args(cap=4 * 64 + 1)) == CAP
    assert f(*args(pool=None)) == NULL
    assert f(*args(pool=FAKE_MIS)) == ALIGN
    assert f(*args(B=-1)) == DIM
    assert f(*args(M=0, T=0)) == OK      # nothing to do on either side


def test_producer_and_rope_validation(lib):
    cfg = v3_cfg()
    c = ctypes.byref(cfg)
    f = lib.mla_kv_produce
    ws = lib.mla_kv_produce_workspace_size
    # workspace: the library's k split x M x (d_c + d_rope) fp32, 256-byte rounded
    need = ws(c, 4, 5120)
    assert need > 0 and need % 256 == 0 and need >= 4 * 576 * 4
    assert ws(c, 0, 5120) == 0
    assert ws(c, 4, 0) == ctypes.c_size_t(-1).value
    # fp32 configs take the generic kernel: one partial slot
    f32 = ctypes.byref(v3_cfg(dtype=0))
    assert ws(f32, 4, 5120) == -(-(4 * 576 * 4) // 256) * 256
    args = lambda **k: [k.get("cfg", c), k.get("hidden", FAKE), k.get("d", 5120),
                        k.get("w_dkv", FAKE), k.get("w_kr", FAKE), k.get("base", 0.0),
                        k.get("pool", FAKE), 10, FAKE, 4, FAKE, k.get("B", 2), k.get("T", 2),
                        k.get("cap", 10), k.get("ws", FAKE), k.get("wsb", need), None]
    assert f(*args(cap=4 * 64 + 1)) == CAP
    assert f(*args(hidden=None)) == NULL
    assert f(*args(w_kr=None)) == NULL                       # d_rope > 0 needs W^KR
    assert f(*args(pool=FAKE_MIS)) == ALIGN
    assert f(*args(d=0)) == DIM
    assert f(*args(base=-1.0)) == DIM
    assert f(*args(base=1.0)) == DIM
    assert f(*args(base=float("inf"))) == DIM
    assert f(*args(cfg=ctypes.byref(v3_cfg(d_rope=63)))) == DIM   # odd rotary width
    assert f(*args(ws=None)) == WS
    assert f(*args(wsb=need - 1)) == WS
    assert f(*args(T=0)) == OK                                  # no new tokens
    r = lib.mla_rope
    assert r(c, None, 128, FAKE, 4, 0.0, None) == NULL
    assert r(c, FAKE, 128, FAKE_MIS, 4, 0.0, None) == ALIGN
    assert r(c, FAKE, 128, FAKE, 4, -2.0, None) == DIM
    assert r(c, FAKE, -1, FAKE, 4, 0.0, None) == DIM
    assert r(c, FAKE, 128, FAKE, 0, 0.0, None) == OK
    assert r(ctypes.byref(v3_cfg(d_rope=0)), FAKE, 128, FAKE, 4, 0.0, None) == OK


def test_output_side_validation(lib):
    """mla_o_proj / mla_fold_uv_o / mla_o_proj_folded: host checks and the
    split-k workspace (a whole number of fp32 [M, d_model] partial slices; for
    the folded product's fp32 rows, after their bf16 copy of M x H*d_c)."""
    cfg = v3_cfg(d_v=40)
    c = ctypes.byref(cfg)
    ws = lib.mla_o_proj_workspace_size
    M, d = 128, 5120
    x16 = -(-(M * cfg.n_heads * cfg.d_c * 2) // 256) * 256
    for folded in (0, 1):
        need = ws(c, M, d, folded)
        parts = need - (x16 if folded else 0)
        assert parts % 256 == 0 and parts >= 2 * M * d * 4          # k is split
        assert parts % (M * d * 4) == 0
    assert ws(c, 0, d, 0) == 0
    assert ws(c, M, 0, 0) == ctypes.c_size_t(-1).value
    assert ws(ctypes.byref(v3_cfg(d_v=0)), M, d, 0) == ctypes.c_size_t(-1).value
    assert ws(ctypes.byref(v3_cfg(dtype=0)), M, d, 0) == 0          # fp32: no split
    need = ws(c, M, d, 0)
    f = lib.mla_o_proj
    assert f(c, None, FAKE, FAKE, M, d, FAKE, need, None) == NULL
    assert f(c, FAKE, FAKE, FAKE_MIS, M, d, FAKE, need, None) == ALIGN
    assert f(c, FAKE, FAKE, FAKE, M, 0, FAKE, need, None) == DIM
    assert f(c, FAKE, FAKE, FAKE, -1, d, FAKE, need, None) == DIM
    assert f(c, FAKE, FAKE, FAKE, M, d, None, 0, None) == WS
    assert f(c, FAKE, FAKE, FAKE, M, d, FAKE, need - 1, None) == WS
    assert f(c, FAKE, FAKE, FAKE, 0, d, None, 0, None) == OK
    g = lib.mla_o_proj_folded
    needf = ws(c, M, d, 1)
    assert g(c, FAKE, None, FAKE, M, d, FAKE, needf, None) == NULL
    assert g(c, FAKE, FAKE, FAKE, M, d, FAKE, needf - 1, None) == WS
    assert g(c, FAKE, FAKE, FAKE, 0, d, None, 0, None) == OK
    h = lib.mla_fold_uv_o
    assert h(c, None, FAKE, FAKE, d, None) == NULL
    assert h(c, FAKE, FAKE, FAKE_MIS, d, None) == ALIGN
    assert h(c, FAKE, FAKE, FAKE, 0, None) == DIM
    assert h(ctypes.byref(v3_cfg(d_v=257)), FAKE, FAKE, FAKE, d, None) == DIM


def test_debug_helpers_validation(lib):
    cfg = v3_cfg()
    c = ctypes.byref(cfg)
    assert lib.mla_gather_rows(c, FAKE, 10, FAKE, 4, FAKE, 2, 4 * 64 + 1, FAKE, None) == CAP
    assert lib.mla_gather_rows(c, FAKE, 10, FAKE, 4, FAKE, 2, 10, None, None) == NULL
    assert lib.mla_gather_rows(c, FAKE, 10, FAKE, 4, FAKE, 0, 10, FAKE, None) == OK
    assert lib.mla_validate_block_table(FAKE, 2, 4, FAKE, 64, 10, None, None) == NULL
    assert lib.mla_validate_block_table(FAKE, 2, 4, FAKE, 64, 10, FAKE + 2, None) == ALIGN
    assert lib.mla_validate_block_table(FAKE, 2, 0, FAKE, 64, 10, FAKE, None) == DIM
    # the streaming-read helper: checks only (bytes == 0 launches nothing)
    for mode in (0, 1):
        assert lib.mla_stream_read(FAKE, 0, FAKE, mode, None) == OK
        assert lib.mla_stream_read(None, 64, FAKE, mode, None) == NULL
        assert lib.mla_stream_read(FAKE, 64, None, mode, None) == NULL
        assert lib.mla_stream_read(FAKE, 72, FAKE, mode, None) == ALIGN
        assert lib.mla_stream_read(FAKE + 8, 64, FAKE, mode, None) == ALIGN
        assert lib.mla_stream_read(FAKE, 64, FAKE + 4, mode, None) == ALIGN
    assert lib.mla_stream_read(FAKE, 64, FAKE, 2, None) == DIM
    assert lib.mla_stream_read(FAKE, 64, FAKE, -1, None) == DIM


def test_binding_rejects_wrong_tensor_types(lib):
    import torch
    cfg = v3_cfg()
    q = torch.zeros(1, 1, 128, 576, dtype=torch.float32)   # wrong dtype for a bf16 config
    with pytest.raises(TypeError):
        mla.mla_decode(cfg, q, q, torch.zeros(1, 1, dtype=torch.int32),
                       torch.zeros(1, dtype=torch.int32), 1, q)
