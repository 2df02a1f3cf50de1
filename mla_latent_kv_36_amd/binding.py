"""Python binding of libmla: the C ABI calls under the same names, taking
torch tensors for device buffers.

Argument marshalling only: each wrapper checks that tensors are contiguous and
of the element type the call expects, passes their device addresses and the
current HIP stream to the C function, and raises ``RuntimeError`` with the
library's message on an error status.  Every step of the computation runs in
the library's HIP kernels.  If ``libmla.so`` is missing, loading fails loudly:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY names another build of the same library to load instead (the
# sanitizer build of the host code, for instance)
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_HERE, "libmla.so")

MLA_F32 = 0
MLA_BF16 = 1
_TORCH_DTYPE = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


class MlaConfig(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


def make_config(n_heads: int, d_c: int, d_rope: int, d_nope: int, d_v: int,
                block_size: int = 64, softmax_scale: float = 0.0,
                dtype: str | int = "bf16") -> MlaConfig:
    if isinstance(dtype, str):
        dtype = {"f32": MLA_F32, "bf16": MLA_BF16}[dtype]
    return MlaConfig(n_heads, d_c, d_rope, d_nope, d_v, block_size, softmax_scale, dtype)


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_CFG = ctypes.POINTER(MlaConfig)
_SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_abi_version": (_I, []),
    "mla_absorb_q": (_I, [_CFG, _P, _P, _P, _P, _I, _P]),
    "mla_cache_append": (_I, [_CFG, _P, _I, _P, _I, _P, _P, _I, _I, _I, _P]),
    "mla_absorb_q_append": (_I, [_CFG, _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _I, _I,
                                 _P]),
    "mla_decode_num_splits": (_I, [_CFG, _I, _I, _I, ctypes.c_int64]),
    "mla_decode_workspace_size": (ctypes.c_size_t, [_CFG, _I, _I, _I, ctypes.c_int64, _I]),
    "mla_decode": (_I, [_CFG, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, ctypes.c_int64, _P,
                        ctypes.c_size_t, _P, _P, _P]),
    "mla_decode_noalloc": (_I, [_CFG, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                ctypes.c_int64, _P, _P, _P]),
    "mla_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "mla_decode_out_proj": (_I, [_CFG, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                 ctypes.c_int64, _P, _P, ctypes.c_size_t, _P, _P, _P, _P]),
    "mla_decode_fused_workspace_size": (ctypes.c_size_t, [_CFG, _I, _I, _I, ctypes.c_int64,
                                                          _I]),
    "mla_decode_fused_counter_bytes": (ctypes.c_size_t, []),
    "mla_decode_fused": (_I, [_CFG, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, ctypes.c_int64,
                              _P, ctypes.c_size_t, _P, _P, _P]),
    "mla_out_proj": (_I, [_CFG, _P, _P, _P, _I, _P]),
    "mla_gather_rows": (_I, [_CFG, _P, _I, _P, _I, _P, _I, _I, _P, _P]),
    "mla_validate_block_table": (_I, [_P, _I, _I, _P, _I, _I, _P, _P]),
    "mla_stream_read": (_I, [_P, ctypes.c_size_t, _P, _I, _P]),
    "mla_kv_produce_workspace_size": (ctypes.c_size_t, [_CFG, _I, _I]),
    "mla_kv_produce": (_I, [_CFG, _P, _I, _P, _P, ctypes.c_float, _P, _I, _P, _I, _P, _I, _I,
                            _I, _P, ctypes.c_size_t, _P]),
    "mla_rope": (_I, [_CFG, _P, _I, _P, _I, ctypes.c_float, _P]),
    "mla_o_proj_workspace_size": (ctypes.c_size_t, [_CFG, _I, _I, _I]),
    "mla_o_proj": (_I, [_CFG, _P, _P, _P, _I, _I, _P, ctypes.c_size_t, _P]),
    "mla_fold_uv_o": (_I, [_CFG, _P, _P, _P, _I, _P]),
    "mla_o_proj_folded": (_I, [_CFG, _P, _P, _P, _I, _I, _P, ctypes.c_size_t, _P]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with "
                              "`python -m mla_latent_kv_36_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise RuntimeError(load().mla_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def mla_status_string(code: int) -> str:
    return load().mla_status_string(code).decode()


def mla_abi_version() -> int:
    return int(load().mla_abi_version())


def mla_absorb_q(cfg: MlaConfig, q_nope: torch.Tensor, q_rope: Optional[torch.Tensor],
                 w_uk: torch.Tensor, q_abs: torch.Tensor, stream=None) -> None:
    """q_abs[m,h] = [q_nope[m,h] . W^UK[h] | q_rope[m,h]]; shapes [M,H,*]."""
    dt = _TORCH_DTYPE[cfg.dtype]
    M = q_nope.shape[0]
    _dev(q_nope, dt, "q_nope"), _dev(w_uk, dt, "w_uk"), _dev(q_abs, dt, "q_abs")
    if q_rope is not None:
        _dev(q_rope, dt, "q_rope")
    _check(load().mla_absorb_q(ctypes.byref(cfg), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                               _ptr(q_abs), M, _stream(stream)))


def mla_cache_append(cfg: MlaConfig, pool: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, new_rows: torch.Tensor, max_seq_len_host: int,
                     stream=None) -> None:
    """Write new_rows [B, T_new, W] after each sequence's seq_lens[b] rows."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(pool, dt, "pool"), _dev(new_rows, dt, "new_rows")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    B, T_new = new_rows.shape[0], new_rows.shape[1]
    _check(load().mla_cache_append(ctypes.byref(cfg), _ptr(pool), pool.shape[0],
                                   _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                   _ptr(new_rows), B, T_new, int(max_seq_len_host),
                                   _stream(stream)))


def mla_absorb_q_append(cfg: MlaConfig, q_nope: torch.Tensor, q_rope: Optional[torch.Tensor],
                        w_uk: torch.Tensor, q_abs: torch.Tensor, pool: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor,
                        new_rows: torch.Tensor, max_seq_len_host: int, stream=None) -> None:
    """mla_absorb_q and mla_cache_append in one call (one launch where the
    MFMA absorb kernel applies)."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(q_nope, dt, "q_nope"), _dev(w_uk, dt, "w_uk"), _dev(q_abs, dt, "q_abs")
    if q_rope is not None:
        _dev(q_rope, dt, "q_rope")
    _dev(pool, dt, "pool"), _dev(new_rows, dt, "new_rows")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    B, T_new = new_rows.shape[0], new_rows.shape[1]
    _check(load().mla_absorb_q_append(ctypes.byref(cfg), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                      _ptr(q_abs), q_nope.shape[0], _ptr(pool), pool.shape[0],
                                      _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                      _ptr(new_rows), B, T_new, int(max_seq_len_host),
                                      _stream(stream)))


def mla_decode_num_splits(cfg: MlaConfig, B: int, T: int, max_seq_len_host: int,
                          total_tokens_host: int = 0) -> int:
    return int(load().mla_decode_num_splits(ctypes.byref(cfg), B, T, int(max_seq_len_host),
                                            int(total_tokens_host)))


def mla_decode_workspace_size(cfg: MlaConfig, B: int, T: int, max_seq_len_host: int,
                              total_tokens_host: int = 0, num_splits: int = 0) -> int:
    n = load().mla_decode_workspace_size(ctypes.byref(cfg), B, T, int(max_seq_len_host),
                                         int(total_tokens_host), int(num_splits))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError("mla_decode_workspace_size: invalid configuration")
    return int(n)


def mla_decode(cfg: MlaConfig, q_abs: torch.Tensor, pool: torch.Tensor,
               block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len_host: int,
               o_lat: torch.Tensor, lse: Optional[torch.Tensor] = None, *, causal: bool = True,
               num_splits: int = 0, total_tokens_host: int = 0,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Latent attention of q_abs [B,T,H,W] over the paged cache -> o_lat [B,T,H,d_c] f32."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(q_abs, dt, "q_abs"), _dev(pool, dt, "pool"), _dev(o_lat, torch.float32, "o_lat")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    B, T = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_decode(ctypes.byref(cfg), _ptr(q_abs), _ptr(pool), pool.shape[0],
                             _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                             int(max_seq_len_host), B, T, 1 if causal else 0, int(num_splits),
                             int(total_tokens_host), _ptr(workspace), ws_bytes, _ptr(o_lat),
                             _ptr(lse), _stream(stream)))


def mla_decode_noalloc(cfg: MlaConfig, q_abs: torch.Tensor, pool: torch.Tensor,
                       block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len_host: int,
                       o_lat: torch.Tensor, lse: Optional[torch.Tensor] = None, *,
                       causal: bool = True, num_splits: int = 0, total_tokens_host: int = 0,
                       stream=None) -> None:
    """mla_decode with the split partials in the library's own scratch array
    (no workspace argument, nothing allocated)."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(q_abs, dt, "q_abs"), _dev(pool, dt, "pool"), _dev(o_lat, torch.float32, "o_lat")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    B, T = q_abs.shape[0], q_abs.shape[1]
    _check(load().mla_decode_noalloc(ctypes.byref(cfg), _ptr(q_abs), _ptr(pool), pool.shape[0],
                                     _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                     int(max_seq_len_host), B, T, 1 if causal else 0,
                                     int(num_splits), int(total_tokens_host), _ptr(o_lat),
                                     _ptr(lse), _stream(stream)))


def mla_decode_noalloc_scratch_bytes() -> int:
    return int(load().mla_decode_noalloc_scratch_bytes())


def mla_decode_out_proj(cfg: MlaConfig, q_abs: torch.Tensor, pool: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len_host: int,
                        w_uv: torch.Tensor, o_lat: torch.Tensor, out: torch.Tensor,
                        lse: Optional[torch.Tensor] = None, *, causal: bool = True,
                        num_splits: int = 0, total_tokens_host: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """mla_decode then mla_out_proj on its o_lat, the merge and the projection
    sharing a launch where they can."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(q_abs, dt, "q_abs"), _dev(pool, dt, "pool"), _dev(o_lat, torch.float32, "o_lat")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    _dev(w_uv, dt, "w_uv"), _dev(out, dt, "out")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    B, T = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_decode_out_proj(ctypes.byref(cfg), _ptr(q_abs), _ptr(pool), pool.shape[0],
                                      _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                      int(max_seq_len_host), B, T, 1 if causal else 0,
                                      int(num_splits), int(total_tokens_host), _ptr(w_uv),
                                      _ptr(workspace), ws_bytes, _ptr(o_lat), _ptr(lse),
                                      _ptr(out), _stream(stream)))


def mla_decode_fused_workspace_size(cfg: MlaConfig, B: int, T: int, max_seq_len_host: int,
                                    total_tokens_host: int = 0, num_splits: int = 0) -> int:
    n = load().mla_decode_fused_workspace_size(ctypes.byref(cfg), B, T, int(max_seq_len_host),
                                               int(total_tokens_host), int(num_splits))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError("mla_decode_fused_workspace_size: unsupported configuration")
    return int(n)


def mla_decode_fused_counter_bytes() -> int:
    return int(load().mla_decode_fused_counter_bytes())


def mla_decode_fused(cfg: MlaConfig, q_abs: torch.Tensor, pool: torch.Tensor,
                     block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len_host: int,
                     o_lat: torch.Tensor, lse: Optional[torch.Tensor] = None, *,
                     workspace: torch.Tensor, causal: bool = True, num_splits: int = 0,
                     total_tokens_host: int = 0, stream=None) -> None:
    """mla_decode in one launch (work queue and in-launch merge).  The first
    mla_decode_fused_counter_bytes() bytes of `workspace` must be zero before
    the first call (each call leaves them zero)."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(q_abs, dt, "q_abs"), _dev(pool, dt, "pool"), _dev(o_lat, torch.float32, "o_lat")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    B, T = q_abs.shape[0], q_abs.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().mla_decode_fused(ctypes.byref(cfg), _ptr(q_abs), _ptr(pool), pool.shape[0],
                                   _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                   int(max_seq_len_host), B, T, 1 if causal else 0,
                                   int(num_splits), int(total_tokens_host), _ptr(workspace),
                                   ws_bytes, _ptr(o_lat), _ptr(lse), _stream(stream)))


def mla_out_proj(cfg: MlaConfig, o_lat: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor,
                 stream=None) -> None:
    """out[m,h,v] = sum_c W^UV[h,v,c] o_lat[m,h,c]; o_lat [M,H,d_c] f32."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(o_lat, torch.float32, "o_lat"), _dev(w_uv, dt, "w_uv"), _dev(out, dt, "out")
    _check(load().mla_out_proj(ctypes.byref(cfg), _ptr(o_lat), _ptr(w_uv), _ptr(out),
                               o_lat.shape[0], _stream(stream)))


def mla_gather_rows(cfg: MlaConfig, pool: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len_host: int, dense: torch.Tensor,
                    stream=None) -> None:
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(pool, dt, "pool"), _dev(dense, dt, "dense")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    _check(load().mla_gather_rows(ctypes.byref(cfg), _ptr(pool), pool.shape[0],
                                  _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                  block_table.shape[0], int(max_seq_len_host), _ptr(dense),
                                  _stream(stream)))


def mla_validate_block_table(block_table: torch.Tensor, seq_lens: torch.Tensor,
                             block_size: int, num_blocks: int, err_flag: torch.Tensor,
                             stream=None) -> None:
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    _dev(err_flag, torch.int32, "err_flag")
    _check(load().mla_validate_block_table(_ptr(block_table), block_table.shape[0],
                                           block_table.shape[1], _ptr(seq_lens), block_size,
                                           num_blocks, _ptr(err_flag), _stream(stream)))


def mla_stream_read(src: torch.Tensor, sink: torch.Tensor, mode: int = 0, stream=None) -> None:
    """Read every byte of the contiguous device tensor src once and XOR its
    16-byte chunks into sink (a device tensor of 16 bytes, updated in place);
    mode 0: loads into registers, 1: direct-to-LDS copies."""
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous() and sink.is_contiguous()):
        raise ValueError("mla_stream_read: contiguous device tensors expected")
    if sink.numel() * sink.element_size() < 16:
        raise ValueError("mla_stream_read: sink must hold 16 bytes")
    _check(load().mla_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                  mode, _stream(stream)))


def mla_kv_produce_workspace_size(cfg: MlaConfig, M: int, d_model: int) -> int:
    n = int(load().mla_kv_produce_workspace_size(ctypes.byref(cfg), M, d_model))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError("mla_kv_produce_workspace_size: invalid arguments")
    return n


def mla_kv_produce(cfg: MlaConfig, hidden: torch.Tensor, w_dkv: torch.Tensor,
                   w_kr: Optional[torch.Tensor], pool: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, max_seq_len_host: int, workspace: torch.Tensor,
                   rope_base: float = 0.0, stream=None) -> None:
    """Rows [W^DKV h | RoPE(W^KR h)] of hidden [B, T_new, d_model] written after
    each sequence's seq_lens[b] rows.  workspace: a device byte tensor of at
    least mla_kv_produce_workspace_size(cfg, B * T_new, d_model) bytes."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(hidden, dt, "hidden"), _dev(w_dkv, dt, "w_dkv"), _dev(pool, dt, "pool")
    if w_kr is not None:
        _dev(w_kr, dt, "w_kr")
    _dev(block_table, torch.int32, "block_table"), _dev(seq_lens, torch.int32, "seq_lens")
    B, T_new, d_model = hidden.shape
    _check(load().mla_kv_produce(ctypes.byref(cfg), _ptr(hidden), d_model, _ptr(w_dkv),
                                 _ptr(w_kr), float(rope_base), _ptr(pool), pool.shape[0],
                                 _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B,
                                 T_new, int(max_seq_len_host), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_rope(cfg: MlaConfig, x: torch.Tensor, positions: torch.Tensor, rope_base: float = 0.0,
             stream=None) -> None:
    """In place: x [M, heads, d_rope], pair i of row m turned by
    positions[m] * base^(-2i/d_rope)."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(x, dt, "x"), _dev(positions, torch.int32, "positions")
    M, heads = x.shape[0], x.shape[1]
    _check(load().mla_rope(ctypes.byref(cfg), _ptr(x), heads, _ptr(positions), M,
                           float(rope_base), _stream(stream)))


def mla_o_proj_workspace_size(cfg: MlaConfig, M: int, d_model: int, folded: bool = False) -> int:
    n = int(load().mla_o_proj_workspace_size(ctypes.byref(cfg), M, d_model, 1 if folded else 0))
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError("mla_o_proj_workspace_size: invalid arguments")
    return n


def _sizes(**named) -> None:
    for name, (t, n) in named.items():
        if t.numel() != n:
            raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")


def _ws(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def mla_o_proj(cfg: MlaConfig, attn: torch.Tensor, w_o: torch.Tensor, y: torch.Tensor,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """y[m] = W^O . attn[m] with the heads of attn [M, H, d_v] concatenated in
    order; w_o [d_model, H * d_v], y [M, d_model]."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(attn, dt, "attn"), _dev(w_o, dt, "w_o"), _dev(y, dt, "y")
    M, d = attn.shape[0], w_o.shape[0]
    _sizes(attn=(attn, M * cfg.n_heads * cfg.d_v), w_o=(w_o, d * cfg.n_heads * cfg.d_v),
           y=(y, M * d))
    ws, nbytes = _ws(workspace)
    _check(load().mla_o_proj(ctypes.byref(cfg), _ptr(attn), _ptr(w_o), _ptr(y), attn.shape[0],
                             w_o.shape[0], ws, nbytes, _stream(stream)))


def mla_fold_uv_o(cfg: MlaConfig, w_uv: torch.Tensor, w_o: torch.Tensor, w_fold: torch.Tensor,
                  stream=None) -> None:
    """w_fold[:, h*d_c:(h+1)*d_c] = W^O[:, h*d_v:(h+1)*d_v] . W^UV[h]."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(w_uv, dt, "w_uv"), _dev(w_o, dt, "w_o"), _dev(w_fold, dt, "w_fold")
    H, d = cfg.n_heads, w_o.shape[0]
    _sizes(w_uv=(w_uv, H * cfg.d_v * cfg.d_c), w_o=(w_o, d * H * cfg.d_v),
           w_fold=(w_fold, d * H * cfg.d_c))
    _check(load().mla_fold_uv_o(ctypes.byref(cfg), _ptr(w_uv), _ptr(w_o), _ptr(w_fold),
                                w_o.shape[0], _stream(stream)))


def mla_o_proj_folded(cfg: MlaConfig, o_lat: torch.Tensor, w_fold: torch.Tensor,
                      y: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """y[m] = w_fold . o_lat[m] with the heads of o_lat [M, H, d_c] (f32)
    concatenated in order; w_fold [d_model, H * d_c], y [M, d_model]."""
    dt = _TORCH_DTYPE[cfg.dtype]
    _dev(o_lat, torch.float32, "o_lat"), _dev(w_fold, dt, "w_fold"), _dev(y, dt, "y")
    M, d = o_lat.shape[0], w_fold.shape[0]
    _sizes(o_lat=(o_lat, M * cfg.n_heads * cfg.d_c), w_fold=(w_fold, d * cfg.n_heads * cfg.d_c),
           y=(y, M * d))
    ws, nbytes = _ws(workspace)
    _check(load().mla_o_proj_folded(ctypes.byref(cfg), _ptr(o_lat), _ptr(w_fold), _ptr(y),
                                    o_lat.shape[0], w_fold.shape[0], ws, nbytes,
                                    _stream(stream)))
