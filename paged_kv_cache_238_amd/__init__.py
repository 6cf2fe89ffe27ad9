"""Python binding of libpa.so: paged-attention decode for AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/pa.h.  torch supplies device
memory and the current stream; nothing here computes attention, and there is
no CPU fallback: if libpa.so is missing or fails to load, importing this
package raises.

Functions mirror the C entry points:
  write_kv(k_new, v_new, slot_mapping, k_pool, v_pool)
  write_kv_int8(k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale)
  write_kv_fp8(k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale)
  decode(q, k_pool, v_pool, block_table, context_lens, ...)
  decode_int8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, ...)
  decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, ...)
  decode_noalloc(q, k_pool, v_pool, block_table, context_lens, ...)
  copy_blocks(k_pool, v_pool, block_pairs, k_scale=None, v_scale=None)

FP8 pools hold raw OCP E4M3 codes: torch.uint8 tensors (a torch.float8_e4m3fn
tensor is accepted and viewed as its bytes).
  decode_partials(...), decode_partials_int8(...), merge_partials(...)
  decode_shared_prefix(q, k_pool, v_pool, block_table, context_lens, prefix_len, ...)
  workspace_size(...), partition_size(...), shared_prefix_workspace_size(...)
  validate(block_table, context_lens, num_blocks, ...)  host check of the caller
      contracts the kernels do not verify (contracts.py)
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "PaError", "LIB_PATH", "lib", "status_string", "write_kv", "write_kv_int8",
    "write_kv_fp8", "partition_size", "workspace_size", "decode", "decode_int8",
    "decode_fp8", "decode_noalloc", "copy_blocks", "decode_partials",
    "decode_partials_int8", "merge_partials", "decode_shared_prefix",
    "shared_prefix_workspace_size", "decode_append", "append_workspace_size", "EXPORTS",
    "validate",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIB", os.path.join(HERE, "libpa.so"))

# torch ships its own HIP runtime (libamdhip64.so.7).  Import it before
# loading libpa.so so that libpa.so binds to that runtime by soname; loading
# libpa.so first would put /opt/rocm's copy in the process under the same
# soname and torch's device calls would then run on a runtime it was not
# built against.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libpa.so not found at {LIB_PATH}; build it with "
        "`python paged_kv_cache_238_amd/build.py` (hipcc, gfx950)")
lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_z = ctypes.c_size_t

# name -> (restype, argtypes); the full exported surface of include/pa.h
EXPORTS = {
    "pa_status_string": (ctypes.c_char_p, [_i]),
    "pa_write_kv": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "pa_write_kv_int8": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "pa_write_kv_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "pa_copy_blocks": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]),
    "pa_decode_partition_size": (_i, [_i, _i, _i, _i, _i, _i]),
    "pa_decode_workspace_size": (_z, [_i, _i, _i, _i, _i, _i]),
    "pa_decode": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                       _p, _z, _p]),
    "pa_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i,
                               _f, _i, _p]),
    "pa_decode_int8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                            _i, _f, _i, _p, _z, _p]),
    "pa_decode_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                           _i, _f, _i, _p, _z, _p]),
    "pa_decode_partials": (_i, [_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                _p, _z, _p]),
    "pa_decode_partials_int8": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                                     _i, _f, _i, _p, _z, _p]),
    "pa_decode_partials_fp8": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                                    _i, _f, _i, _p, _z, _p]),
    "pa_merge_partials": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _z, _p]),
    "pa_decode_append_workspace_size": (_z, [_i, _i, _i, _i, _i, _i]),
    "pa_decode_append": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                              _i, _f, _i, _p, _z, _p]),
    "pa_decode_append_int8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i,
                                   _i, _i, _i, _i, _f, _i, _p, _z, _p]),
    "pa_decode_append_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i,
                                  _i, _i, _i, _i, _f, _i, _p, _z, _p]),
    "pa_decode_shared_prefix_workspace_size": (_z, [_i, _i, _i, _i, _i, _i]),
    "pa_decode_shared_prefix": (_i, [_p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i,
                                     _i, _f, _i, _p, _z, _p]),
    "pa_decode_shared_prefix_int8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i,
                                          _i, _i, _i, _i, _f, _i, _p, _z, _p]),
    "pa_decode_shared_prefix_fp8": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i,
                                         _i, _i, _i, _i, _f, _i, _p, _z, _p]),
}
for _name, (_res, _args) in EXPORTS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

BLOCK_SIZE = 16

from .contracts import validate  # noqa: E402  (host-side contract check)


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def status_string(status: int) -> str:
    return lib.pa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where)


# --- torch marshalling -------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


# The current stream's raw handle for a device index: torch's direct lookup
# (the one its generated kernels use) costs about 0.1 us against about 2 us
# for building the Stream object; the public route is kept where it is absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtype, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def write_kv(k_new, v_new, slot_mapping, k_pool, v_pool) -> None:
    """Copy token i's K/V rows [kv_heads, head_dim] into slot slot_mapping[i]
    of the fp16 pools (negative slots skipped)."""
    torch = _torch()
    _need(k_pool, "k_pool", torch.float16, 4)
    dev = k_pool.device
    _need(v_pool, "v_pool", torch.float16, 4, dev)
    _need(k_new, "k_new", torch.float16, 3, dev)
    _need(v_new, "v_new", torch.float16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int32, 1, dev)
    NB, bs, Hkv, D = k_pool.shape
    T = k_new.shape[0]
    if v_pool.shape != k_pool.shape or k_new.shape != (T, Hkv, D) or v_new.shape != k_new.shape \
            or slot_mapping.shape[0] != T:
        raise ValueError("write_kv: inconsistent shapes")
    _check(lib.pa_write_kv(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_pool),
                           _ptr(v_pool), T, NB, bs, Hkv, D, _stream(k_pool)), "pa_write_kv")


def _codes(t):
    """An FP8 pool as its uint8 codes (float8_e4m3fn tensors are viewed)."""
    torch = _torch()
    fp8 = getattr(torch, "float8_e4m3fn", None)
    if fp8 is not None and isinstance(t, torch.Tensor) and t.dtype == fp8:
        return t.view(torch.uint8)
    return t


def _write_q8(fn, name, pool_dtype, k_new, v_new, slot_mapping, k_pool, v_pool, k_scale,
              v_scale):
    torch = _torch()
    _need(k_pool, "k_pool", pool_dtype, 4)
    dev = k_pool.device
    _need(v_pool, "v_pool", pool_dtype, 4, dev)
    _need(k_scale, "k_scale", torch.float32, 3, dev)
    _need(v_scale, "v_scale", torch.float32, 3, dev)
    _need(k_new, "k_new", torch.float16, 3, dev)
    _need(v_new, "v_new", torch.float16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int32, 1, dev)
    NB, bs, Hkv, D = k_pool.shape
    T = k_new.shape[0]
    if v_pool.shape != k_pool.shape or k_scale.shape != (NB, Hkv, bs) \
            or v_scale.shape != k_scale.shape or k_new.shape != (T, Hkv, D) \
            or v_new.shape != k_new.shape or slot_mapping.shape[0] != T:
        raise ValueError(f"{name}: inconsistent shapes")
    _check(fn(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_pool), _ptr(v_pool),
              _ptr(k_scale), _ptr(v_scale), T, NB, bs, Hkv, D, _stream(k_pool)), name)


def write_kv_int8(k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale) -> None:
    """Quantise token i's K/V rows per (token, kv head) into the int8 pools
    and their fp32 scales at slot slot_mapping[i]."""
    _write_q8(lib.pa_write_kv_int8, "pa_write_kv_int8", _torch().int8, k_new, v_new,
              slot_mapping, k_pool, v_pool, k_scale, v_scale)


def write_kv_fp8(k_new, v_new, slot_mapping, k_pool, v_pool, k_scale, v_scale) -> None:
    """Quantise token i's K/V rows per (token, kv head) to FP8 E4M3 codes in
    the uint8 pools, with their fp32 scales, at slot slot_mapping[i]."""
    _write_q8(lib.pa_write_kv_fp8, "pa_write_kv_fp8", _torch().uint8, k_new, v_new,
              slot_mapping, _codes(k_pool), _codes(v_pool), k_scale, v_scale)


def copy_blocks(k_pool, v_pool, block_pairs, k_scale=None, v_scale=None) -> None:
    """Copy whole blocks src -> dst for each row (src, dst) of block_pairs
    (int32 [n, 2] on the pools' device): K, V and, for 8-bit pools, their
    scales.  dst blocks must be distinct and not also be a src."""
    torch = _torch()
    k_pool, v_pool = _codes(k_pool), _codes(v_pool)
    dev = k_pool.device
    q8 = k_pool.dtype in (torch.int8, torch.uint8)
    _need(k_pool, "k_pool", k_pool.dtype if q8 else torch.float16, 4)
    _need(v_pool, "v_pool", k_pool.dtype, 4, dev)
    _need(block_pairs, "block_pairs", torch.int32, 2, dev)
    NB, bs, Hkv, D = k_pool.shape
    if v_pool.shape != k_pool.shape or block_pairs.shape[1:] != (2,):
        raise ValueError("copy_blocks: inconsistent shapes")
    if q8:
        _need(k_scale, "k_scale", torch.float32, 3, dev)
        _need(v_scale, "v_scale", torch.float32, 3, dev)
        if k_scale.shape != (NB, Hkv, bs) or v_scale.shape != k_scale.shape:
            raise ValueError("copy_blocks: scale shapes must be [num_blocks, kv_heads, block_size]")
    _check(lib.pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale) if q8 else None,
                              _ptr(v_scale) if q8 else None, _ptr(block_pairs),
                              block_pairs.shape[0], NB, bs, Hkv, D, 1 if q8 else 2,
                              _stream(k_pool)), "pa_copy_blocks")


def partition_size(batch, q_heads, kv_heads, head_dim, max_context_len, partition_size=0) -> int:
    return int(lib.pa_decode_partition_size(batch, q_heads, kv_heads, head_dim,
                                            max_context_len, partition_size))


_resolve_partition = partition_size


def workspace_size(batch, q_heads, kv_heads, head_dim, max_context_len, partition_size=0) -> int:
    return int(lib.pa_decode_workspace_size(batch, q_heads, kv_heads, head_dim,
                                            max_context_len, partition_size))


def _decode_args(q, k_pool, v_pool, block_table, context_lens, kv_dtype, max_context_len,
                 k_scale=None, v_scale=None):
    torch = _torch()
    _need(q, "q", torch.float16, 3)
    dev = q.device
    _need(k_pool, "k_pool", kv_dtype, 4, dev)
    _need(v_pool, "v_pool", kv_dtype, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_pool.shape
    if v_pool.shape != k_pool.shape or D2 != D or block_table.shape[0] != B \
            or context_lens.shape[0] != B:
        raise ValueError("decode: inconsistent shapes")
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32, 3, dev)
        _need(v_scale, "v_scale", torch.float32, 3, dev)
        if k_scale.shape != (NB, Hkv, bs) or v_scale.shape != k_scale.shape:
            raise ValueError("decode_int8: scale shapes must be [num_blocks, kv_heads, block_size]")
    if max_context_len is None:
        # host bound from the device lengths (one synchronising read); pass it
        # explicitly to avoid the read
        max_context_len = int(context_lens.max().item()) if B else 0
    return B, Hq, Hkv, D, NB, bs, block_table.shape[1], int(max_context_len)


def _alloc_out(q, out, return_lse):
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
    return out, lse


def _workspace(q, B, Hq, Hkv, D, L, P, workspace):
    torch = _torch()
    need = workspace_size(B, Hq, Hkv, D, L, P)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    return workspace


def decode(q, k_pool, v_pool, block_table, context_lens, scale=None, partition_size=0,
           max_context_len=None, out=None, return_lse=False, workspace=None):
    """fp16 paged decode.  Returns out [B, Hq, D] fp16 (and lse [B, Hq] fp32
    when return_lse)."""
    torch = _torch()
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(q, k_pool, v_pool, block_table, context_lens,
                                                torch.float16, max_context_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    ws = _workspace(q, B, Hq, Hkv, D, L, partition_size, workspace)
    _check(lib.pa_decode(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                         _ptr(block_table), MB, _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB,
                         scale, partition_size, _ptr(ws), ws.numel(), _stream(q)), "pa_decode")
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 64 << 20       # PA_NOALLOC_SCRATCH_BYTES in include/pa.h


def decode_noalloc(q, k_pool, v_pool, block_table, context_lens, scale=None, partition_size=0,
                   max_context_len=None, out=None, return_lse=False):
    """fp16 paged decode through pa_decode_noalloc: no workspace; the
    library's per-device scratch array holds the split-K records (calls that
    overlap on one device race).  Pass `out` (and keep return_lse False) for
    a call that allocates nothing on this side either."""
    torch = _torch()
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(q, k_pool, v_pool, block_table, context_lens,
                                                torch.float16, max_context_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    _check(lib.pa_decode_noalloc(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(block_table), MB, _ptr(context_lens), L, B, Hq, Hkv, D,
                                 bs, NB, scale, partition_size, _stream(q)),
           "pa_decode_noalloc")
    return (out, lse) if return_lse else out


def decode_int8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, scale=None,
                partition_size=0, max_context_len=None, out=None, return_lse=False,
                workspace=None):
    """Paged decode over an int8 cache with fp32 per-(token, kv head) scales."""
    torch = _torch()
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(q, k_pool, v_pool, block_table, context_lens,
                                                torch.int8, max_context_len, k_scale, v_scale)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    ws = _workspace(q, B, Hq, Hkv, D, L, partition_size, workspace)
    _check(lib.pa_decode_int8(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                              _ptr(k_scale), _ptr(v_scale), _ptr(block_table), MB,
                              _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale,
                              partition_size, _ptr(ws), ws.numel(), _stream(q)),
           "pa_decode_int8")
    return (out, lse) if return_lse else out


def decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, scale=None,
               partition_size=0, max_context_len=None, out=None, return_lse=False,
               workspace=None):
    """Paged decode over an FP8 (E4M3 codes, uint8) cache with fp32
    per-(token, kv head) scales."""
    torch = _torch()
    k_pool, v_pool = _codes(k_pool), _codes(v_pool)
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(q, k_pool, v_pool, block_table, context_lens,
                                                torch.uint8, max_context_len, k_scale, v_scale)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    ws = _workspace(q, B, Hq, Hkv, D, L, partition_size, workspace)
    _check(lib.pa_decode_fp8(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                             _ptr(k_scale), _ptr(v_scale), _ptr(block_table), MB,
                             _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale,
                             partition_size, _ptr(ws), ws.numel(), _stream(q)),
           "pa_decode_fp8")
    return (out, lse) if return_lse else out


def append_workspace_size(batch, q_heads, kv_heads, head_dim, max_context_len,
                          partition_size=0) -> int:
    return int(lib.pa_decode_append_workspace_size(batch, q_heads, kv_heads, head_dim,
                                                   max_context_len, partition_size))


def decode_append(q, k_new, v_new, k_pool, v_pool, block_table, context_lens, scale=None,
                  partition_size=0, max_context_len=None, out=None, return_lse=False,
                  workspace=None, k_scale=None, v_scale=None, kv_format=None):
    """Write each sequence's new token (k_new / v_new [B, Hkv, D] fp16, at
    position context_lens[b] - 1) into its slot and decode over the whole
    context, in two launches.  The cache format follows k_pool's dtype
    (float16, int8, or uint8 codes = FP8 E4M3, which needs kv_format="fp8";
    8-bit caches need k_scale / v_scale, which the call updates)."""
    torch = _torch()
    if kv_format is None:
        kv_format = {torch.float16: "fp16", torch.int8: "int8"}.get(k_pool.dtype, "fp8")
    dtype = {"fp16": torch.float16, "int8": torch.int8, "fp8": torch.uint8}[kv_format]
    if kv_format == "fp8":
        k_pool, v_pool = _codes(k_pool), _codes(v_pool)
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(q, k_pool, v_pool, block_table, context_lens,
                                                dtype, max_context_len, k_scale, v_scale)
    _need(k_new, "k_new", torch.float16, 3, q.device)
    _need(v_new, "v_new", torch.float16, 3, q.device)
    if k_new.shape != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("decode_append: k_new / v_new must be [batch, kv_heads, head_dim]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    need = append_workspace_size(B, Hq, Hkv, D, L, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    head = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool))
    tail = (_ptr(block_table), MB, _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale,
            partition_size, _ptr(workspace), workspace.numel(), _stream(q))
    if kv_format == "fp16":
        _check(lib.pa_decode_append(*head, *tail), "pa_decode_append")
    else:
        if k_scale is None or v_scale is None:
            raise ValueError("decode_append: 8-bit caches need k_scale and v_scale")
        fn = lib.pa_decode_append_int8 if kv_format == "int8" else lib.pa_decode_append_fp8
        _check(fn(*head, _ptr(k_scale), _ptr(v_scale), *tail), "pa_decode_append_" + kv_format)
    return (out, lse) if return_lse else out


def decode_partials(q, k_pool, v_pool, block_table, context_lens, workspace, scale=None,
                    partition_size=0, max_context_len=None, k_scale=None, v_scale=None):
    """Stage 1 of decode: write the per-partition records into `workspace`
    (uint8 device tensor of >= workspace_size(...) bytes).  Returns the
    resolved partition size."""
    torch = _torch()
    k_pool, v_pool = _codes(k_pool), _codes(v_pool)
    q8 = k_pool.dtype in (torch.int8, torch.uint8)
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(
        q, k_pool, v_pool, block_table, context_lens, k_pool.dtype if q8 else torch.float16,
        max_context_len, k_scale if q8 else None, v_scale if q8 else None)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    if q8:
        fn = lib.pa_decode_partials_int8 if k_pool.dtype == torch.int8 \
            else lib.pa_decode_partials_fp8
        st = fn(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                _ptr(block_table), MB, _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale,
                partition_size, _ptr(workspace), nbytes, _stream(q))
    else:
        st = lib.pa_decode_partials(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), MB,
                                    _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale,
                                    partition_size, _ptr(workspace), nbytes, _stream(q))
    _check(st, "pa_decode_partials")
    return _resolve_partition(B, Hq, Hkv, D, L, partition_size)


def merge_partials(workspace, context_lens, q_heads, head_dim, partition_size, max_context_len,
                   out=None, return_lse=False):
    """Stage 2 of decode: log-sum-exp merge of the records in `workspace`."""
    torch = _torch()
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    dev = context_lens.device
    if out is None:
        out = torch.empty((B, q_heads, head_dim), dtype=torch.float16, device=dev)
    lse = torch.empty((B, q_heads), dtype=torch.float32, device=dev) if return_lse else None
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.pa_merge_partials(_ptr(out), _ptr(lse), _ptr(context_lens), int(max_context_len),
                                 B, q_heads, head_dim, int(partition_size), _ptr(workspace),
                                 nbytes, _stream(context_lens)), "pa_merge_partials")
    return (out, lse) if return_lse else out


def shared_prefix_workspace_size(batch, q_heads, kv_heads, head_dim, max_context_len,
                                 prefix_len) -> int:
    return int(lib.pa_decode_shared_prefix_workspace_size(batch, q_heads, kv_heads, head_dim,
                                                          max_context_len, prefix_len))


def decode_shared_prefix(q, k_pool, v_pool, block_table, context_lens, prefix_len, scale=None,
                         max_context_len=None, out=None, return_lse=False, workspace=None,
                         k_scale=None, v_scale=None):
    """Decode where every sequence's first `prefix_len` tokens sit in the same
    blocks (row 0's ids); the shared blocks are read once per kv head for all
    sequences.  int8 or fp8 (uint8 codes) pools when k_scale / v_scale are
    given."""
    torch = _torch()
    k_pool, v_pool = _codes(k_pool), _codes(v_pool)
    q8 = k_scale is not None
    B, Hq, Hkv, D, NB, bs, MB, L = _decode_args(
        q, k_pool, v_pool, block_table, context_lens, k_pool.dtype if q8 else torch.float16,
        max_context_len, k_scale, v_scale)
    if q8 and k_pool.dtype not in (torch.int8, torch.uint8):
        raise ValueError("decode_shared_prefix: scaled pools must be int8 or uint8 (fp8) codes")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out, lse = _alloc_out(q, out, return_lse)
    need = shared_prefix_workspace_size(B, Hq, Hkv, D, L, int(prefix_len))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    if q8:
        fn = lib.pa_decode_shared_prefix_int8 if k_pool.dtype == torch.int8 \
            else lib.pa_decode_shared_prefix_fp8
        _check(fn(
            _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
            _ptr(v_scale), _ptr(block_table), MB, _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB,
            scale, int(prefix_len), _ptr(workspace), nbytes, _stream(q)),
            "pa_decode_shared_prefix (8-bit)")
    else:
        _check(lib.pa_decode_shared_prefix(
            _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), MB,
            _ptr(context_lens), L, B, Hq, Hkv, D, bs, NB, scale, int(prefix_len),
            _ptr(workspace), nbytes, _stream(q)), "pa_decode_shared_prefix")
    return (out, lse) if return_lse else out
