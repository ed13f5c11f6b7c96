"""Thin ctypes binding of libpkv (include/pkv.h): argument marshalling only.

Every step of the computation runs in the HIP library; this module turns torch
tensors into device pointers and sizes, passes the current HIP stream, and raises
on a non-zero status.  There is no fallback: without the built library (or on a
machine without a GPU) the compute entry points fail loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_LAUNCH = 0, -1, -2, -3, -4
PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
PKV_MASK_NONE, PKV_MASK_CAUSAL, PKV_MASK_BLOCK_CAUSAL = 0, 1, 2
PKV_CHECK_SLOT_RANGE, PKV_CHECK_SEQ_LEN, PKV_CHECK_TABLE, PKV_CHECK_CU_Q, PKV_CHECK_SPANS = 1, 2, 4, 8, 16
PKV_CHECK_DUP_SLOT = 32

# Every symbol include/pkv.h declares, with its ctypes signature.
_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "pkv_kv_cache_write": (ctypes.c_int, [_P, _P, _I64, _P, _I32, _P, _P, _I64, _I32, _I32, _I32,
                                          _I32, ctypes.c_int, _P]),
    "pkv_kv_cache_write_fp8": (ctypes.c_int, [_P, _P, _I64, _P, _I32, _P, _P, _I64, _I32, _I32,
                                              _I32, _I32, _F, _F, ctypes.c_int, _P]),
    "pkv_kv_cache_gather": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, ctypes.c_int, _P]),
    "pkv_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attention_decode": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32,
                                                  _I32, _I32, _I32, _I32, _F, _I32, _P, _SZ,
                                                  ctypes.c_int, _P]),
    "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P,
                                                          _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                                          _I32, ctypes.c_int, _P]),
    "pkv_paged_attention_decode_fp8": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                                      _I32, _I32, _I32, _I32, _I32, _F, _F, _F,
                                                      _I32, _P, _SZ, ctypes.c_int, _P]),
    "pkv_paged_attention_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                                   ctypes.c_int, _I32, _I32, _I32, ctypes.c_int,
                                                   _P]),
    "pkv_paged_attention_prefill_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _I32,
                                                       _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                       _F, _F, _F, ctypes.c_int, _I32, _I32, _I32,
                                                       ctypes.c_int, _P]),
    "pkv_mixed_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attention_mixed": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32,
                                                 _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                 _F, ctypes.c_int, _I32, _I32, _I32, _P, _SZ,
                                                 ctypes.c_int, _P]),
    "pkv_smallseq_attention_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                                  _I32, _I32, _I32, _I32, _I32, _F, _I32,
                                                  ctypes.c_int, _P]),
    "pkv_smallseq_attention_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _I32,
                                                  _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                                  _I32, _F, _I32, ctypes.c_int, _P]),
    "pkv_paged_attention_prefill_spans": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _I32,
                                                         _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                         _F, _P, _P, _I32, _I32, _I32,
                                                         ctypes.c_int, _P]),
    "pkv_check_slots_unique": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _SZ, _P]),
    "pkv_set_device_checks": (ctypes.c_int, [ctypes.c_int]),
    "pkv_set_log": (ctypes.c_int, [ctypes.c_int]),
    "pkv_check_device_error": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_uint32)]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_int, []),
}

_lib = None


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv status {code}: {msg}")
        self.code = code


def load(path: Optional[str] = None):
    """Load libpkv.so (raises if it was not built).  PKV_LIBRARY in the environment names
    another build of it (a sanitizer build, for instance)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("PKV_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_scaled_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, _lib.pkv_last_error().decode())


def last_error() -> str:
    return load().pkv_last_error().decode()


# ----------------------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    return {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
            torch.uint8: PKV_FP8_E4M3, torch.float8_e4m3fn: PKV_FP8_E4M3}[t.dtype]


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _cache_geometry(key_cache, value_cache):
    """[num_blocks, block_size, num_kv_heads, head_dim] views with dense inner dims."""
    assert key_cache.dim() == 4 and key_cache.shape == value_cache.shape
    assert key_cache.stride(0) == value_cache.stride(0)
    nb, bs, hkv, d = key_cache.shape
    assert key_cache.stride()[1:] == (hkv * d, d, 1) and value_cache.stride()[1:] == (hkv * d, d, 1)
    return nb, bs, hkv, d, key_cache.stride(0)


def kv_cache_write(key, value, slot_mapping, key_cache, value_cache):
    """key/value [T, Hkv, D] (token stride free, inner dims dense); slot_mapping int64 [T]."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T = key.shape[0]
    assert key.shape == value.shape and key.stride() == value.stride()
    assert key.stride()[1:] == (d, 1) and key.shape[1:] == (hkv, d)
    _check(lib.pkv_kv_cache_write(_ptr(key), _ptr(value), key.stride(0), _ptr(slot_mapping), T,
                                  _ptr(key_cache), _ptr(value_cache), bstride, nb, bs, hkv, d,
                                  _dtype_code(key), _stream()))


def kv_cache_write_fp8(key, value, slot_mapping, key_cache, value_cache, k_scale: float,
                       v_scale: float):
    """kv_cache_write into uint8 caches of E4M3 codes (value = code * scale)."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T = key.shape[0]
    assert key.shape == value.shape and key.stride() == value.stride()
    assert key.stride()[1:] == (d, 1) and key.shape[1:] == (hkv, d)
    assert key_cache.element_size() == 1
    _check(lib.pkv_kv_cache_write_fp8(_ptr(key), _ptr(value), key.stride(0), _ptr(slot_mapping),
                                      T, _ptr(key_cache), _ptr(value_cache), bstride, nb, bs, hkv,
                                      d, float(k_scale), float(v_scale), _dtype_code(key),
                                      _stream()))


def check_slots_unique(slot_mapping, num_blocks: int, block_size: int, marks):
    """Flag (in the device error word) a slot that slot_mapping holds twice.  marks: a
    device bitmap of >= ceil(num_blocks * block_size / 32) int32 words, zero on entry and
    left zero."""
    lib = load()
    _check(lib.pkv_check_slots_unique(_ptr(slot_mapping), slot_mapping.shape[0], num_blocks,
                                      block_size, _ptr(marks),
                                      marks.numel() * marks.element_size(), _stream()))


def kv_cache_gather(key_out, value_out, cu_seq_lens, key_cache, value_cache, block_tables,
                    max_seq_len: int):
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S = cu_seq_lens.shape[0] - 1
    _check(lib.pkv_kv_cache_gather(_ptr(key_out), _ptr(value_out), _ptr(cu_seq_lens),
                                   _ptr(key_cache), _ptr(value_cache), bstride,
                                   _ptr(block_tables), block_tables.shape[1], S, key_out.shape[0],
                                   nb, bs, hkv, d, max_seq_len, _dtype_code(key_cache), _stream()))


def decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                          block_size: int, max_seq_len: int) -> int:
    return int(load().pkv_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                 block_size, max_seq_len))


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, seq_lens,
                           scale: float, max_seq_len: int, workspace=None):
    """query/out [S, H, D]; workspace: uint8 tensor of decode_workspace_size() bytes."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S, H, D = query.shape
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode(_ptr(out), _ptr(query), _ptr(key_cache),
                                          _ptr(value_cache), bstride, _ptr(block_tables),
                                          block_tables.shape[1], _ptr(seq_lens), S, H, hkv, D, nb,
                                          bs, float(scale), int(max_seq_len), _ptr(workspace),
                                          ws_bytes, _dtype_code(query), _stream()))


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables, seq_lens,
                                   scale: float, max_seq_len: int):
    """paged_attention_decode with the library's own per-GPU scratch as workspace (the call
    allocates nothing; calls that overlap on one GPU race)."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S, H, D = query.shape
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    _check(lib.pkv_paged_attention_decode_noalloc(_ptr(out), _ptr(query), _ptr(key_cache),
                                                  _ptr(value_cache), bstride, _ptr(block_tables),
                                                  block_tables.shape[1], _ptr(seq_lens), S, H, hkv,
                                                  D, nb, bs, float(scale), int(max_seq_len),
                                                  _dtype_code(query), _stream()))


def paged_attention_decode_fp8(out, query, key_cache, value_cache, block_tables, seq_lens,
                               scale: float, k_scale: float, v_scale: float, max_seq_len: int,
                               workspace=None):
    """paged_attention_decode over uint8 caches of E4M3 codes; query/out bf16 or fp16."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S, H, D = query.shape
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    assert key_cache.element_size() == 1
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode_fp8(_ptr(out), _ptr(query), _ptr(key_cache),
                                              _ptr(value_cache), bstride, _ptr(block_tables),
                                              block_tables.shape[1], _ptr(seq_lens), S, H, hkv, D,
                                              nb, bs, float(scale), float(k_scale), float(v_scale),
                                              int(max_seq_len), _ptr(workspace), ws_bytes,
                                              _dtype_code(query), _stream()))


def paged_attention_prefill(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                            block_tables, scale: float, mask: int, span_len: int, max_q_len: int,
                            max_seq_len: int):
    """query/out [T, H, D] flat over sequences (THD)."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T, H, D = query.shape
    S = seq_lens.shape[0]
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    _check(lib.pkv_paged_attention_prefill(_ptr(out), _ptr(query), _ptr(cu_seqlens_q),
                                           _ptr(seq_lens), _ptr(key_cache), _ptr(value_cache),
                                           bstride, _ptr(block_tables), block_tables.shape[1], S,
                                           T, H, hkv, D, nb, bs, float(scale), int(mask),
                                           int(span_len), int(max_q_len), int(max_seq_len),
                                           _dtype_code(query), _stream()))


def paged_attention_prefill_fp8(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                                block_tables, scale: float, k_scale: float, v_scale: float,
                                mask: int, span_len: int, max_q_len: int, max_seq_len: int):
    """paged_attention_prefill over uint8 caches of E4M3 codes; query/out bf16 or fp16."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T, H, D = query.shape
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    assert key_cache.element_size() == 1
    S = seq_lens.shape[0]
    _check(lib.pkv_paged_attention_prefill_fp8(_ptr(out), _ptr(query), _ptr(cu_seqlens_q),
                                               _ptr(seq_lens), _ptr(key_cache), _ptr(value_cache),
                                               bstride, _ptr(block_tables), block_tables.shape[1],
                                               S, T, H, hkv, D, nb, bs, float(scale),
                                               float(k_scale), float(v_scale), int(mask),
                                               int(span_len), int(max_q_len), int(max_seq_len),
                                               _dtype_code(query), _stream()))


def mixed_workspace_size(num_gen_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                         block_size: int, max_seq_len: int) -> int:
    return int(load().pkv_mixed_workspace_size(num_gen_seqs, num_heads, num_kv_heads, head_dim,
                                                block_size, max_seq_len))


def paged_attention_mixed(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                          block_tables, scale: float, mask: int, span_len: int, max_q_len: int,
                          max_seq_len: int, num_ctx_seqs: int, num_ctx_tokens: int,
                          workspace=None):
    """Context sequences first (rows by cu_seqlens_q), then one-row generation sequences."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T, H, D = query.shape
    S = seq_lens.shape[0]
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_mixed(_ptr(out), _ptr(query), _ptr(cu_seqlens_q),
                                         _ptr(seq_lens), _ptr(key_cache), _ptr(value_cache),
                                         bstride, _ptr(block_tables), block_tables.shape[1], S, T,
                                         int(num_ctx_seqs), int(num_ctx_tokens), H, hkv, D, nb,
                                         bs, float(scale), int(mask), int(span_len),
                                         int(max_q_len), int(max_seq_len), _ptr(workspace),
                                         ws_bytes, _dtype_code(query), _stream()))


def smallseq_attention_fwd(out, weights, query, key_cache, value_cache, block_tables, seq_lens,
                           scale: float, max_seq_len: int):
    """One query row per sequence (<= 16 keys): out [S, H, D], weights [S, H, max_seq_len]."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S, H, D = query.shape
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    assert weights.shape == (S, H, max_seq_len) and weights.is_contiguous()
    _check(lib.pkv_smallseq_attention_fwd(_ptr(out), _ptr(weights), _ptr(query), _ptr(key_cache),
                                          _ptr(value_cache), bstride, _ptr(block_tables),
                                          block_tables.shape[1], _ptr(seq_lens), S, H, hkv, D, nb,
                                          bs, float(scale), int(max_seq_len), _dtype_code(query),
                                          _stream()))


def smallseq_attention_bwd(d_query, d_key, d_value, d_out, query, weights, key_cache,
                           value_cache, block_tables, seq_lens, cu_seq_lens, scale: float,
                           max_seq_len: int):
    """Gradients from the saved weights; d_key/d_value [total_kv, Hkv, D] by cu_seq_lens."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    S, H, D = query.shape
    assert d_query.shape == query.shape == d_out.shape and d_key.shape == d_value.shape
    assert weights.shape == (S, H, max_seq_len)
    _check(lib.pkv_smallseq_attention_bwd(_ptr(d_query), _ptr(d_key), _ptr(d_value), _ptr(d_out),
                                          _ptr(query), _ptr(weights), _ptr(key_cache),
                                          _ptr(value_cache), bstride, _ptr(block_tables),
                                          block_tables.shape[1], _ptr(seq_lens), _ptr(cu_seq_lens),
                                          S, d_key.shape[0], H, hkv, D, nb, bs, float(scale),
                                          int(max_seq_len), _dtype_code(query), _stream()))


def paged_attention_prefill_spans(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                                  block_tables, scale: float, full_spans, cu_spans, max_q_len: int,
                                  max_seq_len: int):
    """Prefill with general span lists: full_spans int32 [N, 2] (start, end) pairs sequence
    by sequence, cu_spans int32 [S+1] offsets into them (N = 0: causal)."""
    lib = load()
    nb, bs, hkv, d, bstride = _cache_geometry(key_cache, value_cache)
    T, H, D = query.shape
    S = seq_lens.shape[0]
    assert D == d and out.shape == query.shape and query.is_contiguous() and out.is_contiguous()
    n = int(full_spans.shape[0]) if full_spans is not None else 0
    _check(lib.pkv_paged_attention_prefill_spans(_ptr(out), _ptr(query), _ptr(cu_seqlens_q),
                                                 _ptr(seq_lens), _ptr(key_cache), _ptr(value_cache),
                                                 bstride, _ptr(block_tables), block_tables.shape[1],
                                                 S, T, H, hkv, D, nb, bs, float(scale),
                                                 _ptr(full_spans if n else None),
                                                 _ptr(cu_spans if n else None), n, int(max_q_len),
                                                 int(max_seq_len), _dtype_code(query), _stream()))


def set_log(enable: bool):
    """Print one line per kernel launch to stderr (kernel, grid, block, variant)."""
    _check(load().pkv_set_log(1 if enable else 0))


def set_device_checks(enable: bool):
    """Device-side precondition checks on (or off) for every later call in this process."""
    _check(load().pkv_set_device_checks(1 if enable else 0))


def check_device_error():
    """Wait for the current stream, read and clear the device error word.
    Returns (bits, message): bits is 0 and message "" when no check failed."""
    lib = load()
    bits = ctypes.c_uint32(0)
    rc = lib.pkv_check_device_error(_stream(), ctypes.byref(bits))
    if rc == PKV_OK:
        return 0, ""
    if rc != PKV_ERR_INVALID_ARG:
        raise PkvError(rc, lib.pkv_last_error().decode())
    return int(bits.value), lib.pkv_last_error().decode()
