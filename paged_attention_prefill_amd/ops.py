"""Thin ctypes binding over libpagedattn.so (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module
turns torch tensors into device pointers, sizes and the current HIP stream,
and turns status codes into exceptions.  It raises if the library has not been
built: there is no fallback path.
"""

import ctypes
import os
import re

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pagedattn.h")

PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_METADATA = \
    0, -1, -2, -3, -4, -5
PA_F32, PA_F16, PA_BF16, PA_FP8_E5M2, PA_FP8_E4M3 = 0, 1, 2, 3, 4
DECODE_MAX_Q = 16
SPLIT_TILE = 32

_TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
                torch.uint8: PA_FP8_E5M2, torch.float8_e5m2: PA_FP8_E5M2, torch.float8_e4m3fn: PA_FP8_E4M3}
_PA_TO_TORCH = {PA_F32: torch.float32, PA_F16: torch.float16, PA_BF16: torch.bfloat16}


class PagedAttentionError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"pagedattn status {status}: {message}")
        self.status = status


class AttnOptions(ctypes.Structure):
    _fields_ = [("sinks", ctypes.c_void_p), ("window_left", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p)]


class KvCache(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("stride_page", ctypes.c_int64), ("stride_token", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("k_head_scales", ctypes.c_void_p), ("v_head_scales", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t


ABI_VERSION = 3  # PA_VERSION of include/pagedattn.h


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_attention_prefill_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.pa_paged_prefill.argtypes = [_P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                       ctypes.POINTER(KvCache), ctypes.c_float, _I, _P, _SZ, _P]
        L.pa_split_kv_decode.argtypes = L.pa_paged_prefill.argtypes
        L.pa_split_kv_decode_fixed.argtypes = L.pa_paged_prefill.argtypes[:14] + [_I, _I, _P, _SZ, _P]
        L.pa_paged_prefill_ex.argtypes = L.pa_paged_prefill.argtypes[:15] + [ctypes.POINTER(AttnOptions), _P, _SZ, _P]
        L.pa_split_kv_decode_ex.argtypes = L.pa_paged_prefill.argtypes[:14] + [_I, _I, ctypes.POINTER(AttnOptions),
                                                                              _P, _SZ, _P]
        L.pa_split_kv_decode_noalloc.argtypes = L.pa_paged_prefill.argtypes[:14] + [_I, _I, ctypes.POINTER(AttnOptions),
                                                                                   _P]
        L.pa_mixed_step.argtypes = [_P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.POINTER(KvCache),
                                    ctypes.c_float, _I, _I, _I, _I, ctypes.POINTER(AttnOptions), _P, _SZ, _P]
        L.pa_mixed_workspace_bytes.argtypes = [_P] + [_I] * 8
        L.pa_mixed_workspace_bytes.restype = _SZ
        L.pa_merge_states.argtypes = [_P, _I, _I, _I, _I, _P, _I, _P, _P]
        L.pa_write_kv.argtypes = [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, ctypes.POINTER(KvCache), _P]
        L.pa_prefill_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.pa_prefill_workspace_bytes.restype = _SZ
        L.pa_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.pa_decode_workspace_bytes.restype = _SZ
        L.pa_check_supported.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_char_p)]
        L.pa_validate_metadata.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I]
        L.pa_prefill_auto_splits.argtypes = [_I] * 8
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_last_error.restype = ctypes.c_char_p
        for name in ("pa_paged_prefill", "pa_split_kv_decode", "pa_split_kv_decode_fixed", "pa_merge_states",
                     "pa_split_kv_decode_noalloc",
                     "pa_write_kv", "pa_paged_prefill_ex", "pa_split_kv_decode_ex", "pa_mixed_step",
                     "pa_check_supported",
                     "pa_validate_metadata", "pa_prefill_auto_splits", "pa_status_string", "pa_version"):
            if name != "pa_status_string":
                getattr(L, name).restype = ctypes.c_int
        L.pa_status_string.argtypes = [ctypes.c_int]
        if L.pa_version() != ABI_VERSION:  # the option struct's layout is tied to the version
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.pa_version()}, this binding expects {ABI_VERSION}: "
                               "rebuild it with `python -m paged_attention_prefill_amd.build`")
        _lib = L
    return _lib


def header_symbols():
    """Function names declared in include/*.h."""
    import glob
    names = set()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER_PATH), "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def _check(status):
    if status != PA_OK:
        L = lib()
        raise PagedAttentionError(status, (L.pa_last_error() or b"").decode() or
                                  L.pa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype(t):
    try:
        return _TORCH_TO_PA[t.dtype]
    except KeyError:
        raise PagedAttentionError(PA_ERR_UNSUPPORTED, f"unsupported dtype {t.dtype}") from None


def kv_cache(k_pages, v_pages, k_scale=1.0, v_scale=1.0, k_head_scales=None, v_head_scales=None):
    """Describe logical [num_pages, page_size, Hkv, D] K/V page tensors (D contiguous);
    fp8 pages may carry per-head scale tensors (float32 [Hkv] on the device)."""
    if k_pages.shape != v_pages.shape or k_pages.stride() != v_pages.stride():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "K and V pages must share shape and strides")
    if k_pages.dtype != v_pages.dtype:
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "K and V pages must share the dtype")
    if k_pages.dim() != 4 or k_pages.stride(3) != 1:
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "pages must be 4-D with a contiguous head dim")
    n, P, H, D = k_pages.shape
    s = k_pages.stride()
    for t, name in ((k_head_scales, "k_head_scales"), (v_head_scales, "v_head_scales")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != H or not t.is_contiguous()):
            raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous float32 [Hkv] tensor")
    return KvCache(k_pages.data_ptr(), v_pages.data_ptr(), s[0], s[1], s[2], n, P, H, D,
                   _dtype(k_pages), float(k_scale), float(v_scale),
                   None if k_head_scales is None else k_head_scales.data_ptr(),
                   None if v_head_scales is None else v_head_scales.data_ptr())


def _i32(t, name):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous int32 tensor")
    return t


def _options(num_q_heads, sinks, window_left, softcap=0.0, alibi_slopes=None):
    """pa_attn_options for the *_ex calls, or None when nothing is set."""
    if sinks is None and (window_left is None or window_left < 0) and not softcap and alibi_slopes is None:
        return None
    for t, name in ((sinks, "sinks"), (alibi_slopes, "alibi_slopes")):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != num_q_heads):
            raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous float32 [Hq] tensor")
    o = AttnOptions(None if sinks is None else sinks.data_ptr(), -1 if window_left is None else int(window_left),
                    float(softcap or 0.0), None if alibi_slopes is None else alibi_slopes.data_ptr())
    return ctypes.byref(o), o  # keep the struct alive with the reference


def prefill_workspace_bytes(total_q, num_q_heads, head_dim, num_kv_splits):
    return int(lib().pa_prefill_workspace_bytes(total_q, num_q_heads, head_dim, num_kv_splits))


def decode_workspace_bytes(total_q, num_q_heads, head_dim, num_splits):
    return int(lib().pa_decode_workspace_bytes(total_q, num_q_heads, head_dim, num_splits))


def _workspace(workspace, nbytes, device):
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)
    return workspace


def _partials_view(workspace, total_q, Hq, D, splits):
    n = total_q * Hq * splits * (D + 2)
    return workspace.view(torch.float32)[:n].view(total_q, Hq, splits, D + 2)


def paged_prefill(q, k_pages, v_pages, cu_seqlens_q, seq_lens, block_tables, max_seqlen_q, scale,
                  *, k_scale=1.0, v_scale=1.0, num_kv_splits=1, out=None, lse=None,
                  return_lse=False, workspace=None, stream=None, merge=True, k_head_scales=None,
                  v_head_scales=None, sinks=None, window_left=-1, softcap=0.0, alibi_slopes=None):
    """pa_paged_prefill(_ex) on torch tensors; returns out (and lse).
    sinks and alibi_slopes (float32 [Hq] on the device), window_left and
    softcap select the options.

    merge=False (num_kv_splits >= 2): runs the first pass only and returns the
    FP32 records [total_q, Hq, num_kv_splits, D + 2] for merge_states."""
    total_q, Hq, D = q.shape
    if not q.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "q must be contiguous")
    kv = kv_cache(k_pages, v_pages, k_scale, v_scale, k_head_scales, v_head_scales)
    if merge:
        out = torch.empty_like(q) if out is None else out
        if return_lse and lse is None:
            lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    else:
        out = lse = None
    B = int(seq_lens.numel())
    ws_bytes = prefill_workspace_bytes(total_q, Hq, D, num_kv_splits)
    workspace = _workspace(workspace, ws_bytes, q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _options(Hq, sinks, window_left, softcap, alibi_slopes)
    _check(lib().pa_paged_prefill_ex(_ptr(q), _dtype(q), _ptr(out), _ptr(lse),
                                     _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")), _ptr(_i32(seq_lens, "seq_lens")),
                                     _ptr(_i32(block_tables, "block_tables")), B, block_tables.shape[-1],
                                     total_q, int(max_seqlen_q), Hq, ctypes.byref(kv), float(scale),
                                     int(num_kv_splits), opts[0] if opts else None, _ptr(workspace), ws_have,
                                     _stream(stream)))
    if not merge:
        return _partials_view(workspace, total_q, Hq, D, num_kv_splits)
    return (out, lse) if return_lse or lse is not None else out


def split_kv_decode(q, k_pages, v_pages, cu_seqlens_q, seq_lens, block_tables, max_q_per_row, scale,
                    *, num_splits=16, part_keys=0, k_scale=1.0, v_scale=1.0, out=None, lse=None,
                    return_lse=False, workspace=None, stream=None, merge=True, k_head_scales=None,
                    v_head_scales=None, sinks=None, window_left=-1, softcap=0.0, alibi_slopes=None):
    """pa_split_kv_decode on torch tensors; returns out (and lse).

    part_keys > 0: pa_split_kv_decode_fixed, num_splits absolute parts of
    part_keys keys each (the last one running on to the row's end).
    merge=False: runs pass 1 only and returns the FP32 records
    [total_q, Hq, num_splits, D + 2] for merge_states."""
    total_q, Hq, D = q.shape
    if not q.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "q must be contiguous")
    kv = kv_cache(k_pages, v_pages, k_scale, v_scale, k_head_scales, v_head_scales)
    if merge:
        out = torch.empty_like(q) if out is None else out
        if return_lse and lse is None:
            lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    else:
        out = lse = None
    B = int(seq_lens.numel())
    ws_bytes = decode_workspace_bytes(total_q, Hq, D, num_splits)
    workspace = _workspace(workspace, ws_bytes, q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _dtype(q), _ptr(out), _ptr(lse), _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")),
            _ptr(_i32(seq_lens, "seq_lens")), _ptr(_i32(block_tables, "block_tables")), B, block_tables.shape[-1],
            total_q, int(max_q_per_row), Hq, ctypes.byref(kv), float(scale))
    opts = _options(Hq, sinks, window_left, softcap, alibi_slopes)
    _check(lib().pa_split_kv_decode_ex(*args, int(num_splits), int(part_keys), opts[0] if opts else None,
                                       _ptr(workspace), ws_have, _stream(stream)))
    if not merge:
        return _partials_view(workspace, total_q, Hq, D, num_splits)
    return (out, lse) if return_lse or lse is not None else out


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # PA_NOALLOC_SCRATCH_BYTES of include/pagedattn.h


def split_kv_decode_noalloc(q, k_pages, v_pages, cu_seqlens_q, seq_lens, block_tables, max_q_per_row, scale, out,
                            *, num_splits=16, part_keys=0, k_scale=1.0, v_scale=1.0, lse=None, stream=None,
                            k_head_scales=None, v_head_scales=None, sinks=None, window_left=-1, softcap=0.0,
                            alibi_slopes=None):
    """pa_split_kv_decode_noalloc: split_kv_decode into the caller's out (and lse)
    with the records in the library's own device buffer; no workspace, nothing
    allocated by the library or by this wrapper."""
    total_q, Hq, D = q.shape
    if not q.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "q must be contiguous")
    kv = kv_cache(k_pages, v_pages, k_scale, v_scale, k_head_scales, v_head_scales)
    opts = _options(Hq, sinks, window_left, softcap, alibi_slopes)
    _check(lib().pa_split_kv_decode_noalloc(
        _ptr(q), _dtype(q), _ptr(out), _ptr(lse), _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")),
        _ptr(_i32(seq_lens, "seq_lens")), _ptr(_i32(block_tables, "block_tables")), int(seq_lens.numel()),
        block_tables.shape[-1], total_q, int(max_q_per_row), Hq, ctypes.byref(kv), float(scale), int(num_splits),
        int(part_keys), opts[0] if opts else None, _stream(stream)))
    return (out, lse) if lse is not None else out


MIXED_DECODE_MAX_Q = 16  # PA_MIXED_DECODE_MAX_Q of include/pagedattn.h


def _host_i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).astype(np.int32))


def mixed_workspace_bytes(host_q_lens, max_pages_per_seq, num_q_heads, head_dim, q_dtype, decode_max_q,
                          decode_splits, prefill_splits):
    ql = _host_i32(host_q_lens)
    return int(lib().pa_mixed_workspace_bytes(ql.ctypes.data, len(ql), max_pages_per_seq, num_q_heads, head_dim,
                                              q_dtype, decode_max_q, decode_splits, prefill_splits))


def mixed_step(q, k_pages, v_pages, cu_seqlens_q, host_q_lens, seq_lens, block_tables, scale, *, decode_max_q=0,
               decode_splits=16, decode_part_keys=0, prefill_splits=0, k_scale=1.0, v_scale=1.0, out=None, lse=None,
               return_lse=False, workspace=None, stream=None, k_head_scales=None, v_head_scales=None, sinks=None,
               window_left=-1, softcap=0.0, alibi_slopes=None):
    """pa_mixed_step: a batch in any order (host_q_lens: the rows' query
    lengths on the host, e.g. a numpy array or list); rows with 1 <= q <=
    decode_max_q (0: the library's default) take the split-KV decode, the
    others the prefill.  Returns out (and lse)."""
    total_q, Hq, D = q.shape
    if not q.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "q must be contiguous")
    kv = kv_cache(k_pages, v_pages, k_scale, v_scale, k_head_scales, v_head_scales)
    out = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    B = int(seq_lens.numel())
    ql = _host_i32(host_q_lens)
    if len(ql) != B:
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "host_q_lens must have one entry per sequence")
    mp = block_tables.shape[-1]
    ws_bytes = mixed_workspace_bytes(ql, mp, Hq, D, _dtype(q), decode_max_q, decode_splits, prefill_splits)
    workspace = _workspace(workspace, ws_bytes, q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _options(Hq, sinks, window_left, softcap, alibi_slopes)
    _check(lib().pa_mixed_step(_ptr(q), _dtype(q), _ptr(out), _ptr(lse), _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")),
                               ql.ctypes.data, _ptr(_i32(seq_lens, "seq_lens")),
                               _ptr(_i32(block_tables, "block_tables")), B, mp, total_q, Hq, ctypes.byref(kv),
                               float(scale), int(decode_max_q), int(decode_splits), int(decode_part_keys),
                               int(prefill_splits), opts[0] if opts else None, _ptr(workspace), ws_have,
                               _stream(stream)))
    return (out, lse) if return_lse or lse is not None else out


def write_kv(k_new, v_new, k_pages, v_pages, cu_seqlens_q, seq_lens, block_tables, max_q, *, k_scale=1.0,
             v_scale=1.0, stream=None, k_head_scales=None, v_head_scales=None):
    """pa_write_kv: k_new / v_new [total_q, Hkv, D] into the pages at each sequence's
    last q_len positions (uint8 / float8_e5m2 pages: E5M2 of x / scale;
    float8_e4m3fn pages: E4M3 of x / scale)."""
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if not t.is_contiguous() or t.dim() != 3:
            raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous [total_q, Hkv, D] tensor")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "k_new and v_new must share shape and dtype")
    kv = kv_cache(k_pages, v_pages, k_scale, v_scale, k_head_scales, v_head_scales)
    B = int(seq_lens.numel())
    _check(lib().pa_write_kv(_ptr(k_new), _ptr(v_new), _dtype(k_new), _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")),
                             _ptr(_i32(seq_lens, "seq_lens")), _ptr(_i32(block_tables, "block_tables")), B,
                             block_tables.shape[-1], int(k_new.shape[0]), int(max_q), ctypes.byref(kv),
                             _stream(stream)))


def merge_states(partials, out_dtype=torch.float32, *, out=None, lse=None, return_lse=False, stream=None):
    """pa_merge_states: partials [N, H, S, D + 2] float32 -> out [N, H, D]."""
    N, H, S, R = partials.shape
    D = R - 2
    if partials.dtype != torch.float32 or not partials.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID_ARGUMENT, "partials must be contiguous float32")
    out = torch.empty((N, H, D), dtype=out_dtype, device=partials.device) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=partials.device)
    _check(lib().pa_merge_states(_ptr(partials), S, N, H, D, _ptr(out), _TORCH_TO_PA[out.dtype],
                                 _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse or lse is not None else out


def check_supported(q_dtype, kv_dtype, head_dim, page_size, num_q_heads, num_kv_heads):
    """(status, reason) of pa_check_supported; dtypes as PA_* codes."""
    r = ctypes.c_char_p()
    st = lib().pa_check_supported(q_dtype, kv_dtype, head_dim, page_size, num_q_heads, num_kv_heads,
                                  ctypes.byref(r))
    return st, r.value.decode()


def validate_metadata(cu_seqlens_q, seq_lens, block_tables, total_q, max_q, page_size, num_pages):
    """pa_validate_metadata on host (numpy) copies; returns (status, message)."""
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    st = lib().pa_validate_metadata(cu.ctypes.data, sl.ctypes.data, bt.ctypes.data, len(sl),
                                    bt.shape[-1], total_q, max_q, page_size, num_pages)
    return st, (lib().pa_last_error() or b"").decode()


def auto_splits(total_q, num_seqs, max_seqlen_q, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype):
    st = lib().pa_prefill_auto_splits(total_q, num_seqs, max_seqlen_q, num_q_heads, num_kv_heads,
                                      head_dim, q_dtype, kv_dtype)
    if st < 0:
        _check(st)
    return st
