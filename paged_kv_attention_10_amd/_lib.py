"""ctypes binding of libpkv.so: argument marshalling only.

Every function here takes torch tensors that already live on the GPU, checks
that they are dense and on the device, and passes raw pointers, sizes and
the current HIP stream to the library.  There is no computation and no
fallback: if libpkv.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")

F32, BF16, F16, I8, FP8 = 0, 1, 2, 3, 4
PAGE_SIZE = 16
_TORCH_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.int8: I8,
               torch.float8_e4m3fn: FP8}

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


ABI_VERSION = 4   # PKV_ABI_VERSION of include/pkv.h this binding marshals for
NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with paged_kv_attention_10_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.pkv_abi_version.restype = _c_int
    lib.pkv_abi_version.argtypes = []
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [_c_int]
    lib.paged_kv_append.restype = _c_int
    lib.paged_kv_append.argtypes = [_vp, _vp, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _vp]
    lib.paged_kv_append_rope.restype = _c_int
    lib.paged_kv_append_rope.argtypes = [_vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _c_int, _c_int,
                                         _c_float, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _vp]
    lib.paged_attn_decode.restype = _c_int
    lib.paged_attn_decode.argtypes = [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp,
                                      _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_float, _c_int, _vp, _c_int, _vp, _c_size, _vp]
    lib.paged_attn_decode_append.restype = _c_int
    lib.paged_attn_decode_append.argtypes = [_vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp,
                                             _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_float, _c_int, _vp, _c_int, _vp,
                                             _c_size, _vp]
    lib.paged_attn_decode_noalloc.restype = _c_int
    lib.paged_attn_decode_noalloc.argtypes = [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int,
                                              _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                              _c_int, _c_float, _c_int, _vp, _c_int, _vp]
    lib.paged_attn_decode_workspace_bytes.restype = _c_size
    lib.paged_attn_decode_workspace_bytes.argtypes = [_c_int] * 6
    lib.paged_attn_prefill_chunk.restype = _c_int
    lib.paged_attn_prefill_chunk.argtypes = [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int,
                                             _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                             _vp, _c_int, _vp, _c_size, _vp]
    lib.paged_attn_prefill_workspace_bytes.restype = _c_size
    lib.paged_attn_prefill_workspace_bytes.argtypes = [_c_int] * 7
    lib.paged_attn_mixed.restype = _c_int
    lib.paged_attn_mixed.argtypes = lib.paged_attn_prefill_chunk.argtypes
    lib.paged_attn_mixed_workspace_bytes.restype = _c_size
    lib.paged_attn_mixed_workspace_bytes.argtypes = [_c_int] * 7
    if lib.pkv_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.pkv_abi_version()}, this binding needs "
                          f"{ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/pkv.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s\*]+([A-Za-z_]\w*)\s*\(", text, flags=re.M)


def _check(fn: str, status: int):
    if status != 0:
        raise PkvError(fn, status, load_library().pkv_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("pkv works on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("pkv needs contiguous tensors")


def _code(t) -> int:
    try:
        return _TORCH_CODE[t.dtype]
    except KeyError:
        raise ValueError(f"dtype {t.dtype} is not a pkv dtype") from None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pkv_abi_version() -> int:
    return load_library().pkv_abi_version()


def pkv_status_string(status: int) -> str:
    return load_library().pkv_status_string(status).decode()


def paged_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales=None, v_scales=None,
                    stream=None) -> None:
    """k_new/v_new [T, Hkv, d]; slot_mapping int64 [T]; pool tensors as in pkv.h."""
    _dev(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales)
    num_pages, hkv, page, d = k_cache.shape
    _check("paged_kv_append", load_library().paged_kv_append(
        _ptr(k_new), _ptr(v_new), _code(k_new), _ptr(slot_mapping), int(slot_mapping.numel()),
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _code(k_cache),
        num_pages, hkv, d, page, _stream(stream)))


ROPE_STYLES = {"half": 1, "interleaved": 2}


def paged_kv_append_rope(k_new, v_new, slot_mapping, positions, k_cache, v_cache, rope_theta,
                         rope_style="half", q=None, k_scales=None, v_scales=None,
                         stream=None) -> None:
    """paged_kv_append with RoPE on K; positions int32 [T]; q (optional)
    [T, Hq, d] is rotated in place.  rope_style "half" or "interleaved"."""
    _dev(k_new, v_new, slot_mapping, positions, k_cache, v_cache, k_scales, v_scales, q)
    num_pages, hkv, page, d = k_cache.shape
    hq = 0 if q is None else int(q.shape[1])
    _check("paged_kv_append_rope", load_library().paged_kv_append_rope(
        _ptr(k_new), _ptr(v_new), _code(k_new), _ptr(slot_mapping), _ptr(positions),
        int(slot_mapping.numel()), _ptr(q), 0 if q is None else _code(q), hq, float(rope_theta),
        ROPE_STYLES[rope_style], _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _code(k_cache), num_pages, hkv, d, page, _stream(stream)))


def paged_attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len, window=0) -> int:
    return int(load_library().paged_attn_decode_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, max_context_len, window))


def paged_attn_prefill_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_q_len,
                                       max_context_len, window=0) -> int:
    return int(load_library().paged_attn_prefill_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, max_q_len, max_context_len, window))


def _workspace(nbytes, workspace, device):
    if nbytes == 0:
        return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                      out=None, out_dtype=torch.float32, k_scales=None, v_scales=None,
                      workspace=None, stream=None, window=0):
    """q [B, Hq, d] -> out [B, Hq, d].  block_tables int32 [B, W],
    context_lens int32 [B] (each <= max_context_len); window 0 = whole context."""
    B, hq, d = q.shape
    num_pages, hkv, page, _ = k_cache.shape
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=q.device)
    _dev(q, k_cache, v_cache, block_tables, context_lens, out, k_scales, v_scales)
    nbytes = paged_attn_decode_workspace_bytes(B, hq, hkv, d, max_context_len, window)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("paged_attn_decode", load_library().paged_attn_decode(
        _ptr(q), _code(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _code(k_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
        int(max_context_len), B, hq, hkv, d, page, num_pages, float(scale), int(window),
        _ptr(out), _code(out), _ptr(workspace), wbytes, _stream(stream)))
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                              scale, out, k_scales=None, v_scales=None, stream=None, window=0):
    """paged_attn_decode with its split partials in the library's static
    device scratch: nothing is allocated (the caller passes `out`)."""
    B, hq, d = q.shape
    num_pages, hkv, page, _ = k_cache.shape
    _dev(q, k_cache, v_cache, block_tables, context_lens, out, k_scales, v_scales)
    _check("paged_attn_decode_noalloc", load_library().paged_attn_decode_noalloc(
        _ptr(q), _code(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _code(k_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
        int(max_context_len), B, hq, hkv, d, page, num_pages, float(scale), int(window),
        _ptr(out), _code(out), _stream(stream)))
    return out


def paged_attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                             max_context_len, scale, out=None, out_dtype=torch.float32,
                             workspace=None, stream=None, window=0, k_scales=None, v_scales=None):
    """One decode step: k_new/v_new [B, Hkv, d] go to position
    context_lens[b] - 1 (int8 / FP8 caches: quantised as paged_kv_append
    does, scales written to k_scales / v_scales), then q [B, Hq, d]
    attends -> out [B, Hq, d]."""
    B, hq, d = q.shape
    num_pages, hkv, page, _ = k_cache.shape
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=q.device)
    _dev(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, out, k_scales, v_scales)
    nbytes = paged_attn_decode_workspace_bytes(B, hq, hkv, d, max_context_len, window)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check("paged_attn_decode_append", load_library().paged_attn_decode_append(
        _ptr(q), _code(q), _ptr(k_new), _ptr(v_new), _code(k_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scales), _ptr(v_scales), _code(k_cache), _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(context_lens),
        int(max_context_len), B, hq, hkv, d, page, num_pages, float(scale), int(window),
        _ptr(out), _code(out), _ptr(workspace), wbytes, _stream(stream)))
    return out


def paged_attn_mixed_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_q_len,
                                     max_context_len, window=0) -> int:
    return int(load_library().paged_attn_mixed_workspace_bytes(
        batch, num_q_heads, num_kv_heads, head_dim, max_q_len, max_context_len, window))


def paged_attn_mixed(q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, max_q_len,
                     max_context_len, scale, out=None, out_dtype=torch.float32, k_scales=None,
                     v_scales=None, workspace=None, stream=None, window=0):
    """Same arguments and result as paged_attn_prefill_chunk; one-token chunks
    run as split decode partitions in the same launch."""
    return _varlen("paged_attn_mixed", paged_attn_mixed_workspace_bytes, q, k_cache, v_cache,
                   block_tables, context_lens, cu_q_lens, max_q_len, max_context_len, scale, out,
                   out_dtype, k_scales, v_scales, workspace, stream, window)


def paged_attn_prefill_chunk(q, k_cache, v_cache, block_tables, context_lens, cu_q_lens,
                             max_q_len, max_context_len, scale, out=None,
                             out_dtype=torch.float32, k_scales=None, v_scales=None,
                             workspace=None, stream=None, window=0):
    """q [T, Hq, d] -> out [T, Hq, d]; cu_q_lens int32 [B+1]; context_lens
    int32 [B] = prefix + chunk; window 0 = the whole causal prefix."""
    return _varlen("paged_attn_prefill_chunk", paged_attn_prefill_workspace_bytes, q, k_cache,
                   v_cache, block_tables, context_lens, cu_q_lens, max_q_len, max_context_len,
                   scale, out, out_dtype, k_scales, v_scales, workspace, stream, window)


def _varlen(fn, ws_query, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, max_q_len,
            max_context_len, scale, out, out_dtype, k_scales, v_scales, workspace, stream, window):
    T, hq, d = q.shape
    B = int(context_lens.shape[0])
    num_pages, hkv, page, _ = k_cache.shape
    if out is None:
        out = torch.empty((T, hq, d), dtype=out_dtype, device=q.device)
    _dev(q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, out, k_scales, v_scales)
    nbytes = ws_query(B, hq, hkv, d, max_q_len, max_context_len, window)
    workspace, wbytes = _workspace(nbytes, workspace, q.device)
    _check(fn, getattr(load_library(), fn)(
        _ptr(q), _code(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _code(k_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
        _ptr(cu_q_lens), T, int(max_q_len), int(max_context_len), B, hq, hkv, d, page,
        num_pages, float(scale), int(window), _ptr(out), _code(out), _ptr(workspace), wbytes,
        _stream(stream)))
    return out
