"""Shared plumbing for the GPU tests: upload oracle-built caches (with
poisoned unused slots), call the library, compare with the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from workloads import custom_workload, make_workload

PS = 16
TOL = {"f32": 2e-5, "bf16": 1e-2, "f16": 1e-2, "i8": 1e-2, "fp8": 1e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "i8": torch.int8,
            "fp8": torch.float8_e4m3fn}
SCALED = ("i8", "fp8")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np_to_gpu(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:          # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.uint8:           # FP8 E4M3 codes
        return torch.from_numpy(np.ascontiguousarray(a)).cuda().view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_to_np_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.double().cpu().numpy()


def oracle_cache(w, dtype=None):
    c = oracle.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, dtype or w.kv_dtype)
    oracle.ref_append(c, w.k, w.v, w.slot_mapping)
    return c


@functools.lru_cache(maxsize=2)
def config_case(name):
    """(workload, oracle cache) for a named configuration, built once."""
    w = make_workload(name)
    return w, oracle_cache(w)


def used_slot_mask(w) -> np.ndarray:
    used = np.zeros((w.num_pages, PS), dtype=bool)
    s = w.slot_mapping
    used[s // PS, s % PS] = True
    return used


def poisoned_gpu_cache(cache, used):
    """GPU copy of the pool where every slot no sequence owns holds NaN
    (int8: code 127 and NaN scales), so a read past a context shows up."""
    k, v = cache.k.copy(), cache.v.copy()
    mk, mv = used[:, None, :, None], used[:, None, None, :]
    if cache.dtype == "bf16":
        k = np.where(mk, k, np.uint16(0x7FC0))
        v = np.where(mv, v, np.uint16(0x7FC0))
    elif cache.dtype == "i8":
        k = np.where(mk, k, np.int8(127))
        v = np.where(mv, v, np.int8(127))
    elif cache.dtype == "fp8":
        k = np.where(mk, k, np.uint8(0x7F))     # the E4M3 NaN code
        v = np.where(mv, v, np.uint8(0x7F))
    else:
        k = np.where(mk, k, np.array(np.nan, dtype=k.dtype))
        v = np.where(mv, v, np.array(np.nan, dtype=v.dtype))
    out = {"k": np_to_gpu(k), "v": np_to_gpu(v), "ks": None, "vs": None}
    if cache.dtype in SCALED:
        ms = used[:, None, :]
        out["ks"] = np_to_gpu(np.where(ms, cache.k_scales, np.float32(np.nan)))
        out["vs"] = np_to_gpu(np.where(ms, cache.v_scales, np.float32(np.nan)))
    return out


def q_tensor(w, dtype="f32"):
    t = torch.from_numpy(w.q).cuda()
    return t.to(TORCH_DT[dtype])


def q_exact_values(qt: torch.Tensor) -> np.ndarray:
    return qt.double().cpu().numpy()


def run_decode(pkv, w, gc, q, out_dtype=torch.float32, max_context_len=None, block_tables=None):
    bt = np_to_gpu(w.block_tables if block_tables is None else block_tables)
    cl = np_to_gpu(w.context_lens)
    mcl = w.max_context_len if max_context_len is None else max_context_len
    out = pkv.paged_attn_decode(q, gc["k"], gc["v"], bt, cl, mcl, w.scale, out_dtype=out_dtype,
                                k_scales=gc["ks"], v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


def run_prefill(pkv, w, gc, q, out_dtype=torch.float32, max_context_len=None):
    bt = np_to_gpu(w.block_tables)
    cl = np_to_gpu(w.context_lens)
    cu = np_to_gpu(w.cu_q_lens)
    mcl = w.max_context_len if max_context_len is None else max_context_len
    out = pkv.paged_attn_prefill_chunk(q, gc["k"], gc["v"], bt, cl, cu, w.max_q_len, mcl,
                                       w.scale, out_dtype=out_dtype, k_scales=gc["ks"],
                                       v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


def small_decode(ctx, hq, hkv, d, kv, seed, **kw):
    return custom_workload(context_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                           kv_dtype=kv, seed=seed, **kw)


def small_prefill(ctx, qlens, hq, hkv, d, kv, seed, **kw):
    return custom_workload(kind="prefill", context_lens=ctx, q_lens=qlens, num_q_heads=hq,
                           num_kv_heads=hkv, head_dim=d, kv_dtype=kv, seed=seed, **kw)
