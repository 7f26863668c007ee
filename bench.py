#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

Headline workload: paged decode with a bf16 KV cache at the Qwen2.5-1.5B
attention shape (batch 64, 12 query / 2 KV heads, head_dim 128, 16-token
pages, context lengths uniform in [512, 4096], pages scattered over a
20k-page pool).  One step = the step's 64 new tokens appended + the decode
over every context, as one fused call (paged_attn_decode_append: the
split-context partition kernel, which also stores the new tokens and, when
a context is split into at most eight partitions, merges them by their
log-sum-exps in the same launch; longer plans add the reduce kernel); the
same step as two calls (append, then decode) is reported beside it.  Before every
timed step a 1 GiB read evicts L2 and the 256 MB MALL, so every step reads
its KV from HBM; each step is timed with HIP events on the stream the
library launches on (the flush is outside the events).

value = effective KV bytes (sum of context tokens x KV heads x head_dim x
2 (K and V) x bytes per element) / mean step time, in GB/s.

Also reported in the same line: the chunked-prefill workload (8 x 512-token
bf16 chunks over prefixes uniform in [0, 3584], Qwen2.5-1.5B heads) in
algorithmic TFLOP/s, the other decode shapes (fp16-KV Stories110M shape,
int8-KV TinyLlama shape, small fp32 case), the roofline of each dominant
kernel, and the CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
ELEM = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1, "fp8": 1}
DESC = {
    "C1": "paged decode, fp32 q/KV/out, batch 4, 9 q / 3 KV heads, head_dim 64, ctx {17,64,133,200}",
    "C2": "paged decode, bf16 KV + fp32 accumulation, Qwen2.5-1.5B shape: batch 64, 12 q / 2 KV heads, head_dim 128, ctx U[512,4096], 20k-page pool",
    "C3": "paged decode, fp16 KV, Stories110M shape: batch 384, 12 q / 12 KV heads, head_dim 64, ctx U[64,1024]",
    "C4": "chunked causal prefill, bf16 q/KV, Qwen2.5-1.5B shape: 8 x 512-token chunks over prefixes U[0,3584], 12 q / 2 KV heads, head_dim 128",
    "C5": "paged decode, int8 KV + per-token-head fp32 scales, TinyLlama-1.1B shape: batch 128, 32 q / 4 KV heads, head_dim 64, ctx 2048",
    "M1": "mixed batch in one call: the C2 decode batch (64 one-token chunks, ctx U[512,4096]) and the C4 chunks (8 x 512 tokens), 12 q / 2 KV heads, head_dim 128, bf16",
    "R1": "append with RoPE on K and q (rotate-half, theta 1e6), the C4 chunks' 4096 new tokens, bf16 K/V/q in and bf16 cache, 12 q / 2 KV heads, head_dim 128",
    "F1": "paged decode, FP8 E4M3 KV + per-token-head fp32 scales, the C2 draw (Qwen2.5-1.5B shape: batch 64, 12 q / 2 KV heads, head_dim 128, ctx U[512,4096])",
    "W1": "sliding-window paged decode, bf16 KV, Qwen2.5-1.5B shape: batch 64, 12 q / 2 KV heads, head_dim 128, ctx U[16384,65536], window 4096, only the window's pages held (earlier block-table entries evicted)",
    "M2": "decode-heavy mixed batch in one call: the C2 decode batch (64 one-token chunks, ctx U[512,4096]) and 4 chunks of 64 tokens over 1024-token prefixes, 12 q / 2 KV heads, head_dim 128, bf16",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def effective_kv_bytes(w) -> int:
    """K and V bytes the decode must read: every context token, or with a
    sliding window the window's tokens."""
    win = int(w.meta.get("window", 0))
    ctx = w.context_lens.astype(np.int64)
    tok = int((np.minimum(ctx, win) if win else ctx).sum())
    b = tok * w.num_kv_heads * w.head_dim * 2 * ELEM[w.kv_dtype]
    if w.kv_dtype in ("i8", "fp8"):
        b += tok * w.num_kv_heads * 2 * 4
    return b


def prefill_flops(w) -> int:
    total = 0
    for b in range(w.batch):
        C = int(w.q_lens[b])
        P = int(w.context_lens[b]) - C
        total += C * P + C * (C + 1) // 2          # sum_i (P + i + 1)
    return 4 * w.head_dim * w.num_q_heads * total


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_attention_10_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(profile_name: str, sha: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha256:\s*(\S+)", text, re.M)
    m_tr = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_tr or m_sha.group(1) != sha:
        return None
    return float(m_tr.group(1))


def profiled_mfma_busy(profile_name: str, sha: str):
    """MFMA busy fraction from a committed counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha256:\s*(\S+)", text, re.M)
    m_u = re.search(r"^mfma_busy_frac:\s*([0-9.eE+-]+)", text, re.M)
    if not m_sha or not m_u or m_sha.group(1) != sha:
        return None
    return float(m_u.group(1))


class Gpu:
    def __init__(self):
        import torch
        import paged_kv_attention_10_amd as pkv
        self.torch, self.pkv = torch, pkv
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.flush_buf = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device=self.dev)

    def flush(self):
        # 1 GiB read (no writes, so no dirty lines are left to drain during
        # the timed call): evicts L2 and the 256 MB MALL
        self.flush_buf.sum()

    def t(self, a):
        return self.torch.from_numpy(a).to(self.dev)

    def pool(self, w):
        torch = self.torch
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "i8": torch.int8,
              "fp8": torch.float8_e4m3fn}[w.kv_dtype]
        k = torch.zeros((w.num_pages, w.num_kv_heads, 16, w.head_dim), dtype=dt, device=self.dev)
        v = torch.zeros((w.num_pages, w.num_kv_heads, w.head_dim, 16), dtype=dt, device=self.dev)
        ks = vs = None
        if w.kv_dtype in ("i8", "fp8"):
            ks = torch.zeros((w.num_pages, w.num_kv_heads, 16), dtype=torch.float32, device=self.dev)
            vs = torch.zeros_like(ks)
        return k, v, ks, vs

    def fill_pool(self, w, pool, rows):
        """Append the tokens at `rows` (fp32 K/V) into the pool on the GPU."""
        k, v, ks, vs = pool
        step = 1 << 17
        for i in range(0, len(rows), step):
            r = rows[i:i + step]
            self.pkv.paged_kv_append(self.t(w.k[r]), self.t(w.v[r]), self.t(w.slot_mapping[r]),
                                     k, v, ks, vs)
        self.torch.cuda.synchronize()

    def timed_steps(self, step_fn, inner_fn, steps, warmup, flush=True):
        """Run warmup, then two timed passes of `steps` steps each, every step
        preceded by the flush (outside the events).  Pass one brackets whole
        steps with events (nothing else recorded inside them); pass two
        brackets only `inner_fn`, the dominant call, so the step time carries
        no event of the inner timing."""
        torch = self.torch
        for _ in range(warmup):
            if flush:
                self.flush()
            step_fn(inner_fn)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush:
                self.flush()
            ev[i][0].record()
            step_fn(inner_fn)
            ev[i][3].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(steps):
            if flush:
                self.flush()
            step_fn(inner_fn, ev[i][1], ev[i][2])
        torch.cuda.synchronize()
        step_ms = [e[0].elapsed_time(e[3]) for e in ev]
        inner_ms = [e[1].elapsed_time(e[2]) for e in ev]
        return step_ms, inner_ms, wall


def stats(xs):
    s = sorted(xs)
    n = len(s)
    return {"mean": sum(s) / n, "median": s[n // 2], "p10": s[int(0.1 * (n - 1))],
            "p90": s[int(0.9 * (n - 1))]}


def bench_decode(g: Gpu, name: str, steps: int, warmup: int):
    """One step = the step's new tokens appended + the decode call, as one
    fused call (paged_attn_decode_append; int8 / FP8 caches quantise the
    new rows in it); the same step as two calls (paged_kv_append, then
    paged_attn_decode) is timed beside it."""
    from workloads import make_workload
    w = make_workload(name)
    log(f"[bench] {name}: building the pool on the GPU")
    pool = g.pool(w)
    new_rows = w.new_token_rows()
    old_mask = g.torch.ones(len(w.slot_mapping), dtype=g.torch.bool).numpy()
    old_mask[new_rows] = False
    g.fill_pool(w, pool, old_mask.nonzero()[0])
    k, v, ks, vs = pool
    k_new, v_new = g.t(w.k[new_rows]), g.t(w.v[new_rows])
    slots_new = g.t(w.slot_mapping[new_rows])
    q = g.t(w.q)
    bt, cl = g.t(w.block_tables), g.t(w.context_lens)
    out = g.torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=g.torch.float32, device=g.dev)
    window = int(w.meta.get("window", 0))
    nws = g.pkv.paged_attn_decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads,
                                                  w.head_dim, w.max_context_len, window)
    ws = g.torch.zeros(max(nws, 16), dtype=g.torch.uint8, device=g.dev)
    fused = True

    def decode():
        g.pkv.paged_attn_decode(q, k, v, bt, cl, w.max_context_len, w.scale, out=out,
                                k_scales=ks, v_scales=vs, workspace=ws, window=window)

    def decode_step():
        g.pkv.paged_attn_decode_append(q, k_new, v_new, k, v, bt, cl, w.max_context_len, w.scale,
                                       out=out, workspace=ws, window=window, k_scales=ks,
                                       v_scales=vs)

    def two_calls(inner, e1=None, e2=None):
        g.pkv.paged_kv_append(k_new, v_new, slots_new, k, v, ks, vs)
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    def one_call(inner, e1=None, e2=None):
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    log(f"[bench] {name}: {warmup} warmup + {steps} timed steps")
    if fused:
        step_ms, inner_ms, wall = g.timed_steps(one_call, decode_step, steps, warmup)
        two_ms, dec_ms, _ = g.timed_steps(two_calls, decode, steps, warmup)
    else:
        step_ms, inner_ms, wall = g.timed_steps(two_calls, decode, steps, warmup)
        two_ms, dec_ms = step_ms, inner_ms
    nbytes = effective_kv_bytes(w)
    st, si, sd = stats(step_ms), stats(inner_ms), stats(dec_ms)
    res = {
        "workload": name, "desc": DESC[name], "effective_kv_bytes": nbytes,
        "step": ("paged_attn_decode_append (the new tokens appended and attended in one launch)"
                 if fused else "paged_kv_append, then paged_attn_decode"),
        "ms_per_step": st["mean"], "step_ms": st, "decode_call_ms": si,
        "two_call_step_ms": stats(two_ms), "decode_only_call_ms": sd,
        "kv_gbs": nbytes / (st["mean"] * 1e-3) / 1e9,
        "seq_tokens_per_s": w.batch / (st["mean"] * 1e-3),
        "context_tokens_per_s": float(w.context_lens.sum()) / (st["mean"] * 1e-3),
        "decode_call_gbs": nbytes / (si["mean"] * 1e-3) / 1e9,
        "decode_only_call_gbs": nbytes / (sd["mean"] * 1e-3) / 1e9,
        "wall_s_timed_region": wall,
        "plan_workspace_bytes": int(nws),
    }
    res["hbm_frac_step"] = res["kv_gbs"] / HBM_PEAK_GBS
    if name == "C2":
        res["paged_overhead"] = paged_overhead(g, w, pool, decode, out, q, ws, steps, warmup)
    return w, res, out


def paged_overhead(g: Gpu, w, pool, decode_scattered, out_scattered, q, ws, steps, warmup):
    """The plain decode call over the same K/V gathered into consecutive
    pages (identity block table: sequence b's logical page i at physical
    page off_b + i) against the scattered pool; the two outputs must agree
    bit for bit (same kernels, same plan, only the page addresses differ).
    Context: TinyLoop's table "KV cache modes" lists paged attention with
    16-token pages at 5.6% overhead."""
    torch = g.torch
    k, v, _, _ = pool
    npg = (w.context_lens.astype(np.int64) + 15) // 16
    off = np.concatenate([[0], np.cumsum(npg)[:-1]])
    src = np.concatenate([w.block_tables[b, :npg[b]] for b in range(w.batch)]).astype(np.int64)
    src_t = g.t(src)
    k_id, v_id = k.index_select(0, src_t), v.index_select(0, src_t)
    bt_id = np.zeros_like(w.block_tables)
    for b in range(w.batch):
        bt_id[b, :npg[b]] = off[b] + np.arange(npg[b])
    bt_id_t, cl = g.t(bt_id), g.t(w.context_lens)
    out_id = torch.empty_like(out_scattered)
    ws_id = torch.zeros_like(ws)

    def decode_identity():
        g.pkv.paged_attn_decode(q, k_id, v_id, bt_id_t, cl, w.max_context_len, w.scale, out=out_id,
                                workspace=ws_id)

    def one_call(inner, e1=None, e2=None):
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    log("[bench] C2: paged overhead (identity block table vs scattered pages)")
    _, sc_ms, _ = g.timed_steps(one_call, decode_scattered, steps, warmup)
    _, id_ms, _ = g.timed_steps(one_call, decode_identity, steps, warmup)
    torch.cuda.synchronize()
    same = bool(torch.equal(out_id.view(torch.int32), out_scattered.view(torch.int32)))
    ss, si = stats(sc_ms), stats(id_ms)
    return {"scattered_call_ms": ss, "identity_call_ms": si,
            "overhead": ss["mean"] / si["mean"] - 1.0, "outputs_bit_identical": same,
            "pages": int(npg.sum())}


PREFILL_VARIANTS = {
    # name: (KV dtype, query dtype)
    "C4": ("bf16", "bf16"),
    "C4i8": ("i8", "bf16"),
    "C4fp8": ("fp8", "bf16"),
    "C4q32": ("bf16", "f32"),
    "C4f32": ("f32", "f32"),
}


def bench_prefill(g: Gpu, steps: int, warmup: int, name: str = "C4"):
    """One step = the chunks' K/V appended + the prefill call, on C4's batch
    with the KV cache and query dtypes of PREFILL_VARIANTS[name]."""
    from workloads import make_workload
    kv, qd = PREFILL_VARIANTS[name]
    w = make_workload("C4")
    w.kv_dtype = kv
    log(f"[bench] {name}: building the prefix pool on the GPU ({kv} KV, {qd} q)")
    pool = g.pool(w)
    new_rows = w.new_token_rows()
    old_mask = g.torch.ones(len(w.slot_mapping), dtype=g.torch.bool).numpy()
    old_mask[new_rows] = False
    g.fill_pool(w, pool, old_mask.nonzero()[0])
    k, v, ks, vs = pool
    k_new, v_new = g.t(w.k[new_rows]), g.t(w.v[new_rows])
    slots_new = g.t(w.slot_mapping[new_rows])
    q = g.t(w.q).to({"bf16": g.torch.bfloat16, "f32": g.torch.float32}[qd])
    peak = FP32_PEAK_TFLOPS if kv == "f32" else BF16_PEAK_TFLOPS
    bt, cl, cu = g.t(w.block_tables), g.t(w.context_lens), g.t(w.cu_q_lens)
    out = g.torch.empty((w.num_query_tokens, w.num_q_heads, w.head_dim), dtype=g.torch.float32,
                        device=g.dev)

    def prefill():
        g.pkv.paged_attn_prefill_chunk(q, k, v, bt, cl, cu, w.max_q_len, w.max_context_len,
                                       w.scale, out=out, k_scales=ks, v_scales=vs)

    def step(inner, e1=None, e2=None):
        g.pkv.paged_kv_append(k_new, v_new, slots_new, k, v, ks, vs)
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    log(f"[bench] {name}: {warmup} warmup + {steps} timed steps")
    step_ms, inner_ms, wall = g.timed_steps(step, prefill, steps, warmup)
    flops = prefill_flops(w)
    st, si = stats(step_ms), stats(inner_ms)
    res = {
        "workload": name, "desc": DESC["C4"], "kv_dtype": kv, "q_dtype": qd,
        "algorithmic_flops": flops,
        "prefix_lens": w.meta["prefix_lens"].tolist(),
        "ms_per_step": st["mean"], "step_ms": st, "prefill_call_ms": si,
        "tflops_step": flops / (st["mean"] * 1e-3) / 1e12,
        "tflops_prefill_call": flops / (si["mean"] * 1e-3) / 1e12,
        "prefill_tokens_per_s": w.num_query_tokens / (st["mean"] * 1e-3),
        "wall_s_timed_region": wall,
    }
    if name != "C4":
        # the peak of the MFMA the kernel runs: bf16 / fp16 dense 2.5 PFLOP/s
        # (16-bit and one-byte caches), fp32 157.3 TFLOP/s (fp32 cache);
        # counters are taken for the bf16 batch only
        res["roofline"] = {"bound": "mfma", "achieved": res["tflops_prefill_call"],
                           "peak": peak, "unit": "TFLOP/s",
                           "frac": res["tflops_prefill_call"] / peak,
                           "traffic": profiled_traffic(f"prefill_{name}_counters.txt",
                                                       source_sha("prefill.hip", "prefill_body.h", "pkv_device.h", "pkv_host.h"))}
        return w, res, out
    res["roofline"] = {"bound": "mfma", "achieved": res["tflops_prefill_call"],
                       "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": res["tflops_prefill_call"] / BF16_PEAK_TFLOPS,
                       "traffic": profiled_traffic("prefill_C4_counters.txt",
                                                   source_sha("prefill.hip", "prefill_body.h", "pkv_device.h", "pkv_host.h")),
                       "mfma_busy_frac_counters": profiled_mfma_busy(
                           "prefill_C4_mfma.txt",
                           source_sha("prefill.hip", "prefill_body.h", "pkv_device.h", "pkv_host.h"))}
    return w, res, out


def mixed_workload(name):
    """M1: C2's 64 decode sequences and C4's eight 512-token chunks in one
    batch.  M2 (decode-heavy): C2's 64 decode sequences and four 64-token
    chunks over 1024-token prefixes.  Same heads, head_dim 128, bf16 q and
    KV, seeded draw (workloads.make_workload)."""
    from workloads import make_workload
    return make_workload(name)


def bench_mixed(g: Gpu, name: str, steps: int, warmup: int):
    w = mixed_workload(name)
    log(f"[bench] {name}: building the pool on the GPU")
    pool = g.pool(w)
    g.fill_pool(w, pool, g.torch.arange(len(w.slot_mapping)).numpy())
    k, v, _, _ = pool
    q = g.t(w.q).to(g.torch.bfloat16)
    bt, cl, cu = g.t(w.block_tables), g.t(w.context_lens), g.t(w.cu_q_lens)
    out = g.torch.empty((w.num_query_tokens, w.num_q_heads, w.head_dim), dtype=g.torch.float32,
                        device=g.dev)
    nws = g.pkv.paged_attn_mixed_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, w.max_q_len, w.max_context_len)
    ws = g.torch.zeros(max(nws, 16), dtype=g.torch.uint8, device=g.dev)

    def mixed():
        g.pkv.paged_attn_mixed(q, k, v, bt, cl, cu, w.max_q_len, w.max_context_len, w.scale,
                               out=out, workspace=ws)

    def prefill_only():
        g.pkv.paged_attn_prefill_chunk(q, k, v, bt, cl, cu, w.max_q_len, w.max_context_len,
                                       w.scale, out=out)

    def step(inner, e1=None, e2=None):
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    log(f"[bench] {name}: {warmup} warmup + {steps} timed steps, mixed and prefill-only calls")
    _, mixed_ms, _ = g.timed_steps(step, mixed, steps, warmup)
    _, pre_ms, _ = g.timed_steps(step, prefill_only, steps, warmup)
    sm, sp = stats(mixed_ms), stats(pre_ms)
    return {
        "workload": name, "desc": DESC[name],
        "mixed_call_ms": sm, "prefill_chunk_call_ms": sp,
        "speedup_vs_prefill_chunk": sp["mean"] / sm["mean"],
        "query_tokens_per_s": w.num_query_tokens / (sm["mean"] * 1e-3),
        "decode_tokens": 64, "prefill_tokens": int(w.num_query_tokens) - 64,
        "plan_workspace_bytes": int(nws),
    }


def bench_ceiling(g: Gpu, sizes, steps: int, warmup: int):
    """The practical streaming-read ceiling: libpkv_probe.so's read-only
    kernel (hand-written HIP, outside the library, see csrc/probe.hip)
    reads `nbytes` of a 1 GiB device buffer once, after the same 1 GiB
    flush as every timed call, HIP events on the stream it runs on.  Five
    grid sizes (256 to 4096 workgroups); the fastest is reported, labelled
    as a measured probe."""
    import ctypes
    torch = g.torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_attention_10_amd", "libpkv_probe.so"))
    lib.pkv_probe_stream_read.restype = ctypes.c_int
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device=g.dev)
    out = torch.zeros(1 << 14, dtype=torch.int32, device=g.dev)
    stream = torch.cuda.current_stream()
    res = []
    for nbytes in sizes:
        nbytes = min(int(nbytes) // 16 * 16, buf.numel())
        best = None
        for wg in (256, 512, 1024, 2048, 4096):
            ms = []
            for i in range(warmup + steps):
                g.flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = lib.pkv_probe_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), wg,
                                               ctypes.c_void_p(stream.cuda_stream))
                e1.record(stream)
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"streaming-read probe failed ({rc})")
                if i >= warmup:
                    ms.append(e0.elapsed_time(e1))
            st = stats(ms)
            gbs = nbytes / (st["median"] * 1e-3) / 1e9
            if best is None or gbs > best["gbs"]:
                best = {"bytes": nbytes, "workgroups": wg, "call_ms": st, "gbs": gbs,
                        "frac_of_peak": gbs / HBM_PEAK_GBS}
        res.append(best)
    return {"kind": "measured streaming-read probe (read-only HIP kernel outside the library, "
                    "16-byte non-temporal loads, cold after the 1 GiB flush); median of the timed "
                    "calls, fastest of 256/512/1024/2048/4096 workgroups",
            "reads": res}


def bench_rope(g: Gpu, steps: int, warmup: int):
    """R1: the fused append with RoPE (K rotated and stored, V stored, q
    rotated in place) against the plain append of the same K/V."""
    from workloads import make_workload
    torch = g.torch
    w = make_workload("C4")
    rows = w.new_token_rows()
    T = len(rows)
    k, v, _, _ = g.pool(w)
    k_new = g.t(w.k[rows]).to(torch.bfloat16)
    v_new = g.t(w.v[rows]).to(torch.bfloat16)
    slots = g.t(w.slot_mapping[rows])
    q = g.t(w.q).to(torch.bfloat16)
    pos = torch.cat([torch.arange(int(c) - int(n), int(c), dtype=torch.int32)
                     for c, n in zip(w.context_lens, w.q_lens)]).to(g.dev)
    assert pos.numel() == T == q.shape[0]

    def fused():
        g.pkv.paged_kv_append_rope(k_new, v_new, slots, pos, k, v, 1e6, "half", q=q)

    def plain():
        g.pkv.paged_kv_append(k_new, v_new, slots, k, v)

    def step(inner, e1=None, e2=None):
        if e1 is not None:
            e1.record()
        inner()
        if e2 is not None:
            e2.record()

    log(f"[bench] R1: {warmup} warmup + {steps} timed steps, fused RoPE append and plain append")
    _, f_ms, _ = g.timed_steps(step, fused, steps, warmup)
    _, p_ms, _ = g.timed_steps(step, plain, steps, warmup)
    sf, sp = stats(f_ms), stats(p_ms)
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    # read K, V, q, slots, positions; write K, V (bf16) and q
    nbytes = T * (2 * (2 * hkv * d + hq * d) * 2 + 8 + 4)
    gbs = nbytes / (sf["mean"] * 1e-3) / 1e9
    return {
        "workload": "R1", "desc": DESC["R1"], "tokens": T,
        "fused_call_ms": sf, "plain_append_call_ms": sp,
        "algorithmic_bytes": nbytes, "fused_gbs": gbs,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("append_rope_R1_counters.txt",
                                                 source_sha("append.hip", "pkv_device.h", "pkv_host.h"))},
    }


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, gpu_out, budget_s: float):
    """The oracle as it stands, timed on the host: one step = oracle append
    of the step's new tokens + oracle decode of the whole batch, repeated
    until `budget_s` of CPU work; also the parity of the GPU output."""
    from threadpoolctl import threadpool_info
    import oracle
    log("[bench] cpu baseline: oracle cache build (untimed)")
    cache = oracle.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, w.kv_dtype)
    new_rows = w.new_token_rows()
    old = np.ones(len(w.slot_mapping), dtype=bool)
    old[new_rows] = False
    oracle.ref_append(cache, w.k[old], w.v[old], w.slot_mapping[old])
    times = []
    ref = None
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.ref_append(cache, w.k[new_rows], w.v[new_rows], w.slot_mapping[new_rows])
        ref = oracle.ref_decode(w.q, cache, w.block_tables, w.context_lens, w.scale,
                                w.num_q_heads)
        times.append(time.perf_counter() - t0)
        log(f"[bench] cpu baseline step {len(times)}: {times[-1]:.2f} s")
        if time.perf_counter() >= t_end:
            break
    mean = sum(times) / len(times)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    err = oracle.max_abs_err(gpu_out.double().cpu().numpy(), ref)
    return {
        "value": effective_kv_bytes(w) / mean / 1e9, "unit": "GB/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"the whole {w.name} batch ({w.batch} sequences), oracle append of the "
                  f"step's {len(new_rows)} new tokens + fp64 numpy decode, {len(times)} steps "
                  f"in {sum(times):.1f} s; affinity {len(os.sched_getaffinity(0))} cores",
        "seconds_per_step": mean,
        "gpu_vs_oracle_max_abs_err": err,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle CPU work for the baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma list of workloads to run (C1..C5, C4i8, C4fp8, C4q32, C4f32, M1, M2, R1, "
                         "W1, F1); default all")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(decode and prefill shard by sequence or KV head with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    only = set(args.only.split(",")) if args.only else {"C1", "C2", "C3", "C4", "C5", "M1", "M2", "R1",
                                                        "W1", "F1", "C4i8", "C4fp8", "C4q32", "C4f32"}

    g = Gpu()
    extras = {}
    head = None
    if "C2" in only:
        w2, head, out2 = bench_decode(g, "C2", args.steps, args.warmup)
    for name in ("C3", "C5", "C1", "W1", "F1"):
        if name in only:
            _, r, _ = bench_decode(g, name, args.steps, args.warmup)
            # the plain decode call (the partition kernel, with the split merge), as profiled
            r["roofline"] = {"bound": "hbm", "achieved": r["decode_only_call_gbs"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": r["decode_only_call_gbs"] / HBM_PEAK_GBS,
                             "traffic": profiled_traffic(f"decode_{name}_counters.txt",
                                                         source_sha("decode.hip", "decode_body.h", "pkv_device.h", "pkv_host.h"))}
            extras[f"decode_{name}"] = r
    if "C4" in only:
        _, rp, _ = bench_prefill(g, args.steps, args.warmup)
        extras["prefill_C4"] = rp
    for name in ("C4i8", "C4fp8", "C4q32", "C4f32"):
        if name in only:
            _, rp, _ = bench_prefill(g, args.steps, args.warmup, name)
            extras[f"prefill_{name}"] = rp
    for name in ("M1", "M2"):
        if name in only:
            extras[f"mixed_{name}"] = bench_mixed(g, name, args.steps, args.warmup)
    if "R1" in only:
        extras["rope_append_R1"] = bench_rope(g, args.steps, args.warmup)

    line = {
        "metric": "decode KV GB/s (% HBM peak) + seq-tokens/s; prefill TFLOP/s (% MFMA)",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/K/V, scattered page tables)",
    }
    ceiling = None
    if "C2" in only:
        ceiling = bench_ceiling(g, [head["effective_kv_bytes"], 1 << 30], args.steps, args.warmup)
        extras["streaming_read_ceiling"] = ceiling
    if head is not None:
        line.update({
            "value": round(head["kv_gbs"], 2),
            "ms_per_step": round(head["ms_per_step"], 5),
            "config": {"workload": DESC["C2"], "batch": 64, "num_q_heads": 12, "num_kv_heads": 2,
                       "head_dim": 128, "page_size": 16, "kv_dtype": "bf16",
                       "context_tokens": int(w2.context_lens.sum()),
                       "step": "64 new tokens appended + decode, one fused call (one partition kernel: the append, the attention and the split merge)",
                       "timing": "HIP events per step on the library's stream; 1 GiB read-only flush before each step, outside the events"},
            "hbm_frac": round(head["hbm_frac_step"], 4),
            "seq_tokens_per_s": round(head["seq_tokens_per_s"], 1),
            "roofline": {"bound": "hbm", "achieved": round(head["decode_call_gbs"], 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(head["decode_call_gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("decode_C2_counters.txt",
                                                     source_sha("decode.hip", "decode_body.h", "pkv_device.h", "pkv_host.h")),
                         "kernel": "paged_attn_decode_append call: decode_partition_kernel<128,bf16,fused> (the split merge in the same launch), events around the call",
                         "algorithmic_bytes_per_launch": head["effective_kv_bytes"],
                         # the same bytes read by the plain streaming probe:
                         # the practical ceiling, not the published peak
                         "practical_ceiling_gbs": round(ceiling["reads"][0]["gbs"], 1) if ceiling else None,
                         "frac_of_practical_ceiling": (round(head["decode_call_gbs"] / ceiling["reads"][0]["gbs"], 4)
                                                       if ceiling else None)},
            "detail_C2": head,
        })
    line["extra"] = extras
    if head is not None and not args.no_cpu_baseline:
        cb = cpu_baseline(w2, out2, args.cpu_budget)
        cb["cpu_model"] = cpu_model()
        # a reported baseline, not a target: the oracle is plain fp64 numpy
        cb["gpu_step_speedup"] = cb["seconds_per_step"] / (head["ms_per_step"] * 1e-3)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
