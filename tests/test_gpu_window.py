"""GPU parity of sliding-window attention (window > 0) in decode, chunked
prefill and the mixed call, against the oracle's window reading: the query
at position p attends (p - W, p].  Block-table entries of pages wholly
before a window are replaced by ids outside the pool, so any read of them
turns the row into NaN (the library's bad-page rule), and the pages they
pointed at hold NaN."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, np_to_gpu, oracle_cache, poisoned_gpu_cache, q_exact_values,
                         q_tensor, say, small_decode, small_prefill, to_f64, used_slot_mask)

pytestmark = pytest.mark.gpu
PS = 16
EVICTED = 10**7


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _evict(w, first_keys):
    """Block table with every page wholly before first_keys[b] evicted, and a
    slot mask with those pages' slots unused (so the GPU copy holds NaN)."""
    bt = w.block_tables.copy()
    used = used_slot_mask(w)
    for b, lo in enumerate(first_keys):
        for pg in range(lo // PS):
            used[int(bt[b, pg])] = False
            bt[b, pg] = EVICTED
    return bt, used


def _decode(pkv, w, gc, q, bt, window, mcl=None):
    out = pkv.paged_attn_decode(q, gc["k"], gc["v"], np_to_gpu(bt), np_to_gpu(w.context_lens),
                                w.max_context_len if mcl is None else mcl, w.scale,
                                k_scales=gc["ks"], v_scales=gc["vs"], window=window)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv,d", [("f32", 64), ("bf16", 128), ("f16", 64), ("i8", 128), ("fp8", 64)])
@pytest.mark.parametrize("window", [1, 7, 16, 17, 32, 33, 100, 1000])
def test_decode_window(pkv, kv, d, window):
    say(f"decode window={window} kv={kv} d={d}")
    ctx = [1, 5, 16, 17, 31, 32, 33, 47, 64, 100, 101, 555, 1000, 1023, 2500]
    w = small_decode(ctx, 8, 2, d, kv, seed=600 + window)
    cache = oracle_cache(w)
    bt, used = _evict(w, [max(0, c - window) for c in ctx])
    gc = poisoned_gpu_cache(cache, used)
    q = q_tensor(w, "f32")
    out = _decode(pkv, w, gc, q, bt, window)
    ref = oracle.ref_decode(q_exact_values(q), cache, bt, w.context_lens, w.scale, 8, window=window)
    assert oracle.max_abs_err(to_f64(out), ref) <= TOL[kv]


def test_decode_window_long_contexts_split(pkv):
    """Contexts far longer than the window, so the window's tiles are split
    over several workgroups and merged; the second case spans 300000 tokens,
    beyond what a decode without a window takes."""
    for window, ctx in ((5000, [20000, 4097, 9000, 1 << 16, 300]), (4096, [300000, 70000, 4100])):
        say(f"decode window={window} long contexts {ctx}")
        mcl = max(ctx)
        w = small_decode(ctx, 12, 2, 128, "bf16", seed=611)
        cache = oracle_cache(w)
        bt, used = _evict(w, [max(0, c - window) for c in ctx])
        gc = poisoned_gpu_cache(cache, used)
        q = q_tensor(w, "bf16")
        assert pkv.paged_attn_decode_workspace_bytes(len(ctx), 12, 2, 128, mcl, window) > 0
        out = _decode(pkv, w, gc, q, bt, window, mcl=mcl)
        ref = oracle.ref_decode(q_exact_values(q), cache, bt, w.context_lens, w.scale, 12,
                                window=window)
        assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2
    assert pkv.paged_attn_decode_workspace_bytes(3, 12, 2, 128, 300000, 0) == 0   # unsupported


def test_decode_window_covering_context_is_plain_decode(pkv):
    ctx = [1, 50, 333, 4096]
    w = small_decode(ctx, 12, 2, 128, "bf16", seed=612)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    full = _decode(pkv, w, gc, q, w.block_tables, 0)
    assert torch.equal(full, _decode(pkv, w, gc, q, w.block_tables, 4096))
    assert torch.equal(full, _decode(pkv, w, gc, q, w.block_tables, 10**9))


def _prefill(pkv, fn, w, gc, q, bt, window):
    out = getattr(pkv, fn)(q, gc["k"], gc["v"], np_to_gpu(bt), np_to_gpu(w.context_lens),
                           np_to_gpu(w.cu_q_lens), w.max_q_len, w.max_context_len, w.scale,
                           k_scales=gc["ks"], v_scales=gc["vs"], window=window)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fn", ["paged_attn_prefill_chunk", "paged_attn_mixed"])
@pytest.mark.parametrize("kv,d,qd", [("bf16", 128, "bf16"), ("f16", 64, "f32"), ("i8", 128, "bf16"),
                                     ("fp8", 64, "f16"), ("f32", 128, "f32")])
@pytest.mark.parametrize("window", [1, 5, 64, 100, 300, 1000])
def test_prefill_window(pkv, fn, kv, d, qd, window):
    say(f"{fn} window={window} kv={kv} d={d} q={qd}")
    ctx = [700, 1, 333, 2049, 45, 129, 64, 1500]
    chunk = [300, 1, 333, 1, 45, 128, 1, 260]
    w = small_prefill(ctx, chunk, 12, 2, d, kv, seed=620 + window)
    cache = oracle_cache(w)
    first = [max(0, c - n - window + 1) for c, n in zip(ctx, chunk)]   # the first row's window
    bt, used = _evict(w, first)
    gc = poisoned_gpu_cache(cache, used)
    q = q_tensor(w, qd)
    out = _prefill(pkv, fn, w, gc, q, bt, window)
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, bt, w.context_lens, w.cu_q_lens,
                                   w.scale, window=window)
    assert oracle.max_abs_err(to_f64(out), ref) <= TOL[kv]


@pytest.mark.parametrize("fn", ["paged_attn_prefill_chunk", "paged_attn_mixed"])
def test_prefill_window_covering_prefix_is_plain(pkv, fn):
    ctx = [700, 333, 129]
    chunk = [300, 1, 128]
    w = small_prefill(ctx, chunk, 12, 2, 128, "bf16", seed=630)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    full = _prefill(pkv, fn, w, gc, q, w.block_tables, 0)
    assert torch.equal(full, _prefill(pkv, fn, w, gc, q, w.block_tables, 700))


def test_decode_window_full_size(pkv):
    """The benchmarked sliding-window decode: batch 64, Qwen2.5-1.5B heads,
    contexts U[16384, 65536], window 4096, only the window's pages held
    (earlier block-table entries are -1); every output checked."""
    from workloads import make_workload
    say("decode window full size (W1)")
    w = make_workload("W1")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "f32")
    out = _decode(pkv, w, gc, q, w.block_tables, w.meta["window"])
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale, 12,
                            window=w.meta["window"])
    assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2
