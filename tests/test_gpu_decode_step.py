"""GPU parity of the fused decode step (paged_attn_decode_append): each
sequence's new K/V row goes to position ctx - 1, then the query attends.
Checked against the oracle's ref_append + ref_decode (output within the
decode tolerance, the whole cache byte for byte) and against the library's
own paged_kv_append + paged_attn_decode (bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, TORCH_DT, gpu_to_np_bits, np_to_gpu, poisoned_gpu_cache,
                         q_exact_values, q_tensor, say, small_decode, to_f64, used_slot_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _setup(w, kv, new_dtype):
    """Oracle cache holding every context token but each sequence's last
    (the new one), its GPU copy with unused slots and the new tokens' slots
    poisoned, and the new rows [B, Hkv, d] in new_dtype on the GPU (zeros
    for a sequence with an empty context).  Returns also the new tokens'
    row index per sequence (-1 when empty)."""
    last = np.array([int(w.token_offsets[b + 1]) - 1 if w.context_lens[b] > 0 else -1
                     for b in range(w.batch)])
    rows = last[last >= 0]
    old = np.ones(len(w.slot_mapping), bool)
    old[rows] = False
    cache = oracle.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, kv)
    oracle.ref_append(cache, w.k[old], w.v[old], w.slot_mapping[old])
    used = used_slot_mask(w)
    s = w.slot_mapping[rows]
    used[s // 16, s % 16] = False                 # the new slots hold NaN until written
    gc = poisoned_gpu_cache(cache, used)
    kb = np.zeros((w.batch, w.num_kv_heads, w.head_dim), np.float32)
    vb = np.zeros_like(kb)
    kb[last >= 0], vb[last >= 0] = w.k[rows], w.v[rows]
    kn = torch.from_numpy(kb).cuda().to(TORCH_DT[new_dtype])
    vn = torch.from_numpy(vb).cuda().to(TORCH_DT[new_dtype])
    return cache, gc, kn, vn, last


def _fused(pkv, w, gc, q, kn, vn, window=0, block_tables=None):
    bt = w.block_tables if block_tables is None else block_tables
    out = pkv.paged_attn_decode_append(q, kn, vn, gc["k"], gc["v"], np_to_gpu(bt),
                                       np_to_gpu(w.context_lens), w.max_context_len, w.scale,
                                       window=window, k_scales=gc["ks"], v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv,new_dtype", [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16"),
                                          ("f32", "f32"), ("f32", "bf16"), ("i8", "f32"),
                                          ("i8", "bf16"), ("fp8", "f32"), ("fp8", "f16")])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(12, 2), (8, 8), (40, 2)])
def test_decode_step_matches_oracle(pkv, kv, new_dtype, d, hq, hkv):
    ctx = [1, 15, 16, 17, 32, 33, 100, 513, 2049, 4096]
    say(f"decode step kv={kv} new={new_dtype} d={d} hq={hq} hkv={hkv}")
    w = small_decode(ctx, hq, hkv, d, kv, seed=700 + d + hq)
    cache, gc, kn, vn, last = _setup(w, kv, new_dtype)
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    oracle.ref_append(cache, kn.float().cpu().numpy(), vn.float().cpu().numpy(), w.slot_mapping[last])
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale, hq)
    assert oracle.max_abs_err(to_f64(out), ref) <= TOL[kv]
    used = used_slot_mask(w)
    mk, mv = used[:, None, :, None], used[:, None, None, :]
    gk, gv = gpu_to_np_bits(gc["k"]), gpu_to_np_bits(gc["v"])
    assert np.array_equal(np.where(mk, gk, 0).view(np.uint8), np.where(mk, cache.k, 0).view(np.uint8))
    assert np.array_equal(np.where(mv, gv, 0).view(np.uint8), np.where(mv, cache.v, 0).view(np.uint8))
    if kv in ("i8", "fp8"):
        for g_s, h_s in ((gc["ks"], cache.k_scales), (gc["vs"], cache.v_scales)):
            got = g_s.cpu().numpy()
            ms = used[:, None, :]
            assert np.array_equal(np.where(ms, got, 0).view(np.uint32), np.where(ms, h_s, 0).view(np.uint32))


def _append_then_decode(pkv, w, gc, q, kn, vn, last, window=0):
    pkv.paged_kv_append(kn, vn, torch.from_numpy(w.slot_mapping[last]).cuda(), gc["k"], gc["v"],
                        gc["ks"], gc["vs"])
    out = pkv.paged_attn_decode(q, gc["k"], gc["v"], np_to_gpu(w.block_tables),
                                np_to_gpu(w.context_lens), w.max_context_len, w.scale, window=window,
                                k_scales=gc["ks"], v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


def _same_cache(gc, gc2):
    for key in ("k", "v", "ks", "vs"):
        if gc[key] is not None:
            assert torch.equal(gc[key].view(torch.uint8), gc2[key].view(torch.uint8)), key


@pytest.mark.parametrize("kv", ["bf16", "f32", "i8", "fp8"])
@pytest.mark.parametrize("window", [0, 40])
def test_decode_step_equals_append_then_decode(pkv, kv, window):
    """The fused step and the two calls give the same cache and the same
    output, bit for bit (splits included)."""
    ctx = [int(x) for x in np.random.default_rng(710).integers(1, 6000, size=48)]
    say(f"decode step vs two calls kv={kv} window={window}")
    w = small_decode(ctx, 12, 2, 128, kv, seed=711)
    _, gc, kn, vn, last = _setup(w, kv, "f32")
    gc2 = {k: (None if t is None else t.clone()) for k, t in gc.items()}
    q = q_tensor(w, "f32")
    fused = _fused(pkv, w, gc, q, kn, vn, window=window)
    two = _append_then_decode(pkv, w, gc2, q, kn, vn, last, window=window)
    assert torch.equal(fused, two)
    _same_cache(gc, gc2)


def test_decode_step_empty_and_bad(pkv):
    """ctx 0: nothing stored, zeros; a bad page id on the new token's page:
    that row is NaN and nothing is stored; other rows unaffected."""
    ctx = [0, 40, 70, 5]
    w = small_decode(ctx, 8, 2, 64, "bf16", seed=720)
    cache, gc, kn, vn, last = _setup(w, "bf16", "bf16")
    q = q_tensor(w, "f32")
    before = gpu_to_np_bits(gc["k"]).copy()
    bt = w.block_tables.copy()
    bt[2, (70 - 1) // 16] = w.num_pages + 5           # sequence 2's new token lives in that page
    out = _fused(pkv, w, gc, q, kn, vn, block_tables=bt).cpu().numpy()
    assert np.all(out[0] == 0)
    assert np.all(np.isnan(out[2])) and np.all(np.isfinite(out[[1, 3]]))
    s2 = int(w.slot_mapping[last[2]])
    assert np.array_equal(gpu_to_np_bits(gc["k"])[s2 // 16, :, s2 % 16], before[s2 // 16, :, s2 % 16])


def test_decode_step_full_size(pkv):
    """The benchmarked step: the bf16 decode workload at the Qwen2.5-1.5B
    shape (64 sequences, contexts U[512, 4096]), fp32 new rows."""
    from workloads import make_workload
    say("decode step full size (C2)")
    w = make_workload("C2")
    cache, gc, kn, vn, last = _setup(w, "bf16", "f32")
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    oracle.ref_append(cache, w.k[last], w.v[last], w.slot_mapping[last])
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale, 12)
    assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2
    s = w.slot_mapping[last]
    assert np.array_equal(gpu_to_np_bits(gc["k"])[s // 16, :, s % 16], cache.k[s // 16, :, s % 16])
    assert np.array_equal(gpu_to_np_bits(gc["v"])[s // 16, :, :, s % 16], cache.v[s // 16, :, :, s % 16])


def test_decode_step_many_workgroups(pkv):
    """A step whose decode needs many rounds of workgroups (the fp16 decode
    workload at the Stories110M shape: 384 sequences x 12 KV heads) stores
    the new tokens with a launch of its own before the decode; same results
    as the two calls, bit for bit, and as the oracle."""
    from workloads import make_workload
    say("decode step C3 (many workgroups)")
    w = make_workload("C3")
    cache, gc, kn, vn, last = _setup(w, "f16", "f32")
    gc2 = {k: (None if t is None else t.clone()) for k, t in gc.items()}
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    pkv.paged_kv_append(kn, vn, torch.from_numpy(w.slot_mapping[last]).cuda(), gc2["k"], gc2["v"])
    two = pkv.paged_attn_decode(q, gc2["k"], gc2["v"], np_to_gpu(w.block_tables),
                                np_to_gpu(w.context_lens), w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    assert torch.equal(gc["k"].view(torch.uint8), gc2["k"].view(torch.uint8))
    assert torch.equal(gc["v"].view(torch.uint8), gc2["v"].view(torch.uint8))
    oracle.ref_append(cache, w.k[last], w.v[last], w.slot_mapping[last])
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale, 12)
    assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2


@pytest.mark.parametrize("name,kv", [("C5", "i8"), ("F1", "fp8")])
def test_decode_step_full_size_one_byte_caches(pkv, name, kv):
    """The benchmarked int8 and FP8 steps in one launch: the new rows are
    quantised in the partition kernel (codes and scales byte for byte those
    of paged_kv_append, output bit for bit that of append + decode) and the
    output is within tolerance of the oracle."""
    from workloads import make_workload
    say(f"decode step full size ({name}, {kv})")
    w = make_workload(name)
    cache, gc, kn, vn, last = _setup(w, kv, "f32")
    gc2 = {k: (None if t is None else t.clone()) for k, t in gc.items()}
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    two = _append_then_decode(pkv, w, gc2, q, kn, vn, last)
    assert torch.equal(out, two)
    _same_cache(gc, gc2)
    oracle.ref_append(cache, w.k[last], w.v[last], w.slot_mapping[last])
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_decode_step_one_byte_many_workgroups(pkv, kv):
    """Many rounds of workgroups (384 sequences x 12 KV heads, head_dim 64)
    over a one-byte cache: the separate store launch quantises as the append
    does; bit for bit the two calls."""
    from workloads import make_workload
    say(f"decode step C3 shape stored as {kv}")
    w = make_workload("C3")
    _, gc, kn, vn, last = _setup(w, kv, "f32")
    gc2 = {k: (None if t is None else t.clone()) for k, t in gc.items()}
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    two = _append_then_decode(pkv, w, gc2, q, kn, vn, last)
    assert torch.equal(out, two)
    _same_cache(gc, gc2)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_decode_step_nan_new_row(pkv, kv):
    """A NaN in a new K row and in a new V row: both get scale NaN and
    codes 0 (the append's rule), the heads of those KV heads read NaN, the
    other rows are untouched; bit for bit the two calls."""
    ctx = [40, 70, 5, 300]
    w = small_decode(ctx, 8, 2, 128, kv, seed=730)
    _, gc, kn, vn, last = _setup(w, kv, "f32")
    kn[1, 0, 17] = float("nan")
    vn[3, 1, 100] = float("nan")
    gc2 = {k: (None if t is None else t.clone()) for k, t in gc.items()}
    q = q_tensor(w, "f32")
    out = _fused(pkv, w, gc, q, kn, vn)
    two = _append_then_decode(pkv, w, gc2, q, kn, vn, last)
    _same_cache(gc, gc2)
    o, t = out.cpu().numpy(), two.cpu().numpy()
    assert np.array_equal(np.isnan(o), np.isnan(t))
    assert np.all(np.isnan(o[1, :4])) and np.all(np.isnan(o[3, 4:]))
    fin = np.isfinite(o)
    assert np.array_equal(o[fin], t[fin])
