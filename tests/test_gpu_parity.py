"""GPU parity: the HIP library against the fp64 oracle, through the C ABI.

Tolerances (max abs error over every output element): 2e-5 for fp32 KV and
1e-2 for bf16/fp16/int8 KV; append is compared byte for byte.  Unused pool
slots are NaN on the GPU, so any read outside a sequence's context fails.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (SCALED, TOL, TORCH_DT, config_case, gpu_to_np_bits, np_to_gpu, oracle_cache,
                         poisoned_gpu_cache, q_exact_values, q_tensor, run_decode, run_prefill,
                         say, small_decode, small_prefill, to_f64, used_slot_mask)
from workloads import custom_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _decode_check(pkv, w, cache, q_dtype="f32", out_dtype=torch.float32, tol=None, **kw):
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, q_dtype)
    out = run_decode(pkv, w, gc, q, out_dtype=out_dtype, **kw)
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    err = oracle.max_abs_err(to_f64(out), ref)
    return err, (TOL[w.kv_dtype] if tol is None else tol)


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("cache_dtype", ["f32", "bf16", "f16", "i8", "fp8"])
@pytest.mark.parametrize("new_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lens", [[37, 16, 1, 90], [37, 16, 1, 90, 2100]], ids=["rows", "segments"])
def test_append_bit_exact(pkv, cache_dtype, new_dtype, d, lens):
    """A few (token, head) rows take the row kernel; past 4096 rows the
    segment kernel with the LDS-transposed V stores."""
    say(f"append cache={cache_dtype} new={new_dtype} d={d} tokens={sum(lens)}")
    w = custom_workload(context_lens=lens, num_q_heads=4, num_kv_heads=2, head_dim=d,
                        kv_dtype=cache_dtype, num_pages=(sum(lens) + 15) // 16 + 8, seed=40 + d)
    k, v = w.k.copy(), w.v.copy()
    # edge values: signed zeros, fp16 subnormals and overflow, bf16 ties, an all-zero vector
    k[0, 0, :8] = [0.0, -0.0, 2.0**-25, 3 * 2.0**-25, 6e-8, 65520.0, 1.00390625, -1.01171875]
    v[1, 1, :] = 0.0
    k[2, 0, :4] = [np.float32(1e-40), -1e-41, 7e4, -1e5]
    if cache_dtype in SCALED:
        # int8 / FP8 quantization is specified for finite vectors only; keep the
        # fp16-overflow values out of its input
        k[0, 0, 5] = 60000.0
        k[2, 0, 2:4] = [6e4, -5e4]
    kt = torch.from_numpy(k).cuda().to(TORCH_DT[new_dtype])
    vt = torch.from_numpy(v).cuda().to(TORCH_DT[new_dtype])
    slots = w.slot_mapping.copy()
    slots[[5, 40]] = -1
    slots[41] = w.num_pages * 16 + 3          # past the pool: skipped like padding
    host = oracle.PagedCache(w.num_pages, 2, d, cache_dtype)
    host.k.view(np.uint8)[:] = 0xA5
    host.v.view(np.uint8)[:] = 0xA5
    if cache_dtype in SCALED:
        host.k_scales.view(np.uint8)[:] = 0xA5
        host.v_scales.view(np.uint8)[:] = 0xA5
    gk, gv = np_to_gpu(host.k), np_to_gpu(host.v)
    gks = np_to_gpu(host.k_scales) if cache_dtype in SCALED else None
    gvs = np_to_gpu(host.v_scales) if cache_dtype in SCALED else None
    pkv.paged_kv_append(kt, vt, torch.from_numpy(slots).cuda(), gk, gv, gks, gvs)
    torch.cuda.synchronize()
    slots[41] = -1
    oracle.ref_append(host, kt.float().cpu().numpy(), vt.float().cpu().numpy(), slots)
    assert np.array_equal(gpu_to_np_bits(gk).view(np.uint8), host.k.view(np.uint8))
    assert np.array_equal(gpu_to_np_bits(gv).view(np.uint8), host.v.view(np.uint8))
    if cache_dtype in SCALED:
        assert np.array_equal(gks.cpu().numpy().view(np.uint32), host.k_scales.view(np.uint32))
        assert np.array_equal(gvs.cpu().numpy().view(np.uint32), host.v_scales.view(np.uint32))


def test_append_full_size_bf16_and_out_of_pool_slots(pkv):
    """Every token of the bf16 decode workload (Qwen2.5-1.5B heads, ~150k
    tokens over a scattered 20k-page pool) appended from fp32 in one call and
    compared byte for byte; tokens whose slot lies past the pool are skipped."""
    w, _ = config_case("C2")
    say("append C2 full size bf16")
    slots = w.slot_mapping.copy()
    beyond = [7, 1000, len(slots) - 1]
    slots[beyond] = w.num_pages * 16 + np.array([0, 5, 10**9])
    host = oracle.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, "bf16")
    gk, gv = np_to_gpu(host.k), np_to_gpu(host.v)
    pkv.paged_kv_append(torch.from_numpy(w.k).cuda(), torch.from_numpy(w.v).cuda(),
                        torch.from_numpy(slots).cuda(), gk, gv)
    torch.cuda.synchronize()
    slots[beyond] = -1                      # the oracle's way of skipping a token
    oracle.ref_append(host, w.k, w.v, slots)
    assert np.array_equal(gpu_to_np_bits(gk), host.k)
    assert np.array_equal(gpu_to_np_bits(gv), host.v)


@pytest.mark.parametrize("name,dt", [("C5", "i8"), ("F1", "fp8")])
def test_append_full_size_scaled(pkv, name, dt):
    """Every token of the int8 (TinyLlama shape) and FP8 (Qwen2.5-1.5B shape)
    decode workloads quantized in one call, codes and scales byte for byte."""
    w, _ = config_case(name)
    say(f"append {name} full size {dt}")
    host = oracle.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, dt)
    gk, gv = np_to_gpu(host.k), np_to_gpu(host.v)
    gks, gvs = np_to_gpu(host.k_scales), np_to_gpu(host.v_scales)
    pkv.paged_kv_append(torch.from_numpy(w.k).cuda(), torch.from_numpy(w.v).cuda(),
                        torch.from_numpy(w.slot_mapping).cuda(), gk, gv, gks, gvs)
    torch.cuda.synchronize()
    oracle.ref_append(host, w.k, w.v, w.slot_mapping)
    assert np.array_equal(gpu_to_np_bits(gk), host.k)
    assert np.array_equal(gpu_to_np_bits(gv), host.v)
    assert np.array_equal(gks.cpu().numpy().view(np.uint32), host.k_scales.view(np.uint32))
    assert np.array_equal(gvs.cpu().numpy().view(np.uint32), host.v_scales.view(np.uint32))


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C5", "F1"])
def test_decode_config_full_size(pkv, name):
    w, cache = config_case(name)
    say(f"decode {name} full size: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} kv={w.kv_dtype}")
    err, tol = _decode_check(pkv, w, cache)
    say(f"  max abs err {err:.3e} (tol {tol})")
    assert err <= tol


@pytest.mark.parametrize("kv", ["f32", "bf16", "f16", "i8", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (9, 3), (8, 1), (32, 2)])
def test_decode_small(pkv, kv, d, hq, hkv):
    ctx = [1, 15, 16, 17, 31, 32, 33, 0, 100, 257, 700]
    w = small_decode(ctx, hq, hkv, d, kv, seed=hq * 7 + d + len(kv))
    say(f"decode small kv={kv} d={d} hq={hq} hkv={hkv}")
    err, tol = _decode_check(pkv, w, oracle_cache(w))
    assert err <= tol, err


@pytest.mark.parametrize("q_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_decode_io_dtypes(pkv, q_dtype, out_dtype):
    w = small_decode([5, 64, 300, 1000], 12, 2, 128, "bf16", seed=7)
    say(f"decode io q={q_dtype} out={out_dtype}")
    err, tol = _decode_check(pkv, w, oracle_cache(w), q_dtype=q_dtype, out_dtype=out_dtype)
    assert err <= tol, err


@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8"])
def test_decode_split_counts_agree(pkv, kv):
    """Raising max_context_len changes how contexts are split into
    partitions (and how many partials the LSE reduce merges); the result
    must stay within tolerance for every split."""
    w = small_decode([3000, 17, 1500, 4096, 600], 8, 2, 64, kv, seed=9, table_width=512)
    cache = oracle_cache(w)
    for mcl in (4096, 5000, 8192):
        say(f"decode split kv={kv} max_context_len={mcl}")
        err, tol = _decode_check(pkv, w, cache, max_context_len=mcl)
        assert err <= tol, (mcl, err)


def test_decode_page_permutation_bit_exact(pkv):
    w = small_decode([40, 300, 77], 6, 2, 128, "bf16", seed=3, num_pages=64)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w)
    out1 = run_decode(pkv, w, gc, q)
    perm = np.random.Generator(np.random.PCG64(1)).permutation(w.num_pages)
    inv = np.argsort(perm)
    gc2 = dict(gc)
    gc2["k"] = gc["k"][torch.from_numpy(perm).cuda()].contiguous()
    gc2["v"] = gc["v"][torch.from_numpy(perm).cuda()].contiguous()
    out2 = run_decode(pkv, w, gc2, q, block_tables=inv[w.block_tables].astype(np.int32))
    assert torch.equal(out1, out2)


def test_decode_bad_page_id_gives_nan(pkv):
    w = small_decode([40, 50], 4, 2, 64, "f16", seed=5)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    bt = w.block_tables.copy()
    bt[1, 1] = w.num_pages + 100          # out of the pool
    out = run_decode(pkv, w, gc, q_tensor(w), block_tables=bt)
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isfinite(o[0]))


def test_decode_memory_stable(pkv):
    w = small_decode([100, 2000, 50], 12, 2, 128, "bf16", seed=2)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w)
    run_decode(pkv, w, gc, q)
    before = torch.cuda.memory_allocated()
    for _ in range(5):
        out = run_decode(pkv, w, gc, q)
        del out
    assert torch.cuda.memory_allocated() == before


# ------------------------------------------------------------------ prefill
def _prefill_check(pkv, w, cache, q_dtype="bf16", out_dtype=torch.float32):
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, q_dtype)
    out = run_prefill(pkv, w, gc, q, out_dtype=out_dtype)
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    return oracle.max_abs_err(to_f64(out), ref)


def test_prefill_config_full_size(pkv):
    w, cache = config_case("C4")
    say(f"prefill C4 full size: prefixes {w.meta['prefix_lens'].tolist()}")
    err = _prefill_check(pkv, w, cache)
    say(f"  max abs err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("case", ["spread_many_blocks", "spread_few_blocks", "uniform", "batch_over_256",
                                  "batch_256_grid_512"])
def test_prefill_row_block_order(pkv, case):
    """Every row block is computed exactly once whichever order the workgroups
    take them in: contexts that differ (ranked order, with more and with fewer
    row blocks than the first round of 256 workgroups), contexts within 25% of
    each other (grid order) and more than 256 sequences (grid order).  The
    output starts as NaN, so a row no workgroup wrote fails.  The last case is
    the largest grid that takes the ranked order: 256 sequences, 512
    workgroups."""
    rng = np.random.Generator(np.random.PCG64(77))
    if case == "spread_many_blocks":       # 12 sequences x 2 KV heads x 12 row blocks = 288 > 256
        ql = [256] * 12
        pre = rng.integers(0, 1200, size=12).tolist()
        hq, hkv = 12, 2
    elif case == "spread_few_blocks":
        ql = [40, 90, 7, 130]
        pre = [900, 0, 333, 61]
        hq, hkv = 6, 2
    elif case == "uniform":
        ql = [128] * 10
        pre = [500 + 10 * i for i in range(10)]
        hq, hkv = 6, 2
    elif case == "batch_over_256":
        ql = rng.integers(1, 6, size=300).tolist()
        pre = rng.integers(0, 120, size=300).tolist()
        hq, hkv = 4, 2
    else:                                  # the largest ranked grid: 256 x 2 KV heads x 1 row block
        ql = rng.integers(1, 9, size=256).tolist()
        pre = rng.integers(0, 300, size=256).tolist()
        hq, hkv = 4, 2
    ctx = [p + c for p, c in zip(pre, ql)]
    w = small_prefill(ctx, ql, hq, hkv, 64, "bf16", seed=len(ctx))
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = torch.full((int(w.cu_q_lens[-1]), hq, 64), float("nan"), device="cuda")
    say(f"prefill row-block order: {case}, batch {len(ctx)}")
    pkv.paged_attn_prefill_chunk(q, gc["k"], gc["v"], np_to_gpu(w.block_tables),
                                 np_to_gpu(w.context_lens), np_to_gpu(w.cu_q_lens), w.max_q_len,
                                 w.max_context_len, w.scale, out=out)
    torch.cuda.synchronize()
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    got = to_f64(out)
    assert not np.isnan(got).any()
    assert oracle.max_abs_err(got, ref) <= 1e-2


@pytest.mark.parametrize("kv", ["f32", "bf16", "f16", "i8", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (6, 2), (12, 2), (3, 1)])
def test_prefill_small(pkv, kv, d, hq, hkv):
    ctx = [16, 40, 17, 200, 33, 130]
    ql = [16, 7, 17, 150, 1, 64]           # prefixes 0, 33, 0, 50, 32, 66
    w = small_prefill(ctx, ql, hq, hkv, d, kv, seed=hq + d)
    say(f"prefill small kv={kv} d={d} hq={hq} hkv={hkv}")
    err = _prefill_check(pkv, w, oracle_cache(w), q_dtype=kv if kv in ("f32", "bf16", "f16") else "bf16")
    assert err <= TOL[kv], err


@pytest.mark.parametrize("kv,q_dtype", [("bf16", "f32"), ("bf16", "f16"), ("i8", "f32"), ("i8", "f16"),
                                        ("fp8", "f32"), ("fp8", "f16"), ("f32", "bf16"), ("f32", "f16")])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_q_other_dtype(pkv, kv, q_dtype, d):
    w = small_prefill([300, 90], [100, 90], 6, 2, d, kv, seed=8)
    say(f"prefill {kv} KV d={d} with q={q_dtype}")
    err = _prefill_check(pkv, w, oracle_cache(w), q_dtype=q_dtype)
    assert err <= TOL[kv], err


def test_prefill_bench_batch_stored_fp32(pkv):
    """The benchmarked prefill batch with an fp32 cache and fp32 query:
    every row within the fp32 tolerance."""
    w = make_workload("C4")
    say("prefill C4 batch stored as f32")
    cache = oracle_cache(w, "f32")
    err = _prefill_check(pkv, w, cache, q_dtype="f32")
    say(f"  max abs err {err:.3e}")
    assert err <= TOL["f32"]


def test_prefill_rows_match_decode(pkv):
    """Chunk row i equals a decode over the first P+i+1 tokens."""
    w = small_prefill([90], [40], 6, 2, 128, "bf16", seed=4)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    pre = run_prefill(pkv, w, gc, q)
    P = 50
    for i in (0, 13, 39):
        wd = small_decode([P + i + 1], 6, 2, 128, "bf16", seed=4)
        wd.block_tables = w.block_tables.copy()
        wd.q = w.q[i:i + 1].copy()
        dec = run_decode(pkv, wd, gc, q[i:i + 1].contiguous())
        assert torch.max(torch.abs(dec[0] - pre[i])).item() <= 1e-2


# ------------------------------------------------------------------ errors
def test_error_codes_with_device_buffers(pkv):
    w = small_decode([20], 4, 2, 64, "bf16", seed=1)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w)
    bt, cl = np_to_gpu(w.block_tables), np_to_gpu(w.context_lens)
    lib = pkv.load_library()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = torch.empty((1, 4, 64), device="cuda")
    nws = pkv.paged_attn_decode_workspace_bytes(1, 4, 2, 64, 20)
    assert nws == 0                       # one partition: no workspace

    def call(**over):
        args = dict(q=P(q), qd=0, k=P(gc["k"]), v=P(gc["v"]), ks=None, vs=None, kvd=1, bt=P(bt),
                    mb=int(w.block_tables.shape[1]), cl=P(cl), mcl=20, B=1, hq=4, hkv=2, d=64,
                    ps=16, np_=w.num_pages, sc=0.125, win=0, out=P(out), od=0, ws=None, wsb=0,
                    st=None)
        args.update(over)
        return lib.paged_attn_decode(*args.values())

    assert call() == 0
    torch.cuda.synchronize()
    assert call(q=None) == 1
    assert call(hq=5) == 1
    assert call(ps=8) == 2
    assert call(d=96) == 2
    assert call(kvd=3) == 1                       # int8 without scales
    assert call(qd=3) == 1                        # int8 query
    assert call(mcl=10000) == 1                   # beyond the block table
    assert call(win=-1) == 1                      # negative window
    assert call(q=ctypes.c_void_p(q.data_ptr() + 4)) == 3
    assert call(mcl=20, B=1, hq=4, hkv=2) == 0
    torch.cuda.synchronize()
