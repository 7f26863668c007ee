"""GPU: value ranges beyond N(0,1) data, and non-finite inputs.

* Attention is linear in V, so a V scaled by c is held to c times the
  absolute tolerance: the same bar as unscaled data, at magnitudes where an
  fp16 intermediate could overflow.
* A NaN in a new K/V vector stored as int8 or FP8 gives that vector a NaN
  scale and zero codes (the append's stated handling), and every query that
  attends the token gets NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (SCALED, TORCH_DT, gpu_to_np_bits, np_to_gpu, oracle_cache,
                         poisoned_gpu_cache, q_tensor, run_decode, say, to_f64, used_slot_mask)
from workloads import custom_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _jump_workload(kv, v_gain, seed):
    """128 sequences (4 query heads on one KV head, head_dim 64, contexts
    900-1100 so each takes two splits of five tiles per wave).  Keys are
    tiny except at positions 64k + 40, whose key is aligned with the
    sequence's first query head so that head's log2-score there is 6: a
    wave whose run starts on a tile without such a key meets probabilities
    of about 2^6 under the running max.  V is N(0,1) times v_gain."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(900, 1100, size=128, endpoint=True).tolist()
    w = custom_workload(context_lens=ctx, num_q_heads=4, num_kv_heads=1, head_dim=64,
                        kv_dtype=kv, seed=seed)
    w.k *= np.float32(0.02)
    w.v *= np.float32(v_gain)
    log2e = 1.0 / np.log(2.0)
    for b in range(w.batch):
        q0 = w.q[b, 0].astype(np.float64)
        alpha = 6.0 / (float(q0 @ q0) * float(w.scale) * log2e)
        t0 = int(w.token_offsets[b])
        for pos in range(40, int(w.context_lens[b]), 64):
            w.k[t0 + pos, 0] = (alpha * q0).astype(np.float32)
    return w


@pytest.mark.parametrize("kv,v_gain", [("fp8", 3.0e3), ("i8", 3.0e5), ("bf16", 3.0e3)])
def test_decode_large_v_with_late_high_scores(pkv, kv, v_gain):
    """FP8 V with absmax ~1e4 and int8 V with absmax ~1e6: the probability
    times the V scale that the PV product takes in fp16 would pass 65504
    without the kernel's power-of-two normalisation of the scales."""
    w = _jump_workload(kv, v_gain, seed=11 if kv == "fp8" else 12)
    say(f"decode large V kv={kv} gain={v_gain:g}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    out = run_decode(pkv, w, gc, q_tensor(w))
    ref = oracle.ref_decode(w.q.astype(np.float64), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    err = oracle.max_abs_err(got, ref)
    say(f"  max abs err {err:.3e} (tol {1e-2 * v_gain:.3e}, linear in V)")
    assert err <= 1e-2 * v_gain


@pytest.mark.parametrize("kv", ["fp8", "i8"])
def test_decode_tiny_v_scales(pkv, kv):
    """V of absmax ~1e-6: the normalised scales keep the probabilities'
    products in fp16's normal range (tolerance scaled by linearity)."""
    w = _jump_workload(kv, 3.0e-7, seed=13)
    say(f"decode tiny V kv={kv}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    out = run_decode(pkv, w, gc, q_tensor(w))
    ref = oracle.ref_decode(w.q.astype(np.float64), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    err = oracle.max_abs_err(to_f64(out), ref)
    assert err <= 1e-2 * 3.0e-7, err


@pytest.mark.parametrize("cache_dtype", SCALED)
@pytest.mark.parametrize("new_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens", [[37, 16, 1, 90], [37, 16, 1, 90, 2100]], ids=["rows", "segments"])
def test_append_nan_vector_gets_nan_scale(pkv, cache_dtype, new_dtype, lens):
    """A NaN in a K row and in a V row: scale NaN and codes 0 for exactly
    those (token, head) vectors, every other byte as the oracle stores it;
    the decode of a sequence over the token is NaN for the heads that read
    it, the other sequences unaffected."""
    say(f"append NaN vector cache={cache_dtype} new={new_dtype} tokens={sum(lens)}")
    w = custom_workload(context_lens=lens, num_q_heads=4, num_kv_heads=2, head_dim=64,
                        kv_dtype=cache_dtype, num_pages=(sum(lens) + 15) // 16 + 8, seed=77)
    k, v = w.k.copy(), w.v.copy()
    k[40, 1, 17] = np.nan           # sequence 0 (37 tokens) owns rows 0..36; row 40 is sequence 1
    v[3, 0, 60] = np.nan            # sequence 0
    kt = torch.from_numpy(k).cuda().to(TORCH_DT[new_dtype])
    vt = torch.from_numpy(v).cuda().to(TORCH_DT[new_dtype])
    host = oracle.PagedCache(w.num_pages, 2, 64, cache_dtype)
    gk, gv = np_to_gpu(host.k), np_to_gpu(host.v)
    gks, gvs = np_to_gpu(host.k_scales), np_to_gpu(host.v_scales)
    pkv.paged_kv_append(kt, vt, torch.from_numpy(w.slot_mapping).cuda(), gk, gv, gks, gvs)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        oracle.ref_append(host, kt.float().cpu().numpy(), vt.float().cpu().numpy(), w.slot_mapping)
    assert np.array_equal(gpu_to_np_bits(gk).view(np.uint8), host.k.view(np.uint8))
    assert np.array_equal(gpu_to_np_bits(gv).view(np.uint8), host.v.view(np.uint8))
    for g_s, h_s in ((gks, host.k_scales), (gvs, host.v_scales)):
        got = g_s.cpu().numpy()
        nan = np.isnan(h_s)
        assert nan.sum() == 1 and np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), h_s[~nan].view(np.uint32))
    out = pkv.paged_attn_decode(q_tensor(w), gk, gv, np_to_gpu(w.block_tables),
                                np_to_gpu(w.context_lens), w.max_context_len, w.scale,
                                k_scales=gks, v_scales=gvs)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[0, :2]))               # V NaN in KV head 0 of sequence 0
    assert np.all(np.isnan(o[1, 2:]))               # K NaN in KV head 1 of sequence 1
    assert np.all(np.isfinite(o[2:])) and np.all(np.isfinite(o[0, 2:])) and np.all(np.isfinite(o[1, :2]))


@pytest.mark.parametrize("scale", [0.0, -0.125, -0.7, 3.0])
@pytest.mark.parametrize("kv", ["bf16", "f16"])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_prefill_and_mixed_any_finite_scale(pkv, scale, kv, q_dtype):
    """A zero scale averages V over each row's keys, a negative one favours
    the keys with the lowest dot products; masked keys stay out either way.
    Prefill (chunks over a prefix, ragged tails) and the mixed call (the
    same chunks plus one-token rows) against the oracle at that scale."""
    from gpu_helpers import small_prefill
    say(f"prefill/mixed scale={scale} kv={kv} q={q_dtype}")
    w = small_prefill([300, 77, 1, 200, 17], [140, 77, 1, 1, 9], 12, 2, 128, kv, seed=31,
                      scale=scale)
    assert float(w.scale) == float(np.float32(scale))
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = torch.from_numpy(w.q).cuda().to(TORCH_DT[q_dtype])
    ref = oracle.ref_prefill_chunk(q.double().cpu().numpy(), cache, w.block_tables,
                                   w.context_lens, w.cu_q_lens, w.scale)
    args = (q, gc["k"], gc["v"], np_to_gpu(w.block_tables), np_to_gpu(w.context_lens),
            np_to_gpu(w.cu_q_lens), w.max_q_len, w.max_context_len, w.scale)
    for fn in (pkv.paged_attn_prefill_chunk, pkv.paged_attn_mixed):
        out = fn(*args)
        torch.cuda.synchronize()
        err = oracle.max_abs_err(to_f64(out), ref)
        say(f"  {fn.__name__}: max abs err {err:.3e}")
        assert err <= 1e-2


@pytest.mark.parametrize("scale", [0.0, -0.2])
@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8"])
def test_decode_any_finite_scale(pkv, scale, kv):
    w = custom_workload(context_lens=[1, 40, 300, 1000], num_q_heads=8, num_kv_heads=2,
                        head_dim=64, kv_dtype=kv, seed=32, scale=scale)
    say(f"decode scale={scale} kv={kv}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    out = run_decode(pkv, w, gc, q_tensor(w))
    ref = oracle.ref_decode(w.q.astype(np.float64), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    assert oracle.max_abs_err(to_f64(out), ref) <= (2e-5 if kv == "f32" else 1e-2)


@pytest.mark.parametrize("kv", ["f16", "i8", "fp8", "bf16", "f32"])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k", [-60, 40])
def test_decode_query_outside_fp16_range(pkv, kv, q_dtype, k):
    """The query times 2^k with the scale times 2^-k (the same scores): the
    fp16-operand decodes (fp16, int8 and FP8 caches) scale each head's query
    by a power of two before the head + remainder split, so a query of 2^40
    (past fp16's largest value) or 2^-60 (below its smallest) is held to
    the usual tolerance."""
    w = custom_workload(context_lens=[1, 40, 300, 1000, 2500], num_q_heads=8, num_kv_heads=2,
                        head_dim=128, kv_dtype=kv, seed=33)
    w.q = (w.q.astype(np.float64) * 2.0 ** k).astype(np.float32)
    w.scale = np.float32(float(w.scale) * 2.0 ** -k)
    say(f"decode kv={kv} q={q_dtype} query x 2^{k}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = torch.from_numpy(w.q).cuda().to(TORCH_DT[q_dtype])
    assert torch.all(torch.isfinite(q))
    out = run_decode(pkv, w, gc, q)
    ref = oracle.ref_decode(q.double().cpu().numpy(), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    assert oracle.max_abs_err(to_f64(out), ref) <= (2e-5 if kv == "f32" else 1e-2)
