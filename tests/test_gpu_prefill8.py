"""GPU parity of the chunked prefill and the mixed call over int8 and FP8 KV
caches, against the fp64 oracle on the stored codes and scales.

The kernel converts the codes to fp16 exactly, multiplies the scores by the
K scales, and folds the V scales into the fp16 probabilities under a
power-of-two normaliser.  The query row is scaled by a power of two before
it is rounded to fp16.  Beyond the shapes: V scales that span many binades
within a sequence, queries far outside fp16's range, NaN scales at one
position, and the one-token rows of a mixed call, which must equal the
decode bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TORCH_DT, np_to_gpu, oracle_cache, poisoned_gpu_cache, q_exact_values,
                         q_tensor, run_decode, run_prefill, say, small_prefill, to_f64,
                         used_slot_mask)
from workloads import make_workload

pytestmark = pytest.mark.gpu
PS = 16


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _ref(w, cache, q, window=0):
    return oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                    w.cu_q_lens, w.scale, window=window)


def _mixed(pkv, w, gc, q):
    out = pkv.paged_attn_mixed(q, gc["k"], gc["v"], np_to_gpu(w.block_tables),
                               np_to_gpu(w.context_lens), np_to_gpu(w.cu_q_lens), w.max_q_len,
                               w.max_context_len, w.scale, k_scales=gc["ks"], v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_prefill8_bench_batch_full_size(pkv, kv):
    """The benchmarked prefill batch (8 chunks of 512 over prefixes of 289
    to 3499 tokens, 12 query heads on 2 KV heads, head_dim 128) stored as
    int8 / FP8: every row against the oracle."""
    w = make_workload("C4")
    say(f"prefill C4 batch stored as {kv}: {w.num_query_tokens} query rows")
    cache = oracle_cache(w, kv)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = run_prefill(pkv, w, gc, q)
    err = oracle.max_abs_err(to_f64(out), _ref(w, cache, q))
    say(f"  max abs err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("plan", ["long_chunks", "short_chunks"])
def test_mixed8_matches_oracle(pkv, kv, d, plan):
    """Mixed batches over a one-byte cache: one-token rows as decode
    partitions, longer chunks as prefill row blocks, each plan of the
    one-token rows (long chunks present, or short chunks only)."""
    if plan == "long_chunks":
        ctx = [700, 1, 333, 2049, 45, 0, 5000, 129, 64]
        chunk = [1, 1, 300, 1, 45, 0, 1, 128, 1]
    else:
        ctx = [2, 1500, 40, 5, 700, 128, 3000, 17, 260]
        chunk = [2, 1, 33, 5, 1, 127, 1, 16, 100]
    say(f"mixed kv={kv} d={d} {plan}")
    w = small_prefill(ctx, chunk, 12, 2, d, kv, seed=801 + d)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = _mixed(pkv, w, gc, q)
    assert oracle.max_abs_err(to_f64(out), _ref(w, cache, q)) <= 1e-2
    pre = run_prefill(pkv, w, gc, q)
    assert torch.max(torch.abs(out - pre)).item() <= 1e-2


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_mixed8_one_token_batch_is_decode_bit_for_bit(pkv, kv):
    rng = np.random.default_rng(805)
    ctx = [int(x) for x in rng.integers(1, 5000, size=30)]
    w = small_prefill(ctx, [1] * 30, 12, 2, 128, kv, seed=805)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "f32")
    mixed = _mixed(pkv, w, gc, q)
    dec = run_decode(pkv, w, gc, q)
    assert torch.equal(dec, mixed)


def _spread_v(w, lo_exp, hi_exp):
    """Scale each token's V by 10^e, e running linearly from lo_exp at
    position 0 to hi_exp at the sequence's last position; returns the gain
    of each (sequence, position)."""
    gains = []
    for b in range(w.batch):
        t0, t1 = int(w.token_offsets[b]), int(w.token_offsets[b + 1])
        n = t1 - t0
        g = 10.0 ** np.linspace(lo_exp, hi_exp, n)
        w.v[t0:t1] *= g[:, None, None].astype(np.float32)
        gains.append(g)
    return gains


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_prefill8_v_scales_across_binades(pkv, kv, direction):
    """V magnitudes from 1e-6 to 1e6 along each sequence (rising: the
    normaliser is raised again and again as the walk goes on; falling: later
    scales lie far below it).  Attention is linear in V, so each row is held
    to 1e-2 times the largest gain among the positions it attends."""
    ctx, chunk = [900, 400, 1300], [300, 400, 129]
    w = small_prefill(ctx, chunk, 6, 2, 128, kv, seed=811)
    gains = _spread_v(w, -6.0, 6.0) if direction == "rising" else _spread_v(w, 6.0, -6.0)
    say(f"prefill {kv} V across binades ({direction})")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    for name, out in (("prefill", run_prefill(pkv, w, gc, q)), ("mixed", _mixed(pkv, w, gc, q))):
        got, ref = to_f64(out), _ref(w, cache, q)
        assert np.all(np.isfinite(got)), name
        for b in range(w.batch):
            r0, r1 = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
            P = ctx[b] - chunk[b]
            for i in range(r1 - r0):
                tol = 1e-2 * float(np.max(gains[b][:P + i + 1]))
                err = float(np.max(np.abs(got[r0 + i] - ref[r0 + i])))
                assert err <= tol, (name, b, i, err, tol)


@pytest.mark.parametrize("kv", ["i8", "fp8", "f16"])
@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k", [-60, -20, 20, 40])
def test_prefill_query_outside_fp16_range(pkv, kv, q_dtype, k):
    """The query times 2^k with the scale times 2^-k (the same scores): a
    query of magnitude 2^40 overflows fp16 and one of 2^-60 underflows it,
    and the fp16-operand paths (one-byte caches, and an fp16 cache with a
    bf16 or fp32 query) scale each row by a power of two first."""
    w = small_prefill([300, 90, 17], [200, 90, 17], 6, 2, 64, kv, seed=820)
    w.q = (w.q.astype(np.float64) * 2.0 ** k).astype(np.float32)
    w.scale = np.float32(float(w.scale) * 2.0 ** -k)
    say(f"prefill kv={kv} q={q_dtype} query x 2^{k}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, q_dtype)
    assert torch.all(torch.isfinite(q))
    out = run_prefill(pkv, w, gc, q)
    assert oracle.max_abs_err(to_f64(out), _ref(w, cache, q)) <= 1e-2


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_prefill8_query_rows_with_tiny_elements(pkv, kv):
    """Rows whose elements alternate between unit size and 1e-6: the small
    ones keep their bits after the row's power-of-two scaling."""
    w = small_prefill([400], [256], 6, 2, 128, kv, seed=821)
    w.q[:, :, 1::2] *= np.float32(1e-6)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    for qd in ("bf16", "f32"):
        q = q_tensor(w, qd)
        out = run_prefill(pkv, w, gc, q)
        assert oracle.max_abs_err(to_f64(out), _ref(w, cache, q)) <= 1e-2


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("which", ["k", "v"])
def test_prefill8_nan_scale_reaches_only_rows_that_attend_it(pkv, kv, which):
    """A NaN K or V scale at position p of a chunk (the append's encoding of
    a vector holding a NaN): rows that attend p are NaN in the query heads
    of that KV head; rows before p, and the other KV head's query heads,
    equal the oracle (the zero probability of a masked key times a NaN V
    scale contributes nothing)."""
    w = small_prefill([330, 100], [250, 100], 6, 2, 128, kv, seed=830)
    P, p = 80, 80 + 137
    cache = oracle_cache(w)
    page, off = int(w.block_tables[0, p // PS]), p % PS
    getattr(cache, f"{which}_scales")[page, 1, off] = np.nan
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    with np.errstate(invalid="ignore"):
        ref = _ref(w, cache, q)
    for name, out in (("prefill", run_prefill(pkv, w, gc, q)), ("mixed", _mixed(pkv, w, gc, q))):
        got = to_f64(out)
        hit = p - P                             # first row of sequence 0 that attends p
        assert np.all(np.isnan(got[hit:250, 3:])), name
        keep = np.ones(got.shape[:2], bool)
        keep[hit:250, 3:] = False
        assert np.all(np.isfinite(got[keep])), name
        assert np.max(np.abs(got[keep] - ref[keep])) <= 1e-2, name


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_prefill8_every_code_converts_exactly(pkv, kv):
    """K and V vectors drawn from every finite E4M3 code (FP8) or every int8
    code, each vector holding the top code so its scale is the same power
    of two for all: the stored values are the codes' own, times that power.
    A large softmax scale makes most rows attend one key, so a row returns
    that key's V vector.  Each element is held to 2^-9 relative to the
    oracle's sum of weight x |V| (the fp16 rounding of the scaled
    probability is 2^-11).  A code converted to a neighbouring value is off
    by at least 2^-4 (FP8) or 1/127 (int8) relative."""
    w = small_prefill([192], [64], 4, 1, 128, kv, seed=840)
    rng = np.random.default_rng(840)
    if kv == "fp8":
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        vals = oracle.e4m3_bits_to_f64(finite).astype(np.float32)
        top = np.float32(448.0)
    else:
        vals = np.arange(-127, 128, dtype=np.float32)
        top = np.float32(127.0)
    for arr in (w.k, w.v):
        for t in range(arr.shape[0]):
            x = np.concatenate([[top], rng.choice(vals, size=127)]).astype(np.float32)
            arr[t, 0] = x[rng.permutation(128)]
    w.k *= np.float32(1.0 / 64)
    w.scale = np.float32(200.0 / 64)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = to_f64(run_prefill(pkv, w, gc, q))
    ref = _ref(w, cache, q)
    absv = cache.copy()
    absv.v = np.abs(absv.v) if kv == "i8" else absv.v & np.uint8(0x7F)
    bound = _ref(w, absv, q)               # sum over keys of weight x |V|
    assert np.all(np.isfinite(out))
    excess = np.abs(out - ref) - (2.0 ** -9 * bound + 1e-6)
    assert np.max(excess) <= 0, float(np.max(excess))
