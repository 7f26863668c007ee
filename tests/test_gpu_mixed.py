"""GPU parity of the mixed prefill/decode call (paged_attn_mixed): one launch
where one-token chunks run as split decode partitions and longer chunks as
MFMA prefill row blocks.  Same semantics as paged_attn_prefill_chunk, so the
same oracle (ref_prefill_chunk) checks it; structural checks compare the
one-token rows with paged_attn_decode bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (np_to_gpu, oracle_cache, poisoned_gpu_cache, q_exact_values, q_tensor,
                         say, small_prefill, to_f64, used_slot_mask)
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def run_mixed(pkv, w, gc, q, out_dtype=torch.float32, max_context_len=None):
    mcl = w.max_context_len if max_context_len is None else max_context_len
    out = pkv.paged_attn_mixed(q, gc["k"], gc["v"], np_to_gpu(w.block_tables), np_to_gpu(w.context_lens),
                               np_to_gpu(w.cu_q_lens), w.max_q_len, mcl, w.scale, out_dtype=out_dtype,
                               k_scales=gc["ks"], v_scales=gc["vs"])
    torch.cuda.synchronize()
    return out


def ref(w, cache, q):
    return oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                    w.cu_q_lens, w.scale)


@pytest.mark.parametrize("kv,d,qd", [("bf16", 128, "bf16"), ("f16", 64, "f16"), ("bf16", 64, "f32"),
                                     ("f16", 128, "bf16"), ("f32", 128, "f32"), ("f32", 64, "bf16")])
def test_mixed_matches_oracle(pkv, kv, d, qd):
    ctx = [700, 1, 333, 2049, 45, 0, 5000, 129, 64]
    chunk = [1, 1, 300, 1, 45, 0, 1, 128, 1]
    say(f"mixed kv={kv} d={d} q={qd}")
    w = small_prefill(ctx, chunk, 12, 2, d, kv, seed=301)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, qd)
    out = run_mixed(pkv, w, gc, q)
    assert oracle.max_abs_err(to_f64(out), ref(w, cache, q)) <= (2e-5 if kv == "f32" else 1e-2)


def test_mixed_decode_rows_equal_decode_and_rest_equals_prefill(pkv):
    rng = np.random.default_rng(302)
    ctx = [int(x) for x in rng.integers(512, 4097, size=24)] + [900, 3000]
    chunk = [1] * 24 + [256, 512]
    w = small_prefill(ctx, chunk, 12, 2, 128, "bf16", seed=302)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    mixed = run_mixed(pkv, w, gc, q)
    pre = pkv.paged_attn_prefill_chunk(q, gc["k"], gc["v"], np_to_gpu(w.block_tables),
                                       np_to_gpu(w.context_lens), np_to_gpu(w.cu_q_lens),
                                       w.max_q_len, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(mixed - pre)).item() <= 1e-2
    # the decode entry point over all 26 sequences (a prefill chunk's last row
    # attends to its whole context, like a decode token); with chunks in the
    # batch the mixed call does not split the one-token rows, so they agree
    # within rounding rather than bit for bit
    last = [int(w.cu_q_lens[b]) if b < 24 else int(w.cu_q_lens[b + 1]) - 1 for b in range(26)]
    rows = torch.tensor(last, device="cuda")
    dec = pkv.paged_attn_decode(q[rows].contiguous(), gc["k"], gc["v"], np_to_gpu(w.block_tables),
                                np_to_gpu(w.context_lens), w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(dec[:24] - mixed[rows[:24]])).item() <= 1e-5
    assert torch.max(torch.abs(dec[24:] - mixed[rows[24:]])).item() <= 1e-2


def test_mixed_one_token_batch_is_decode_bit_for_bit(pkv):
    """A batch of one-token chunks is planned and computed exactly as the
    decode entry point (same splits and merge)."""
    rng = np.random.default_rng(305)
    ctx = [int(x) for x in rng.integers(1, 6000, size=40)]
    w = small_prefill(ctx, [1] * 40, 12, 2, 128, "bf16", seed=305)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "f32")
    mixed = run_mixed(pkv, w, gc, q)
    dec = pkv.paged_attn_decode(q, gc["k"], gc["v"], np_to_gpu(w.block_tables),
                                np_to_gpu(w.context_lens), w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(dec, mixed)
    assert oracle.max_abs_err(to_f64(mixed), ref(w, cache, q)) <= 1e-2


def test_mixed_pure_decode_batch(pkv):
    ctx = [17, 64, 133, 200, 4096, 1]
    w = small_prefill(ctx, [1] * 6, 9, 3, 64, "f16", seed=303)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "f16")
    out = run_mixed(pkv, w, gc, q, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    assert oracle.max_abs_err(to_f64(out), ref(w, cache, q)) <= 1e-2


def test_mixed_bad_inputs_give_nan_rows(pkv):
    ctx = [300, 40, 90]
    chunk = [100, 1, 1]
    w = small_prefill(ctx, chunk, 6, 2, 128, "bf16", seed=304)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    good = ref(w, cache, q)
    page = int(w.block_tables[1, 1])
    w.block_tables[1, 1] = w.num_pages + 3          # decode row 100 reads page 1 (tokens 16..31)
    out = run_mixed(pkv, w, gc, q).cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(out[100])) and np.all(np.isfinite(out[[0, 99, 101]]))
    assert oracle.max_abs_err(out[:100], good[:100]) <= 1e-2     # the chunk's 100 rows
    assert oracle.max_abs_err(out[101:], good[101:]) <= 1e-2
    w.block_tables[1, 1] = page
    w.context_lens[2] = 0                            # a one-token chunk longer than its context
    out = run_mixed(pkv, w, gc, q).cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(out[101]))
    assert oracle.max_abs_err(out[:101], good[:101]) <= 1e-2


@pytest.mark.parametrize("name", ["M1", "M2"])
def test_mixed_bench_batches_full_size(pkv, name):
    """The two mixed batches the benchmark times, every row against the
    oracle: M1 (C2's 64 decode rows and C4's 512-token chunks: long chunks,
    so the one-token rows take the fewest splits) and M2 (the same decode
    rows and four 64-token chunks: short chunks, so the one-token rows are
    split as in a decode call)."""
    w = make_workload(name)
    say(f"mixed {name} full size: {w.batch} sequences, {w.num_query_tokens} query rows")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = run_mixed(pkv, w, gc, q)
    err = oracle.max_abs_err(to_f64(out), ref(w, cache, q))
    say(f"  max abs err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_short_chunks_every_row(pkv, d):
    """Chunks of 2 to 127 tokens beside one-token rows (the plan that splits
    the one-token rows as a decode call), every row against the oracle."""
    ctx = [2, 1500, 40, 5, 700, 128, 3000, 17, 260]
    chunk = [2, 1, 33, 5, 1, 127, 1, 16, 100]
    w = small_prefill(ctx, chunk, 8, 2, d, "bf16", seed=306)
    say(f"mixed short chunks d={d}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = run_mixed(pkv, w, gc, q)
    assert oracle.max_abs_err(to_f64(out), ref(w, cache, q)) <= 1e-2
