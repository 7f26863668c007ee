"""Seeded randomised GPU parity (shapes, dtypes, lengths) and structural
properties of the HIP path, through the C ABI, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, np_to_gpu, oracle_cache, poisoned_gpu_cache, q_exact_values,
                         q_tensor, run_decode, run_prefill, say, small_decode, small_prefill,
                         to_f64, used_slot_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _lengths(rng, n, hi):
    """Context lengths mixing page/tile boundaries, tiny and long ones."""
    special = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257]
    out = []
    for _ in range(n):
        out.append(int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(1, hi + 1)))
    return out


@pytest.mark.parametrize("it", range(24))
def test_decode_fuzz(pkv, it):
    rng = np.random.default_rng(1000 + it)
    kv = ["f32", "bf16", "f16", "i8", "fp8"][it % 5]
    d = [64, 128][(it // 4) % 2]
    hkv = int(rng.choice([1, 2, 3, 4]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 20]))
    B = int(rng.integers(1, 13))
    ctx = _lengths(rng, B, 3000)
    slack = int(rng.integers(0, 200))
    w = small_decode(ctx, hkv * G, hkv, d, kv, seed=2000 + it,
                     table_width=max(1, (max(ctx) + slack + 15) // 16))
    q_dtype = ["f32", "bf16", "f16"][it % 3]
    say(f"decode fuzz {it}: kv={kv} d={d} Hkv={hkv} G={G} B={B} ctx={ctx} q={q_dtype}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, q_dtype)
    mcl = max(ctx) + slack
    out = run_decode(pkv, w, gc, q, max_context_len=mcl)
    ref = oracle.ref_decode(q_exact_values(q), cache, w.block_tables, w.context_lens, w.scale,
                            w.num_q_heads)
    err = oracle.max_abs_err(to_f64(out), ref)
    assert err <= TOL[kv], err


@pytest.mark.parametrize("it", range(20))
def test_prefill_fuzz(pkv, it):
    rng = np.random.default_rng(3000 + it)
    kv = ["bf16", "f16", "i8", "fp8", "f32"][it % 5]
    d = [64, 128][(it // 5) % 2]
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 3, 6, 8]))
    B = int(rng.integers(1, 6))
    prefix = [int(x) for x in rng.integers(0, 700, size=B)]
    chunk = [int(rng.choice([0, 1, 7, 32, 33, 100, 300])) for _ in range(B)]
    ctx = [p + c for p, c in zip(prefix, chunk)]
    w = small_prefill(ctx, chunk, hkv * G, hkv, d, kv, seed=4000 + it)
    say(f"prefill fuzz {it}: kv={kv} d={d} Hkv={hkv} G={G} P={prefix} C={chunk}")
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, kv if kv in ("bf16", "f16") else ["bf16", "f16", "f32"][it % 3])
    tol = TOL[kv]
    out = run_prefill(pkv, w, gc, q)
    assert out.shape == q.shape
    if w.num_query_tokens == 0:            # every chunk empty: a no-op
        return
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    assert oracle.max_abs_err(to_f64(out), ref) <= tol


def test_mixed_prefill_and_decode_rows(pkv):
    """One prefill call carrying decode rows (chunks of one token) beside long
    chunks equals the oracle, and its one-token rows equal decode calls."""
    ctx = [700, 1, 300, 2049, 45]
    chunk = [1, 1, 256, 1, 45]
    w = small_prefill(ctx, chunk, 12, 2, 128, "bf16", seed=77)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out = run_prefill(pkv, w, gc, q)
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2
    for b in (0, 1, 3):
        row = int(w.cu_q_lens[b])
        wd = small_decode([ctx[b]], 12, 2, 128, "bf16", seed=5)
        wd.block_tables = w.block_tables[b:b + 1].copy()
        dec = run_decode(pkv, wd, gc, q[row:row + 1].contiguous())
        assert torch.max(torch.abs(dec[0] - out[row])).item() <= 1e-2


def test_prefill_chunk_split_equivalence(pkv):
    """Prefilling [0, C) in one call or as [0, C1) then [C1, C) gives the
    same rows (within tolerance): a chunk sees only its prefix."""
    w = small_prefill([600], [400], 6, 2, 128, "bf16", seed=91)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    full = run_prefill(pkv, w, gc, q)
    bt, out = np_to_gpu(w.block_tables), []
    for lo, hi in ((0, 150), (150, 400)):
        cl = torch.tensor([200 + hi], dtype=torch.int32, device="cuda")
        cu = torch.tensor([0, hi - lo], dtype=torch.int32, device="cuda")
        out.append(pkv.paged_attn_prefill_chunk(q[lo:hi].contiguous(), gc["k"], gc["v"], bt, cl, cu,
                                                hi - lo, 600, w.scale))
    torch.cuda.synchronize()
    assert torch.max(torch.abs(torch.cat(out) - full)).item() <= 2e-3


def test_prefill_causal_future_is_invisible(pkv):
    """Changing K/V at positions after a row's limit (inside the context)
    leaves that row bit-identical on the GPU and changes later rows."""
    w = small_prefill([500], [300], 6, 2, 128, "bf16", seed=92)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    out1 = run_prefill(pkv, w, gc, q)
    p = 200 + 123                          # rows i < 123 must not see it
    page, off = int(w.block_tables[0, p // 16]), p % 16
    gc["k"][page, :, off, :] += 1.0
    gc["v"][page, :, :, off] -= 2.0
    out2 = run_prefill(pkv, w, gc, q)
    assert torch.equal(out1[:123], out2[:123])
    assert not torch.equal(out1[123:], out2[123:])


def test_prefill_output_dtypes_and_bad_page(pkv):
    w = small_prefill([300, 90], [100, 90], 6, 2, 128, "bf16", seed=93)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    for od in (torch.bfloat16, torch.float16):
        out = run_prefill(pkv, w, gc, q, out_dtype=od)
        assert out.dtype == od
        assert oracle.max_abs_err(to_f64(out), ref) <= 1e-2
    # sequence 1 (no prefix, rows 100..189 at positions 0..89) gets a bad id
    # for its third page (positions 32..47): every row that must read it is
    # NaN, rows that need not read it are NaN or correct, sequence 0 is correct
    w.block_tables[1, 2] = w.num_pages + 7
    out = run_prefill(pkv, w, gc, q).cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(out[132:]))
    head = out[100:132]
    ok = np.isnan(head).all(axis=(1, 2)) | (np.abs(head - ref[100:132]).max(axis=(1, 2)) <= 1e-2)
    assert ok.all()
    assert oracle.max_abs_err(out[:100], ref[:100]) <= 1e-2


def test_prefill_bad_context_length_gives_nan(pkv):
    """A context length past max_context_len (device data the host cannot
    check) turns that sequence's rows into NaN and leaves the others exact,
    also when the workgroups take the row blocks in ranked order (the
    contexts differ, so the bad value takes part in the ranking)."""
    w = small_prefill([200, 60, 130], [64, 60, 30], 6, 2, 64, "bf16", seed=95)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    q = q_tensor(w, "bf16")
    ref = oracle.ref_prefill_chunk(q_exact_values(q), cache, w.block_tables, w.context_lens,
                                   w.cu_q_lens, w.scale)
    w.context_lens[1] = 10 ** 6
    out = run_prefill(pkv, w, gc, q, max_context_len=200).cpu().numpy().astype(np.float64)
    lo, hi = int(w.cu_q_lens[1]), int(w.cu_q_lens[2])
    assert np.all(np.isnan(out[lo:hi]))
    keep = np.r_[0:lo, hi:out.shape[0]]
    assert oracle.max_abs_err(out[keep], ref[keep]) <= 1e-2


def test_decode_bad_context_length_gives_nan(pkv):
    w = small_decode([40, 50], 4, 2, 64, "bf16", seed=94)
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    w.context_lens[1] = 10 ** 6            # beyond max_context_len and the table row
    out = run_decode(pkv, w, gc, q_tensor(w), max_context_len=50).cpu().numpy()
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[0]))
