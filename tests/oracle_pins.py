"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle module ``O`` and raises AssertionError (or any
exception) when the oracle violates what the pages and the mathematics fix:
brute force with ``math.fsum`` on tiny inputs, torch's fp64 SDPA on the CPU,
closed forms, invariants, the causal structure, library cross-checks of the
conversions and hand-derived golden values.  The same pins run against the
real oracle (they must all pass) and against deliberately broken copies of it
(each copy must fail at least one), so a plausible slip in the oracle cannot
hide.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from workloads import custom_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PS = 16


# ------------------------------------------------------------------ helpers
def _seq(w, arr, b):
    return arr[int(w.token_offsets[b]):int(w.token_offsets[b + 1])]


def write_paged_f32(O, seqs_k, seqs_v, block_tables, num_pages, hkv, d):
    """Lay dense per-sequence K/V ([n, Hkv, d] each) into an fp32 pool with
    explicit loops over the layout definition: K[page, g, off, i] and
    V[page, g, i, off] for token t at page block_tables[b][t // 16],
    offset t % 16."""
    cache = O.PagedCache(num_pages, hkv, d, "f32")
    for b, (ks, vs) in enumerate(zip(seqs_k, seqs_v)):
        for t in range(len(ks)):
            page, off = int(block_tables[b][t // PS]), t % PS
            for g in range(hkv):
                for i in range(d):
                    cache.k[page, g, off, i] = ks[t][g][i]
                    cache.v[page, g, i, off] = vs[t][g][i]
    return cache


def brute_attention_row(qrow, ks, vs, g, scale):
    """softmax over keys of scale*q.k, then the weighted sum of V, with
    Python floats and math.fsum (no numpy)."""
    d = len(qrow)
    scores = [scale * math.fsum(float(qrow[i]) * float(k[g][i]) for i in range(d)) for k in ks]
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = math.fsum(e)
    return [math.fsum(e[t] * float(vs[t][g][i]) for t in range(len(ks))) / z for i in range(d)]


def _dense_stored(x_f32, dtype, O):
    """Stored values as float64, derived with torch's own casts (not the
    oracle's) for bf16/f16; int8 uses the quantizer under test."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32))
    if dtype == "f32":
        return t.double().numpy()
    if dtype == "bf16":
        return t.to(torch.bfloat16).double().numpy()
    if dtype == "f16":
        return t.to(torch.float16).double().numpy()
    if dtype == "fp8":
        # absmax scale in fp32, then torch's own E4M3 rounding of the ratio
        x = np.asarray(x_f32, np.float32)
        sc = (np.max(np.abs(x), axis=-1) / np.float32(448.0)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        r = np.clip((x / safe[..., None]).astype(np.float32), -448, 448).astype(np.float32)
        codes = torch.from_numpy(r).to(torch.float8_e4m3fn).double().numpy()
        return np.where((sc > 0)[..., None], codes, 0.0) * sc.astype(np.float64)[..., None]
    codes, sc = O.quantize_int8(x_f32)
    return codes.astype(np.float64) * sc.astype(np.float64)[..., None]


def _filled_cache(O, w, dtype=None):
    c = O.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim, dtype or w.kv_dtype)
    O.ref_append(c, w.k, w.v, w.slot_mapping)
    return c


def _sdpa(q, k, v, scale, mask=None):
    """torch fp64 SDPA on the CPU; q [Hq, L, d], k/v [Hq, n, d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
        scale=scale)[0].numpy()


# ------------------------------------------------------------------ attention pins
def pin_bruteforce_decode(O):
    w = custom_workload(context_lens=[1, 5, 37, 16], num_q_heads=4, num_kv_heads=2,
                        head_dim=8, num_pages=12, seed=11)
    ks = [_seq(w, w.k, b) for b in range(w.batch)]
    vs = [_seq(w, w.v, b) for b in range(w.batch)]
    cache = write_paged_f32(O, ks, vs, w.block_tables, w.num_pages, 2, 8)
    out = O.ref_decode(w.q, cache, w.block_tables, w.context_lens, w.scale, 4)
    for b in range(w.batch):
        for h in range(4):
            g = h * 2 // 4
            ref = brute_attention_row(w.q[b, h], ks[b], vs[b], g, w.scale)
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12, (b, h)


def pin_bruteforce_prefill(O):
    w = custom_workload(kind="prefill", context_lens=[9, 21, 18], q_lens=[9, 5, 1],
                        num_q_heads=2, num_kv_heads=1, head_dim=4, num_pages=8, seed=12)
    ks = [_seq(w, w.k, b) for b in range(w.batch)]
    vs = [_seq(w, w.v, b) for b in range(w.batch)]
    cache = write_paged_f32(O, ks, vs, w.block_tables, w.num_pages, 1, 4)
    out = O.ref_prefill_chunk(w.q, cache, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    for b in range(w.batch):
        n, C = int(w.context_lens[b]), int(w.q_lens[b])
        P = n - C
        for i in range(C):
            row = int(w.cu_q_lens[b]) + i
            for h in range(2):
                ref = brute_attention_row(w.q[row, h], ks[b][:P + i + 1], vs[b][:P + i + 1], 0, w.scale)
                assert np.max(np.abs(out[row, h] - ref)) <= 1e-12, (b, i, h)


def pin_sdpa_decode_all_dtypes(O):
    for dtype in ("f32", "bf16", "f16", "i8", "fp8"):
        w = custom_workload(context_lens=[16, 17, 33, 70], num_q_heads=6, num_kv_heads=2,
                            head_dim=16, kv_dtype=dtype, num_pages=24, seed=13)
        cache = _filled_cache(O, w)
        out = O.ref_decode(w.q, cache, w.block_tables, w.context_lens, w.scale, 6)
        for b in range(w.batch):
            K = _dense_stored(_seq(w, w.k, b), dtype, O)
            V = _dense_stored(_seq(w, w.v, b), dtype, O)
            k = np.repeat(K.transpose(1, 0, 2), 3, axis=0)
            v = np.repeat(V.transpose(1, 0, 2), 3, axis=0)
            ref = _sdpa(w.q[b][:, None, :].astype(np.float64), k, v, w.scale)[:, 0, :]
            assert np.max(np.abs(out[b] - ref)) <= 1e-12, (dtype, b)


def pin_sdpa_prefill_bottom_right(O):
    w = custom_workload(kind="prefill", context_lens=[20, 40, 35, 16], q_lens=[20, 17, 1, 16],
                        num_q_heads=4, num_kv_heads=1, head_dim=8, num_pages=16, seed=14)
    cache = _filled_cache(O, w)
    out = O.ref_prefill_chunk(w.q, cache, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    for b in range(w.batch):
        n, C = int(w.context_lens[b]), int(w.q_lens[b])
        P = n - C
        K = _seq(w, w.k, b).astype(np.float64)
        V = _seq(w, w.v, b).astype(np.float64)
        mask = np.array([[j <= P + i for j in range(n)] for i in range(C)])
        r0 = int(w.cu_q_lens[b])
        q = w.q[r0:r0 + C].transpose(1, 0, 2).astype(np.float64)
        k = np.repeat(K.transpose(1, 0, 2), 4, axis=0)
        v = np.repeat(V.transpose(1, 0, 2), 4, axis=0)
        ref = _sdpa(q, k, v, w.scale, mask).transpose(1, 0, 2)
        assert np.max(np.abs(out[r0:r0 + C] - ref)) <= 1e-12, b


def pin_golden_closed_forms(O):
    with open(os.path.join(GOLDEN, "attention_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q = np.array(case["q"], dtype=np.float32)[None]          # [1, Hq, d]
        k = np.array(case["k"], dtype=np.float32)                 # [n, Hkv, d]
        v = np.array(case["v"], dtype=np.float32)
        n, hkv, d = k.shape
        bt = np.array([[3, 1]], dtype=np.int32)
        cache = write_paged_f32(O, [k], [v], bt, 4, hkv, d)
        out = O.ref_decode(q, cache, bt, np.array([n], np.int32), case["scale"], q.shape[1])
        err = np.max(np.abs(out[0] - np.array(case["out"])))
        assert err <= case["tol"], (case["name"], err)


def pin_single_token_returns_v(O):
    for dtype in ("f32", "bf16", "f16", "i8"):
        w = custom_workload(context_lens=[1, 1, 1], num_q_heads=4, num_kv_heads=2,
                            head_dim=16, kv_dtype=dtype, seed=15)
        out = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 4)
        for b in range(3):
            Vd = _dense_stored(_seq(w, w.v, b), dtype, O)[0]          # [Hkv, d]
            assert np.array_equal(out[b], np.repeat(Vd, 2, axis=0)), (dtype, b)


def pin_empty_context_is_zero(O):
    w = custom_workload(context_lens=[0, 3, 0], num_q_heads=2, num_kv_heads=2, head_dim=8, seed=16)
    out = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 2)
    assert np.all(out[0] == 0) and np.all(out[2] == 0) and np.any(out[1] != 0)


def pin_scale_zero_is_mean(O):
    w = custom_workload(context_lens=[7, 40], num_q_heads=3, num_kv_heads=1, head_dim=8,
                        scale=0.0, seed=17)
    out = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, 0.0, 3)
    for b in range(2):
        mean = _seq(w, w.v, b).astype(np.float64).mean(axis=0)[0]
        assert np.max(np.abs(out[b] - mean[None])) <= 1e-14


def pin_shift_and_hull(O):
    # V drawn on a coarse grid so that V + 1 is exact in fp32.
    w = custom_workload(context_lens=[5, 33, 64], num_q_heads=2, num_kv_heads=1, head_dim=8, seed=18)
    w.v[:] = np.round(w.v * 8) / 8
    c0 = _filled_cache(O, w)
    out0 = O.ref_decode(w.q, c0, w.block_tables, w.context_lens, w.scale, 2)
    w.v[:] += 1.0
    out1 = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 2)
    assert np.max(np.abs(out1 - (out0 + 1.0))) <= 1e-13
    for b in range(w.batch):
        V = _seq(w, w.v, b).astype(np.float64)[:, 0, :]
        assert np.all(out1[b] >= V.min(axis=0) - 1e-13) and np.all(out1[b] <= V.max(axis=0) + 1e-13)


def pin_page_permutation_invariance(O):
    w = custom_workload(context_lens=[20, 50, 3], num_q_heads=4, num_kv_heads=2, head_dim=8,
                        kv_dtype="bf16", num_pages=20, seed=19)
    c = _filled_cache(O, w)
    out = O.ref_decode(w.q, c, w.block_tables, w.context_lens, w.scale, 4)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(w.num_pages)
    inv = np.argsort(perm)               # new page p holds old page perm[p]
    c2 = c.copy()
    c2.k, c2.v = c.k[perm], c.v[perm]
    bt2 = inv[w.block_tables].astype(np.int32)
    out2 = O.ref_decode(w.q, c2, bt2, w.context_lens, w.scale, 4)
    assert np.array_equal(out, out2)


def pin_gqa_equals_repeated_mha(O):
    w = custom_workload(context_lens=[9, 30], num_q_heads=6, num_kv_heads=2, head_dim=8, seed=20)
    out = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 6)
    w.k = np.repeat(w.k, 3, axis=1)
    w.v = np.repeat(w.v, 3, axis=1)
    w.num_kv_heads = 6
    out_mha = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 6)
    assert np.array_equal(out, out_mha)


def pin_group_locality(O):
    w = custom_workload(context_lens=[9, 30], num_q_heads=6, num_kv_heads=3, head_dim=8, seed=21)
    out = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 6)
    w.v[:, 1, :] += 0.5
    out2 = O.ref_decode(w.q, _filled_cache(O, w), w.block_tables, w.context_lens, w.scale, 6)
    changed = np.any(out != out2, axis=(0, 2))
    assert list(changed) == [False, False, True, True, False, False], changed


def pin_causal_structure(O):
    w = custom_workload(kind="prefill", context_lens=[45], q_lens=[20], num_q_heads=2,
                        num_kv_heads=1, head_dim=8, seed=22)
    P = 25
    out = O.ref_prefill_chunk(w.q, _filled_cache(O, w), w.block_tables, w.context_lens,
                              w.cu_q_lens, w.scale)
    for p in (P + 3, P + 11, 44):
        w2 = custom_workload(kind="prefill", context_lens=[45], q_lens=[20], num_q_heads=2,
                             num_kv_heads=1, head_dim=8, seed=22)
        w2.k[p] += 2.0
        w2.v[p] -= 3.0
        out2 = O.ref_prefill_chunk(w2.q, _filled_cache(O, w2), w2.block_tables,
                                   w2.context_lens, w2.cu_q_lens, w2.scale)
        for i in range(20):
            same = np.array_equal(out[i], out2[i])
            assert same == (P + i < p), (p, i)


def pin_prefill_row_equals_decode(O):
    w = custom_workload(kind="prefill", context_lens=[37, 16], q_lens=[12, 16], num_q_heads=4,
                        num_kv_heads=2, head_dim=8, seed=23)
    c = _filled_cache(O, w)
    out = O.ref_prefill_chunk(w.q, c, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    for b in range(2):
        n, C = int(w.context_lens[b]), int(w.q_lens[b])
        for i in range(C):
            row = int(w.cu_q_lens[b]) + i
            dec = O.ref_decode(w.q[row][None], c, w.block_tables[b:b + 1],
                               np.array([n - C + i + 1], np.int32), w.scale, 4)
            assert np.max(np.abs(out[row] - dec[0])) <= 1e-13, (b, i)
    # P = 0, i = 0 attends to the first token only
    b1 = int(w.cu_q_lens[1])
    v0 = _seq(w, w.v, 1)[0].astype(np.float64)
    assert np.array_equal(out[b1], np.repeat(v0, 2, axis=0))


def pin_chunk_split(O):
    w = custom_workload(kind="prefill", context_lens=[50], q_lens=[30], num_q_heads=2,
                        num_kv_heads=1, head_dim=8, seed=24)
    c = _filled_cache(O, w)
    full = O.ref_prefill_chunk(w.q, c, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    a = O.ref_prefill_chunk(w.q[:11], c, w.block_tables, np.array([31], np.int32),
                            np.array([0, 11], np.int32), w.scale)
    b = O.ref_prefill_chunk(w.q[11:], c, w.block_tables, np.array([50], np.int32),
                            np.array([0, 19], np.int32), w.scale)
    assert np.max(np.abs(np.concatenate([a, b]) - full)) <= 1e-13


def pin_prefill_unseen_nonfinite_v(O):
    """A position a chunk row does not attend (after its causal limit, or
    before its window) takes no part in that row, even when its V holds NaN
    or inf: such rows equal the rows computed with that V finite, and the
    rows that do attend it are non-finite in the heads of its KV head."""
    import warnings
    w = custom_workload(kind="prefill", context_lens=[40], q_lens=[24], num_q_heads=4,
                        num_kv_heads=2, head_dim=8, seed=25)
    P, p = 16, 16 + 9                       # rows 0..8 do not attend position p
    c = _filled_cache(O, w)
    clean = O.ref_prefill_chunk(w.q, c, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    page, off = int(w.block_tables[0, p // PS]), p % PS
    for bad in (np.nan, np.inf):
        c2 = _filled_cache(O, w)
        c2.v[page, 1, 3, off] = bad          # KV head 1 serves query heads 2 and 3
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            out = O.ref_prefill_chunk(w.q, c2, w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
        assert np.max(np.abs(out[:p - P] - clean[:p - P])) <= 1e-13
        assert np.all(~np.isfinite(out[p - P:, 2:, 3]))
        assert np.array_equal(out[p - P:, :2], clean[p - P:, :2])
    # a window of 4: row i attends (P+i-4, P+i], so rows from i = p-P+4 on
    # no longer see p
    c2 = _filled_cache(O, w)
    c2.v[page, 1, 3, off] = np.nan
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ref = O.ref_prefill_chunk(w.q, c, w.block_tables, w.context_lens, w.cu_q_lens, w.scale, window=4)
        out = O.ref_prefill_chunk(w.q, c2, w.block_tables, w.context_lens, w.cu_q_lens, w.scale, window=4)
    seen = [P + i - 4 < p <= P + i for i in range(24)]
    for i in range(24):
        if seen[i]:
            assert np.all(np.isnan(out[i, 2:, 3]))
        else:
            assert np.max(np.abs(out[i] - ref[i])) <= 1e-13, i


# ------------------------------------------------------------------ conversion pins
def _golden_conv():
    with open(os.path.join(GOLDEN, "conversions.json")) as f:
        return json.load(f)


def pin_bf16_golden_and_torch(O):
    for case in _golden_conv()["bf16"]:
        x = np.array([int(case["f32_bits"], 16)], dtype=np.uint32).view(np.float32)
        got = int(O.f32_to_bf16_bits(x)[0])
        assert got == int(case["bf16_bits"], 16), case
    rng = np.random.Generator(np.random.PCG64(30))
    x = np.concatenate([rng.standard_normal(20000, dtype=np.float32),
                        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), ref)
    assert np.array_equal(O.bf16_bits_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def pin_f16_golden_and_torch(O):
    for case in _golden_conv()["f16"]:
        got = int(O.f32_to_f16(np.array([case["value"]], np.float32)).view(np.uint16)[0])
        assert got == int(case["f16_bits"], 16), case
    rng = np.random.Generator(np.random.PCG64(31))
    x = np.concatenate([rng.standard_normal(20000, dtype=np.float32),
                        (rng.standard_normal(20000) * 1e-5).astype(np.float32),
                        (rng.standard_normal(2000) * 7e4).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float16).numpy()
    assert np.array_equal(O.f32_to_f16(x).view(np.uint16), ref.view(np.uint16))


def pin_int8_golden(O):
    for case in _golden_conv()["int8"]:
        codes, sc = O.quantize_int8(np.array([case["x"]], np.float32))
        assert float(sc[0]) == case["scale"], case
        assert codes[0].tolist() == case["codes"], case


def pin_int8_bounds(O):
    rng = np.random.Generator(np.random.PCG64(32))
    x = rng.standard_normal((3000, 64), dtype=np.float32)
    codes, sc = O.quantize_int8(x)
    s = sc.astype(np.float64)[:, None]
    assert np.all(np.abs(x - codes * s) <= s * (0.5 + 1e-5))
    assert np.all(np.abs(codes[np.arange(3000), np.argmax(np.abs(x), axis=1)]) == 127)
    assert np.all(np.abs(codes) <= 127)
    c2, s2 = O.quantize_int8(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, sc)


def pin_append_layout(O):
    w = custom_workload(context_lens=[19, 33], num_q_heads=2, num_kv_heads=2, head_dim=8,
                        num_pages=8, seed=33)
    slots = w.slot_mapping.copy()
    slots[[3, 20]] = -1                  # padding tokens are skipped
    c = O.PagedCache(w.num_pages, 2, 8, "f32")
    O.ref_append(c, w.k, w.v, slots)
    e = O.PagedCache(w.num_pages, 2, 8, "f32")
    for j, s in enumerate(slots):
        if s < 0:
            continue
        for g in range(2):
            for i in range(8):
                e.k[s // PS, g, s % PS, i] = w.k[j, g, i]
                e.v[s // PS, g, i, s % PS] = w.v[j, g, i]
    assert np.array_equal(c.k, e.k) and np.array_equal(c.v, e.v)
    ci = O.PagedCache(w.num_pages, 2, 8, "i8")
    O.ref_append(ci, w.k, w.v, slots)
    for j, s in enumerate(slots):
        if s < 0:
            continue
        kq, ks = O.quantize_int8(w.k[j])
        vq, vs = O.quantize_int8(w.v[j])
        assert np.array_equal(ci.k[s // PS, :, s % PS, :], kq)
        assert np.array_equal(ci.v[s // PS, :, :, s % PS], vq)
        assert np.array_equal(ci.k_scales[s // PS, :, s % PS], ks)
        assert np.array_equal(ci.v_scales[s // PS, :, s % PS], vs)
    for s in w.slot_mapping[[3, 20]]:
        assert np.all(ci.k[s // PS, :, s % PS, :] == 0) and np.all(ci.v_scales[s // PS, :, s % PS] == 0)


# ------------------------------------------------------------------ RoPE
def _unit(d, i):
    x = np.zeros((1, 1, d), dtype=np.float32)
    x[0, 0, i] = 1.0
    return x


def pin_rope_golden_angles(O):
    """Hand-derived angles: with theta = 2^16 and d = 8 the four pairs turn at
    1, 1/16, 1/256, 1/4096 rad per position (exact in fp32), so position 4096
    turns them by 4096, 256, 16 and 1 rad; with theta = 256 and d = 4,
    position 16 turns the two pairs by 16 and 1 rad.  With theta = 10^4 and
    d = 8 the rates are 1, 1/10, 1/100, 1/1000 up to their fp32 rounding
    (relative 2^-24), so position 1000 turns by 1000, 100, 10, 1 rad within
    about 1e-5.  A unit vector on a pair's first coordinate goes to (cos, sin)
    on (first, second); one on the second coordinate to (-sin, cos) -- a
    rotation by +angle, as in the published definition."""
    for d, theta, pos, angles, tol in ((8, 65536.0, 4096, (4096.0, 256.0, 16.0, 1.0), 1e-12),
                                       (4, 256.0, 16, (16.0, 1.0), 1e-12),
                                       (8, 1e4, 1000, (1000.0, 100.0, 10.0, 1.0), 1e-4)):
        for style in ("half", "interleaved"):
            for i, ang in enumerate(angles):
                first, second = (i, i + d // 2) if style == "half" else (2 * i, 2 * i + 1)
                want = np.zeros(d)
                want[first], want[second] = math.cos(ang), math.sin(ang)
                got = O.rope_f64(_unit(d, first), [pos], theta, style)[0, 0]
                assert np.max(np.abs(got - want)) < tol, (d, style, i)
                want = np.zeros(d)
                want[first], want[second] = -math.sin(ang), math.cos(ang)
                got = O.rope_f64(_unit(d, second), [pos], theta, style)[0, 0]
                assert np.max(np.abs(got - want)) < tol, (d, style, i)


def pin_rope_group_laws(O):
    """Position 0 is the identity, rotations compose additively in position,
    position -m undoes m, and every coordinate pair keeps its length."""
    rng = np.random.default_rng(71)
    for d in (8, 64, 128):
        x = rng.standard_normal((5, 3, d)).astype(np.float32)
        m = np.array([0, 1, 17, 4095, 262143])
        n = np.array([3, 0, 1000, 7, 11])
        for style in ("half", "interleaved"):
            assert np.array_equal(O.rope_f64(x, np.zeros(5, dtype=np.int64), 1e4, style),
                                  x.astype(np.float64))
            once = O.rope_f64(x, m + n, 1e4, style)
            twice = O.rope_f64(O.rope_f64(x, m, 1e4, style), n, 1e4, style)
            assert np.max(np.abs(once - twice)) < 1e-9
            back = O.rope_f64(O.rope_f64(x, m, 5e5, style), -m, 5e5, style)
            assert np.max(np.abs(back - x)) < 1e-9
            r = O.rope_f64(x, m, 1e4, style)
            if style == "half":
                pn = lambda y: y[..., : d // 2] ** 2 + y[..., d // 2:] ** 2   # noqa: E731
            else:
                pn = lambda y: y[..., 0::2] ** 2 + y[..., 1::2] ** 2          # noqa: E731
            assert np.max(np.abs(pn(r) - pn(x.astype(np.float64)))) < 1e-9


def pin_rope_relative_position(O):
    """The score between a rotated query and a rotated key depends only on the
    distance between their positions (the property RoPE is built for)."""
    rng = np.random.default_rng(72)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64)).astype(np.float32)
    for style in ("half", "interleaved"):
        ref = float(np.sum(O.rope_f64(q, [40], 1e4, style) * O.rope_f64(k, [13], 1e4, style)))
        for shift in (1, 500, 100000):
            got = float(np.sum(O.rope_f64(q, [40 + shift], 1e4, style) *
                               O.rope_f64(k, [13 + shift], 1e4, style)))
            assert abs(got - ref) < 1e-9


def pin_append_rope(O):
    """Append with RoPE: V lands exactly as a plain append puts it; K of a
    token at position 0 too; K of the golden unit vector lands as the float32
    of (cos, sin) in every storage type."""
    w = custom_workload(context_lens=[40], num_q_heads=2, num_kv_heads=2, head_dim=8, kv_dtype="f32",
                        num_pages=4, seed=74)
    T = w.k.shape[0]
    pos = np.arange(T) * 37
    for dt in ("f32", "bf16", "f16", "i8"):
        plain = O.PagedCache(w.num_pages, 2, 8, dt)
        O.ref_append(plain, w.k, w.v, w.slot_mapping)
        rot = O.PagedCache(w.num_pages, 2, 8, dt)
        O.ref_append_rope(rot, w.k, w.v, w.slot_mapping, pos, 1e4, "half")
        assert np.array_equal(plain.v, rot.v)
        if dt == "i8":
            assert np.array_equal(plain.v_scales, rot.v_scales)
        s0 = int(w.slot_mapping[0])
        assert np.array_equal(plain.k[s0 // PS, :, s0 % PS], rot.k[s0 // PS, :, s0 % PS])
    c = O.PagedCache(1, 1, 8, "f32")      # pair 1 turns at 1/16 rad per position: 100 rad
    O.ref_append_rope(c, _unit(8, 1), np.zeros((1, 1, 8), np.float32), [5], [1600], 65536.0, "half")
    want = np.zeros(8, np.float32)
    want[1], want[5] = np.float32(math.cos(100.0)), np.float32(math.sin(100.0))
    assert np.array_equal(c.k[0, 0, 5], want)
    # queries: position 0 keeps every dtype's values; the golden vector turns
    # like the key, then rounds to the query dtype
    # (values compared through torch's bf16, so -0 and +0 count as equal)
    q = w.k[:3].astype(np.float32)
    bf = lambda y: torch.from_numpy(np.ascontiguousarray(y).view(np.int16)).view(torch.bfloat16).double().numpy()  # noqa: E731
    for dt, conv, val in (("f32", lambda y: y, lambda y: y), ("f16", lambda y: y.astype(np.float16), lambda y: y),
                          ("bf16", lambda y: torch.from_numpy(y).to(torch.bfloat16).double().numpy(), bf)):
        assert np.array_equal(val(O.ref_rope_q(q, [0, 0, 0], 1e4, "interleaved", dt)), conv(q))
        got = val(O.ref_rope_q(_unit(8, 1), [1600], 65536.0, "half", dt))
        assert np.array_equal(got[0, 0], conv(want))


# ------------------------------------------------------------------ sliding window
def pin_window_bruteforce(O):
    """Sliding window of W tokens: the query at position p attends exactly
    the positions (p - W, p], checked with math.fsum brute force for decode
    and for every chunk row (rows near the chunk start see keys of the
    prefix, rows further on only keys of the chunk)."""
    w = custom_workload(kind="prefill", context_lens=[40, 21, 18, 3], q_lens=[9, 21, 1, 3],
                        num_q_heads=2, num_kv_heads=1, head_dim=4, num_pages=12, seed=81)
    ks = [_seq(w, w.k, b) for b in range(w.batch)]
    vs = [_seq(w, w.v, b) for b in range(w.batch)]
    cache = write_paged_f32(O, ks, vs, w.block_tables, w.num_pages, 1, 4)
    for W in (1, 5, 16, 17):
        out = O.ref_prefill_chunk(w.q, cache, w.block_tables, w.context_lens, w.cu_q_lens, w.scale,
                                  window=W)
        for b in range(w.batch):
            n, C = int(w.context_lens[b]), int(w.q_lens[b])
            P = n - C
            for i in range(C):
                p = P + i
                lo = max(0, p - W + 1)
                row = int(w.cu_q_lens[b]) + i
                for h in range(2):
                    ref = brute_attention_row(w.q[row, h], ks[b][lo:p + 1], vs[b][lo:p + 1], 0, w.scale)
                    assert np.max(np.abs(out[row, h] - ref)) <= 1e-12, (W, b, i, h)
        qd = np.stack([w.q[int(w.cu_q_lens[b + 1]) - 1] for b in range(w.batch)])
        dec = O.ref_decode(qd, cache, w.block_tables, w.context_lens, w.scale, 2, window=W)
        for b in range(w.batch):
            n = int(w.context_lens[b])
            lo = max(0, n - W)
            for h in range(2):
                ref = brute_attention_row(qd[b, h], ks[b][lo:n], vs[b][lo:n], 0, w.scale)
                assert np.max(np.abs(dec[b, h] - ref)) <= 1e-12, (W, b, h)


def pin_window_special_cases(O):
    """A window covering the whole context is full attention (bit for bit);
    a window of one token returns the query's own V; block-table entries of
    pages wholly before the window are never read (they hold ids far outside
    the pool here)."""
    w = custom_workload(kind="prefill", context_lens=[70, 33, 16], q_lens=[20, 33, 1],
                        num_q_heads=4, num_kv_heads=2, head_dim=8, kv_dtype="bf16",
                        num_pages=20, seed=82)
    c = _filled_cache(O, w)
    args = (w.block_tables, w.context_lens, w.cu_q_lens, w.scale)
    full = O.ref_prefill_chunk(w.q, c, *args)
    assert np.array_equal(O.ref_prefill_chunk(w.q, c, *args, window=70), full)
    qd = np.stack([w.q[int(w.cu_q_lens[b + 1]) - 1] for b in range(w.batch)])
    dfull = O.ref_decode(qd, c, w.block_tables, w.context_lens, w.scale, 4)
    assert np.array_equal(O.ref_decode(qd, c, w.block_tables, w.context_lens, w.scale, 4, window=10**6), dfull)
    one = O.ref_prefill_chunk(w.q, c, *args, window=1)
    for b in range(w.batch):
        n, C = int(w.context_lens[b]), int(w.q_lens[b])
        for i in range(C):
            p = n - C + i
            page, off = int(w.block_tables[b][p // PS]), p % PS
            v = O.bf16_bits_to_f64(c.v[page, :, :, off])            # [Hkv, d]
            row = int(w.cu_q_lens[b]) + i
            for h in range(4):
                assert np.max(np.abs(one[row, h] - v[h // 2])) <= 1e-15
    # evicted pages: ids outside the pool before the window's first page
    bt = w.block_tables.copy()
    W = 20
    for b in range(w.batch):
        n, C = int(w.context_lens[b]), int(w.q_lens[b])
        first_page = max(0, n - C - W + 1) // PS
        bt[b, :first_page] = 10**7
    got = O.ref_prefill_chunk(w.q, c, bt, w.context_lens, w.cu_q_lens, w.scale, window=W)
    assert np.array_equal(got, O.ref_prefill_chunk(w.q, c, *args, window=W))
    for b in range(w.batch):
        bt[b, :max(0, int(w.context_lens[b]) - W) // PS] = 10**7
    got = O.ref_decode(qd, c, bt, w.context_lens, w.scale, 4, window=W)
    assert np.array_equal(got, O.ref_decode(qd, c, w.block_tables, w.context_lens, w.scale, 4, window=W))


# ------------------------------------------------------------------ fp8 (E4M3)
def _e4m3_torch(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def pin_fp8_encoding_matches_torch(O):
    """E4M3 rounding against torch's float8_e4m3fn cast: every bf16 value in
    [-448, 448], log-uniform fp32 draws, and the exact midpoints between
    neighbouring E4M3 values (ties go to the even code)."""
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    v = b.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    rng = np.random.default_rng(91)
    r = (rng.standard_normal(100000) * np.exp(rng.uniform(-14, 6.1, 100000))).astype(np.float32)
    r = np.clip(r, -448, 448)
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # exact in fp32
    for arr in (v, r, mids, -mids):
        assert np.array_equal(O.f32_to_e4m3_bits(arr), _e4m3_torch(arr))


def pin_fp8_decoding_matches_torch(O):
    codes = np.arange(256, dtype=np.uint8)
    finite = (codes & 0x7F) != 0x7F
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_bits_to_f64(codes)
    assert np.array_equal(got[finite], ref[finite]) and np.all(np.isnan(got[~finite]))


def pin_fp8_golden(O):
    """Hand-derived: absmax 448 gives scale 1; 448 -> 0x7E (exponent field
    15, mantissa 6), -1 -> 0xB8, 0.5 -> 0x30, 1e-3 -> 0x01 (subnormal
    1e-3 * 2^9 = 0.512 rounds to 1), 0 -> 0x00, -0 -> 0x80, 3 -> 0x44,
    17 -> 0x58 (17/2 = 8.5 ties to the even 8: 16 = 2^4)."""
    x = np.array([[448, -1, 0.5, 1e-3, 0, -0.0, 3.0, 17.0]], np.float32)
    codes, sc = O.quantize_fp8(x)
    assert sc[0] == np.float32(1.0)
    assert codes[0].tolist() == [0x7E, 0xB8, 0x30, 0x01, 0x00, 0x80, 0x44, 0x58]
    z, zs = O.quantize_fp8(np.zeros((2, 8), np.float32))
    assert np.all(z == 0) and np.all(zs == 0)


def pin_fp8_bounds(O):
    """Per element the stored value is within half a grid step of x: 2^-4
    relative for ratios of 2^-6 and up, scale * 2^-10 below; the absmax
    element stores +-448 * scale; codes are sign-symmetric."""
    rng = np.random.default_rng(92)
    x = (rng.standard_normal((300, 64)) * np.exp(rng.uniform(-20, 20, (300, 1)))).astype(np.float32)
    codes, sc = O.quantize_fp8(x)
    got = O.e4m3_bits_to_f64(codes) * sc.astype(np.float64)[:, None]
    xd = x.astype(np.float64)
    s = sc.astype(np.float64)[:, None]
    bound = np.maximum(np.abs(xd) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(got - xd) <= bound)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(O.e4m3_bits_to_f64(codes[np.arange(300), am])) == 448.0)
    c2, s2 = O.quantize_fp8(-x)
    assert np.array_equal(s2, sc) and np.array_equal(c2 ^ 0x80, codes)


def pin_comparator(O):
    """max_abs_err, the measure every parity test asserts through, against
    values fixed by hand: a difference of either sign counts by its
    magnitude, one large element is not averaged away among equal ones, both
    sides are widened to fp64 before the difference (fp32 0.1 differs from
    fp64 0.1 by 2^-27 * 0.2 exactly), a NaN or an infinity on either side
    gives +inf, and arrays of different shapes are refused rather than
    broadcast."""
    r = np.linspace(-1.0, 1.0, 1000).reshape(10, 100)
    assert O.max_abs_err(r.copy(), r) == 0.0
    g = r.copy()
    g[3, 7] -= 0.5                       # gpu below the reference
    assert O.max_abs_err(g, r) == 0.5
    g = r.copy()
    g[9, 99] += 0.25                     # one element among 1000
    assert O.max_abs_err(g, r) == 0.25
    g = r.copy()
    g[0, 0] += 0.125
    g[5, 5] -= 0.375
    assert O.max_abs_err(g, r) == 0.375  # the largest magnitude, not the largest signed value
    x32 = np.float32(0.1)
    exact = abs(float(x32) - 0.1)
    assert exact > 0 and O.max_abs_err(np.array([x32]), np.array([0.1])) == exact
    for bad in (np.nan, np.inf, -np.inf):
        g = r.copy()
        g[2, 2] = bad
        assert O.max_abs_err(g, r) == float("inf")
        rr = r.copy()
        rr[4, 4] = bad
        assert O.max_abs_err(r.copy(), rr) == float("inf")
    assert O.max_abs_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    for shape in ((100,), (1, 10, 100), (10, 1), (100, 10)):
        try:
            O.max_abs_err(np.zeros(shape), r)
        except ValueError:
            continue
        raise AssertionError(f"shape {shape} against {r.shape} was compared")


def pin_quantizers_non_finite(O):
    """A NaN anywhere in a vector makes its int8/FP8 scale NaN and its codes
    0; an infinity makes the scale +inf; other rows of the same call are
    untouched (the library's stated handling of non-finite inputs)."""
    import warnings
    rng = np.random.default_rng(93)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    x[1, 9] = np.nan
    x[2, 0] = -np.inf
    clean = np.delete(x, [1, 2], axis=0)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for quant in (O.quantize_int8, O.quantize_fp8):
            codes, sc = quant(x)
            assert np.isnan(sc[1]) and np.all(codes[1].view(np.uint8) == 0)
            assert sc[2] == np.inf
            c0, s0 = quant(clean)
            assert np.array_equal(s0, sc[[0, 3]]) and np.array_equal(c0, codes[[0, 3]])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
