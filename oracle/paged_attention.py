"""CPU oracle for attention over a paged KV cache (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke entry point and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

What it computes, and where that is defined
-------------------------------------------
* Attention is ``softmax(q K^T * scale) V`` evaluated exactly (up to fp64
  rounding) on the values stored in the cache.  The pages name the operation
  and its pieces: paged attention over 16-token pages (TinyLoop "Current
  Status", table "KV cache modes", row "Paged attention"), cached decode
  (same page, table "Core inference", row "Generation"), GQA with fewer KV
  heads than query heads (same page, table "Model architecture support", row
  "GQA"), chunked prefill (same table, row "Chunked prefill"; Tiny-LLM
  "Project Status", the supported-features list and the release paragraph
  naming the chunked-prefill SDPA path).
* KV storage dtypes fp32 / bf16 / fp16 / int8: Tiny-LLM "Project Status"
  (dtype-contract paragraph: separate compute and KV-cache dtypes, a BF16 KV
  cache with its own paged kernel), mini-llm README (hardware table: FP16 KV
  cache), TinyLoop "Current Status" (table "KV cache modes", row "INT8 KV
  cache").

Readings taken where the pages are silent (each is also listed in the design
notes):
* Layout: K pages are ``[num_pages, Hkv, 16, d]``; V pages are stored with
  the token index innermost, ``[num_pages, Hkv, d, 16]``; int8 scales are
  ``[num_pages, Hkv, 16]`` float32 for K and for V.
* GQA map: query head ``h`` reads KV head ``h // (Hq // Hkv)``.
* Decode: ``context_lens[b]`` counts the query token itself (its K/V are in
  the cache already); the query attends to positions ``[0, ctx_b)``.
  ``ctx_b == 0`` yields zeros.
* Prefill: the chunk's K/V are in the cache; ``context_lens[b] = P_b + C_b``
  where ``C_b`` is the chunk length from ``cu_q_lens``; chunk row ``i`` sits at
  absolute position ``P_b + i`` and attends to ``[0, P_b + i]`` (causal,
  aligned at the bottom right).
* int8: symmetric absmax per (token, KV head): ``scale = absmax / 127`` in
  IEEE fp32, ``code = clip(rint(x / scale), -127, 127)`` with ties to even;
  an all-zero vector gets scale 0 and codes 0.  The pages say only "INT8 KV",
  so this convention is parity unpinned beyond its own definition; the
  pinned properties are the rounding bound, the +-127 code at the absmax and
  sign symmetry.
* bf16 from fp32: round to nearest even on the bit pattern; NaN stays NaN.
* fp8: OCP FP8 E4M3 codes (1 sign, 4 exponent bits of bias 7, 3 mantissa
  bits; largest finite 448; no infinities; S.1111.111 is NaN), the "FP8 KV
  cache" the stylome.io "Classifier receipt" names beside INT8.  Symmetric
  absmax per (token, KV head) like int8: ``scale = absmax / 448`` in IEEE
  fp32, ``code = e4m3(x / scale)`` rounded to the nearest e4m3 value (ties
  to even) after clamping to +-448; the sign bit is the sign of the fp32
  ratio (so -0.0 and a negative value that rounds to zero store 0x80); an
  all-zero vector gets scale 0 and codes 0.
"""
from __future__ import annotations

import numpy as np

PAGE_SIZE = 16
DTYPES = ("f32", "bf16", "f16", "i8", "fp8")
E4M3_MAX = 448.0


# ---------------------------------------------------------------- conversions
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the
    16-bit patterns as uint16."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    rounded = np.where(nan, (u >> 16) | 0x0040, rounded)
    return (rounded & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 -> fp32 is a 16-bit shift)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_f16(x) -> np.ndarray:
    """fp32 -> fp16, nearest-even with subnormals (numpy's IEEE cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def quantize_int8(x):
    """Symmetric absmax int8 over the last axis, all arithmetic in fp32.

    Returns (codes int8 [..., d], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(ratio), -127, 127)
    codes = np.where((scale > 0)[..., None], codes, 0).astype(np.int8)
    return codes, scale


def f32_to_e4m3_bits(x) -> np.ndarray:
    """Finite float32 values with |x| <= 448 -> OCP E4M3 codes (uint8), to
    the nearest representable value with ties to even.  Normal values
    2^e (1 + m/8) have e in [-6, 8]; below 2^-6 the grid is m * 2^-9."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    _, ex = np.frexp(a)                                  # a = frac * 2^ex, frac in [0.5, 1)
    e = np.maximum(ex - 1, -6)                           # exponent of a's binade, floored at -6
    step = np.ldexp(1.0, e - 3)                          # grid spacing in that binade
    q = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    _, qx = np.frexp(q)
    qe = qx - 1
    normal = q >= 2.0 ** -6
    mant_normal = np.where(normal, q / np.ldexp(1.0, np.where(normal, qe, 0)) * 8 - 8, 0)
    bits = np.where(normal, ((qe + 7) << 3) + mant_normal, q / 2.0 ** -9)
    bits = bits.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)
    return bits.astype(np.uint8)


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """OCP E4M3 codes -> float64 (exact); 0x7F / 0xFF are NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def quantize_fp8(x):
    """Symmetric absmax FP8 (E4M3) over the last axis: scale in fp32, the
    ratio x / scale in fp32, clamped to +-448, then rounded to E4M3.

    Returns (codes uint8 [..., d], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)
    ratio = np.clip(ratio, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = f32_to_e4m3_bits(ratio)
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def storage_from_f32(x, dtype: str):
    """Convert float32 values to the cache's storage representation.

    f32 -> float32, bf16 -> uint16 bit patterns, f16 -> float16,
    i8 -> (int8 codes, float32 scales over the last axis)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).copy()
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16(x)
    if dtype == "i8":
        return quantize_int8(x)
    if dtype == "fp8":
        return quantize_fp8(x)
    raise ValueError(dtype)


def upcast(stored, dtype: str, scales=None) -> np.ndarray:
    """Stored cache values -> float64, exactly."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(stored)
    if dtype == "f16":
        return np.asarray(stored, dtype=np.float16).astype(np.float64)
    if dtype == "i8":
        return np.asarray(stored, dtype=np.int8).astype(np.float64) * \
            np.asarray(scales, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_bits_to_f64(stored) * np.asarray(scales, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- cache
_STORE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16, "i8": np.int8, "fp8": np.uint8}
SCALED = ("i8", "fp8")   # dtypes with per-(token, head) fp32 scales


class PagedCache:
    """Host copy of a paged KV pool in its storage representation."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, dtype: str):
        if dtype not in DTYPES:
            raise ValueError(dtype)
        self.num_pages, self.num_kv_heads, self.head_dim, self.dtype = \
            num_pages, num_kv_heads, head_dim, dtype
        st = _STORE[dtype]
        self.k = np.zeros((num_pages, num_kv_heads, PAGE_SIZE, head_dim), dtype=st)
        self.v = np.zeros((num_pages, num_kv_heads, head_dim, PAGE_SIZE), dtype=st)
        if dtype in SCALED:
            self.k_scales = np.zeros((num_pages, num_kv_heads, PAGE_SIZE), np.float32)
            self.v_scales = np.zeros((num_pages, num_kv_heads, PAGE_SIZE), np.float32)
        else:
            self.k_scales = self.v_scales = None

    def copy(self) -> "PagedCache":
        c = PagedCache.__new__(PagedCache)
        c.num_pages, c.num_kv_heads, c.head_dim, c.dtype = \
            self.num_pages, self.num_kv_heads, self.head_dim, self.dtype
        c.k, c.v = self.k.copy(), self.v.copy()
        c.k_scales = None if self.k_scales is None else self.k_scales.copy()
        c.v_scales = None if self.v_scales is None else self.v_scales.copy()
        return c


def ref_append(cache: PagedCache, k_new, v_new, slot_mapping) -> None:
    """Write new tokens into the pool through the slot mapping (in place).

    ``k_new``/``v_new`` are [T, Hkv, d] float32 (the exact values of whatever
    dtype the caller holds them in).  Token ``j`` with ``slot >= 0`` goes to
    page ``slot // 16``, offset ``slot % 16``; negative slots are skipped."""
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots, k_new, v_new = slots[keep], k_new[keep], v_new[keep]
    page, off = slots // PAGE_SIZE, slots % PAGE_SIZE
    if cache.dtype in SCALED:
        kq, ks = storage_from_f32(k_new, cache.dtype)
        vq, vs = storage_from_f32(v_new, cache.dtype)
        cache.k[page, :, off, :] = kq
        cache.v[page, :, :, off] = vq
        cache.k_scales[page, :, off] = ks
        cache.v_scales[page, :, off] = vs
    else:
        cache.k[page, :, off, :] = storage_from_f32(k_new, cache.dtype)
        cache.v[page, :, :, off] = storage_from_f32(v_new, cache.dtype)


def rope_f64(x, positions, theta, style: str = "half") -> np.ndarray:
    """Rotary position embedding, float64 and unrounded.

    RoPE with a configurable base theta runs in every forward path (TinyLoop
    "Current Status", table "Model architecture support", row "RoPE"); the
    runtimes serve LLaMA/SmolLM2-compatible and Qwen2-family checkpoints
    (Tiny-LLM "Project Status", supported models).  The rotation follows its
    published definition (RoFormer, Su et al. 2021): the d/2 coordinate pairs of a head vector are
    rotated in their planes, pair i by the angle ``pos * theta**(-2 i / d)``,
    ``(a, b) -> (a cos - b sin, b cos + a sin)``.  style "half" pairs
    coordinate i with i + d/2 (the pairing of the Llama and Qwen reference
    implementations); "interleaved" pairs 2i with 2i + 1.

    x [T, H, d]; positions [T] integers; theta the base (taken at the fp32
    value the library receives).  The pair frequencies theta^(-2i/d) are held
    as fp32 numbers (the power evaluated in float64, rounded once), the usual
    storage of a RoPE frequency table; the angle, its cosine and sine and the
    rotation are float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    i = np.arange(h, dtype=np.float64)
    inv_freq = (np.float64(np.float32(theta)) ** (-2.0 * i / d)).astype(np.float32).astype(np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    if style == "half":
        a, b = x[..., :h], x[..., h:]
    elif style == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        raise ValueError(style)
    ra = a * c - b * s
    rb = b * c + a * s
    out = np.empty_like(x)
    if style == "half":
        out[..., :h], out[..., h:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out


def ref_append_rope(cache: PagedCache, k_new, v_new, slot_mapping, positions, theta,
                    style: str = "half") -> None:
    """Append with RoPE applied to K first: the rotation is evaluated in
    float64 and rounded to float32, then K and V are stored as ref_append
    stores them (V is not rotated)."""
    k_rot = rope_f64(np.asarray(k_new, dtype=np.float32), positions, theta, style)
    ref_append(cache, k_rot.astype(np.float32), v_new, slot_mapping)


def ref_rope_q(q, positions, theta, style: str, dtype: str) -> np.ndarray:
    """Queries rotated as the fused append rotates them: each query row of
    token j turns by its position, the float64 result is rounded to float32
    and then to the query's own dtype (storage representation of
    storage_from_f32)."""
    rot = rope_f64(np.asarray(q, dtype=np.float32), positions, theta, style)
    return storage_from_f32(rot.astype(np.float32), dtype)


def gather_sequence(cache: PagedCache, block_row, n: int, start: int = 0):
    """Contiguous float64 K, V [n - start, Hkv, d] of the tokens at positions
    [start, n) of one sequence (block-table entries of earlier pages are not
    read)."""
    t = np.arange(start, n)
    page = np.asarray(block_row, dtype=np.int64)[t // PAGE_SIZE]
    off = t % PAGE_SIZE
    ks = None if cache.k_scales is None else cache.k_scales[page, :, off][..., None]
    vs = None if cache.v_scales is None else cache.v_scales[page, :, off][..., None]
    K = upcast(cache.k[page, :, off, :], cache.dtype, ks)
    V = upcast(cache.v[page, :, :, off], cache.dtype, vs)
    return K, V


# ---------------------------------------------------------------- attention
def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def ref_decode(q, cache: PagedCache, block_tables, context_lens, scale,
               num_q_heads: int, window: int = 0) -> np.ndarray:
    """Batched decode: out[b, h] = softmax(scale * K_b q_bh) V_b over the
    positions [lo_b, ctx_b): lo_b = 0, or with a sliding window of `window`
    tokens (TinyLoop "Current Status", table "KV cache modes", row
    "Sliding-window cache") lo_b = max(0, ctx_b - window), so the query at
    position ctx_b - 1 sees its `window` most recent positions, itself
    included.

    q: [B, Hq, d] (any float dtype, widened exactly).  Returns float64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    G = Hq // cache.num_kv_heads
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        lo = max(0, n - window) if window > 0 else 0
        K, V = gather_sequence(cache, block_tables[b], n, lo)
        for h in range(Hq):
            g = h // G
            s = sc * (K[:, g, :] @ q[b, h])
            w = _softmax_rows(s)
            out[b, h] = w @ V[:, g, :]
    return out


def ref_prefill_chunk(q, cache: PagedCache, block_tables, context_lens, cu_q_lens,
                      scale, window: int = 0) -> np.ndarray:
    """Chunked causal prefill.  q: [T, Hq, d]; sequence b's chunk is rows
    cu_q_lens[b]:cu_q_lens[b+1]; row i of it attends to [0, P_b + i] with
    P_b = context_lens[b] - C_b, or with a sliding window of `window` tokens
    to (P_b + i - window, P_b + i].  Positions a row does not attend take no
    part in its sum, also when their V holds NaN or inf.  Returns float64
    [T, Hq, d]."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    G = Hq // cache.num_kv_heads
    sc = float(np.float32(scale))
    out = np.zeros((T, Hq, d), dtype=np.float64)
    for b in range(len(context_lens)):
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        C, n = r1 - r0, int(context_lens[b])
        if C == 0:
            continue
        P = n - C
        if P < 0:
            raise ValueError("context shorter than its query chunk")
        lo = max(0, P - window + 1) if window > 0 else 0
        K, V = gather_sequence(cache, block_tables[b], n, lo)
        keypos = np.arange(lo, n)[None, :]
        rowpos = P + np.arange(C)[:, None]
        seen = keypos <= rowpos
        if window > 0:
            seen = seen & (keypos > rowpos - window)
        for h in range(Hq):
            g = h // G
            s = np.where(seen, sc * (q[r0:r1, h, :] @ K[:, g, :].T), -np.inf)
            w = _softmax_rows(s)
            Vg = V[:, g, :]
            if np.all(np.isfinite(Vg)):
                out[r0:r1, h] = w @ Vg
            else:
                # a zero weight times a non-finite value would be NaN: sum
                # each row over the positions it attends only
                for i in range(C):
                    out[r0 + i, h] = w[i, seen[i]] @ Vg[seen[i]]
    return out


# ---------------------------------------------------------------- comparison
def max_abs_err(gpu_out, ref) -> float:
    """The parity measure: max |gpu - ref| over every element, each side
    widened to fp64 before the difference.  The two arrays must have the
    same shape (no broadcasting: a missing axis is an error, not a smaller
    comparison).  A NaN or an infinity on either side gives +inf, so such an
    output fails every tolerance.  Empty arrays give 0."""
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"compared arrays differ in shape: {g.shape} vs {r.shape}")
    if g.size == 0:
        return 0.0
    if not (np.all(np.isfinite(g)) and np.all(np.isfinite(r))):
        return float("inf")
    return float(np.max(np.abs(g - r)))
