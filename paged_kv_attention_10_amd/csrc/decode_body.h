// Device code of the paged decode partition (shared by the decode entry
// point and the mixed prefill/decode kernel).  The algorithm is described
// in decode.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;   // null, or a mixed batch's chunk offsets (decode rows: chunks of one)
  void* out;
  float* part_o;
  float* part_lse;
  // In-kernel merge (null: the partials go to decode_reduce_kernel): one
  // arrival counter per (sequence, KV head x head tile), tagged with the
  // call's epoch (distinct per call) in its upper 56 bits, so that whatever
  // a counter held before (an earlier call's count, or anything at all in a
  // fresh workspace) reads as no arrivals yet.
  unsigned long long* merge_cnt = nullptr;
  unsigned long long epoch = 0;
  int q_dtype, out_dtype;
  int max_blocks, max_context_len;
  int batch, hq, hkv, group, head_tiles, num_pages;
  int tiles_per_split, nsplits;
  int window;                 // sliding window in tokens, 0 = the whole context
  float scale_log2;
  // Fused decode step (null k_new: none): each sequence's new K/V row
  // [batch][hkv][D] in new_dtype is stored at position ctx - 1 (through the
  // block table) and attended from registers; k_store/v_store (and for
  // int8 / FP8 ks_store/vs_store) are the writable cache pointers.
  const void* k_new;
  const void* v_new;
  int new_dtype;
  void* k_store;
  void* v_store;
  float* ks_store;
  float* vs_store;
};

// First position a query at position ctx - 1 attends: ctx - window with a
// sliding window, else 0.
__device__ __forceinline__ int window_start(int ctx, int window) {
  return window > 0 ? max(0, ctx - window) : 0;
}

constexpr float kDecodeLazyRescale = 8.0f;

// Context length as the kernels use it; flags lengths the block table
// cannot hold.
__device__ __forceinline__ int checked_ctx(int raw, int max_ctx, int max_blocks, bool& bad) {
  int lim = min(max_ctx, max_blocks * kPage);
  if (raw < 0) { bad = true; return 0; }
  if (raw > lim) { bad = true; return lim; }
  return raw;
}

template <int D, int KV>
struct DecodeTile {
  // K fragments: 16-byte loads per MFMA row-half u.
  static constexpr int KL = (KV == PKV_F32) ? D / 16 : (kv_code8(KV) ? D / 64 : D / 32);
  u32x4 k[2][KL];
  // V^T fragments, one per 16-row block of d.
  u32x4 v[kv_code8(KV) ? 1 : D / 16][(KV == PKV_F32) ? 2 : 1];
  u32x2 v8[kv_code8(KV) ? D / 16 : 1];
  f32x4 ks[2], vs[2];
};

// Register ring depth: tiles in flight per wave, sized so the ring, the
// query fragments and the accumulators stay within the VGPR budget.
template <int D, int KV>
constexpr int ring_depth() {
  return (KV == PKV_F32 && D == 128) ? 1 : 2;
}

template <int D, int KV>
__device__ __forceinline__ void load_tile(DecodeTile<D, KV>& t, const DecodeArgs& a, int g,
                                          int pa, int pb, int lane) {
  const int r = lane & 15, kg = lane >> 4;
  const int page_k = (r < 8) ? pa : pb;
  const int rows_tok = 8 * ((r >> 2) & 1) + (r & 3);  // + 4*u
  constexpr int ES = (KV == PKV_F32) ? 4 : (kv_code8(KV) ? 1 : 2);
  const char* kbase = static_cast<const char*>(a.k_cache) +
                      ((long)page_k * a.hkv + g) * (long)(kPage * D) * ES;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const char* row = kbase + (long)(rows_tok + 4 * u) * D * ES;
#pragma unroll
    for (int s = 0; s < DecodeTile<D, KV>::KL; ++s) {
      int d0;
      if constexpr (KV == PKV_F32) d0 = 16 * s + 4 * kg;
      else if constexpr (kv_code8(KV)) d0 = 64 * s + 16 * kg;
      else d0 = 32 * s + 8 * kg;
      t.k[u][s] = *reinterpret_cast<const u32x4*>(row + (long)d0 * ES);
    }
  }
  const int page_v = (kg < 2) ? pa : pb;
  const char* vbase = static_cast<const char*>(a.v_cache) +
                      ((long)page_v * a.hkv + g) * (long)(D * kPage) * ES;
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk) {
    const char* p = vbase + ((long)(16 * blk + r) * kPage + 8 * (kg & 1)) * ES;
    if constexpr (kv_code8(KV)) {
      t.v8[blk] = *reinterpret_cast<const u32x2*>(p);
    } else if constexpr (KV == PKV_F32) {
      t.v[blk][0] = *reinterpret_cast<const u32x4*>(p);
      t.v[blk][1] = *reinterpret_cast<const u32x4*>(p + 16);
    } else {
      t.v[blk][0] = *reinterpret_cast<const u32x4*>(p);
    }
  }
  if constexpr (kv_code8(KV)) {
    // scales of the 8 tokens 8*kg..8*kg+7 this lane holds scores for
    const long sidx = ((long)page_v * a.hkv + g) * kPage + 8 * (kg & 1);
    t.ks[0] = *reinterpret_cast<const f32x4*>(a.k_scales + sidx);
    t.ks[1] = *reinterpret_cast<const f32x4*>(a.k_scales + sidx + 4);
    t.vs[0] = *reinterpret_cast<const f32x4*>(a.v_scales + sidx);
    t.vs[1] = *reinterpret_cast<const f32x4*>(a.v_scales + sidx + 4);
  }
}

// Fused decode step.  The new token's K row and V column, converted to the
// cache's storage format, are stashed per wave in LDS (the merge area,
// unused while tiles stream: 2 * D * ES bytes per wave, K as 16-byte
// chunks (s, k-group), V by d) and patched into the tile holding position
// ctx - 1 when it comes up.  In load_tile's lane layout, K row `tau` of the
// tile is MFMA row half u of the lanes with tile_row_of_lane(r) + 4u == tau
// (all four k-groups), and V column `tau` is element tau % 8 of the lanes of
// k-group tau / 8, d = 16 * blk + r.
__device__ __forceinline__ int tile_row_of_lane(int r) {
  return (r < 8 ? 0 : 16) + 8 * ((r >> 2) & 1) + (r & 3);
}

// The new token's values this lane converts: for 16- and 32-bit caches K
// chunk `lane` (16 bytes of storage, 16/ES elements) for lanes below
// D*ES/16, for one-byte caches K elements d = lane + 64h; V elements
// d = lane + 64h.  Loaded as fp32 (exact for every input dtype; an fp32
// value's bits are kept).
template <int D>
struct NewRaw {
  float k[8];
  float v[D / 64];
};

// Bytes of the per-wave stash of the new token: K and V as stored plus,
// for one-byte caches, the two scales.
template <int D>
constexpr int kStashBytes = 2 * D * 4;

template <int D, int KV>
__device__ __forceinline__ void load_new_token(NewRaw<D>& nr, const DecodeArgs& a, int b, int g,
                                               int lane) {
  const long nrow = ((long)b * a.hkv + g) * D;
  if constexpr (kv_code8(KV)) {
    with_io_dtype(a.new_dtype, [&](auto ndt) {
      constexpr int NT = decltype(ndt)::value;
      uint32_t kb[D / 64], vb[D / 64];
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        kb[h] = io_bits<NT>(a.k_new, nrow + lane + 64 * h);
        vb[h] = io_bits<NT>(a.v_new, nrow + lane + 64 * h);
      }
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        nr.k[h] = io_value<NT>(kb[h]);
        nr.v[h] = io_value<NT>(vb[h]);
      }
    });
    return;
  }
  constexpr int ES = (KV == PKV_F32) ? 4 : 2;
  constexpr int KE = 16 / ES;                       // K elements per chunk
  const int kc = lane < D * ES / 16 ? lane : 0;     // lanes past the chunks reload chunk 0
  with_io_dtype(a.new_dtype, [&](auto ndt) {
    constexpr int NT = decltype(ndt)::value;
    uint32_t kb[KE], vb[D / 64];
    io_bits_vec<KE, NT>(a.k_new, nrow + kc * KE, kb);
#pragma unroll
    for (int h = 0; h < D / 64; ++h) vb[h] = io_bits<NT>(a.v_new, nrow + lane + 64 * h);
#pragma unroll
    for (int e = 0; e < KE; ++e) nr.k[e] = io_value<NT>(kb[e]);
#pragma unroll
    for (int h = 0; h < D / 64; ++h) nr.v[h] = io_value<NT>(vb[h]);
  });
}

// One-byte caches: quantises the new K and V vectors as the append does
// (code8_scale / code8 on the wave's absmax), writes the codes (K at stash
// byte d, V at D + d) and the two scales (bytes 2D and 2D + 4) to the
// stash and, with `store`, the codes and scales to the cache slot.
template <int D, int KV>
__device__ __forceinline__ void stash_new_token8(char* stash, const NewRaw<D>& nr,
                                                 const DecodeArgs& a, int g, long page, int off,
                                                 bool store, int lane) {
  constexpr bool kI8 = (KV == PKV_I8);
  uint32_t kam = 0u, vam = 0u;
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    kam = max(kam, abs_key(nr.k[h]));
    vam = max(vam, abs_key(nr.v[h]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kam = max(kam, (uint32_t)__shfl_xor((int)kam, m));
    vam = max(vam, (uint32_t)__shfl_xor((int)vam, m));
  }
  const float ksc = code8_scale(__uint_as_float(kam), kI8);
  const float vsc = code8_scale(__uint_as_float(vam), kI8);
  const long head = page * a.hkv + g;
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    const int d = lane + 64 * h;
    const uint8_t kc = (uint8_t)code8(nr.k[h], ksc, kI8);
    const uint8_t vc = (uint8_t)code8(nr.v[h], vsc, kI8);
    reinterpret_cast<uint8_t*>(stash)[d] = kc;
    reinterpret_cast<uint8_t*>(stash)[D + d] = vc;
    if (store) {
      static_cast<uint8_t*>(a.k_store)[(head * kPage + off) * D + d] = kc;
      static_cast<uint8_t*>(a.v_store)[(head * D + d) * kPage + off] = vc;
    }
  }
  if (lane == 0) {
    reinterpret_cast<float*>(stash + 2 * D)[0] = ksc;
    reinterpret_cast<float*>(stash + 2 * D)[1] = vsc;
    if (store) {
      a.ks_store[head * kPage + off] = ksc;
      a.vs_store[head * kPage + off] = vsc;
    }
  }
}

// Converts the loaded new token into the wave's stash and, with `store`,
// writes it to the cache slot (page, off), rounding as the append rounds.
template <int D, int KV>
__device__ __forceinline__ void stash_new_token(char* stash, const NewRaw<D>& nr,
                                                const DecodeArgs& a, int g, long page, int off,
                                                bool store, int lane) {
  if constexpr (kv_code8(KV)) {
    stash_new_token8<D, KV>(stash, nr, a, g, page, off, store, lane);
    return;
  }
  constexpr int ES = (KV == PKV_F32) ? 4 : 2;
  auto conv = [](float x) -> uint32_t {
    if constexpr (KV == PKV_F32) return __float_as_uint(x);
    else if constexpr (KV == PKV_BF16) return f32_to_bf16_bits(x);
    else return f32_to_f16_bits(x);
  };
  if (lane < D * ES / 16) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ES == 4) w[e] = conv(nr.k[e]);
      else w[e] = conv(nr.k[2 * e]) | (conv(nr.k[2 * e + 1]) << 16);
    }
    *reinterpret_cast<u32x4*>(stash + 16 * lane) = w;
    if (store) {
      char* krow = static_cast<char*>(a.k_store) + ((page * a.hkv + g) * kPage + off) * (long)D * ES;
      *reinterpret_cast<u32x4*>(krow + 16 * lane) = w;
    }
  }
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    const int d = lane + 64 * h;
    const uint32_t bits = conv(nr.v[h]);
    if constexpr (ES == 4) reinterpret_cast<uint32_t*>(stash + D * ES)[d] = bits;
    else reinterpret_cast<uint16_t*>(stash + D * ES)[d] = (uint16_t)bits;
    if (store) {
      const long vi = ((page * a.hkv + g) * (long)D + d) * kPage + off;
      if constexpr (ES == 4) static_cast<uint32_t*>(a.v_store)[vi] = bits;
      else static_cast<uint16_t*>(a.v_store)[vi] = (uint16_t)bits;
    }
  }
}

// Puts the stashed new token (tile position tau) into a loaded tile.  Every
// register index is static (selects on the lane's role): a runtime index
// into the tile's registers would move the tile to scratch memory.
template <int D, int KV>
__device__ __forceinline__ void patch_new_token(DecodeTile<D, KV>& t, const char* stash, int tau,
                                                int lane) {
  constexpr int ES = (KV == PKV_F32) ? 4 : (kv_code8(KV) ? 1 : 2);
  constexpr int KL = DecodeTile<D, KV>::KL;
  const int r = lane & 15, kg = lane >> 4;
  const int base = tile_row_of_lane(r);
  const bool k0 = tau == base, k1 = tau == base + 4;
#pragma unroll
  for (int s = 0; s < KL; ++s) {
    const int d0 = (KV == PKV_F32) ? 16 * s + 4 * kg : (kv_code8(KV) ? 64 * s + 16 * kg : 32 * s + 8 * kg);
    const u32x4 w = *reinterpret_cast<const u32x4*>(stash + d0 * ES);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t.k[0][s][e] = k0 ? w[e] : t.k[0][s][e];
      t.k[1][s][e] = k1 ? w[e] : t.k[1][s][e];
    }
  }
  const bool vl = kg == (tau >> 3);
  const int e = tau & 7;
  if constexpr (kv_code8(KV)) {
    // V code byte e of the lane's 8 tokens, and the two scales of token e
    const float ksc = reinterpret_cast<const float*>(stash + 2 * D)[0];
    const float vsc = reinterpret_cast<const float*>(stash + 2 * D)[1];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      t.ks[q >> 2][q & 3] = (vl && q == e) ? ksc : t.ks[q >> 2][q & 3];
      t.vs[q >> 2][q & 3] = (vl && q == e) ? vsc : t.vs[q >> 2][q & 3];
    }
#pragma unroll
    for (int blk = 0; blk < D / 16; ++blk) {
      const uint32_t nv = reinterpret_cast<const uint8_t*>(stash + D)[16 * blk + r];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t w = t.v8[blk][q];
        const int sh = 8 * (e & 3);
        const uint32_t pw = (w & ~(0xffu << sh)) | (nv << sh);
        t.v8[blk][q] = (vl && q == (e >> 2)) ? pw : w;
      }
    }
    return;
  }
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk) {
    const int d = 16 * blk + r;
    if constexpr (KV == PKV_F32) {
      const uint32_t nv = reinterpret_cast<const uint32_t*>(stash + D * ES)[d];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        t.v[blk][q >> 2][q & 3] = (vl && q == e) ? nv : t.v[blk][q >> 2][q & 3];
    } else {
      const uint32_t nv = reinterpret_cast<const uint16_t*>(stash + D * ES)[d];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = t.v[blk][0][q];
        const uint32_t pw = (e & 1) ? ((w & 0x0000ffffu) | (nv << 16)) : ((w & 0xffff0000u) | nv);
        t.v[blk][0][q] = (vl && q == (e >> 1)) ? pw : w;
      }
    }
  }
}

// LDS of one partition workgroup: the wave merge (per wave and head its
// output row, max and sum), the split's page ids and the bad-page flag.
template <int D>
struct DecodeSmem {
  static constexpr int o = 0;                                       // float [W][16][D+1]
  static constexpr int m = o + kDecodeWaves * 16 * (D + 1) * 4;      // float [W][16]
  static constexpr int l = m + kDecodeWaves * 16 * 4;                // float [W][16]
  static constexpr int pid = l + kDecodeWaves * 16 * 4;              // int [2 * max tiles]
  static constexpr int bad = pid + 2 * kDecodeMaxTilesPerSplit * 4;  // int
  static constexpr int total = bad + 16;
};

// One partition workgroup: (split, KV head x head tile gy, sequence b).
// Called by all threads of a 64*kDecodeWaves-thread workgroup; `smem` holds
// DecodeSmem<D>::total bytes.  With a.cu_q_lens set (a mixed batch), only
// sequences with a one-token chunk are processed, their query and output
// rows being cu_q_lens[b].
template <int D, int KV, bool FUSE = false>
__device__ __forceinline__ void decode_partition_body(const DecodeArgs& a, char* smem, int split,
                                                      int gy, int b) {
  constexpr bool kF32 = (KV == PKV_F32);
  constexpr bool kI8 = kv_code8(KV);   // int8 or FP8 codes, exact in fp16
  constexpr bool kBF16 = (KV == PKV_BF16);
  using H8 = typename std::conditional<kBF16, bf16x8, f16x8>::type;
  constexpr int NSTEP = kF32 ? D / 4 : D / 32;    // QK MFMA k-steps
  constexpr int NBLK = D / 16;
  constexpr int R = ring_depth<D, KV>();

  const int g = gy / a.head_tiles;
  const int ht = gy % a.head_tiles;
  int qb = b;                         // query / output row of the sequence
  if (a.cu_q_lens) {
    qb = a.cu_q_lens[b];
    if (a.cu_q_lens[b + 1] - qb != 1) return;
  }
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int h0 = g * a.group + ht * 16;
  const int nh = min(16, a.group - ht * 16);

  // ---- one round trip for the context length, the query and the page ids
  //      of the whole split (loaded before the context length says which of
  //      them the split uses and how its tiles divide over the waves; entries
  //      past the context are never used).  The query's loads go out first
  //      and convert only after the page ids are in LDS: the page ids' wait
  //      then covers both.  With a sliding window the split's pages follow
  //      from the window start, so the context length comes first and
  //      entries of pages wholly before the window are not read.
  const int raw_ctx = a.context_lens[b];
  bool bad = a.cu_q_lens && raw_ctx < 1;   // a chunk of one needs a context of at least one
  using SM = DecodeSmem<D>;
  int* const s_pid = reinterpret_cast<int*>(smem + SM::pid);

  // the query's raw words (decoded below); columns past the group's heads
  // load the group's first row and are zeroed when decoded
  const bool q_live = c < nh;
  const long qrow = ((long)qb * a.hq + h0 + (q_live ? c : 0)) * D;
  constexpr int QRUN = kF32 ? 4 : 8;                 // elements per run
  uint32_t qw[NSTEP / (kF32 ? 4 : 1)][QRUN];
#pragma unroll
  for (int r = 0; r < NSTEP / (kF32 ? 4 : 1); ++r) {
    // fp32 KV: qf[4r + e] holds d = 16r + 4j + e; else run r starts at d0
    const int d0 = kF32 ? 16 * r + 4 * j : (kI8 ? (64 * (r >> 1) + 16 * j + 8 * (r & 1)) : (32 * r + 8 * j));
    io_words_rt<QRUN>(a.q, qrow + d0, a.q_dtype, qw[r]);
  }

  int lo = 0, t_lo = 0;                    // window start and its tile
  if (a.window > 0) {
    bool dummy = false;
    lo = window_start(checked_ctx(raw_ctx, a.max_context_len, a.max_blocks, dummy), a.window);
    t_lo = lo >> 5;
  }
  {
    const int sp0 = 2 * (t_lo + split * a.tiles_per_split);   // the split's first page
    const int i = threadIdx.x;
    if (i < 2 * a.tiles_per_split && sp0 + i < a.max_blocks && sp0 + i >= (lo >> 4))
      s_pid[i] = a.block_tables[(long)b * a.max_blocks + sp0 + i];
  }

  float qf[kF32 ? NSTEP : 1];
  H8 qhi[kF32 ? 1 : NSTEP], qlo[kF32 ? 1 : NSTEP];
  float head_c = a.scale_log2;   // scale * log2(e) * 2^-e for this lane's head
  // columns past the group's heads are zeroed with a mask rather than a
  // branch per element (which would put a wait and a branch around every
  // conversion ahead of the first tile loads)
  const uint32_t q_mask = q_live ? 0xffffffffu : 0u;
  if constexpr (kF32) {
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
      qf[s] = __uint_as_float(__float_as_uint(io_value_sel(io_word_bits(qw[s >> 2], s & 3, a.q_dtype), a.q_dtype)) & q_mask);
  } else {
    float x[NSTEP][8];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[s][e] = __uint_as_float(__float_as_uint(io_value_sel(io_word_bits(qw[s], e, a.q_dtype), a.q_dtype)) & q_mask);
    if constexpr (!kBF16) {
      // fp16 operands (fp16, int8 and FP8 caches): the head's query is scaled
      // by the power of two 2^e that puts its largest magnitude in
      // [2^14, 2^15), so that fp16's range holds it (a head of magnitude
      // 1e6 would overflow otherwise); the scores take 2^-e.  The head's
      // elements lie in lanes c, c+16, c+32, c+48.
      uint32_t amk = 0;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) amk = max(amk, abs_key(x[s][e]));
      amk = max(amk, (uint32_t)__shfl_xor((int)amk, 16));
      amk = max(amk, (uint32_t)__shfl_xor((int)amk, 32));
      const float am = __uint_as_float(amk);
      // zero, inf or NaN heads keep e = 0
      const int e2 = (am > 0.f && am <= 3.402823466e38f) ? 15 - __builtin_amdgcn_frexp_expf(am) : 0;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] = __builtin_ldexpf(x[s][e], e2);
      head_c = __builtin_ldexpf(a.scale_log2, -e2);
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if constexpr (kBF16) {
        auto sp = split_bf16(x[s]);
        qhi[s] = sp.hi;
        qlo[s] = sp.lo;
      } else {
        auto sp = split_f16(x[s]);
        qhi[s] = sp.hi;
        qlo[s] = sp.lo;
      }
    }
  }

  const int ctx = checked_ctx(raw_ctx, a.max_context_len, a.max_blocks, bad);
  const int ntiles = (ctx + 31) >> 5;
  const int nsplit_b = (ntiles - t_lo + a.tiles_per_split - 1) / a.tiles_per_split;
  if (split >= (nsplit_b > 0 ? nsplit_b : 1)) return;
  const int npages = (ctx + kPage - 1) / kPage;
  const int p_lo = lo >> 4;                                  // first page inside the window
  // the split's tiles, divided evenly over the waves in contiguous runs
  const int st0 = t_lo + split * a.tiles_per_split;
  const int stn = max(0, min(ntiles - st0, a.tiles_per_split));
  const int per = (stn + kDecodeWaves - 1) / kDecodeWaves;   // <= 32
  const int wt0 = st0 + wave * per;                          // first tile of the wave
  const int ntw = max(0, min(st0 + stn - wt0, per));
  const int wp0 = 2 * wt0;                                   // its first page
  const int npw = max(0, min(npages - wp0, 2 * ntw));
  __syncthreads();   // the split's page ids are in LDS
  const bool ctx_ok = !bad;
  int pid = 0, pid_ok = 1;
  if (lane < npw) {
    // a page wholly before the window (the first tile's first page at most)
    // takes the window's first page instead; its keys are masked
    pid = s_pid[max(wp0 + lane, p_lo) - 2 * st0];
    if ((unsigned)pid >= (unsigned)a.num_pages) { bad = true; pid = 0; pid_ok = 0; }
  }

  // ---- fused decode step: the wave whose tiles hold position ctx - 1 takes
  //      the new token from k_new / v_new (loaded now, ahead of its tiles),
  //      stores it to the cache (the first head tile only) and patches it
  //      into the tile it streams
  constexpr bool kFusable = FUSE;
  char* const stash = smem + SM::o + wave * kStashBytes<D>;
  int t_new = -1, tau_new = 0, page_new = 0;
  bool store_new = false;
  NewRaw<D> nr;
  if constexpr (kFusable) {
    if (ctx >= 1) {
      const int tl = (ctx - 1) >> 5;
      if (tl >= wt0 && tl < wt0 + ntw) {
        t_new = tl - wt0;
        tau_new = (ctx - 1) & 31;
        const int pl = ((ctx - 1) >> 4) - wp0;                 // the new token's page, lane of pid
        page_new = __builtin_amdgcn_readlane(pid, pl);
        store_new = ctx_ok && __builtin_amdgcn_readlane(pid_ok, pl) != 0 && ht == 0;
        load_new_token<D, KV>(nr, a, b, g, lane);
      }
    }
  }

  f32x4 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_part = 0.f;
  // 8-bit caches: acc holds the output times 2^-(v_exp - 4), where
  // v_exp is the binade of the largest V scale seen (see compute)
  int v_exp = -1000;

  auto issue = [&](DecodeTile<D, KV>& dst, int li) {
    const int pa = __builtin_amdgcn_readlane(pid, 2 * li);
    const int pb = (2 * li + 1 < npw) ? __builtin_amdgcn_readlane(pid, 2 * li + 1) : pa;
    load_tile<D, KV>(dst, a, g, pa, pb, lane);
  };

  auto compute = [&](const DecodeTile<D, KV>& cur, int li) {
    // ---- S^T = K * Q^T for the 32 tile tokens
    f32x4 s2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kF32) {
#pragma unroll
        for (int s4 = 0; s4 < D / 16; ++s4) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc = mfma16x16x4(__uint_as_float(cur.k[u][s4][e]), qf[4 * s4 + e], sacc);
        }
      } else if constexpr (kI8) {
#pragma unroll
        for (int s2i = 0; s2i < D / 64; ++s2i) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f16x8 kf;
            const u32x2 codes = u32x2{cur.k[u][s2i][2 * h], cur.k[u][s2i][2 * h + 1]};
            if constexpr (KV == PKV_FP8) fp8x8_to_f16x8_value(codes, kf);
            else i8x8_to_f16x8(codes, kf);
            sacc = mfma16x16x32(kf, qhi[2 * s2i + h], sacc);
            sacc = mfma16x16x32(kf, qlo[2 * s2i + h], sacc);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
          H8 kf = __builtin_bit_cast(H8, cur.k[u][s]);
          sacc = mfma16x16x32(kf, qhi[s], sacc);
          sacc = mfma16x16x32(kf, qlo[s], sacc);
        }
      }
      s2[u] = sacc;
    }

    // ---- scores of head c for tile tokens 8j + e, e = 4u + i; only the
    //      tiles holding the context end or the window start need masking
    const int t = wt0 + li;
    const int tok0 = 32 * t + 8 * j;
    const bool partial = (32 * t + 32 > ctx) || (32 * t < lo);
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = s2[e >> 2][e & 3] * head_c;
      if constexpr (kI8) x *= cur.ks[e >> 2][e & 3];
      sc[e] = x;
    }
    if (partial) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tok0 + e >= ctx || tok0 + e < lo) sc[e] = -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sc[e]);
    mt = wave_max_xor_16_32(mt);
    // lazy running max: the accumulator is rescaled only when the max grows
    // by more than 2^8; the stale max cancels in the final normalisation
    if (__any(mt > m_run + kDecodeLazyRescale)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < NBLK; ++i) acc[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      lsum += p[e];
    }
    l_part += lsum;

    // ---- O^T += V^T * P^T
    if constexpr (kF32) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = __uint_as_float(cur.v[blk][e >> 2][e & 3]);
          if (partial && (tok0 + e >= ctx || tok0 + e < lo)) v = 0.f;
          acc[blk] = mfma16x16x4(v, p[e], acc[blk]);
        }
      }
    } else {
      float pv[8];
      if constexpr (kI8) {
        // The V scale folds into the probability, which the PV MFMA takes
        // as fp16 (head + remainder).  To keep p * scale inside fp16's range
        // for any scale, the scales are multiplied by 2^(4 - v_exp), v_exp
        // being the binade of the largest in-context scale the wave has met
        // (wave-uniform; raised, and the accumulator scaled down by the same
        // power of two, only when a tile's largest scale lies more than two
        // binades above it): p <= 2^8 under the lazy max, so p * scale stays
        // below 2^14.  Scales of masked tokens may hold anything and are
        // left out.
        float vsc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vsc[e] = (tok0 + e < ctx && tok0 + e >= lo) ? cur.vs[e >> 2][e & 3] : 0.f;
        float vmax = vsc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) vmax = fmaxf(vmax, vsc[e]);
        vmax = wave_max_xor_16_32(vmax);
        const int et = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(vmax));
        if (et > v_exp + 2) {
#pragma unroll
          for (int i = 0; i < NBLK; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_ldexpf(acc[i][r], v_exp - et);
          v_exp = et;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = p[e] * __builtin_ldexpf(vsc[e], 4 - v_exp);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = p[e];
      }
      // V of tokens at or past the context end or before the window may
      // hold anything (NaN; for FP8 the NaN codes): zero them.  int8 codes
      // are always finite and take a zero scale above instead.
      u32x4 vmask = {~0u, ~0u, ~0u, ~0u};
      u32x2 cmask = {~0u, ~0u};
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (tok0 + e >= ctx || tok0 + e < lo) {
            vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            cmask[e >> 2] &= ~(0xffu << (8 * (e & 3)));
          }
      }
      H8 phi, plo;
      if constexpr (kBF16) {
        auto sp = split_bf16(pv);
        phi = sp.hi;
        plo = sp.lo;
      } else {
        auto sp = split_f16(pv);
        phi = sp.hi;
        plo = sp.lo;
      }
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        H8 vf;
        if constexpr (kI8) {
          f16x8 tmp;
          if constexpr (KV == PKV_FP8) fp8x8_to_f16x8_value(partial ? cur.v8[blk] & cmask : cur.v8[blk], tmp);
          else i8x8_to_f16x8(cur.v8[blk], tmp);
          vf = tmp;
        } else {
          u32x4 wv = cur.v[blk][0];
          if (partial) wv &= vmask;
          vf = __builtin_bit_cast(H8, wv);
        }
        acc[blk] = mfma16x16x32(vf, phi, acc[blk]);
        acc[blk] = mfma16x16x32(vf, plo, acc[blk]);
      }
    }
  };

  // ---- stream the wave's tiles through the register ring.  The loop body
  //      holds no conditional loads or stores: the wait before a tile
  //      computes then covers only that tile's loads, not the next tile's
  //      issued just before (a load skipped on some path makes the wait
  //      count for every path the worst one).  The wave's last tile (or
  //      last two) run after the loop: the fused step's new token, at
  //      position ctx - 1, always lies in the wave's last tile (the tile
  //      holding ctx - 1 is the context's last, and a wave's tiles are a
  //      contiguous run), so it is patched in there, outside the loop (a
  //      conditional patch inside it made the compiler copy and drain the
  //      ring on every iteration).
  DecodeTile<D, KV> ring[R];
  if constexpr (kFusable) {
    // the new token's loads went out ahead of the first tile's, so this
    // waits only for them
    if (t_new >= 0) stash_new_token<D, KV>(stash, nr, a, g, page_new, tau_new & 15, store_new, lane);
  }
  if constexpr (R == 1) {
    int i = 0;
    for (; i + 1 < ntw; ++i) {
      issue(ring[0], i);
      compute(ring[0], i);
    }
    if (i < ntw) {
      issue(ring[0], i);
      if constexpr (kFusable) {
        if (t_new == i) patch_new_token<D, KV>(ring[0], stash, tau_new, lane);
      }
      compute(ring[0], i);
    }
  } else {
    static_assert(R == 2, "a ring of one or two tiles");
    if (ntw > 0) issue(ring[0], 0);
    int i = 0;
    for (; i + 2 < ntw; i += 2) {
      issue(ring[1], i + 1);
      compute(ring[0], i);
      issue(ring[0], i + 2);
      compute(ring[1], i + 1);
    }
    if (i + 1 < ntw) {          // two tiles left, i in ring[0]
      issue(ring[1], i + 1);
      compute(ring[0], i);
      if constexpr (kFusable) {
        if (t_new == i + 1) patch_new_token<D, KV>(ring[1], stash, tau_new, lane);
      }
      compute(ring[1], i + 1);
    } else if (i < ntw) {       // one tile left, in ring[0]
      if constexpr (kFusable) {
        if (t_new == i) patch_new_token<D, KV>(ring[0], stash, tau_new, lane);
      }
      compute(ring[0], i);
    }
  }
  const float l_run = wave_sum_xor_16_32(l_part);
  if constexpr (kI8) {
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_ldexpf(acc[i][r], v_exp - 4);
  }

  // ---- merge the four waves in LDS
  typedef float OrowT[16][D + 1];
  OrowT* const s_o = reinterpret_cast<OrowT*>(smem + SM::o);
  float (*const s_m)[16] = reinterpret_cast<float (*)[16]>(smem + SM::m);
  float (*const s_l)[16] = reinterpret_cast<float (*)[16]>(smem + SM::l);
  int* const s_bad = reinterpret_cast<int*>(smem + SM::bad);
  if (threadIdx.x == 0) *s_bad = 0;
  __syncthreads();
  if (bad) atomicOr(s_bad, 1);
  if (j == 0) {
    s_m[wave][c] = m_run;
    s_l[wave][c] = l_run;
  }
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][c][16 * blk + 4 * j + i] = acc[blk][i];
  }
  __syncthreads();
  const bool any_bad = *s_bad != 0;
  const bool direct = nsplit_b <= 1;
  for (int idx = threadIdx.x; idx < nh * D; idx += 64 * kDecodeWaves) {
    const int hc = idx / D, d = idx - hc * D;
    float M = s_m[0][hc];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][hc]);
    float num = 0.f, den = 0.f;
    // a NaN score (e.g. a token whose K scale is NaN) makes a wave's sum NaN
    // while the max skips it: such a row is NaN, not zero
    bool nan_l = false;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) nan_l |= s_l[w][hc] != s_l[w][hc];
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        float f = __builtin_amdgcn_exp2f(s_m[w][hc] - M);
        num += s_o[w][hc][d] * f;
        den += s_l[w][hc] * f;
      }
    }
    const bool poison = any_bad || nan_l;
    float val = den > 0.f ? num / den : 0.f;
    if (poison) val = NAN;
    const long row = (long)b * a.hq + h0 + hc;
    if (direct) {
      store_from_f32(a.out, ((long)qb * a.hq + h0 + hc) * D + d, a.out_dtype, val);
    } else {
      const long prow = row * a.nsplits + split;
      const float lse = poison ? NAN : (den > 0.f ? M + log2f(den) : -INFINITY);
      if (a.merge_cnt) {
        // agent-coherent stores: the sequence's other splits, on any XCD,
        // read them with agent-coherent loads
        __hip_atomic_store(&a.part_o[prow * D + d], val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) __hip_atomic_store(&a.part_lse[prow], lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        a.part_o[prow * D + d] = val;
        if (d == 0) a.part_lse[prow] = lse;
      }
    }
  }
  if (direct || !a.merge_cnt) return;

  // ---- in-kernel merge: every split waits until its own partial stores
  //      have completed (agent-coherent, so visible to every XCD), then
  //      counts itself in with an atomic on the (sequence, gy) counter; the
  //      split that arrives last reads all nsplit_b partials back with
  //      agent-coherent loads and writes the output, as decode_reduce_kernel
  //      does (log-sum-exp weights, NaN from a poisoned split).  Completed
  //      stores before the counter, and the counter's returned value before
  //      the loads, order the two sides.  The counter goes from any value
  //      of another epoch to (epoch, 1) and then counts up: a compare-and-
  //      swap loop that fails only when another split counted in first, so
  //      it ends within nsplit_b + 1 tries.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are done
  __syncthreads();
  int* const s_last = s_bad + 1;
  if (threadIdx.x == 0) {
    unsigned long long* cnt = a.merge_cnt + (long)b * (a.hkv * a.head_tiles) + gy;
    unsigned long long cur = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long want = 0;
    bool done = false;
    for (int it = 0; it <= kDecodeMaxSplits + 1 && !done; ++it) {
      want = ((cur >> 8) == a.epoch ? cur : (a.epoch << 8)) + 1;
      done = __hip_atomic_compare_exchange_strong(cnt, &cur, want, __ATOMIC_RELAXED,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_last = done && (int)(want & 0xff) == nsplit_b;
  }
  __syncthreads();
  if (!*s_last) return;
  for (int idx = threadIdx.x; idx < nh * D; idx += 64 * kDecodeWaves) {
    const int hc = idx / D, d = idx - hc * D;
    const long row = (long)b * a.hq + h0 + hc;
    // eight splits' lse and element per round trip, folded into a running
    // log-sum-exp
    float M = -INFINITY, num = 0.f, den = 0.f;
    bool nan_in = false;
    for (int s0 = 0; s0 < nsplit_b; s0 += 8) {
      float l8[8], o8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const long prow = row * a.nsplits + s0 + k;
        const bool in = s0 + k < nsplit_b;
        l8[k] = in ? __hip_atomic_load(&a.part_lse[prow], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : -INFINITY;
        o8[k] = in ? __hip_atomic_load(&a.part_o[prow * D + d], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0.f;
      }
      float m8 = M;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        nan_in |= l8[k] != l8[k];
        m8 = fmaxf(m8, l8[k]);
      }
      if (m8 != -INFINITY) {
        const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - m8);
        num *= r;
        den *= r;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float w = l8[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l8[k] - m8);
          num += o8[k] * w;
          den += w;
        }
        M = m8;
      }
    }
    float val = den > 0.f ? num / den : 0.f;
    if (!ctx_ok || nan_in) val = NAN;
    store_from_f32(a.out, ((long)qb * a.hq + h0 + hc) * D + d, a.out_dtype, val);
  }
}

// Log-sum-exp merge of the split partials of one (sequence, query head):
// out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s.
// One wave per row; the context length, every split's lse and every
// partial element this lane needs are loaded together, so the merge costs
// one memory round trip.  Rows whose sequence fit one split were written by
// the partition kernel and are skipped.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  int qb = b;                         // output row (mixed batch: cu_q_lens[b])
  if (a.cu_q_lens) {
    qb = a.cu_q_lens[b];
    if (a.cu_q_lens[b + 1] - qb != 1) return;
  }
  const long row = (long)b * a.hq + h;
  const int S = a.nsplits;                       // <= kDecodeMaxSplits
  const int raw_ctx = a.context_lens[b];
  const float lse_l = lane < S ? a.part_lse[row * S + lane] : -INFINITY;
  float o[kDecodeMaxSplits][PER];
#pragma unroll
  for (int s = 0; s < kDecodeMaxSplits; ++s) {
    if (s < S) {
#pragma unroll
      for (int e = 0; e < PER; ++e) o[s][e] = a.part_o[(row * S + s) * D + lane + 64 * e];
    }
  }
  bool bad = a.cu_q_lens && raw_ctx < 1;
  const int ctx = checked_ctx(raw_ctx, a.max_context_len, a.max_blocks, bad);
  const int ntiles = (ctx + 31) >> 5;
  const int t_lo = window_start(ctx, a.window) >> 5;
  const int ns = (ntiles - t_lo + a.tiles_per_split - 1) / a.tiles_per_split;
  if (ns <= 1) return;
  const float mine = lane < ns ? lse_l : -INFINITY;
  float M = mine;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
  const float w_l = (M == -INFINITY || lane >= ns) ? 0.f : __builtin_amdgcn_exp2f(mine - M);
  float den = w_l;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m);
  // a NaN partial (a split that met a bad page id) poisons the row
  const bool nan_in = __any(mine != mine);
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kDecodeMaxSplits; ++s) {
    if (s < ns) {
      const float w = __shfl(w_l, s);
#pragma unroll
      for (int e = 0; e < PER; ++e) num[e] += o[s][e] * w;
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float val = den > 0.f ? num[e] / den : 0.f;
    if (bad || nan_in) val = NAN;
    store_from_f32(a.out, ((long)qb * a.hq + h) * D + lane + 64 * e, a.out_dtype, val);
  }
}

}  // namespace pkv
