// Chunked causal prefill over a paged prefix (TinyLoop "Current Status",
// table "Model architecture support", rows "Chunked prefill" and "GQA";
// Tiny-LLM "Project Status", supported features: chunked prefill with a
// paged KV cache).  Chunk row i of sequence b sits at position P_b + i and
// attends to keys [0, P_b + i].
//
// Rows.  The query rows of one (sequence, KV head) are the chunk positions
// times the G query heads that share the KV head, flattened head-fastest:
// row r -> position r / G, head g*G + r % G.  A workgroup of 4 waves owns 128
// consecutive rows, a wave 32; every wave walks the key tiles its rows need
// (32 keys = two pages per tile), so the G heads of a position reuse each
// K/V fragment.
//
// MFMA mapping (32x32x16, wave64).  S^T = K * Q^T: A = K (row = key),
// B = Q^T (column = query row).  The A-operand row rho loads key
// 16*(rho/16) + 8*((rho/4)&1) + 4*((rho/8)&1) + rho%4, which makes lane
// (c + 32*h) hold, for query row c, the scores of keys 8h..8h+7 of the first
// page (registers 0-7) and of the second page (registers 8-15): the
// B-operand layout of O^T = V^T * P^T with no data movement.  The V page is
// stored token-innermost, so each V^T A-operand load is a contiguous 8-key
// run.  The causal mask is applied only to tiles that cross a row's limit.
//
// Precision: q and K/V in the cache's 16-bit type (an fp32 or other-typed
// q is split into head + remainder and multiplied twice), P rounded to the
// 16-bit type (the normaliser sums the rounded values), fp32 accumulation.
#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerBlock = kPrefillRowsPerWave * kPrefillWaves;

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  void* out;
  int q_dtype, out_dtype;
  int max_blocks, max_context_len, max_q_len;
  int batch, hq, hkv, group, num_pages, nrowblocks;
  float scale_log2;
};

template <int D, int KV, bool QSPLIT>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr bool kBF16 = (KV == PKV_BF16);
  using H8 = typename std::conditional<kBF16, bf16x8, f16x8>::type;
  constexpr int NSTEP = D / 16;  // QK k-steps of 16
  constexpr int NDB = D / 32;    // 32-row blocks of d for PV

  const int b = blockIdx.x;
  const int g = blockIdx.y;
  const int rb = a.nrowblocks - 1 - (int)blockIdx.z;  // heavier (later) rows first
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int G = a.group;

  bool bad = false;
  const int q0 = a.cu_q_lens[b];
  int C = a.cu_q_lens[b + 1] - q0;
  if (C < 0 || C > a.max_q_len) { bad = true; C = C < 0 ? 0 : a.max_q_len; }
  int ctx = a.context_lens[b];
  const int ctx_lim = min(a.max_context_len, a.max_blocks * kPage);
  if (ctx < C || ctx > ctx_lim) { bad = true; ctx = max(C, min(ctx, ctx_lim)); }
  const int P = ctx - C;
  const int rows_b = C * G;
  const int r0 = rb * kPrefillRowsPerBlock + wave * kPrefillRowsPerWave;
  if (r0 >= rows_b) return;  // no barrier in this kernel: waves leave independently

  const int row = r0 + col;
  const bool live = row < rows_b;
  const int pos = live ? row / G : 0;
  const int h = g * G + (live ? row - pos * G : 0);
  const int limit = live ? P + pos : -1;
  const int last_row = min(rows_b - 1, r0 + kPrefillRowsPerWave - 1);
  const int lim_max = P + last_row / G;
  const int lim_min = P + r0 / G;
  const int ntiles = (lim_max + 1 + 31) >> 5;
  const int npages = (ctx + kPage - 1) / kPage;
  const long qrow = ((long)(q0 + pos) * a.hq + h) * D;

  // ---- Q^T fragments (B operand): column col, k-chunk d = 16*s + 8*hh
  H8 qhi[NSTEP], qlo[QSPLIT ? NSTEP : 1];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int d0 = 16 * s + 8 * hh;
    if constexpr (!QSPLIT) {
      u32x4 w = live ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qrow + d0)
                     : u32x4{0u, 0u, 0u, 0u};
      qhi[s] = __builtin_bit_cast(H8, w);
    } else {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = live ? load_as_f32(a.q, qrow + d0 + e, a.q_dtype) : 0.f;
      if constexpr (kBF16) {
        auto sp = split_bf16(x);
        qhi[s] = sp.hi;
        qlo[s] = sp.lo;
      } else {
        auto sp = split_f16(x);
        qhi[s] = sp.hi;
        qlo[s] = sp.lo;
      }
    }
  }

  const int32_t* bt = a.block_tables + (long)b * a.max_blocks;
  auto page_of = [&](int idx) -> int {
    int p = bt[idx];
    if ((unsigned)p >= (unsigned)a.num_pages) { bad = true; p = 0; }
    return p;
  };
  // K A-operand row of this lane and the key it carries
  const int krow = col;
  const int kpage_sel = krow >> 4;  // 0: first page of the tile, 1: second
  const int ktok = 8 * ((krow >> 2) & 1) + 4 * ((krow >> 3) & 1) + (krow & 3);
  const long head_elems = (long)kPage * D;

  auto load_k = [&](u32x4 (&kf)[NSTEP], int pa, int pb) {
    const int pg = kpage_sel ? pb : pa;
    const uint16_t* base = static_cast<const uint16_t*>(a.k_cache) +
                           ((long)pg * a.hkv + g) * head_elems + (long)ktok * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) kf[s] = *reinterpret_cast<const u32x4*>(base + 16 * s);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  u32x4 kcur[NSTEP], knxt[NSTEP];
  int pa_cur = 0, pb_cur = 0;
  if (ntiles > 0) {
    pa_cur = page_of(0);
    pb_cur = (1 < npages) ? page_of(1) : pa_cur;
    load_k(kcur, pa_cur, pb_cur);
  }
  for (int t = 0; t < ntiles; ++t) {
    // V^T fragments of this tile: A operand rows d = 32*db + col, keys 8*hh..+7
    u32x4 vf[NDB][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pg = u ? pb_cur : pa_cur;
      const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) +
                              ((long)pg * a.hkv + g) * head_elems + 8 * hh;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        vf[db][u] = *reinterpret_cast<const u32x4*>(vbase + (long)(32 * db + col) * kPage);
    }
    // next tile's K
    int pa_n = pa_cur, pb_n = pb_cur;
    if (t + 1 < ntiles) {
      pa_n = page_of(2 * t + 2);
      pb_n = (2 * t + 3 < npages) ? page_of(2 * t + 3) : pa_n;
      load_k(knxt, pa_n, pb_n);
    }

    // ---- S^T = K * Q^T
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      H8 kf = __builtin_bit_cast(H8, kcur[st]);
      s = mfma32x32x16(kf, qhi[st], s);
      if constexpr (QSPLIT) s = mfma32x32x16(kf, qlo[st], s);
    }

    // ---- online softmax for query row `col`; register r holds key
    //      32t + 16*(r/8) + 8*hh + r%8
    const int kbase_tok = 32 * t + 8 * hh;
    const bool need_mask = (32 * t + 31 > lim_min);
    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * a.scale_log2;
      if (need_mask && kbase_tok + 16 * (r >> 3) + (r & 7) > limit) x = -INFINITY;
      sc[r] = x;
    }
    float mt = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    H8 p16[2];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(sc[r] - m_use);
      if constexpr (kBF16) {
        __bf16 hv = (__bf16)p;
        p16[r >> 3][r & 7] = hv;
        lsum += (float)hv;
      } else {
        _Float16 hv = (_Float16)p;
        p16[r >> 3][r & 7] = hv;
        lsum += (float)hv;
      }
    }
    l_part = l_part * alpha + lsum;
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] *= alpha;

    // keys at or past the context end may hold anything: zero their V
    if (32 * t + 32 > ctx) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (32 * t + 16 * u + 8 * hh + e >= ctx) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              vf[db][u][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
    }
    // ---- O^T += V^T * P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      acc[db] = mfma32x32x16(__builtin_bit_cast(H8, vf[db][0]), p16[0], acc[db]);
      acc[db] = mfma32x32x16(__builtin_bit_cast(H8, vf[db][1]), p16[1], acc[db]);
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) kcur[st] = knxt[st];
    pa_cur = pa_n;
    pb_cur = pb_n;
  }
  const float l_run = l_part + __shfl_xor(l_part, 32);
  if (!live) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const long orow = ((long)(q0 + pos) * a.hq + h) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
      float v = acc[db][r] * inv;
      if (bad) v = NAN;
      store_from_f32(a.out, orow + d, a.out_dtype, v);
    }
  }
}

template <int D, int KV>
static void dispatch_prefill_q(const PrefillArgs& a, pkv_stream_t stream) {
  dim3 grid(a.batch, a.hkv, a.nrowblocks);
  if (a.q_dtype == KV)
    hipLaunchKernelGGL((prefill_kernel<D, KV, false>), grid, dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, KV, true>), grid, dim3(256), 0, (hipStream_t)stream, a);
}

template <int D>
static void dispatch_prefill(int kv, const PrefillArgs& a, pkv_stream_t stream) {
  if (kv == PKV_BF16) dispatch_prefill_q<D, PKV_BF16>(a, stream);
  else dispatch_prefill_q<D, PKV_F16>(a, stream);
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attn_prefill_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                                     int head_dim, int max_q_len,
                                                     int max_context_len) {
  (void)batch; (void)num_q_heads; (void)num_kv_heads; (void)head_dim; (void)max_q_len;
  (void)max_context_len;
  return 0;
}

extern "C" int paged_attn_prefill_chunk(const void* q, int q_dtype, const void* k_cache,
                                        const void* v_cache, const float* k_scales,
                                        const float* v_scales, int kv_dtype,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, const int32_t* cu_q_lens,
                                        int num_tokens, int max_q_len, int max_context_len,
                                        int batch, int num_q_heads, int num_kv_heads,
                                        int head_dim, int page_size, int num_pages, float scale,
                                        void* out, int out_dtype, void* workspace,
                                        size_t workspace_bytes, pkv_stream_t stream) {
  (void)workspace; (void)workspace_bytes;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens || !out)
    return PKV_ERR_INVALID_ARG;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      num_pages <= 0 || max_blocks_per_seq <= 0 || num_tokens < 0 || max_q_len < 0 ||
      max_context_len < 0 || max_q_len > max_context_len ||
      (long)max_context_len > (long)max_blocks_per_seq * PKV_PAGE_SIZE)
    return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(q_dtype) || !io_dtype_ok(out_dtype) || !kv_dtype_ok(kv_dtype))
    return PKV_ERR_INVALID_ARG;
  if ((kv_dtype == PKV_I8) != (k_scales != nullptr) || (kv_dtype == PKV_I8) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_F16) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(block_tables) || !aligned16(context_lens) || !aligned16(cu_q_lens))
    return PKV_ERR_MISALIGNED;
  if (num_tokens == 0 || max_q_len == 0) return PKV_OK;

  PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = cu_q_lens;
  a.out = out;
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  a.max_blocks = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.max_q_len = max_q_len;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_pages = num_pages;
  a.nrowblocks = ceil_div((long)max_q_len * a.group, kPrefillRowsPerBlock);
  a.scale_log2 = scale * kLog2e;
  if (a.nrowblocks > 65535 || batch > 0x7fffffff) return PKV_ERR_INVALID_ARG;

  clear_launch_error();
  if (head_dim == 64) dispatch_prefill<64>(kv_dtype, a, stream);
  else dispatch_prefill<128>(kv_dtype, a, stream);
  return launch_status();
}
