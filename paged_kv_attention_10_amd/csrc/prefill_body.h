// Device code of the chunked causal prefill (shared by the prefill entry
// point and the mixed prefill/decode kernel).  The algorithm is described
// in prefill.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from global memory into LDS at l + 16 * lane (l must be
// the same in every lane of the wave).
__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerBlock = kPrefillRowsPerWave * kPrefillWaves;
constexpr int kPrefillTileKeys = 64;  // 4 pages, one per wave

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
  // scale * log2(e) enters as c = |scale| * log2(e) > 0 (log2(e) for a zero
  // scale) with the query multiplied by the sign of the scale (0 for a zero
  // scale) as it is loaded: exact, and the raw-score max and the -inf masks
  // below then need a positive c
  float scale_log2;
  uint32_t q_xor, q_and;   // applied to packed 16-bit query words
  float q_mul;             // applied to an fp32 query value
  int skip_single;   // mixed batch: chunks of one token are left to the decode path
  int window;        // sliding window in tokens, 0 = the whole causal prefix
};

template <int D>
struct PrefillLds {
  static constexpr int kRow = 2 * D;                 // bytes of one K row
  static constexpr int kPageBytes = kPage * kRow;    // one page of K (= one page of V^T)
  static constexpr int vOff = 4 * kPageBytes;        // V^T blocks after the 64 K rows
  static constexpr int stage = 8 * kPageBytes;
  static constexpr int dmaPerPage = kPageBytes / 1024;
  static constexpr int chunksPerRow = D / 8;
};

// 16-byte-chunk swizzle of K row rr (its offset in the page): chunk c of the
// row is stored in slot c ^ swz(rr).
template <int D>
__device__ __forceinline__ int k_swizzle(int rr) {
  if constexpr (D == 128) return (rr ^ ((rr & 8) >> 1)) & 15;
  else return (rr ^ (rr >> 3)) & 7;
}

constexpr float kLazyRescale = 8.0f;

// Which row block a prefill workgroup takes.  Workgroup ids are dealt round
// robin to the XCDs and, within one, to its CUs in turn, and two workgroups
// share a CU; a row block's time grows with its sequence's context.  In the
// grid order (sequence fastest, then KV head, then row block, heavier row
// blocks first) each sequence's row blocks share one XCD and its L2.  When
// the whole grid fits two workgroups per CU (at most kPrefillSortMaxGrid;
// larger grids queue, and the queue balances them) and holds at most
// kPrefillSortMaxBatch sequences whose contexts differ (among those with
// rows, the longest more than 25% above the shortest), every workgroup
// ranks the sequences by context length (ties by index) from the same
// loads, so all agree on one order of the row blocks that hold rows: the
// first kPrefillFirstRound ids (one per CU of a 256-CU
// MI355X) take the heaviest and the next ids the rest lightest first, so
// that a CU's second workgroup tends to be a light one and every XCD gets a
// share of the long sequences; ids past the last such row block have no work.
constexpr int kPrefillSortMaxBatch = 256;
constexpr long kPrefillFirstRound = 256;
constexpr long kPrefillSortMaxGrid = 2 * kPrefillFirstRound;

// `id` is the workgroup's position in the grid order.  Returns false (and
// leaves b, g, rb alone) when the grid order is kept; a workgroup left
// without work gets rb = nrowblocks, which prefill_body turns away.  Called
// by all 256 threads; uses 3 KB of `sh`, free again on return.
__device__ __forceinline__ bool prefill_item(const PrefillArgs& a, int* sh, long id, int& b,
                                             int& g, int& rb) {
  const int B = a.batch, H = a.hkv, R = a.nrowblocks;
  int* weight = sh;                                 // per sequence: context, -1 without rows
  int* seq_of = sh + kPrefillSortMaxBatch;          // per rank: sequence
  int* items_of = sh + 2 * kPrefillSortMaxBatch;    // per rank: row blocks holding rows x H
  const int t = threadIdx.x;
  int items = 0;
  if (t < B) {
    // the rows prefill_body gives the sequence (the same clamping)
    int C = a.cu_q_lens[t + 1] - a.cu_q_lens[t];
    C = C < 0 ? 0 : min(C, a.max_q_len);
    const int rows = (a.skip_single && C == 1) ? 0 : C * a.group;
    items = (rows + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock * H;
    weight[t] = items > 0 ? max(a.context_lens[t], 0) : -1;
  }
  __syncthreads();
  const int w = t < B ? weight[t] : 0;
  int rank = 0, live = 0, lo = 0x7fffffff, hi = -1;
  for (int u = 0; u < B; ++u) {
    const int x = weight[u];
    rank += (x > w) || (x == w && u < t);
    if (x >= 0) {
      ++live;
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  if (live == 0 || (long)hi <= (long)lo + lo / 4) {   // all threads agree (same loads)
    __syncthreads();
    return false;
  }
  if (t < B) {
    seq_of[rank] = t;
    items_of[rank] = items;
  }
  __syncthreads();
  long n_items = 0;
  for (int r = 0; r < B; ++r) n_items += items_of[r];
  if (id >= n_items) {
    rb = R;
  } else {
    long p = id;                                   // position in the ranked order
    if (id >= kPrefillFirstRound) p = n_items - 1 + kPrefillFirstRound - id;
    long acc = 0;
    int r = 0;
    while (p >= acc + items_of[r]) acc += items_of[r++];
    const int q = (int)(p - acc);
    b = seq_of[r];
    rb = items_of[r] / H - 1 - q / H;              // heavier (later) row blocks first
    g = q % H;
  }
  __syncthreads();
  return true;
}

// One row block: the 128 rows rb of (sequence b, KV head g).  Called by all
// 256 threads of the workgroup; `lds` holds two tile stages (1024-aligned).
template <int D, int KV, bool QSPLIT>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, char* lds, int b, int g, int rb) {
  constexpr bool kBF16 = (KV == PKV_BF16);
  using H8 = typename std::conditional<kBF16, bf16x8, f16x8>::type;
  using L = PrefillLds<D>;
  constexpr int NSTEP = D / 16;  // QK k-steps of 16
  constexpr int NDB = D / 32;    // 32-row blocks of d for PV
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
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
  const int rows_b = (a.skip_single && C == 1) ? 0 : C * G;
  const int wg_r0 = rb * kPrefillRowsPerBlock;
  if (wg_r0 >= rows_b) return;  // the whole workgroup, before any barrier

  // the workgroup's key range and this wave's.  With a sliding window of W
  // tokens row position p sees keys (p - W, p]: the workgroup starts at the
  // tile of its first row's window, and pages wholly before that window are
  // never read.
  const int wg_last = min(rows_b - 1, wg_r0 + kPrefillRowsPerBlock - 1);
  const int ntiles = (P + wg_last / G + kPrefillTileKeys) / kPrefillTileKeys;
  const int W = a.window;
  const int wg_lo = W > 0 ? max(0, P + wg_r0 / G - W + 1) : 0;   // first key of the workgroup
  const int t_first = wg_lo / kPrefillTileKeys;
  const int p_first = wg_lo / kPage;                             // first page read
  const int r0 = wg_r0 + wave * kPrefillRowsPerWave;
  const int lim_min = P + r0 / G;      // smallest causal limit among the wave's rows
  // largest window start among the wave's rows: tiles starting below it need
  // the window mask
  const int win_max = W > 0 ? P + min(rows_b - 1, r0 + kPrefillRowsPerWave - 1) / G - W + 1 : 0;
  const int row = r0 + col;
  const bool live = row < rows_b;
  const int pos = live ? row / G : 0;
  const int h = g * G + (live ? row - pos * G : 0);
  const int limit = live ? P + pos : -1;
  const int wlo = W > 0 ? limit - W + 1 : 0;   // this row's first key
  const int npages = (ctx + kPage - 1) / kPage;
  const long qrow = ((long)(q0 + pos) * a.hq + h) * D;

  // ---- Q^T fragments (B operand): column col, k-chunk d = 16*s + 8*hh
  H8 qhi[NSTEP], qlo[QSPLIT ? NSTEP : 1];
  if constexpr (!QSPLIT) {
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const int d0 = 16 * s + 8 * hh;
      u32x4 w = live ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qrow + d0)
                     : u32x4{0u, 0u, 0u, 0u};
      w = (w ^ a.q_xor) & a.q_and;
      qhi[s] = __builtin_bit_cast(H8, w);
    }
  } else {
    // a dead row's qrow is the chunk's first row (valid): loaded, then zeroed
    with_io_dtype(a.q_dtype, [&](auto qdt) {
      constexpr int QT = decltype(qdt)::value;
      uint32_t bits[NSTEP][8];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) io_bits_vec<8, QT>(a.q, qrow + 16 * s + 8 * hh, bits[s]);
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? io_value<QT>(bits[s][e]) * a.q_mul : 0.f;
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
    });
  }

  // ---- page ids: a window of 64 consecutive entries of the block-table row,
  //      one per lane, and the next window loaded ahead
  const int32_t* bt = a.block_tables + (long)b * a.max_blocks;
  auto load_window = [&](int win) {
    const int i = 64 * win + lane;
    return i < npages ? bt[i] : 0;
  };
  int pid_cur = load_window(t_first >> 4);
  int pid_next = ntiles > (t_first | 15) + 1 ? load_window((t_first >> 4) + 1) : 0;

  // ---- tile copy: wave w moves page 4t + w of the tile (K rows swizzled,
  //      V^T block as is) into stage `stg`; pages past the context are not
  //      read (their keys are masked and their V is zeroed in registers)
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  int koff[L::dmaPerPage];
#pragma unroll
  for (int j = 0; j < L::dmaPerPage; ++j) {
    const int byte = 1024 * j + 16 * lane;          // position inside the page's K block
    const int rr = byte / L::kRow, slot = (byte % L::kRow) / 16;
    koff[j] = rr * L::kRow + ((slot ^ k_swizzle<D>(rr)) * 16);
  }
  auto issue_tile = [&](int t, int stg) {
    if ((t & 15) == 0 && t > t_first) {
      pid_cur = pid_next;
      pid_next = load_window((t >> 4) + 1);
    }
    const int pi = 4 * t + wave;
    if (pi < npages && pi >= p_first) {
      int pid = __builtin_amdgcn_readlane(pid_cur, pi & 63);
      if ((unsigned)pid >= (unsigned)a.num_pages) { bad = true; pid = 0; }
      const long blk = ((long)pid * a.hkv + g) * L::kPageBytes;
      char* lk = lds + stg * L::stage + wave * L::kPageBytes;
      char* lv = lds + stg * L::stage + L::vOff + wave * L::kPageBytes;
#pragma unroll
      for (int j = 0; j < L::dmaPerPage; ++j) {
        dma16(kc + blk + koff[j], lk + 1024 * j);
        dma16(vc + blk + 1024 * j + 16 * lane, lv + 1024 * j);
      }
    }
  };

  // per-lane LDS offsets of the fragment reads
  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);
  int kaddr[NSTEP];
#pragma unroll
  for (int k = 0; k < NSTEP; ++k)
    kaddr[k] = krow * L::kRow + (((2 * k + hh) ^ k_swizzle<D>(krow & 15)) * 16);
  const int vaddr = L::vOff + col * 32 + hh * 16;

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // one 64-key tile (keys kb .. kb+63; half hf = pages 2hf and 2hf+1)
  auto compute_tile = [&](const char* st, int kb) {
    // ---- S^T = K * Q^T for both halves: all K fragment reads first (one
    //      LDS latency), then two independent MFMA chains
    u32x4 kfr[2][NSTEP];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int k = 0; k < NSTEP; ++k)
        kfr[hf][k] = *reinterpret_cast<const u32x4*>(st + hf * 32 * L::kRow + kaddr[k]);
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const H8 kf = __builtin_bit_cast(H8, kfr[hf][k]);
        s[hf] = mfma32x32x16(kf, qhi[k], s[hf]);
        if constexpr (QSPLIT) s[hf] = mfma32x32x16(kf, qlo[k], s[hf]);
      }
    // keep the K reads ahead of the MFMAs (the default schedule pairs them
    // and waits for LDS between every two MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NSTEP, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, (QSPLIT ? 4 : 2) * NSTEP, 0);
    // ---- V^T fragments (their LDS latency hides behind the softmax)
    u32x4 vfr[2][NDB][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          vfr[hf][db][j] = *reinterpret_cast<const u32x4*>(
              st + vaddr + (2 * hf + j) * L::kPageBytes + db * 32 * 32);
    // keys at or past the context end, or in pages not read because they
    // lie wholly before the window, may hold anything: zero their V
    if (kb + 64 > ctx || kb < kPage * p_first) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int key0 = kb + 32 * hf + 16 * j + 8 * hh;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool out = key0 + e >= ctx || key0 + e < kPage * p_first;
            const uint32_t m = out ? ((e & 1) ? 0x0000ffffu : 0xffff0000u) : 0xffffffffu;
#pragma unroll
            for (int db = 0; db < NDB; ++db) vfr[hf][db][j][e >> 1] &= m;
          }
        }
    }
    // ---- online softmax for query row `col`; register r of half hf holds
    //      key kb + 32*hf + 16*(r/8) + 8*hh + r%8, masked when that exceeds
    //      `limit`.  Raw scores are masked and maximised; the log2e-prescaled
    //      scale (positive) is applied inside the exponent: p = 2^(s*c - m).
    if (kb + 63 > lim_min) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rel = limit - (kb + 32 * hf + 8 * hh);   // largest allowed 16*(r/8) + r%8
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) > rel) s[hf][r] = -INFINITY;
      }
    }
    if (kb < win_max) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rel = wlo - (kb + 32 * hf + 8 * hh);     // smallest allowed 16*(r/8) + r%8
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) < rel) s[hf][r] = -INFINITY;
      }
    }
    float mt = s[0][0];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[hf][r]);
    mt = max_xor32(mt) * a.scale_log2;
    const bool grow = mt > m_run + kLazyRescale;
    if (__any(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) acc[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      H8 p16[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][r], a.scale_log2, -m_use));
        if constexpr (kBF16) p16[r >> 3][r & 7] = (__bf16)p;
        else p16[r >> 3][r & 7] = (_Float16)p;
      }
      // the row sum takes the rounded probabilities the PV multiplies, two
      // per packed dot product with (1, 1)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        if constexpr (kBF16) {
          const bf16x2 pair = {p16[r >> 3][r & 7], p16[r >> 3][(r & 7) + 1]};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pair, bf16x2{(__bf16)1.f, (__bf16)1.f}, lsum, false);
        } else {
          const f16x2 pair = {p16[r >> 3][r & 7], p16[r >> 3][(r & 7) + 1]};
          lsum = __builtin_amdgcn_fdot2(pair, f16x2{(_Float16)1.f, (_Float16)1.f}, lsum, false);
        }
      }
      // ---- O^T += V^T * P^T
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32x32x16(__builtin_bit_cast(H8, vfr[hf][db][j]), p16[j], acc[db]);
    }
    l_part += lsum;
  };

  // ---- pipeline: tile t computes from LDS while tile t+1 is copied in
  issue_tile(t_first, t_first & 1);
  __syncthreads();  // waits for this wave's copies, then for every wave's
  for (int t = t_first; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue_tile(t + 1, (t + 1) & 1);
    const char* st = lds + (t & 1) * L::stage;
    const int kb = t * kPrefillTileKeys;
    // every wave computes every tile: a tile past all of a wave's rows is
    // fully masked (p = 0), and branching around it would make the compiler
    // copy the accumulators at each join
    compute_tile(st, kb);
    __syncthreads();
  }
  bad = __syncthreads_or(bad);

  const float l_run = sum_xor32(l_part);
  if (!live) return;
  // a NaN score makes the row sum NaN while the max skips it: NaN, not zero
  const float inv = (bad || l_run != l_run) ? NAN : (l_run > 0.f ? 1.f / l_run : 0.f);
  const long orow = ((long)(q0 + pos) * a.hq + h) * D;
  // lane (col + 32*hh), register r of block db holds d = 32*db + 8*(r/4) + 4*hh + r%4:
  // four consecutive d per group of four registers
  auto write = [&](auto tag) {
    using T = decltype(tag);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const long o = orow + 32 * db + 8 * r4 + 4 * hh;
        f32x4 v = {acc[db][4 * r4] * inv, acc[db][4 * r4 + 1] * inv, acc[db][4 * r4 + 2] * inv,
                   acc[db][4 * r4 + 3] * inv};
        if constexpr (std::is_same<T, float>::value) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = v;
        } else {
          u32x2 pk;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            uint32_t lo, hi;
            if constexpr (std::is_same<T, __bf16>::value) {
              lo = f32_to_bf16_bits(v[2 * e]);
              hi = f32_to_bf16_bits(v[2 * e + 1]);
            } else {
              lo = f32_to_f16_bits(v[2 * e]);
              hi = f32_to_f16_bits(v[2 * e + 1]);
            }
            pk[e] = lo | (hi << 16);
          }
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = pk;
        }
      }
    }
  };
  if (a.out_dtype == PKV_F32) write(0.f);
  else if (a.out_dtype == PKV_BF16) write((__bf16)0.f);
  else write((_Float16)0.f);
}

}  // namespace pkv
