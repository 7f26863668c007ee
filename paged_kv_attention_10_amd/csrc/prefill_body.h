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

// The same copy issued from inline asm: the compiler does not count it among
// its vector-memory operations, so it neither waits for it before LDS reads
// of the other stage (it cannot tell the stages apart) nor keeps it out of a
// run of MFMAs.  The copy has no register result and reads its address
// registers when it issues; M0 carries the LDS address (the compiler sets
// M0 again before any use of its own).  Its caller waits for it with
// wait_vmcnt0 before the barrier that hands the stage to the other waves;
// the compiler's own vector-memory waits stay correct (a copy it does not
// count only makes them wait longer).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved: nothing else keeps a value in it here
__device__ __forceinline__ void dma16_async(const void* g, void* l) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)l;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(la)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0) with the other counters unbounded
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerBlock = kPrefillRowsPerWave * kPrefillWaves;
constexpr int kPrefillTileKeys = 64;  // 4 pages, one per wave

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;   // int8 / FP8 caches only
  const float* v_scales;
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

// One tile stage in LDS: four pages of K rows, then four V^T page blocks,
// then (int8 / FP8) each page's 16 K scales and 16 V scales.
template <int D, int KV>
struct PrefillLds {
  // bytes per element in LDS: fp32 caches 4, the others 2 (one-byte codes
  // are converted to fp16 as the tile is staged)
  static constexpr int ES = KV == PKV_F32 ? 4 : 2;
  static constexpr int kRow = ES * D;                // bytes of one K row
  static constexpr int kPageBytes = kPage * kRow;    // one page of K (= one page of V^T)
  static constexpr int vOff = 4 * kPageBytes;        // V^T blocks after the 64 K rows
  // one-byte caches: per page 16 K scales and 16 V scales, then the four
  // pages' largest in-range V scale
  static constexpr int sOff = 8 * kPageBytes;
  static constexpr int pmOff = sOff + 4 * 128;
  static constexpr int stage = 8 * kPageBytes + (kv_code8(KV) ? 1024 : 0);
  static constexpr int dmaPerPage = kPageBytes / 1024;
};

// 16-byte-chunk swizzle of K row rr (its offset in the page): chunk c of the
// row is stored in slot c ^ swz(rr).
template <int D>
__device__ __forceinline__ int k_swizzle(int rr) {
  if constexpr (D == 128) return (rr ^ ((rr & 8) >> 1)) & 15;
  else return (rr ^ (rr >> 3)) & 7;
}

// 16-bit V^T rows (16 keys, two 16-byte chunks): chunk c of row d is
// stored in slot c ^ v_swizzle16(d).  A fragment read has lanes c .. c+15
// on rows d .. d+15 and one chunk: without the swap rows d and d + 8 share
// a 16-byte bank slot (a two-way conflict in every 16-lane group).
__device__ __forceinline__ int v_swizzle16(int d) { return (d >> 3) & 1; }

// Workgroups a CU can hold for this stage size (160 KB of LDS per CU): two
// for the 16-bit and one-byte caches, one for fp32 at head_dim 128.
template <int D, int KV>
constexpr int prefill_workgroups_per_cu() {
  return 2 * (2 * PrefillLds<D, KV>::stage) <= 160 * 1024 ? 2 : 1;
}

// fp32 K rows (D/4 chunks): chunk c in slot c ^ swz(rr) with the 16-slot
// pattern above (rows are a multiple of 256 bytes, so the 16 rows a 16-lane
// read touches land in 16 different slots).  fp32 V^T rows (16 keys, four
// chunks): chunk c of row d in slot c ^ vswz(d), which puts the 16 rows of
// a 16-lane read (64 bytes apart) in 16 different 16-byte bank slots.
__device__ __forceinline__ int k_swizzle32(int rr) { return (rr ^ ((rr & 8) >> 1)) & 15; }
__device__ __forceinline__ int v_swizzle32(int d) { return ((d >> 2) ^ (d >> 1)) & 3; }

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
// leaves b, g, rb alone) when the caller's order is kept (also when more
// than kPrefillSortMaxGrid row blocks hold rows); a workgroup left without
// work gets rb = nrowblocks, which prefill_body turns away.  Called by all
// 256 threads; uses 3 KB of `sh`, free again on return.
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
  if (n_items > kPrefillSortMaxGrid) {   // more than two rounds: keep the caller's order
    __syncthreads();
    return false;
  }
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

// x * y with 0 * anything = 0 (NaN and inf included): v_mul_legacy_f32,
// reached through its LLVM intrinsic (not inline asm, so that the compiler
// sees the instruction and keeps the wait states it needs, e.g. after a
// transcendental that produced x).
extern "C" __device__ float pkv_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");
__device__ __forceinline__ float mul_zero_wins(float x, float y) { return pkv_fmul_legacy(x, y); }

// int8 / FP8 codes (8 per 64 bits) -> fp16 values, exact.
template <int KV>
__device__ __forceinline__ f16x8 codes8_to_f16(u32x2 w) {
  f16x8 r;
  if constexpr (KV == PKV_FP8) fp8x8_to_f16x8_value(w, r);
  else i8x8_to_f16x8(w, r);
  return r;
}

// One row block: the 128 rows rb of (sequence b, KV head g).  Called by all
// 256 threads of the workgroup; `lds` holds two tile stages (1024-aligned).
//
// int8 / FP8 caches: each tile's codes are converted once, exactly, to fp16
// as the tile is staged in LDS (int8 with the v_perm + subtract trick, FP8
// with the hardware convert), so the compute reads fp16 fragments as the
// 16-bit path does.  The query row is scaled by the power of two 2^e that
// puts its largest magnitude in [2^14, 2^15) and rounded to fp16 (split
// into head + remainder for an fp32 query); a bf16 or fp16 query is then
// exact down to 2^-32 of that largest magnitude.  The scores take the K
// scale and c * 2^-e.  The V scale multiplies the probability (0 * anything
// = 0 there, so a NaN scale of a masked key stays out), normalised as in
// the decode: scales are multiplied by 2^(4 - v_exp), v_exp the binade of
// the largest in-range scale met so far (the same in every wave: each tile
// stages its pages' largest scales), raised (with the accumulator scaled
// down to match) when a tile's largest scale lies more than two binades
// above it, so p * scale stays below 2^14 in fp16; the power of two goes
// back on at the end.
template <int D, int KV, bool QSPLIT>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, char* lds, int b, int g, int rb) {
  constexpr bool kI8 = kv_code8(KV);
  constexpr bool kF32 = (KV == PKV_F32);
  static_assert(!(kF32 && QSPLIT), "an fp32 cache takes the query in fp32");
  constexpr bool kBF16 = (KV == PKV_BF16);
  using H8 = typename std::conditional<kBF16, bf16x8, f16x8>::type;
  using L = PrefillLds<D, KV>;
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

  // ---- Q^T fragments (B operand), column col, k-chunk d = 16*s + 8*hh.
  //      A query in the cache's own 16-bit type is used as it is; otherwise
  //      the row goes through fp32 (times the sign of the scale) and, when
  //      the MFMA takes fp16, is scaled by the power of two 2^e that puts its
  //      largest magnitude in [2^14, 2^15) (fp16's range then holds it, and
  //      a bf16 or fp16 row is exact down to 2^-32 of that magnitude); it is
  //      rounded to the MFMA type, split into head + remainder for an fp32
  //      or other-typed query, and the scores take c * 2^-e.
  H8 qhi[NSTEP], qlo[QSPLIT ? NSTEP : 1];
  float qf[kF32 ? D / 2 : 1];   // fp32 cache: q[col][s + (D/2)*hh], exact in fp32
  float row_c = a.scale_log2;   // c * 2^-e for this row
  if constexpr (kF32) {
    with_io_dtype(a.q_dtype, [&](auto qdt) {
      constexpr int QT = decltype(qdt)::value;
      uint32_t bits[D / 16][8];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) io_bits_vec<8, QT>(a.q, qrow + (D / 2) * hh + 8 * s, bits[s]);
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[8 * s + i] = live ? io_value<QT>(bits[s][i]) * a.q_mul : 0.f;
    });
  } else if constexpr (!kI8 && !QSPLIT) {
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
      for (int s = 0; s < NSTEP; ++s)
        io_bits_vec<8, QT>(a.q, qrow + 16 * s + 8 * hh, bits[s]);
      float x[NSTEP][8];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[s][i] = live ? io_value<QT>(bits[s][i]) * a.q_mul : 0.f;
      if constexpr (!kBF16) {
        uint32_t amk = 0;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) amk = max(amk, abs_key(x[s][i]));
        amk = max(amk, (uint32_t)__shfl_xor((int)amk, 32));
        const float am = __uint_as_float(amk);
        // zero, inf or NaN rows keep e = 0
        const int e = (am > 0.f && am <= 3.402823466e38f) ? 15 - __builtin_amdgcn_frexp_expf(am) : 0;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) x[s][i] = __builtin_ldexpf(x[s][i], e);
        row_c = __builtin_ldexpf(a.scale_log2, -e);
      }
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        if constexpr (QSPLIT && kBF16) {
          const auto sp = split_bf16(x[s]);
          qhi[s] = sp.hi;
          qlo[s] = sp.lo;
        } else if constexpr (QSPLIT) {
          const auto sp = split_f16(x[s]);
          qhi[s] = sp.hi;
          qlo[s] = sp.lo;
        } else if constexpr (!kBF16) {
#pragma unroll
          for (int i = 0; i < 8; ++i) qhi[s][i] = (_Float16)x[s][i];
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

  // ---- page id of page 4t + w of tile t for wave w (the page-id window
  //      advanced every 16 tiles; called once per tile, in order), or -1
  //      for a page not read (past the context, or wholly before the
  //      window: its keys are masked and its V zeroed or weighted by zero)
  auto tile_page = [&](int t) {
    if ((t & 15) == 0 && t > t_first) {
      pid_cur = pid_next;
      pid_next = load_window((t >> 4) + 1);
    }
    const int pi = 4 * t + wave;
    if (pi >= npages || pi < p_first) return -1;
    int pid = __builtin_amdgcn_readlane(pid_cur, pi & 63);
    if ((unsigned)pid >= (unsigned)a.num_pages) { bad = true; pid = 0; }
    return pid;
  };

  // ---- tile copy (16- and 32-bit caches): wave w moves page 4t + w of the
  //      tile (K rows swizzled, V^T block as is) into stage `stg` with LDS
  //      DMA
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  int koff[kI8 ? 1 : L::dmaPerPage];
  // lane l's V^T chunk of a 1 KB block: row l/2 of the block, the chunk
  // that lands in slot l%2
  int voff = 32 * (lane >> 1) + 16 * ((lane & 1) ^ v_swizzle16(lane >> 1));
  if constexpr (!kI8) {
#pragma unroll
    for (int j = 0; j < L::dmaPerPage; ++j) {
      const int byte = 1024 * j + 16 * lane;          // position inside the page's K block
      const int rr = byte / L::kRow, slot = (byte % L::kRow) / 16;
      if constexpr (kF32) koff[j] = rr * L::kRow + ((slot ^ k_swizzle32(rr & 15)) * 16);
      else koff[j] = rr * L::kRow + ((slot ^ k_swizzle<D>(rr)) * 16);
    }
    // fp32 V^T rows are 64 bytes: the swizzle of row d = 16*j + lane/4 does
    // not depend on j
    if constexpr (kF32) voff = 64 * (lane >> 2) + (((lane & 3) ^ v_swizzle32(lane >> 2)) * 16);
  }
  // part j of the copy of page pid into stage stg: K and V^T chunks j
  auto copy_part = [&](int pid, int stg, int j) {
    const long blk = ((long)pid * a.hkv + g) * L::kPageBytes;
    char* lk = lds + stg * L::stage + wave * L::kPageBytes;
    char* lv = lds + stg * L::stage + L::vOff + wave * L::kPageBytes;
    dma16_async(kc + blk + koff[j], lk + 1024 * j);
    dma16_async(vc + blk + 1024 * j + voff, lv + 1024 * j);
  };
  auto issue_tile = [&](int t, int stg) {
    const int pid = tile_page(t);
    if (pid >= 0) {
#pragma unroll
      for (int j = 0; j < L::dmaPerPage; ++j) copy_part(pid, stg, j);
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  int v_exp = -1000;   // one-byte caches: acc holds the output times 2^-(v_exp - 4)

  // ---- pipeline: tile t computes from LDS while tile t+1 is copied in
  auto run_tiles = [&](auto&& compute_tile) {
    issue_tile(t_first, t_first & 1);
    wait_vmcnt0();
    __syncthreads();  // this wave's copies have landed; now every wave's
    for (int t = t_first; t < ntiles; ++t) {
      const char* st = lds + (t & 1) * L::stage;
      const int kb = t * kPrefillTileKeys;
      // every wave computes every tile: a tile past all of a wave's rows is
      // fully masked (p = 0), and branching around it would make the compiler
      // copy the accumulators at each join.  compute_tile calls issue_next
      // (the copy of tile t+1 into the other stage) where the copies' issue
      // best overlaps its own work.
      // The copy is unconditional (no branch between it and the MFMAs it
      // is interleaved with): a page not read, or the tile after the last,
      // copies page 0 instead, into a stage whose keys are then masked
      // (their V zeroed) or never computed on.  issue_next(j) issues part j
      // of L::dmaPerPage.
      const int pid_next = max(tile_page(t + 1), 0);
      auto issue_next = [&](int j) { copy_part(pid_next, (t + 1) & 1, j); };
      compute_tile(st, kb, issue_next);
      wait_vmcnt0();
      __syncthreads();
    }
  };

  // ---- causal and window masks on the S^T registers: register r of half
  //      hf holds key kb + base(hf) + roff(r), roff(r) a constant; keys past
  //      the row's limit, or before its window, get -inf (only tiles that
  //      cross one need the test).  The comparisons are against the row's
  //      bound minus the half's base, so each register costs one compare
  //      with a constant.
  auto apply_masks = [&](f32x16 (&s)[2], int kb, auto base, auto roff) {
    if (kb + 63 > lim_min) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rel = limit - (kb + base(hf));   // largest allowed roff
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (roff(r) > rel) s[hf][r] = -INFINITY;
      }
    }
    if (kb < win_max) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rel = wlo - (kb + base(hf));     // smallest allowed roff
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (roff(r) < rel) s[hf][r] = -INFINITY;
      }
    }
  };
  // ---- lazy running max (log2 units): the accumulator is rescaled only when
  //      a row's max grows by more than 2^8; returns the max to subtract
  auto update_max = [&](float mt) {
    const bool grow = mt > m_run + kLazyRescale;
    if (__any(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) acc[i] *= alpha;
      m_run = m_new;
    }
    return (m_run == -INFINITY) ? 0.f : m_run;
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mt = s[0][0];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[hf][r]);
    return max_xor32(mt);
  };
  // keys at or past the context end, or in pages not read because they lie
  // wholly before the window, may hold anything
  auto edge_tile = [&](int kb) { return kb + 64 > ctx || kb < kPage * p_first; };
  // the register layout of the 16-bit and fp32 paths: the A-operand row
  // rho of S^T reads key 16*(rho/16) + 8*((rho/4)&1) + 4*((rho/8)&1) + rho%4,
  // so register r of half hf holds key 32*hf + 16*(r/8) + 8*hh + r%8
  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);
  auto base16 = [&](int hf) { return 32 * hf + 8 * hh; };
  auto roff16 = [](int r) { return 16 * (r >> 3) + (r & 7); };

  if constexpr (!kI8 && !kF32) {
    // per-lane LDS offsets of the fragment reads
    int kaddr[NSTEP];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
      kaddr[k] = krow * L::kRow + (((2 * k + hh) ^ k_swizzle<D>(krow & 15)) * 16);
    const int vaddr = L::vOff + col * 32 + 16 * (hh ^ v_swizzle16(col));

    // one 64-key tile (keys kb .. kb+63; half hf = pages 2hf and 2hf+1)
    run_tiles([&](const char* st, int kb, auto&& issue_next) {
      // ---- S^T = K * Q^T for both halves
      f32x16 s[2] = {f32x16{}, f32x16{}};
      if constexpr (!QSPLIT) {
        // all K fragment reads first (one LDS latency), then two
        // independent MFMA chains; the next tile's copies are issued while
        // the K reads are in flight
        u32x4 kfr[2][NSTEP];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int k = 0; k < NSTEP; ++k)
            kfr[hf][k] = *reinterpret_cast<const u32x4*>(st + hf * 32 * L::kRow + kaddr[k]);
        // keep the K reads ahead of the MFMAs (the default schedule pairs
        // them and waits for LDS between every two MFMAs); the next tile's
        // copies go in pairs after the first MFMA pairs, issued while the
        // matrix core runs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            s[hf] = mfma32x32x16(__builtin_bit_cast(H8, kfr[hf][k]), qhi[k], s[hf]);
          if (k < L::dmaPerPage) {
            issue_next(k);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < L::dmaPerPage; ++j) issue_next(j);
        // head and remainder of q take 2*NSTEP fragments: one half's K
        // fragments at a time (two MFMAs per fragment hide the second LDS
        // latency), so that both halves' fragments are not live together
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 kfr[NSTEP];
#pragma unroll
          for (int k = 0; k < NSTEP; ++k)
            kfr[k] = *reinterpret_cast<const u32x4*>(st + hf * 32 * L::kRow + kaddr[k]);
#pragma unroll
          for (int k = 0; k < NSTEP; ++k) {
            const H8 kf = __builtin_bit_cast(H8, kfr[k]);
            s[hf] = mfma32x32x16(kf, qhi[k], s[hf]);
            s[hf] = mfma32x32x16(kf, qlo[k], s[hf]);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, NSTEP, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NSTEP, 0);
        }
      }
      // ---- V^T fragments of half hf; out-of-range keys may hold anything
      //      (NaN): their V is zeroed.  Both halves are read here, their
      //      LDS latency hidden behind the softmax; with a split query (two
      //      q fragments live) each half is read as its softmax starts, so
      //      that both halves' fragments are not live together.
      u32x4 vfr[QSPLIT ? 1 : 2][NDB][2];
      auto load_v = [&](int hf, u32x4 (&vf)[NDB][2]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            vf[db][j] = *reinterpret_cast<const u32x4*>(
                st + vaddr + (2 * hf + j) * L::kPageBytes + db * 32 * 32);
        if (edge_tile(kb)) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int key0 = kb + 32 * hf + 16 * j + 8 * hh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool out = key0 + e >= ctx || key0 + e < kPage * p_first;
              const uint32_t m = out ? ((e & 1) ? 0x0000ffffu : 0xffff0000u) : 0xffffffffu;
#pragma unroll
              for (int db = 0; db < NDB; ++db) vf[db][j][e >> 1] &= m;
            }
          }
        }
      };
      if constexpr (!QSPLIT) {
        load_v(0, vfr[0]);
        load_v(1, vfr[QSPLIT ? 0 : 1]);
      }
      // ---- online softmax for query row `col` on raw scores; the
      //      log2e-prescaled scale (positive) is applied inside the
      //      exponent: p = 2^(s*c - m)
      apply_masks(s, kb, base16, roff16);
      const float m_use = update_max(tile_max(s) * row_c);
      float lsum = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (QSPLIT) load_v(hf, vfr[0]);
        H8 p16[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][r], row_c, -m_use));
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
            acc[db] = mfma32x32x16(__builtin_bit_cast(H8, vfr[QSPLIT ? 0 : hf][db][j]), p16[j], acc[db]);
      }
      l_part += lsum;
    });
  } else if constexpr (kF32) {
    // fp32 cache, 32x32x2 fp32 MFMA: k-step s of the QK product pairs lane
    // hh's d = (D/2)*hh + s, so a lane reads one contiguous half of its K
    // row; PV k-step (page pg, e) pairs lane hh's key 16*pg + 8*hh + e, so a
    // lane reads 8 contiguous keys of its V^T row d = 32*db + col per page
    const int kbase = krow * L::kRow;
    const int ksw = k_swizzle32(krow & 15);
    const int vsw = v_swizzle32(col);          // the swizzle of row 32*db + col
    const int vrow = L::vOff + col * 64;
    run_tiles([&](const char* st, int kb, auto&& issue_next) {
#pragma unroll
      for (int j = 0; j < L::dmaPerPage; ++j) issue_next(j);
      // ---- S^T = K * Q^T, the two halves' MFMA chains interleaved
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        f32x4 kf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          kf[hf] = *reinterpret_cast<const f32x4*>(st + hf * 2 * L::kPageBytes + kbase +
                                                   ((((D / 8) * hh + c) ^ ksw) * 16));
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            s[hf] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[hf][e], qf[4 * c + e], s[hf], 0, 0, 0);
      }
      // ---- online softmax on raw scores, P kept in fp32
      apply_masks(s, kb, base16, roff16);
      const float m_use = update_max(tile_max(s) * row_c);
      float lsum = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[hf][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][r], row_c, -m_use));
          lsum += s[hf][r];
        }
      l_part += lsum;
      // ---- O^T += V^T * P^T; out-of-range keys may hold anything (NaN):
      //      their V is zeroed
      const bool edge = edge_tile(kb);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
          const int key0 = kb + 32 * hf + 16 * pg + 8 * hh;
          const int nv = key0 < kPage * p_first ? 0 : ctx - key0;   // in-range keys of the 8
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const char* vp = st + vrow + (2 * hf + pg) * L::kPageBytes + db * 32 * 64;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(vp + (((2 * hh) ^ vsw) * 16));
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(vp + (((2 * hh + 1) ^ vsw) * 16));
            float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            if (edge) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (e >= nv) v[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[e], s[hf][8 * pg + e], acc[db], 0, 0, 0);
          }
        }
    });
  } else {
    // ---- one-byte caches.  Wave w loads the codes of page 4t + w of the
    //      next tile into registers (lane l: D/4 bytes of the K page and two
    //      V^T rows, see kVSwap; lanes 0-7 the page's 16 K and 16 V scales)
    //      while the current tile computes, then converts them, each code
    //      once, to fp16 in the next stage in the 16-bit layout (K rows
    //      swizzled, V^T row halves swapped), zeroes the V of keys past the context or before
    //      the window, stores the scales (those keys' V scales as 0) and the
    //      page's largest V scale.  The compute reads fp16 fragments as the
    //      16-bit path does; register r of half hf holds key
    //      32*hf + 16*(r/8) + 8*hh + r%8, i.e. key 8*hh + r%8 of page
    //      2*hf + r/8.
    constexpr int KQ = D / 64;                      // 16-byte code chunks per lane and page
    // Lane l stages V^T rows l and l + 64 with their halves swapped as in
    // the 16-bit layout (staging writes and fragment reads free of bank
    // conflicts), except with a split query, whose kernel keeps rows 2l and
    // 2l + 1 unswapped: measured, the conflict-free layout speeds the
    // 16-bit-query kernels up by 4-6% and slows the split-query ones (at
    // 256 VGPRs) by 7%
    constexpr bool kVSwap = !QSPLIT;
    auto vrow_of = [&](int i) { return kVSwap ? lane + 64 * i : KQ * lane + i; };
    struct Codes {
      u32x4 k[KQ], v[KQ], sc;
    };
    const char* sc_src =
        reinterpret_cast<const char*>(lane < 4 ? a.k_scales : a.v_scales) + 16 * (lane & 3);
    auto load_codes = [&](int t, Codes& c) {
      const int pid = tile_page(t);
      if (pid >= 0) {
        const long blk = ((long)pid * a.hkv + g) * (long)(kPage * D);
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
          c.k[i] = *reinterpret_cast<const u32x4*>(kc + blk + 16 * (KQ * lane + i));
          c.v[i] = *reinterpret_cast<const u32x4*>(vc + blk + 16 * vrow_of(i));
        }
        if (lane < 8)
          c.sc = *reinterpret_cast<const u32x4*>(sc_src + ((long)pid * a.hkv + g) * (kPage * 4));
      }
    };
    auto stage_codes = [&](int t, int stg, const Codes& c) {
      char* F = lds + stg * L::stage;
      // in-range keys of the page (none for a page not read)
      const int pi = 4 * t + wave;
      const int nv = (pi >= npages || pi < p_first) ? 0 : min(max(ctx - kPage * pi, 0), kPage);
      // K row lane/4 of the page, d = (D/4)*(lane%4) ..: 2*KQ fp16 chunks
      const int kr = lane >> 2;
      char* krow = F + wave * L::kPageBytes + kr * L::kRow;
#pragma unroll
      for (int i = 0; i < KQ; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ch = 2 * KQ * (lane & 3) + 2 * i + h;
          *reinterpret_cast<f16x8*>(krow + ((ch ^ k_swizzle<D>(kr)) * 16)) =
              codes8_to_f16<KV>(u32x2{c.k[i][2 * h], c.k[i][2 * h + 1]});
        }
      // V^T row vrow_of(i) (16 keys), keys at or past nv zeroed, its two
      // 16-byte halves swapped as the 16-bit copy swaps them (kVSwap): the
      // 16 lanes of a write then cover 16 different bank slots
#pragma unroll
      for (int i = 0; i < KQ; ++i) {
        f16x8 lo = codes8_to_f16<KV>(u32x2{c.v[i][0], c.v[i][1]});
        f16x8 hi = codes8_to_f16<KV>(u32x2{c.v[i][2], c.v[i][3]});
        if (nv < kPage) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (e >= nv) lo[e] = (_Float16)0.f;
            if (8 + e >= nv) hi[e] = (_Float16)0.f;
          }
        }
        const int vd = vrow_of(i);
        char* vrow = F + L::vOff + wave * L::kPageBytes + vd * 32;
        const int vsw = kVSwap ? v_swizzle16(vd) : 0;
        *reinterpret_cast<f16x8*>(vrow + 16 * vsw) = lo;
        *reinterpret_cast<f16x8*>(vrow + 16 * (1 ^ vsw)) = hi;
      }
      // scales: lanes 0-3 the K scales of keys 4*lane.., lanes 4-7 the V
      // scales of keys 4*(lane-4)..; the page's largest in-range V scale
      float pm = 0.f;
      if (lane < 8) {
        f32x4 x = __builtin_bit_cast(f32x4, c.sc);
        if (lane >= 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (4 * (lane - 4) + e >= nv) x[e] = 0.f;
            pm = fmaxf(pm, x[e]);
          }
        }
        *reinterpret_cast<f32x4*>(F + L::sOff + 128 * wave + 16 * lane) = x;
      }
      pm = fmaxf(pm, __shfl_xor(pm, 1));
      pm = fmaxf(pm, __shfl_xor(pm, 2));
      if (lane == 4) reinterpret_cast<float*>(F + L::pmOff)[wave] = pm;
    };

    // K fragment k of this lane: row krow, chunk (2k + hh) ^ swz (the swizzle
    // is below 16, so it only flips the low bits of the chunk index)
    const int kbase = krow * L::kRow;
    const int kswz = k_swizzle<D>(krow & 15);
    const int vaddr = L::vOff + col * 32 + 16 * (kVSwap ? (hh ^ v_swizzle16(col)) : hh);
    const int saddr = L::sOff + 32 * hh;

    auto compute_tile = [&](const char* st, int kb, auto&& issue_next) {
      // ---- S^T = K * Q^T, one half at a time; the next tile's code loads
      //      are issued while the first half's K reads are in flight
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 kfr[NSTEP];
#pragma unroll
        for (int k = 0; k < NSTEP; ++k)
          kfr[k] = *reinterpret_cast<const u32x4*>(st + hf * 32 * L::kRow + kbase +
                                                   (((2 * k + hh) ^ kswz) * 16));
        if (hf == 0) issue_next();
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
          const f16x8 kf = __builtin_bit_cast(f16x8, kfr[k]);
          s[hf] = mfma32x32x16(kf, qhi[k], s[hf]);
          if constexpr (QSPLIT) s[hf] = mfma32x32x16(kf, qlo[k], s[hf]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NSTEP, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, (QSPLIT ? 2 : 1) * NSTEP, 0);
      }
      // ---- scores in log2 units: K scale times c * 2^-e
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const char* sp = st + saddr + 128 * (2 * hf + j);
          const f32x4 k0 = *reinterpret_cast<const f32x4*>(sp);
          const f32x4 k1 = *reinterpret_cast<const f32x4*>(sp + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[hf][8 * j + e] *= k0[e] * row_c;
            s[hf][8 * j + 4 + e] *= k1[e] * row_c;
          }
        }
      apply_masks(s, kb, base16, roff16);
      const float m_use = update_max(tile_max(s));
      // ---- V normaliser from the four pages' largest in-range V scales
      const f32x4 pm = *reinterpret_cast<const f32x4*>(st + L::pmOff);
      const float vmax = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
      const int et = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(vmax));
      if (et > v_exp + 2) {
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] = __builtin_ldexpf(acc[i][r], v_exp - et);
        v_exp = et;
      }
      // ---- P (times the normalised V scale) and O^T += V^T * P^T, one
      //      16-key page at a time
      float lsum = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 vfr[NDB];
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            vfr[db] = *reinterpret_cast<const u32x4*>(
                st + vaddr + (2 * hf + j) * L::kPageBytes + db * 32 * 32);
          const char* sp = st + saddr + 128 * (2 * hf + j) + 64;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(sp);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(sp + 16);
          f16x8 p16;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(s[hf][8 * j + e] - m_use);
            lsum += p;
            const float vsc = e < 4 ? v0[e] : v1[e - 4];
            p16[e] = (_Float16)mul_zero_wins(p, __builtin_ldexpf(vsc, 4 - v_exp));
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32x32x16(__builtin_bit_cast(f16x8, vfr[db]), p16, acc[db]);
        }
      l_part += lsum;
    };

    // ---- pipeline: tile t computes from one stage while tile t+1's codes
    //      are in flight to registers; they are staged into the other stage
    //      after the compute, one barrier per tile
    Codes cr = {};
    load_codes(t_first, cr);
    stage_codes(t_first, t_first & 1, cr);
    __syncthreads();
    for (int t = t_first; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      compute_tile(lds + (t & 1) * L::stage, t * kPrefillTileKeys, [&]() {
        if (more) load_codes(t + 1, cr);
      });
      if (more) stage_codes(t + 1, (t + 1) & 1, cr);
      __syncthreads();
    }
  }
  bad = __syncthreads_or(bad);

  const float l_run = sum_xor32(l_part);
  if (!live) return;
  // a NaN score makes the row sum NaN while the max skips it: NaN, not zero
  const float inv = (bad || l_run != l_run) ? NAN : (l_run > 0.f ? 1.f / l_run : 0.f);
  const int o_exp = v_exp - 4;   // one-byte caches
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
        if constexpr (kI8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_ldexpf(v[e], o_exp);
        }
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
