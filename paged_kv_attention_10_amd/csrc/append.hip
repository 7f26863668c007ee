// Append: new K/V tokens are written into the paged pool through a slot
// mapping and converted to the cache dtype (TinyLoop "Current Status", table
// "KV cache modes", rows "Paged attention" and "INT8 KV cache"; Tiny-LLM
// "Project Status", dtype-contract paragraph on a separate KV-cache dtype),
// optionally with rotary position embedding on K and the queries (same
// page, table "Model architecture support", row "RoPE": every forward path,
// configurable theta).
//
// Work split.  Small plain appends (up to 4096 (token, KV head) rows, e.g.
// a decode step) take one wave per (token, KV head).  Otherwise a row is one
// head vector of one token (a K row, a V row, or
// with RoPE a query row); a thread owns a 16-element segment of a row and
// loads it with 16-byte loads, so a row of D elements takes D/16
// consecutive lanes.  K/V workgroups take as many whole tokens as their 256
// threads cover (at most 16); K segments go to the token's page row with
// 16-byte stores, V values are gathered in LDS as [head][d][token] and
// stored with consecutive lanes on consecutive tokens of a (head, d) column
// of the token-innermost V page.  With RoPE on the queries, query rows are
// rotated in place by workgroups of their own after the K/V workgroups.  A
// workgroup builds the RoPE angle table of its tokens once in LDS.  int8
// takes the absmax of the (token, head) row with a shuffle over the row's
// lanes, then scale = absmax/127 (IEEE fp32 division) and
// code = clamp(rint(x/scale), -127, 127) with ties to even.  The absmax is
// taken on the bit patterns so that a NaN element gives a NaN scale (and
// codes 0): attention over such a token comes out NaN instead of reading
// plausible codes.
//
// RoPE: coordinate pair i turns by pos * f_i radians, f_i = theta^(-2i/D)
// held as an fp32 number (the power evaluated in double and rounded once,
// the usual storage of a frequency table; computed on the host per call).
// The angle, its cosine and sine and the rotation
// (a, b) -> (a cos - b sin, b cos + a sin) are evaluated in double without
// contraction; the result is rounded once to fp32 and then converted as an
// fp32 input would be.  PKV_ROPE_HALF pairs coordinate i with i + D/2, so a
// segment holds elements [8s, 8s+8) and their partners [D/2+8s, D/2+8s+8);
// PKV_ROPE_INTERLEAVED pairs 2i with 2i+1 and a segment is 16 consecutive
// elements.  Either way segment s holds pairs [8s, 8s+8).
#include <math.h>

#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

constexpr int kSegElems = 16;
constexpr int kAppendThreads = 256;
constexpr int kMaxRopePairs = 64;   // D/2 for the largest head_dim built

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  float* k_scales;
  float* v_scales;
  const int32_t* positions;   // RoPE only
  void* q;                    // RoPE only, may be null
  int new_dtype, cache_dtype, q_dtype;
  int num_tokens, hkv, hq;    // hq = 0 when no query rows are rotated
  int style;
  int kv_tokens_per_block;    // whole tokens a K/V workgroup covers
  int q_tokens_per_block;     // whole tokens a query workgroup covers
  int kv_blocks;              // K/V workgroups first, then query workgroups
  int v_via_lds;              // V columns transposed through LDS before the store
  long num_slots;
  float inv_freq[kMaxRopePairs];
};

constexpr int kMaxTokensPerBlock = 16;
constexpr int kVTileBytes = 8192;

// Elements e0..e0+7 and e1..e1+7 of a row in a 16- or 32-bit dtype: their
// values and storage bits (an fp32 input keeps its bits; a 16-bit one's
// value bits as fp32).  Both 16- or 32-byte loads issue before either
// converts.
__device__ __forceinline__ void load8x2(const void* row, int dtype, int e0, int e1, float* x,
                                        uint32_t* raw) {
  with_io_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    uint32_t b[16];
    io_bits_vec<8, DT>(row, e0, b);
    io_bits_vec<8, DT>(row, e1, b + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[j] = io_value<DT>(b[j]);
      raw[j] = DT == PKV_F32 ? b[j] : __float_as_uint(x[j]);
    }
  });
}

// Storage bits of one element in a 16- or 32-bit dtype.
__device__ __forceinline__ uint32_t storage_bits(int dtype, float x, uint32_t raw) {
  return dtype == PKV_F32 ? raw : dtype == PKV_BF16 ? f32_to_bf16_bits(x) : f32_to_f16_bits(x);
}

// Eight consecutive elements of a row (fp32, bf16 or fp16 storage).
__device__ __forceinline__ void store8(void* row, int dtype, int e0, const float* x, const uint32_t* raw) {
  if (dtype == PKV_F32) {
    u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint32_t*>(row) + e0);
    p[0] = u32x4{raw[0], raw[1], raw[2], raw[3]};
    p[1] = u32x4{raw[4], raw[5], raw[6], raw[7]};
  } else {
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = storage_bits(dtype, x[j], raw[j]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(row) + e0) =
        u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

// (cos, sin) of every (token, pair) angle of the workgroup's tokens.
template <int D>
__device__ __forceinline__ void build_rope_table(const AppendArgs& a, long tok0, int ntok, double2* cs) {
  constexpr int PAIRS = D / 2;
  for (int e = threadIdx.x; e < ntok * PAIRS; e += kAppendThreads) {
    const long tok = tok0 + e / PAIRS;
    if (tok < a.num_tokens) {
      const double ang = (double)a.positions[tok] * (double)a.inv_freq[e % PAIRS];
      double sn, cn;
      sincos(ang, &sn, &cn);
      cs[e] = double2{cn, sn};
    }
  }
}

// Rotates the 8 pairs a segment holds (pairs [8s, 8s+8) of the table row).
__device__ __forceinline__ void rotate16(float* x, uint32_t* raw, const double2* tab, bool split) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ia = split ? j : 2 * j, ib = split ? j + 8 : 2 * j + 1;
    const double2 c = tab[j];
    const double xa = x[ia], xb = x[ib];
    double ra, rb;
    {
#pragma clang fp contract(off)
      const double ac = xa * c.x, bs = xb * c.y, bc = xb * c.x, as = xa * c.y;
      ra = ac - bs;
      rb = bc + as;
    }
    x[ia] = (float)ra;
    x[ib] = (float)rb;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) raw[j] = __float_as_uint(x[j]);
}

// Workgroups that rotate query rows in place (RoPE with queries only).
template <int D>
__device__ void query_block(const AppendArgs& a, long qb, double2* cs) {
  constexpr int NSEG = D / kSegElems;
  const int tpb = a.q_tokens_per_block;
  const long tok0 = qb * tpb;
  const int segs = a.hq * NSEG;
  const int es = a.q_dtype == PKV_F32 ? 4 : 2;
  const bool split = a.style == PKV_ROPE_HALF;
  // item t: token lt, head h, segment s; its row and first column
  auto item = [&](int t, int& lt, int& s, char*& row, int& c0, int& c1) {
    lt = t / segs;
    const int rem = t - lt * segs;
    const int h = rem / NSEG;
    s = rem - h * NSEG;
    c0 = split ? 8 * s : kSegElems * s;
    c1 = split ? D / 2 + 8 * s : kSegElems * s + 8;
    row = static_cast<char*>(a.q) + ((tok0 + lt) * a.hq + h) * D * es;
  };
  // the first pass's query segment is loaded before the angle table is
  // built (the same memory round trip as the positions)
  const int t_first = threadIdx.x;
  float x0[16];
  uint32_t raw0[16];
  if (t_first < tpb * segs && tok0 + t_first / segs < a.num_tokens) {
    int lt, s, c0, c1;
    char* row;
    item(t_first, lt, s, row, c0, c1);
    load8x2(row, a.q_dtype, c0, c1, x0, raw0);
  }
  build_rope_table<D>(a, tok0, tpb, cs);
  __syncthreads();
  for (int t = t_first; t < tpb * segs; t += kAppendThreads) {
    int lt, s, c0, c1;
    char* row;
    item(t, lt, s, row, c0, c1);
    if (tok0 + lt >= a.num_tokens) continue;
    float x[16];
    uint32_t raw[16];
    if (t == t_first) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x[j] = x0[j];
        raw[j] = raw0[j];
      }
    } else {
      load8x2(row, a.q_dtype, c0, c1, x, raw);
    }
    rotate16(x, raw, cs + lt * (D / 2) + 8 * s, split);
    store8(row, a.q_dtype, c0, x, raw);
    store8(row, a.q_dtype, c1, x + 8, raw + 8);
  }
}

// Workgroups that append K (rotated with RoPE) and V for whole tokens.  A
// thread owns a 16-element segment of a K or V row.  K segments are stored
// straight into the token's page row.  V columns are token-innermost in the
// page, so a V segment is 16 elements 32 B apart; with `v_via_lds` the
// converted V values are first gathered in LDS as [head][d][token] and then
// stored with consecutive lanes on consecutive tokens, so the tokens of one
// page that share a workgroup write one contiguous run per (head, d).
template <int D, bool ROPE>
__device__ void kv_block(const AppendArgs& a, long kb, double2* cs, unsigned char* vt,
                         int64_t* s_slot) {
  constexpr int NSEG = D / kSegElems;
  const int tpb = a.kv_tokens_per_block;
  const long tok0 = kb * tpb;
  const int segs = 2 * a.hkv * NSEG;
  const int items = tpb * segs;
  // item t: token lt, row (K heads, then V heads), 16-element segment s
  auto item = [&](int t, int& lt, int& row, int& s) {
    lt = t / segs;
    const int rem = t - lt * segs;
    row = rem / NSEG;
    s = rem - row * NSEG;
  };
  auto seg_cols = [&](int row, int s, int& c0, int& c1) {
    const bool split = ROPE && row < a.hkv && a.style == PKV_ROPE_HALF;
    c0 = split ? 8 * s : kSegElems * s;
    c1 = split ? D / 2 + 8 * s : kSegElems * s + 8;
  };
  auto load_item = [&](int t, float* x, uint32_t* raw) {
    int lt, row, s, c0, c1;
    item(t, lt, row, s);
    seg_cols(row, s, c0, c1);
    const bool is_v = row >= a.hkv;
    const int h = is_v ? row - a.hkv : row;
    const char* src = static_cast<const char*>(is_v ? a.v_new : a.k_new) +
                      ((tok0 + lt) * a.hkv + h) * D * (a.new_dtype == PKV_F32 ? 4 : 2);
    load8x2(src, a.new_dtype, c0, c1, x, raw);
  };
  // the first pass's input segment does not depend on the slot: loaded
  // before the barrier, in the same memory round trip as the slots
  float x0[16];
  uint32_t raw0[16];
  const int t_first = threadIdx.x;
  if (t_first < items && tok0 + t_first / segs < a.num_tokens) load_item(t_first, x0, raw0);
  if (threadIdx.x < tpb) {
    const long tok = tok0 + threadIdx.x;
    int64_t slot = tok < a.num_tokens ? a.slots[tok] : -1;
    if (slot >= a.num_slots) slot = -1;   // outside the pool: skipped like padding
    s_slot[threadIdx.x] = slot < 0 ? -1 : slot;
  }
  if (ROPE) build_rope_table<D>(a, tok0, tpb, cs);
  __syncthreads();

  const int ces = a.cache_dtype == PKV_F32 ? 4 : kv_scaled(a.cache_dtype) ? 1 : 2;
  for (int t = t_first; t < items; t += kAppendThreads) {
    // a row's NSEG lanes are consecutive and aligned and share a token, so
    // the int8 shuffle stays inside a group of lanes active together
    int lt, row, s, c0, c1;
    item(t, lt, row, s);
    const int64_t slot = s_slot[lt];
    if (slot < 0) continue;
    seg_cols(row, s, c0, c1);
    const bool is_v = row >= a.hkv;
    const int h = is_v ? row - a.hkv : row;
    const long page = slot / kPage;
    const int off = (int)(slot - page * kPage);
    const bool rotate = ROPE && !is_v;
    const bool split = rotate && a.style == PKV_ROPE_HALF;
    float x[16];
    uint32_t raw[16];
    if (t == t_first) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x[j] = x0[j];
        raw[j] = raw0[j];
      }
    } else {
      load_item(t, x, raw);
    }
    if (rotate) rotate16(x, raw, cs + lt * (D / 2) + 8 * s, split);

    const long head = page * a.hkv + h;
    uint32_t bits[16];
    if (kv_scaled(a.cache_dtype)) {
      uint32_t amk = 0u;   // absmax as a sort key: a NaN element makes the scale NaN
#pragma unroll
      for (int j = 0; j < 16; ++j) amk = max(amk, abs_key(x[j]));
#pragma unroll
      for (int m = 1; m < NSEG; m <<= 1) amk = max(amk, (uint32_t)__shfl_xor((int)amk, m));
      const bool i8 = a.cache_dtype == PKV_I8;
      const float sc = code8_scale(__uint_as_float(amk), i8);
#pragma unroll
      for (int j = 0; j < 16; ++j) bits[j] = code8(x[j], sc, i8);
      if (s == 0) (is_v ? a.v_scales : a.k_scales)[head * kPage + off] = sc;
      if (!is_v) {
        int8_t* dst = static_cast<int8_t*>(a.k_cache) + (head * kPage + off) * D;
        *reinterpret_cast<u32x2*>(dst + c0) =
            u32x2{bits[0] | bits[1] << 8 | bits[2] << 16 | bits[3] << 24,
                  bits[4] | bits[5] << 8 | bits[6] << 16 | bits[7] << 24};
        *reinterpret_cast<u32x2*>(dst + c1) =
            u32x2{bits[8] | bits[9] << 8 | bits[10] << 16 | bits[11] << 24,
                  bits[12] | bits[13] << 8 | bits[14] << 16 | bits[15] << 24};
        continue;
      }
    } else {
      if (!is_v) {
        char* dst = static_cast<char*>(a.k_cache) + (head * kPage + off) * D * ces;
        store8(dst, a.cache_dtype, c0, x, raw);
        store8(dst, a.cache_dtype, c1, x + 8, raw + 8);
        continue;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) bits[j] = storage_bits(a.cache_dtype, x[j], raw[j]);
    }
    // V: 16 consecutive d (never rotated), c0 = 16 s
    if (a.v_via_lds) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = (h * D + c0 + j) * tpb + lt;
        if (ces == 4) reinterpret_cast<uint32_t*>(vt)[i] = bits[j];
        else if (ces == 2) reinterpret_cast<uint16_t*>(vt)[i] = (uint16_t)bits[j];
        else vt[i] = (unsigned char)bits[j];
      }
    } else {
      char* dst = static_cast<char*>(a.v_cache) + ((head * D + c0) * kPage + off) * ces;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        char* p = dst + j * kPage * ces;
        if (ces == 4) *reinterpret_cast<uint32_t*>(p) = bits[j];
        else if (ces == 2) *reinterpret_cast<uint16_t*>(p) = (uint16_t)bits[j];
        else *reinterpret_cast<unsigned char*>(p) = (unsigned char)bits[j];
      }
    }
  }
  if (!a.v_via_lds) return;
  __syncthreads();
  // consecutive lanes: consecutive tokens of one (head, d) column
  for (int u = threadIdx.x; u < tpb * a.hkv * D; u += kAppendThreads) {
    const int lt = u % tpb, hd = u / tpb;
    const int64_t slot = s_slot[lt];
    if (slot < 0) continue;
    const int h = hd / D, d = hd - h * D;
    const long page = slot / kPage;
    const int off = (int)(slot - page * kPage);
    const long di = ((page * a.hkv + h) * D + d) * kPage + off;
    if (ces == 4) static_cast<uint32_t*>(a.v_cache)[di] = reinterpret_cast<const uint32_t*>(vt)[u];
    else if (ces == 2) static_cast<uint16_t*>(a.v_cache)[di] = reinterpret_cast<const uint16_t*>(vt)[u];
    else static_cast<unsigned char*>(a.v_cache)[di] = vt[u];
  }
}

// Small appends (a decode step's new tokens): one wave per (token, KV head)
// moves the token's K row and V row, each lane D/64 consecutive elements.
// Its chain per token is short and its waves spread over many CUs, which
// beats the segment kernel's LDS staging below a few thousand (token, head)
// rows.  No RoPE (that path shares angle tables across a token's heads).
// The lane's D/64 elements of one new row: values and storage bits (an
// fp32 input keeps its bits).
template <int D>
struct RowIn {
  float x[D / 64];
  uint32_t raw[D / 64];
};
template <int D>
__device__ __forceinline__ RowIn<D> load_row(const AppendArgs& a, const void* src, long row, int lane) {
  constexpr int PER = D / 64;
  RowIn<D> r;
  with_io_dtype(a.new_dtype, [&](auto ndt) {
    constexpr int NT = decltype(ndt)::value;
    uint32_t bits[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) bits[e] = io_bits<NT>(src, row * D + lane * PER + e);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      r.x[e] = io_value<NT>(bits[e]);
      r.raw[e] = NT == PKV_F32 ? bits[e] : __float_as_uint(r.x[e]);
    }
  });
  return r;
}
template <int D>
__device__ __forceinline__ void row_append(const AppendArgs& a, const RowIn<D>& in, void* cache,
                                           float* scales, long page, int off, int g, bool is_v,
                                           int lane) {
  constexpr int PER = D / 64;
  const float* x = in.x;
  const uint32_t* raw = in.raw;
  const long head = page * a.hkv + g;
  auto dst_index = [&](int d) -> long {
    return is_v ? (head * D + d) * kPage + off : (head * kPage + off) * D + d;
  };
  if (kv_scaled(a.cache_dtype)) {
    uint32_t amk = 0u;   // absmax as a sort key: a NaN element makes the scale NaN
#pragma unroll
    for (int e = 0; e < PER; ++e) amk = max(amk, abs_key(x[e]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amk = max(amk, (uint32_t)__shfl_xor((int)amk, m));
    const bool i8 = a.cache_dtype == PKV_I8;
    const float sc = code8_scale(__uint_as_float(amk), i8);
#pragma unroll
    for (int e = 0; e < PER; ++e)
      static_cast<uint8_t*>(cache)[dst_index(lane * PER + e)] = (uint8_t)code8(x[e], sc, i8);
    if (lane == 0) scales[head * kPage + off] = sc;
    return;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const long di = dst_index(lane * PER + e);
    if (a.cache_dtype == PKV_F32) static_cast<uint32_t*>(cache)[di] = raw[e];
    else static_cast<uint16_t*>(cache)[di] = (uint16_t)storage_bits(a.cache_dtype, x[e], raw[e]);
  }
}

template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_rows_kernel(AppendArgs a) {
  const long w = (long)blockIdx.x * (kAppendThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long)a.num_tokens * a.hkv) return;
  const long tok = w / a.hkv;
  const int g = (int)(w - tok * a.hkv);
  const long row = tok * a.hkv + g;
  // the new rows do not depend on the slot: loaded in the same memory round
  // trip as it
  const RowIn<D> kin = load_row<D>(a, a.k_new, row, lane);
  const RowIn<D> vin = load_row<D>(a, a.v_new, row, lane);
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= a.num_slots) return;
  const long page = slot / kPage;
  const int off = (int)(slot - page * kPage);
  row_append<D>(a, kin, a.k_cache, a.k_scales, page, off, g, false, lane);
  row_append<D>(a, vin, a.v_cache, a.v_scales, page, off, g, true, lane);
}

// (token, KV head) rows up to which a plain append takes the row kernel.
constexpr long kRowAppendMaxRows = 4096;

// Consecutive workgroup ids go to different XCDs (and L2s); remap them so
// that runs of consecutive K/V workgroups (neighbouring tokens, often one
// page) share an XCD.
__device__ __forceinline__ long xcd_grouped(long id, long n) {
  const long x = id % 8, i = id / 8, q = n / 8, r = n % 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int D, bool ROPE>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  __shared__ double2 cs[ROPE ? kMaxTokensPerBlock * D / 2 : 1];   // (cos, sin) per (token, pair)
  __shared__ __attribute__((aligned(16))) unsigned char vt[kVTileBytes];
  __shared__ int64_t s_slot[kMaxTokensPerBlock];
  if (ROPE && (long)blockIdx.x >= a.kv_blocks) {
    query_block<D>(a, blockIdx.x - a.kv_blocks, cs);
    return;
  }
  kv_block<D, ROPE>(a, xcd_grouped(blockIdx.x, a.kv_blocks), cs, vt, s_slot);
}

// Shared checks and launch of both entry points.
static int append_launch(AppendArgs& a, int head_dim, bool rope, pkv_stream_t stream) {
  if (!rope && (long)a.num_tokens * a.hkv <= kRowAppendMaxRows) {
    const long blocks = ((long)a.num_tokens * a.hkv + kAppendThreads / 64 - 1) / (kAppendThreads / 64);
    clear_launch_error();
    if (head_dim == 64)
      hipLaunchKernelGGL(append_rows_kernel<64>, dim3((unsigned)blocks), dim3(kAppendThreads), 0,
                         (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL(append_rows_kernel<128>, dim3((unsigned)blocks), dim3(kAppendThreads), 0,
                         (hipStream_t)stream, a);
    return launch_status();
  }
  const int nseg = head_dim / kSegElems;
  auto tokens_per_block = [](long segs) {
    long t = kAppendThreads / segs;
    return (int)(t < 1 ? 1 : t > kMaxTokensPerBlock ? kMaxTokensPerBlock : t);
  };
  a.kv_tokens_per_block = tokens_per_block(2L * a.hkv * nseg);
  const int ces = a.cache_dtype == PKV_F32 ? 4 : kv_scaled(a.cache_dtype) ? 1 : 2;
  a.v_via_lds = (long)a.kv_tokens_per_block * a.hkv * head_dim * ces <= kVTileBytes &&
                a.kv_tokens_per_block > 1;
  const long kvb = ((long)a.num_tokens + a.kv_tokens_per_block - 1) / a.kv_tokens_per_block;
  long qb = 0;
  if (a.hq > 0) {
    a.q_tokens_per_block = tokens_per_block((long)a.hq * nseg);
    qb = ((long)a.num_tokens + a.q_tokens_per_block - 1) / a.q_tokens_per_block;
  } else {
    a.q_tokens_per_block = 1;
  }
  if (kvb + qb > 0x7fffffffL) return PKV_ERR_INVALID_ARG;
  a.kv_blocks = (int)kvb;
  const dim3 grid((unsigned)(kvb + qb)), block(kAppendThreads);
  clear_launch_error();
  if (head_dim == 64) {
    if (rope) hipLaunchKernelGGL((append_kernel<64, true>), grid, block, 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((append_kernel<64, false>), grid, block, 0, (hipStream_t)stream, a);
  } else {
    if (rope) hipLaunchKernelGGL((append_kernel<128, true>), grid, block, 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((append_kernel<128, false>), grid, block, 0, (hipStream_t)stream, a);
  }
  return launch_status();
}

static void append_args_common(AppendArgs& a, const void* k_new, const void* v_new, int new_dtype,
                               const int64_t* slot_mapping, int num_tokens, void* k_cache,
                               void* v_cache, float* k_scales, float* v_scales, int cache_dtype,
                               int num_pages, int num_kv_heads) {
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.positions = nullptr;
  a.q = nullptr;
  a.new_dtype = new_dtype;
  a.cache_dtype = cache_dtype;
  a.q_dtype = PKV_F32;
  a.num_tokens = num_tokens;
  a.hkv = num_kv_heads;
  a.hq = 0;
  a.style = PKV_ROPE_HALF;
  a.num_slots = (long)num_pages * PKV_PAGE_SIZE;
  for (int i = 0; i < kMaxRopePairs; ++i) a.inv_freq[i] = 0.f;
}

}  // namespace pkv

using namespace pkv;

extern "C" int paged_kv_append(const void* k_new, const void* v_new, int new_dtype,
                               const int64_t* slot_mapping, int num_tokens, void* k_cache,
                               void* v_cache, float* k_scales, float* v_scales, int cache_dtype,
                               int num_pages, int num_kv_heads, int head_dim, int page_size,
                               pkv_stream_t stream) {
  if (num_tokens < 0 || num_pages <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(new_dtype) || !kv_dtype_ok(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (kv_scaled(cache_dtype) != (k_scales != nullptr) || kv_scaled(cache_dtype) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return PKV_ERR_MISALIGNED;
  AppendArgs a;
  append_args_common(a, k_new, v_new, new_dtype, slot_mapping, num_tokens, k_cache, v_cache,
                     k_scales, v_scales, cache_dtype, num_pages, num_kv_heads);
  return append_launch(a, head_dim, false, stream);
}

extern "C" int paged_kv_append_rope(const void* k_new, const void* v_new, int new_dtype,
                                    const int64_t* slot_mapping, const int32_t* positions,
                                    int num_tokens, void* q, int q_dtype, int num_q_heads,
                                    float rope_theta, int rope_style, void* k_cache, void* v_cache,
                                    float* k_scales, float* v_scales, int cache_dtype, int num_pages,
                                    int num_kv_heads, int head_dim, int page_size,
                                    pkv_stream_t stream) {
  if (num_tokens < 0 || num_pages <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(new_dtype) || !kv_dtype_ok(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (kv_scaled(cache_dtype) != (k_scales != nullptr) || kv_scaled(cache_dtype) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (rope_style != PKV_ROPE_HALF && rope_style != PKV_ROPE_INTERLEAVED) return PKV_ERR_INVALID_ARG;
  if (!(rope_theta > 0.f) || !isfinite(rope_theta)) return PKV_ERR_INVALID_ARG;
  if (q && (num_q_heads <= 0 || !io_dtype_ok(q_dtype))) return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !positions || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)) ||
      (q && !aligned16(q)) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) ||
      (reinterpret_cast<uintptr_t>(positions) & 3u))
    return PKV_ERR_MISALIGNED;
  AppendArgs a;
  append_args_common(a, k_new, v_new, new_dtype, slot_mapping, num_tokens, k_cache, v_cache,
                     k_scales, v_scales, cache_dtype, num_pages, num_kv_heads);
  a.positions = positions;
  a.q = q;
  a.q_dtype = q ? q_dtype : PKV_F32;
  a.hq = q ? num_q_heads : 0;
  a.style = rope_style;
  // pair frequencies theta^(-2i/D): the power in double, rounded once to fp32
  for (int i = 0; i < head_dim / 2; ++i)
    a.inv_freq[i] = (float)pow((double)rope_theta, (-2.0 * i) / head_dim);
  return append_launch(a, head_dim, true, stream);
}
