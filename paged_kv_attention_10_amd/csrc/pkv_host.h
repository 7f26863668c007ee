// Host-side helpers shared by the pkv entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>

#include "../../include/pkv.h"

namespace pkv {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool head_dim_built(int d) { return d == 64 || d == 128; }
inline bool io_dtype_ok(int dt) { return dt == PKV_F32 || dt == PKV_BF16 || dt == PKV_F16; }
__host__ __device__ inline bool kv_scaled(int dt) { return dt == PKV_I8 || dt == PKV_FP8; }
inline bool kv_dtype_ok(int dt) { return io_dtype_ok(dt) || kv_scaled(dt); }
// Whether the prefill splits the query into head + remainder: a 16-bit
// cache multiplies q in its own type (exact when q has that type), an
// int8 / FP8 cache in fp16 (exact after a power-of-two row scaling for a
// bf16 or fp16 q), an fp32 cache in fp32.
inline bool prefill_q_split(int kv, int q_dtype) {
  if (kv == PKV_F32) return false;   // fp32 MFMA: q exact in fp32
  return kv_scaled(kv) ? q_dtype == PKV_F32 : q_dtype != kv;
}
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
inline bool scale_ok(float scale) { return std::isfinite(scale); }

// The prefill's form of a softmax scale: a positive exponent factor and the
// query's sign (see PrefillArgs).
struct ScaleForm {
  float c;
  uint32_t q_xor, q_and;
  float q_mul;
};
inline ScaleForm scale_form(float scale, float log2e) {
  ScaleForm f;
  f.c = (scale != 0.f ? (scale < 0.f ? -scale : scale) : 1.f) * log2e;
  f.q_xor = scale < 0.f ? 0x80008000u : 0u;
  f.q_and = scale != 0.f ? 0xffffffffu : 0u;
  f.q_mul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  return f;
}

// Clears any stale error, so the check after a launch sees only ours.
inline void clear_launch_error() { (void)hipGetLastError(); }
inline int launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// How a decode call is cut into work: contexts are processed in tiles of 32
// tokens (two pages); a workgroup of 4 waves owns `tiles_per_split` tiles of
// one (sequence, KV head, head tile), its waves an equal share of the tiles
// the split actually holds; `nsplits` workgroups cover the longest context.
// A pure function of the shapes, so the workspace query and the launch agree.
struct DecodePlan {
  int head_tiles;
  int tiles_per_split;
  int nsplits;
};

constexpr int kDecodeTileTokens = 32;
// Waves of a decode workgroup (8 measured slower).
constexpr int kDecodeWaves = 4;
// A wave's page ids are held one per lane, so a wave takes at most 32 tiles.
constexpr int kDecodeMaxTilesPerSplit = 32 * kDecodeWaves;
// The merge kernel holds one split per lane.
constexpr int kDecodeMaxSplits = 64;
// Longest context a decode call takes.
constexpr long kDecodeMaxContext = (long)kDecodeMaxSplits * kDecodeMaxTilesPerSplit * kDecodeTileTokens;
// A split takes at least two tiles per wave: a call of a few short
// contexts (a handful of sequences of a few hundred tokens) then runs as
// one split per sequence and skips the merge launch, which costs more than
// the splits would save.
constexpr int kDecodeMinTilesPerSplit = 2 * kDecodeWaves;
// Aim for about this many workgroups per call: one per CU of a 256-CU
// MI355X.  Fewer, longer splits measured faster than more, shorter ones:
// every split pays a few dependent memory round trips before its first
// tile streams and leaves a partial for the merge.
constexpr long kDecodeTargetWorkgroups = 256;

// Tiles a sequence's keys span at most: its whole context, or with a
// sliding window of `window` tokens the window, which may start anywhere in
// a tile.
inline int decode_tiles(int max_context_len, int window) {
  int t = max_context_len > 0 ? ceil_div(max_context_len, kDecodeTileTokens) : 1;
  if (window > 0) {
    const int tw = (window - 1) / kDecodeTileTokens + 2;
    if (tw < t) t = tw;
  }
  return t;
}

// Whether the split plan covers that span (at most kDecodeMaxContext tokens).
inline bool decode_span_supported(int max_context_len, int window) {
  return (long)decode_tiles(max_context_len, window) * kDecodeTileTokens <= kDecodeMaxContext;
}

// target_workgroups = 0 asks for the fewest splits the context allows (a
// mixed batch, where the prefill row blocks set the critical path and a
// decode split would only add the merge).
inline DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len,
                              int window, long target_workgroups = kDecodeTargetWorkgroups) {
  DecodePlan p;
  int group = num_q_heads / num_kv_heads;
  p.head_tiles = ceil_div(group, 16);
  int tiles_max = decode_tiles(max_context_len, window);
  long units = (long)batch * num_kv_heads * p.head_tiles;
  long want = (target_workgroups + units - 1) / units;
  if (want < 1) want = 1;
  int tps = ceil_div(tiles_max, want);
  tps = ceil_div(tps, kDecodeWaves) * kDecodeWaves;
  if (tps < kDecodeMinTilesPerSplit) tps = kDecodeMinTilesPerSplit;
  if (tps > kDecodeMaxTilesPerSplit) tps = kDecodeMaxTilesPerSplit;
  p.tiles_per_split = tps;
  p.nsplits = ceil_div(tiles_max, tps);   // <= kDecodeMaxSplits for spans <= kDecodeMaxContext
  return p;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Plans of up to this many splits merge inside the partition launch (the
// last split reads every partial in one round trip of eight); longer ones
// use decode_reduce_kernel.  C2 (two splits): fused step 44.5 -> 42.7 us; a
// 16k-64k-token plan of many splits measured 1.4% slower merged in-kernel.
constexpr int kMergeInKernelSplits = 8;

// Epochs of the in-kernel merge's arrival counters: distinct for every call
// in the process (56 bits).
inline unsigned long long next_merge_epoch() {
  static std::atomic<unsigned long long> epoch{1};
  return epoch.fetch_add(1, std::memory_order_relaxed) & ((1ull << 56) - 1);
}

// Workspace of a split decode: normalised partial outputs and their
// log2-sum-exp, [batch][num_q_heads][nsplits] rows.  Contents on entry do
// not matter.
// Split partials (o, then lse) and, for the in-kernel merge, one 64-bit
// arrival counter per (sequence, KV head x head tile).
struct DecodeWorkspace {
  size_t part_o_offset, part_lse_offset, cnt_offset, total;
};

inline DecodeWorkspace decode_workspace_layout(int batch, int num_q_heads, int num_kv_heads,
                                               int head_dim, const DecodePlan& p,
                                               bool merge_counters) {
  DecodeWorkspace w = {0, 0, 0, 0};
  if (p.nsplits <= 1) return w;
  size_t rows = (size_t)batch * num_q_heads * p.nsplits;
  w.part_o_offset = 0;
  w.part_lse_offset = align_up(rows * head_dim * sizeof(float), 256);
  w.cnt_offset = w.part_lse_offset + align_up(rows * sizeof(float), 256);
  w.total = w.cnt_offset +
            (merge_counters ? align_up((size_t)batch * num_kv_heads * p.head_tiles * 8, 256) : 0);
  return w;
}

}  // namespace pkv
