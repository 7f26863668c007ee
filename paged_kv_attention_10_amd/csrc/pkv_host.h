// Host-side helpers shared by the pkv entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool head_dim_built(int d) { return d == 64 || d == 128; }
inline bool io_dtype_ok(int dt) { return dt == PKV_F32 || dt == PKV_BF16 || dt == PKV_F16; }
inline bool kv_dtype_ok(int dt) { return io_dtype_ok(dt) || dt == PKV_I8; }
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Clears any stale error, so the check after a launch sees only ours.
inline void clear_launch_error() { (void)hipGetLastError(); }
inline int launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// How a decode call is cut into work: contexts are processed in tiles of 32
// tokens (two pages); a workgroup of 4 waves owns `tiles_per_split` tiles of
// one (sequence, KV head, head tile); `nsplits` workgroups cover the
// longest context.  Pure function of the shapes, so the workspace query and
// the launch agree.
struct DecodePlan {
  int head_tiles;
  int tiles_per_split;
  int nsplits;
};

constexpr int kDecodeTileTokens = 32;
constexpr int kDecodeWaves = 4;
// Aim for about this many workgroups per call: four per CU on a 256-CU
// MI355X, so short and long sequences interleave across the chip.
constexpr long kDecodeTargetWorkgroups = 1024;

inline DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len) {
  DecodePlan p;
  int group = num_q_heads / num_kv_heads;
  p.head_tiles = ceil_div(group, 16);
  int tiles_max = max_context_len > 0 ? ceil_div(max_context_len, kDecodeTileTokens) : 1;
  long units = (long)batch * num_kv_heads * p.head_tiles;
  long want = (kDecodeTargetWorkgroups + units - 1) / units;
  if (want < 1) want = 1;
  int tps = ceil_div(tiles_max, want);
  if (tps < kDecodeWaves) tps = kDecodeWaves;
  tps = ceil_div(tps, kDecodeWaves) * kDecodeWaves;
  p.tiles_per_split = tps;
  p.nsplits = ceil_div(tiles_max, tps);
  return p;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, const DecodePlan& p) {
  if (p.nsplits <= 1) return 0;
  size_t rows = (size_t)batch * num_q_heads * p.nsplits;
  return align_up(rows * head_dim * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

}  // namespace pkv
