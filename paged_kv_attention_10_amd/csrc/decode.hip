// Batched paged decode: one query token per sequence attends over its
// 16-token pages with GQA (TinyLoop "Current Status", tables "Core
// inference" row "Generation", "KV cache modes" row "Paged attention",
// "Model architecture support" row "GQA").
//
// Work split.  A workgroup of 4 waves owns one (sequence b, KV head g, tile
// of up to 16 query heads, context split).  The context is walked in tiles
// of 32 tokens (two pages); the tiles a split actually has are divided
// evenly over the four waves in contiguous runs.  The split's page ids are
// loaded into LDS in the same round trip as the context length and the
// query (lane i of a wave then holds the i-th page id of its run); tiles
// stream through a ring of register buffers, the next tile's loads in
// flight while the current one computes.  Each wave keeps its own running
// max / sum / accumulator (the max updated lazily: the accumulator is
// rescaled only when it grows by more than 2^8); the four waves merge in
// LDS.  A sequence whose context needs several splits writes normalised
// partials and a log2-sum-exp per split.  With at most kMergeInKernelSplits
// splits the split that finishes last merges them inside the launch: the
// partials go out as agent-coherent stores (visible across the XCDs'
// separate L2 caches without writing back or invalidating a whole L2, which
// a fenced version did and measured 3-7x slower), each split counts itself
// in on an epoch-tagged arrival counter once its stores have completed, and
// the last reads the partials back with agent-coherent loads.  Longer plans
// merge with decode_reduce_kernel on the same stream, whose one-wave-per-row
// grid reads many splits in one round trip.
//
// Fused decode step (paged_attn_decode_append).  The wave whose tiles hold
// position ctx - 1 loads the sequence's new K/V row with its first tiles,
// converts it as the append rounds, stashes it in the workgroup's merge area
// of LDS (free while tiles stream), stores it to the cache and patches it
// into the tile it streams, so the attention sees exactly the stored values.
// When the partition grid needs more than one round of workgroups, the
// in-kernel V column stores measured slower than a launch of their own, and
// append_step_kernel stores the rows before the plain decode instead.
//
// MFMA mapping (16x16 tiles, wave64).  Scores are computed transposed,
// S^T = K * Q^T: A = K (row = token), B = Q^T (column = query head of the
// group, padded to 16).  The output layout puts, in lane (c + 16*j), the
// scores of head c for the 8 consecutive tile tokens 8j..8j+7 - exactly the
// B-operand layout PV needs, so O^T = V^T * P^T runs with no data movement:
// A = V^T (row = d), B = P^T.  The V page is stored token-innermost, so every
// A-operand load of V^T is a contiguous 8-token run.  The A-operand row of
// K for tile token tau is chosen so that this holds: MFMA u (0/1), row r
// loads token 8*(r/4) + 4*u + r%4.
//
// Precision.  bf16/fp16 KV use the 16x16x32 MFMA; the fp32 query and the
// fp32 probabilities are each split into a 16-bit head plus remainder and
// multiplied twice, so products carry ~16 significant bits.  int8 codes are
// converted exactly to fp16; the per-token K scale multiplies the score and
// the per-token V scale folds into the probability.  fp32 KV uses the fp32
// 16x16x4 MFMA.  exp is exp2 of a log2e-prescaled score.
#include <mutex>

#include "decode_body.h"

namespace pkv {

// Decode workgroups a CU holds at once (the register budget: 256 VGPRs).
constexpr int kDecodeWorkgroupsPerCu = 2;

template <int D, int KV, bool FUSE>
__global__ __launch_bounds__(64 * kDecodeWaves, kDecodeWorkgroupsPerCu) void decode_partition_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DecodeSmem<D>::total];
  decode_partition_body<D, KV, FUSE>(a, smem, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Decode step with many rounds of workgroups: one wave per (sequence, KV
// head) stores the new token's K row and V column at position ctx - 1
// (through the block table), converted as in the fused path, before the
// plain decode runs.  Rows with an invalid context or page id store nothing.
template <int D, int KV>
__global__ __launch_bounds__(256) void append_step_kernel(DecodeArgs a) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long)a.batch * a.hkv) return;
  const int b = (int)(w / a.hkv), g = (int)(w - (long)b * a.hkv);
  NewRaw<D> nr;
  load_new_token<D, KV>(nr, a, b, g, lane);   // independent of the slot: in flight meanwhile
  bool bad = false;
  const int ctx = checked_ctx(a.context_lens[b], a.max_context_len, a.max_blocks, bad);
  if (bad || ctx < 1) return;
  const int page = a.block_tables[(long)b * a.max_blocks + ((ctx - 1) >> 4)];
  if ((unsigned)page >= (unsigned)a.num_pages) return;
  __shared__ __attribute__((aligned(16))) char stash[4][kStashBytes<D>];
  stash_new_token<D, KV>(stash[threadIdx.x >> 6], nr, a, g, page, (ctx - 1) & 15, true, lane);
}

// The fused decode step stores the new token from inside the partition
// kernel, which measured faster while the grid is one round of workgroups;
// with more rounds the in-kernel V column stores cost more than a separate
// launch (fp16 decode of 384 sequences x 12 heads: 134 us fused against
// 115 + 5 us).
constexpr long kFuseMaxWorkgroups = 512;

template <int D, int KV>
static void launch_decode(const DecodeArgs& a, pkv_stream_t stream) {
  dim3 grid(a.nsplits, a.hkv * a.head_tiles, a.batch);
  const bool fuse = a.k_new && (long)grid.x * grid.y * grid.z <= kFuseMaxWorkgroups;
  if (a.k_new && !fuse)
    hipLaunchKernelGGL((append_step_kernel<D, KV>), dim3((unsigned)(((long)a.batch * a.hkv + 3) / 4)),
                       dim3(256), 0, (hipStream_t)stream, a);
  if (!fuse)
    hipLaunchKernelGGL((decode_partition_kernel<D, KV, false>), grid, dim3(64 * kDecodeWaves), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<D, KV, true>), grid, dim3(64 * kDecodeWaves), 0,
                       (hipStream_t)stream, a);
  if (a.nsplits > 1 && !a.merge_cnt)
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(a.hq, a.batch), dim3(64), 0,
                       (hipStream_t)stream, a);
}

template <int D>
static void dispatch_kv(int kv, const DecodeArgs& a, pkv_stream_t stream) {
  switch (kv) {
    case PKV_F32: launch_decode<D, PKV_F32>(a, stream); break;
    case PKV_BF16: launch_decode<D, PKV_BF16>(a, stream); break;
    case PKV_F16: launch_decode<D, PKV_F16>(a, stream); break;
    case PKV_I8: launch_decode<D, PKV_I8>(a, stream); break;
    default: launch_decode<D, PKV_FP8>(a, stream); break;
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attn_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                                    int head_dim, int max_context_len, int window) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      !head_dim_built(head_dim) || max_context_len < 0 || window < 0 ||
      !decode_span_supported(max_context_len, window))
    return 0;
  DecodePlan p = plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, window);
  return decode_workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, p, true).total;
}

// Checks and launch shared by paged_attn_decode and paged_attn_decode_append
// (k_new null for the former).
static int decode_call(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                       const float* k_scales, const float* v_scales, int kv_dtype,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, int max_context_len, int batch,
                       int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                       int num_pages, float scale, int window, void* out, int out_dtype,
                       void* workspace, size_t workspace_bytes, const void* k_new,
                       const void* v_new, int new_dtype, pkv_stream_t stream) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKV_ERR_INVALID_ARG;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      num_pages <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      (long)max_context_len > (long)max_blocks_per_seq * PKV_PAGE_SIZE || batch > 65535 ||
      window < 0)
    return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(q_dtype) || !io_dtype_ok(out_dtype) || !kv_dtype_ok(kv_dtype) || !scale_ok(scale))
    return PKV_ERR_INVALID_ARG;
  if (kv_scaled(kv_dtype) != (k_scales != nullptr) || kv_scaled(kv_dtype) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim) ||
      !decode_span_supported(max_context_len, window))
    return PKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(block_tables) || !aligned16(context_lens) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)) ||
      (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
    return PKV_ERR_MISALIGNED;

  DecodePlan p = plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, window);
  DecodeWorkspace ws = decode_workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, p, true);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (workspace && !aligned16(workspace)) return PKV_ERR_MISALIGNED;

  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = nullptr;
  a.out = out;
  char* wsb = static_cast<char*>(workspace);
  a.part_o = ws.total ? reinterpret_cast<float*>(wsb + ws.part_o_offset) : nullptr;
  a.part_lse = ws.total ? reinterpret_cast<float*>(wsb + ws.part_lse_offset) : nullptr;
  a.merge_cnt = ws.total && p.nsplits <= kMergeInKernelSplits
                    ? reinterpret_cast<unsigned long long*>(wsb + ws.cnt_offset)
                    : nullptr;
  a.epoch = next_merge_epoch();
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  a.max_blocks = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_tiles = p.head_tiles;
  a.num_pages = num_pages;
  a.tiles_per_split = p.tiles_per_split;
  a.nsplits = p.nsplits;
  a.window = window;
  a.scale_log2 = scale * kLog2e;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  a.k_store = const_cast<void*>(k_cache);
  a.v_store = const_cast<void*>(v_cache);
  a.ks_store = const_cast<float*>(k_scales);
  a.vs_store = const_cast<float*>(v_scales);

  clear_launch_error();
  if (head_dim == 64) dispatch_kv<64>(kv_dtype, a, stream);
  else dispatch_kv<128>(kv_dtype, a, stream);
  return launch_status();
}

extern "C" int paged_attn_decode(const void* q, int q_dtype, const void* k_cache,
                                 const void* v_cache, const float* k_scales,
                                 const float* v_scales, int kv_dtype,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, int batch,
                                 int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                 int num_pages, float scale, int window, void* out, int out_dtype,
                                 void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
  return decode_call(q, q_dtype, k_cache, v_cache, k_scales, v_scales, kv_dtype, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, page_size, num_pages, scale, window, out, out_dtype,
                     workspace, workspace_bytes, nullptr, nullptr, PKV_F32, stream);
}

extern "C" int paged_attn_decode_append(const void* q, int q_dtype, const void* k_new,
                                        const void* v_new, int new_dtype, void* k_cache,
                                        void* v_cache, float* k_scales, float* v_scales,
                                        int kv_dtype, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* context_lens,
                                        int max_context_len, int batch, int num_q_heads,
                                        int num_kv_heads, int head_dim, int page_size,
                                        int num_pages, float scale, int window, void* out,
                                        int out_dtype, void* workspace, size_t workspace_bytes,
                                        pkv_stream_t stream) {
  if (!k_new || !v_new) return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(new_dtype) || !kv_dtype_ok(kv_dtype)) return PKV_ERR_INVALID_ARG;
  return decode_call(q, q_dtype, k_cache, v_cache, k_scales, v_scales, kv_dtype, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, page_size, num_pages, scale, window, out, out_dtype,
                     workspace, workspace_bytes, k_new, v_new, new_dtype, stream);
}

// ------------------------------------------------ allocation-free decode
// Split partials of paged_attn_decode_noalloc live in this file-scope device
// array instead of a caller workspace.  Each GPU holds its own copy (at its
// own address) from when the library's code is loaded on it until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: host code uses only the address hipGetSymbolAddress returns
// for the device, looked up once per device and kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The device address of `scratch` on the device `stream` runs on (the
// current device for the null stream), looked up with that device current
// on the first call for it.
int scratch_address(pkv_stream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PKV_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PKV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return PKV_ERR_HIP;
    if (e != hipSuccess || !p) return PKV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int paged_attn_decode_noalloc(const void* q, int q_dtype, const void* k_cache,
                                         const void* v_cache, const float* k_scales,
                                         const float* v_scales, int kv_dtype,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int max_context_len,
                                         int batch, int num_q_heads, int num_kv_heads,
                                         int head_dim, int page_size, int num_pages, float scale,
                                         int window, void* out, int out_dtype,
                                         pkv_stream_t stream) {
  // the split partials the plan needs (0 for shapes decode_call rejects)
  const size_t need = paged_attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                        head_dim, max_context_len, window);
  if (need > kNoAllocScratchBytes) return PKV_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(stream, &ws);
    if (st != PKV_OK) return st;
  }
  return decode_call(q, q_dtype, k_cache, v_cache, k_scales, v_scales, kv_dtype, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, page_size, num_pages, scale, window, out, out_dtype,
                     ws, need > 0 ? kNoAllocScratchBytes : 0, nullptr, nullptr, PKV_F32, stream);
}
