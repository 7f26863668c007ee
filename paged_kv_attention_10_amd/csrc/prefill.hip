// Chunked causal prefill over a paged prefix (TinyLoop "Current Status",
// table "Model architecture support", rows "Chunked prefill" and "GQA";
// Tiny-LLM "Project Status", supported features: chunked prefill with a
// paged KV cache).  Chunk row i of sequence b sits at position P_b + i and
// attends to keys [0, P_b + i].
//
// Rows.  The query rows of one (sequence, KV head) are the chunk positions
// times the G query heads that share the KV head, flattened head-fastest:
// row r -> position r / G, head g*G + r % G.  A workgroup of 4 waves owns 128
// consecutive rows, a wave 32.  The workgroup walks the key range its rows
// need in tiles of 64 keys (4 pages).  Wave w copies page w of the next tile
// (its K block and its V^T block) straight from HBM into LDS with
// global_load_lds (no register staging) while all four waves compute on
// the current tile, so the G heads of a position and the 32-row blocks of
// the chunk share every load; one barrier per 64 keys.  Page ids come from a
// 64-page window held one per lane and read with readlane.
//
// LDS (per stage, double-buffered): K as 64 key rows of D elements whose
// 16-byte chunks are XOR-swizzled by the row's position in its page, and
// V^T as four page blocks [d][16 keys] as they lie in HBM except that the
// two 16-byte halves of the rows with bit 3 of d set trade places.  Both
// fragment reads below are free of bank conflicts on gfx950 (64 banks of 4
// bytes; a 16-byte read is served 16 lanes at a time, and each group of 16
// lanes touches 16 different 16-byte slots of the 256-byte bank space:
// measured, the LDS bank-conflict cycles of the C4 prefill went from a third
// of the LDS busy cycles to none).
//
// MFMA mapping (32x32x16, wave64), per 32-key half of a tile: S^T = K * Q^T
// with A = K (row = key), B = Q^T (column = query row).  The A-operand row
// rho reads key 16*(rho/16) + 8*((rho/4)&1) + 4*((rho/8)&1) + rho%4, which
// makes lane (c + 32*h) hold, for query row c, the scores of keys 8h..8h+7
// of the half's first page (registers 0-7) and of its second page
// (registers 8-15): the B-operand layout of O^T = V^T * P^T with no data
// movement.  Each V^T A-operand read is a contiguous 8-key run of one d row.
// The causal mask runs only on halves that cross a row's limit.
//
// Softmax.  exp2 of log2e-prescaled scores with a lazily updated running
// max: the accumulator is rescaled only when a row's max grows by more than
// 2^8 (the stale max cancels in the final normalisation, and probabilities
// stay below 256).
//
// Precision: q and K/V in the cache's 16-bit type (an fp32 or other-typed
// q is split into head + remainder and multiplied twice), P rounded to the
// 16-bit type for PV (the normaliser sums those same rounded values, two
// per packed dot product), fp32 accumulation.  int8 / FP8 caches (Tiny-LLM
// "Classifier receipt", KV cache point: INT8 or FP8 KV cache): wave w loads
// the codes of page w of the next tile into registers (no DMA) and, after
// the current tile's compute, converts each code once, exactly, to fp16 into
// the next stage in the 16-bit layout, with the page's scales beside it; q
// is scaled by a power of two and rounded to fp16 (split for an fp32 q), the
// K scale goes on the score and the V scale on the fp16 probability
// (prefill_body.h states the ranges).
// fp32 caches: the 32x32x2 fp32 MFMA with P kept in fp32 (two stages of
// 64 KB at head_dim 128: one workgroup per CU).
#include "prefill_body.h"

namespace pkv {

template <int D, int KV, bool QSPLIT>
__global__ __launch_bounds__(256, (prefill_workgroups_per_cu<D, KV>())) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * PrefillLds<D, KV>::stage];
  int b = blockIdx.x, g = blockIdx.y;
  int rb = a.nrowblocks - 1 - (int)blockIdx.z;   // heavier (later) row blocks first
  const long id = blockIdx.x + (long)a.batch * (blockIdx.y + (long)a.hkv * blockIdx.z);
  if (a.batch <= kPrefillSortMaxBatch && (long)a.batch * a.hkv * a.nrowblocks <= kPrefillSortMaxGrid)
    prefill_item(a, reinterpret_cast<int*>(lds), id, b, g, rb);
  prefill_body<D, KV, QSPLIT>(a, lds, b, g, rb);
}

template <int D, int KV>
static void dispatch_prefill_q(const PrefillArgs& a, pkv_stream_t stream) {
  dim3 grid(a.batch, a.hkv, a.nrowblocks);
  if constexpr (KV != PKV_F32) {
    if (prefill_q_split(KV, a.q_dtype)) {
      hipLaunchKernelGGL((prefill_kernel<D, KV, true>), grid, dim3(256), 0, (hipStream_t)stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((prefill_kernel<D, KV, false>), grid, dim3(256), 0, (hipStream_t)stream, a);
}

template <int D>
static void dispatch_prefill(int kv, const PrefillArgs& a, pkv_stream_t stream) {
  switch (kv) {
    case PKV_BF16: dispatch_prefill_q<D, PKV_BF16>(a, stream); break;
    case PKV_F16: dispatch_prefill_q<D, PKV_F16>(a, stream); break;
    case PKV_I8: dispatch_prefill_q<D, PKV_I8>(a, stream); break;
    case PKV_FP8: dispatch_prefill_q<D, PKV_FP8>(a, stream); break;
    default: dispatch_prefill_q<D, PKV_F32>(a, stream); break;
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attn_prefill_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                                     int head_dim, int max_q_len,
                                                     int max_context_len, int window) {
  (void)batch; (void)num_q_heads; (void)num_kv_heads; (void)head_dim; (void)max_q_len;
  (void)max_context_len; (void)window;
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
                                        int window, void* out, int out_dtype, void* workspace,
                                        size_t workspace_bytes, pkv_stream_t stream) {
  (void)workspace; (void)workspace_bytes;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens ||
      ((!q || !out) && num_tokens > 0))
    return PKV_ERR_INVALID_ARG;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      num_pages <= 0 || max_blocks_per_seq <= 0 || num_tokens < 0 || max_q_len < 0 ||
      max_context_len < 0 || max_q_len > max_context_len || window < 0 ||
      (long)max_context_len > (long)max_blocks_per_seq * PKV_PAGE_SIZE)
    return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(q_dtype) || !io_dtype_ok(out_dtype) || !kv_dtype_ok(kv_dtype) || !scale_ok(scale))
    return PKV_ERR_INVALID_ARG;
  if (kv_scaled(kv_dtype) != (k_scales != nullptr) || kv_scaled(kv_dtype) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(block_tables) || !aligned16(context_lens) || !aligned16(cu_q_lens) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)))
    return PKV_ERR_MISALIGNED;
  if (num_tokens == 0 || max_q_len == 0) return PKV_OK;

  PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
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
  const ScaleForm sf = scale_form(scale, kLog2e);
  a.scale_log2 = sf.c;
  a.q_xor = sf.q_xor;
  a.q_and = sf.q_and;
  a.q_mul = sf.q_mul;
  a.skip_single = 0;
  a.window = window;
  if (a.nrowblocks > 65535 || batch > 0x7fffffff) return PKV_ERR_INVALID_ARG;

  clear_launch_error();
  if (head_dim == 64) dispatch_prefill<64>(kv_dtype, a, stream);
  else dispatch_prefill<128>(kv_dtype, a, stream);
  return launch_status();
}
