// Mixed batch: prefill chunks and decode tokens in one varlen call
// (Tiny-LLM "Project Status", supported features: chunked prefill/decode
// scheduling over a paged KV cache; TinyLoop "Current Status", table "Model
// architecture support", row "Chunked prefill").  The semantics are those of
// paged_attn_prefill_chunk: chunk row i of sequence b sits at position
// P_b + i and attends to [0, P_b + i]; a decode token is a chunk of one.
//
// One launch holds two kinds of workgroups.  The first part of the grid is
// the prefill row blocks that hold rows, found on the device (see
// mixed_prefill_item) so that the part is sized by the token count rather
// than by batch x row blocks, most of which a decode-heavy batch leaves
// empty.  The second part is the decode kernel's partitions, which take
// exactly the single-token sequences (their query and output rows mapped
// through cu_q_lens): a decode token is walked by four waves with
// 16-query-head MFMA tiles instead of occupying a 128-row prefill block.
// When the batch holds only short chunks the one-token rows are split
// across the context as in paged_attn_decode; with long chunks present they
// take the fewest splits their context allows.  Both kinds share the
// workgroup's LDS buffer and its register budget; split partials are merged
// as in a decode call (inside the launch by the last split for plans of up
// to eight splits, else by the decode reduce kernel afterwards).

#include <algorithm>

#include "decode_body.h"
#include "prefill_body.h"

namespace pkv {

template <int D, int KV>
constexpr int mixed_lds_bytes() {
  return 2 * PrefillLds<D, KV>::stage > DecodeSmem<D>::total ? 2 * PrefillLds<D, KV>::stage
                                                             : DecodeSmem<D>::total;
}

static_assert(64 * kDecodeWaves == 256, "both kinds of workgroup have 256 threads");

// The prefill part of a mixed launch holds only as many workgroups as row
// blocks can hold rows (host bound: KV heads x (ceil(tokens x G / 128) +
// batch), since the chunks' lengths sum to the token count), and each
// workgroup finds its row block here: the id-th item of the list of row
// blocks that hold rows, KV head fastest, then the sequences in order, each
// sequence's row blocks heaviest (last) first.  Every workgroup derives the
// same list from cu_q_lens with prefix sums of the sequences' row-block
// counts, 256 sequences per pass.  A workgroup past the list's end gets
// rb = nrowblocks (no work).  Called by all 256 threads; uses 1 KB of `sh`,
// free again on return.
__device__ __forceinline__ void mixed_prefill_item(const PrefillArgs& a, int* sh, int id, int& b,
                                                   int& g, int& rb) {
  const int t = threadIdx.x;
  const int j = id / a.hkv;          // the (sequence, row block) item
  g = id - j * a.hkv;
  b = 0;
  rb = a.nrowblocks;
  int* scan = sh;                    // [256] inclusive prefix within the pass
  int* found = sh + 256;             // sequence and row block of item j
  if (t == 0) found[0] = -1;
  int base = 0;                      // items before the pass
  for (int p0 = 0; p0 < a.batch; p0 += 256) {
    const int s = p0 + t;
    int n = 0;
    if (s < a.batch) {
      // the rows prefill_body gives the sequence (the same clamping)
      int C = a.cu_q_lens[s + 1] - a.cu_q_lens[s];
      C = C < 0 ? 0 : min(C, a.max_q_len);
      const int rows = (a.skip_single && C == 1) ? 0 : C * a.group;
      n = (rows + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
    }
    scan[t] = n;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = t >= off ? scan[t - off] : 0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    const int incl = base + scan[t];
    if (n > 0 && j >= incl - n && j < incl) {
      found[0] = s;
      found[1] = incl - 1 - j;       // heavier (later) row blocks first
    }
    base += scan[255];
    __syncthreads();
    if (found[0] >= 0 || base > j) break;   // the same in every thread
  }
  if (found[0] >= 0) {
    b = found[0];
    rb = found[1];
  }
  __syncthreads();
}

template <int D, int KV, bool QSPLIT>
__global__ __launch_bounds__(256, (prefill_workgroups_per_cu<D, KV>()))
void mixed_kernel(DecodeArgs da, PrefillArgs pa, int n_prefill) {
  __shared__ __attribute__((aligned(1024))) char lds[mixed_lds_bytes<D, KV>()];
  const int id = blockIdx.x;
  if (id < n_prefill) {
    // the prefill kernel's ranked order when it applies (at most 256
    // sequences, contexts that differ, at most two rounds of row blocks),
    // else the list order
    int b = 0, g = 0, rb = 0;
    if (pa.batch > kPrefillSortMaxBatch || !prefill_item(pa, reinterpret_cast<int*>(lds), id, b, g, rb))
      mixed_prefill_item(pa, reinterpret_cast<int*>(lds), id, b, g, rb);
    prefill_body<D, KV, QSPLIT>(pa, lds, b, g, rb);
  } else {
    const int j = id - n_prefill;
    const int ny = da.hkv * da.head_tiles;
    const int split = j % da.nsplits, r = j / da.nsplits;
    decode_partition_body<D, KV>(da, lds, split, r % ny, r / ny);
  }
}

template <int D, int KV>
static void launch_mixed(const DecodeArgs& da, const PrefillArgs& pa, int n_prefill, int n_decode,
                         pkv_stream_t stream) {
  const dim3 grid(n_prefill + n_decode);
  bool split = false;
  if constexpr (KV != PKV_F32) split = prefill_q_split(KV, pa.q_dtype);
  if (split)
    hipLaunchKernelGGL((mixed_kernel<D, KV, KV != PKV_F32>), grid, dim3(256), 0, (hipStream_t)stream,
                       da, pa, n_prefill);
  else
    hipLaunchKernelGGL((mixed_kernel<D, KV, false>), grid, dim3(256), 0, (hipStream_t)stream, da, pa,
                       n_prefill);
  if (da.nsplits > 1 && !da.merge_cnt)
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(da.hq, da.batch), dim3(64), 0,
                       (hipStream_t)stream, da);
}

template <int D>
static void dispatch_mixed(int kv, const DecodeArgs& da, const PrefillArgs& pa, int n_prefill,
                           int n_decode, pkv_stream_t stream) {
  switch (kv) {
    case PKV_BF16: launch_mixed<D, PKV_BF16>(da, pa, n_prefill, n_decode, stream); break;
    case PKV_F16: launch_mixed<D, PKV_F16>(da, pa, n_prefill, n_decode, stream); break;
    case PKV_I8: launch_mixed<D, PKV_I8>(da, pa, n_prefill, n_decode, stream); break;
    case PKV_FP8: launch_mixed<D, PKV_FP8>(da, pa, n_prefill, n_decode, stream); break;
    default: launch_mixed<D, PKV_F32>(da, pa, n_prefill, n_decode, stream); break;
  }
}

// Split plan of the one-token rows.  With long chunks in the batch
// (max_q_len >= kMixedLongChunk) the prefill row blocks set the critical
// path, so the one-token rows take the fewest splits their context allows (a
// split would only add the merge); otherwise the one-token rows
// dominate and are planned as a decode call.
constexpr int kMixedLongChunk = 128;
static DecodePlan mixed_plan(int batch, int num_q_heads, int num_kv_heads, int max_q_len,
                             int max_context_len, int window) {
  return max_q_len >= kMixedLongChunk
             ? plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, window, 0)
             : plan_decode(batch, num_q_heads, num_kv_heads, max_context_len, window);
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attn_mixed_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                                   int head_dim, int max_q_len, int max_context_len,
                                                   int window) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      !head_dim_built(head_dim) || max_q_len < 0 || max_context_len < 0 || window < 0 ||
      !decode_span_supported(max_context_len, window))
    return 0;
  return decode_workspace_layout(batch, num_q_heads, num_kv_heads, head_dim,
                                 mixed_plan(batch, num_q_heads, num_kv_heads, max_q_len,
                                            max_context_len, window),
                                 true).total;
}

extern "C" int paged_attn_mixed(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                                const float* k_scales, const float* v_scales, int kv_dtype,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* cu_q_lens,
                                int num_tokens, int max_q_len, int max_context_len, int batch,
                                int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                int num_pages, float scale, int window, void* out, int out_dtype,
                                void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
  if (!k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens ||
      ((!q || !out) && num_tokens > 0))
    return PKV_ERR_INVALID_ARG;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      num_pages <= 0 || max_blocks_per_seq <= 0 || num_tokens < 0 || max_q_len < 0 ||
      max_context_len < 0 || max_q_len > max_context_len || batch > 65535 || window < 0 ||
      (long)max_context_len > (long)max_blocks_per_seq * PKV_PAGE_SIZE)
    return PKV_ERR_INVALID_ARG;
  if (!io_dtype_ok(q_dtype) || !io_dtype_ok(out_dtype) || !kv_dtype_ok(kv_dtype) || !scale_ok(scale))
    return PKV_ERR_INVALID_ARG;
  if (kv_scaled(kv_dtype) != (k_scales != nullptr) || kv_scaled(kv_dtype) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim) ||
      !decode_span_supported(max_context_len, window))
    return PKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(block_tables) || !aligned16(context_lens) || !aligned16(cu_q_lens) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)))
    return PKV_ERR_MISALIGNED;
  if (num_tokens == 0 || max_q_len == 0) return PKV_OK;

  const DecodePlan p = mixed_plan(batch, num_q_heads, num_kv_heads, max_q_len, max_context_len, window);
  const DecodeWorkspace ws = decode_workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, p, true);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (workspace && !aligned16(workspace)) return PKV_ERR_MISALIGNED;

  DecodeArgs da;
  da.q = q;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.k_scales = k_scales;
  da.v_scales = v_scales;
  da.block_tables = block_tables;
  da.context_lens = context_lens;
  da.cu_q_lens = cu_q_lens;
  da.out = out;
  char* wsb = static_cast<char*>(workspace);
  da.part_o = ws.total ? reinterpret_cast<float*>(wsb + ws.part_o_offset) : nullptr;
  da.part_lse = ws.total ? reinterpret_cast<float*>(wsb + ws.part_lse_offset) : nullptr;
  // decode rows merge as in a decode call: inside the launch for plans of up
  // to kMergeInKernelSplits splits, else with the reduce kernel
  da.merge_cnt = ws.total && p.nsplits <= kMergeInKernelSplits
                     ? reinterpret_cast<unsigned long long*>(wsb + ws.cnt_offset)
                     : nullptr;
  da.epoch = next_merge_epoch();
  da.q_dtype = q_dtype;
  da.out_dtype = out_dtype;
  da.max_blocks = max_blocks_per_seq;
  da.max_context_len = max_context_len;
  da.batch = batch;
  da.hq = num_q_heads;
  da.hkv = num_kv_heads;
  da.group = num_q_heads / num_kv_heads;
  da.head_tiles = p.head_tiles;
  da.num_pages = num_pages;
  da.tiles_per_split = p.tiles_per_split;
  da.nsplits = p.nsplits;
  da.window = window;
  da.scale_log2 = scale * kLog2e;
  da.k_new = da.v_new = nullptr;
  da.new_dtype = PKV_F32;
  da.k_store = da.v_store = nullptr;
  da.ks_store = da.vs_store = nullptr;

  PrefillArgs pa;
  pa.q = q;
  pa.k_cache = k_cache;
  pa.v_cache = v_cache;
  pa.k_scales = k_scales;
  pa.v_scales = v_scales;
  pa.block_tables = block_tables;
  pa.context_lens = context_lens;
  pa.cu_q_lens = cu_q_lens;
  pa.out = out;
  pa.q_dtype = q_dtype;
  pa.out_dtype = out_dtype;
  pa.max_blocks = max_blocks_per_seq;
  pa.max_context_len = max_context_len;
  pa.max_q_len = max_q_len;
  pa.batch = batch;
  pa.hq = num_q_heads;
  pa.hkv = num_kv_heads;
  pa.group = num_q_heads / num_kv_heads;
  pa.num_pages = num_pages;
  pa.nrowblocks = ceil_div((long)max_q_len * pa.group, kPrefillRowsPerBlock);
  const ScaleForm sf = scale_form(scale, kLog2e);
  pa.scale_log2 = sf.c;
  pa.q_xor = sf.q_xor;
  pa.q_and = sf.q_and;
  pa.q_mul = sf.q_mul;
  pa.skip_single = 1;
  pa.window = window;
  if (pa.nrowblocks > 65535) return PKV_ERR_INVALID_ARG;

  // no row block can hold work when every chunk has at most one token;
  // otherwise at most KV heads x (ceil(tokens x G / 128) + batch) row
  // blocks hold rows (the chunk lengths sum to num_tokens)
  const long n_prefill =
      max_q_len > 1 ? std::min((long)batch * num_kv_heads * pa.nrowblocks,
                               (long)num_kv_heads * (ceil_div((long)num_tokens * pa.group,
                                                              kPrefillRowsPerBlock) + batch))
                    : 0;
  const long n_decode = (long)p.nsplits * num_kv_heads * p.head_tiles * batch;
  if (n_prefill + n_decode > 0x7fffffffL) return PKV_ERR_INVALID_ARG;

  clear_launch_error();
  if (head_dim == 64) dispatch_mixed<64>(kv_dtype, da, pa, (int)n_prefill, (int)n_decode, stream);
  else dispatch_mixed<128>(kv_dtype, da, pa, (int)n_prefill, (int)n_decode, stream);
  return launch_status();
}
