/*
 * pkv.h - attention over a paged KV cache on MI355X (gfx950), C ABI.
 *
 * The operation: softmax(q K^T * scale) V over a KV cache held in fixed
 * 16-token pages that each sequence indexes through its row of a block table
 * (TinyLoop "Current Status", table "KV cache modes", row "Paged attention":
 * 16-token pages).  Two query shapes are served: batched decode, one query
 * token per sequence (same page, table "Core inference", row "Generation";
 * mini-llm README, architecture overview: true batched decode), and chunked
 * causal prefill, a block of query tokens over its paged prefix (TinyLoop
 * "Current Status", table "Model architecture support", row "Chunked
 * prefill"; Tiny-LLM "Project Status", supported-features list).  Query heads
 * share KV heads in groups (GQA/MQA; TinyLoop table "Model architecture
 * support", row "GQA").  KV storage is fp32, bf16, fp16, or int8 or FP8
 * (E4M3) codes with per-token-per-head fp32 scales (Tiny-LLM "Project
 * Status", dtype-contract paragraph; mini-llm README hardware table, FP16 KV
 * cache; TinyLoop table "KV cache modes", row "INT8 KV cache"; stylome.io
 * "Classifier receipt", KV cache point: INT8 or FP8 KV cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a device pointer (HBM) allocated by the
 * caller, dense and row-major in the layout stated, aligned to 16 bytes.
 * The library never allocates, frees or synchronises, and keeps no pointer
 * after it returns.  All work is enqueued, in order, on `stream` (a
 * hipStream_t; NULL is the null stream) and the call returns without
 * waiting.  Calls on one stream are ordered; calls on different streams that
 * write the same buffers race.
 *
 * Cache layout (page size 16, the only size built):
 *   k_cache   [num_pages][num_kv_heads][16][head_dim]   token-major page
 *   v_cache   [num_pages][num_kv_heads][head_dim][16]   token index innermost
 *   k_scales, v_scales [num_pages][num_kv_heads][16] float32 (int8 and FP8 only)
 * Token t of sequence b lives in page block_tables[b][t / 16] at offset
 * t % 16.  The V page is stored with tokens innermost so that the PV
 * contraction (over tokens) reads contiguous runs.
 *
 * GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Errors.  Arguments are checked on the host before anything is enqueued;
 * a non-zero status means nothing was launched.  Device-resident data
 * (context lengths, block-table entries, slots) is not read by the host.  A
 * kernel that meets an out-of-range page id or a context length beyond the
 * block-table row or beyond max_context_len writes NaN for the affected
 * outputs instead of reading out of bounds; an append slot outside the pool
 * is skipped.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 4
#define PKV_PAGE_SIZE 16

/* Element types.  PKV_BF16 is bfloat16 bits; PKV_I8 (int8 codes) and PKV_FP8
 * (OCP FP8 E4M3 codes: bias 7, largest finite 448) are KV-only and carry
 * per-(token, KV head) fp32 scales. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_F16 = 2, PKV_I8 = 3, PKV_FP8 = 4 };

/* Status codes. */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,          /* null pointer, non-positive size, Hq % Hkv != 0, ... */
  PKV_ERR_UNSUPPORTED = 2,          /* page size, head_dim or dtype combination not built */
  PKV_ERR_MISALIGNED = 3,           /* a tensor pointer is not 16-byte aligned */
  PKV_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes below the size the query returns */
  PKV_ERR_HIP = 5,                  /* a kernel launch failed */
  PKV_ERR_SCRATCH_TOO_SMALL = 6     /* paged_attn_decode_noalloc: the call needs more split
                                       scratch than PKV_NOALLOC_SCRATCH_BYTES */
};

typedef struct ihipStream_t* pkv_stream_t; /* the same type as hipStream_t */

/* ABI version of the loaded library (PKV_ABI_VERSION at build time). */
int pkv_abi_version(void);

/* Static, human-readable name of a status code; never NULL. */
const char* pkv_status_string(int status);

/*
 * paged_kv_append - write new K/V tokens into the pool through a slot map.
 *
 * Defines the write side of the paged cache: each new token of a sequence
 * is stored in a page slot of the pool (TinyLoop "Current Status", table "KV
 * cache modes", rows "Paged attention" and "INT8 KV cache"), converted to
 * the cache's dtype (Tiny-LLM "Project Status", dtype-contract paragraph).
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim], dtype new_dtype
 *                  (PKV_F32, PKV_BF16 or PKV_F16); read only.
 *   slot_mapping   [num_tokens] int64; token j goes to page slot/16, offset
 *                  slot%16.  A negative slot skips the token (padding); a
 *                  slot >= num_pages*16 is skipped too.  Two tokens with the
 *                  same slot in one call leave either one (undefined which).
 *   k_cache, v_cache  the pool (layout above), dtype cache_dtype; written.
 *   k_scales, v_scales  required (non-NULL) iff cache_dtype is PKV_I8 or
 *                  PKV_FP8, and must be NULL otherwise; written.
 *
 * Conversions: fp32 is copied bit for bit; fp16 and bf16 round to nearest
 * even (fp16 keeps subnormals; a bf16 NaN stays NaN); int8 is symmetric
 * absmax per (token, KV head): scale = absmax/127 in IEEE fp32, code =
 * clamp(rint(x/scale), -127, 127) with ties to even, scale 0 and codes 0 for
 * an all-zero vector; FP8 likewise with scale = absmax/448 and code = the
 * E4M3 value nearest to clamp(x/scale, -448, 448) (ties to even; the sign
 * bit is that of the fp32 ratio, so -0 stores 0x80).  An int8 or FP8
 * vector holding a NaN stores scale NaN and codes 0 (attention over that
 * token then gives NaN); one holding an infinity (and no NaN) stores scale
 * +inf with unspecified codes.  num_tokens == 0
 * is a no-op returning PKV_OK.
 */
int paged_kv_append(const void* k_new, const void* v_new, int new_dtype,
                    const int64_t* slot_mapping, int num_tokens,
                    void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                    int cache_dtype, int num_pages, int num_kv_heads, int head_dim,
                    int page_size, pkv_stream_t stream);

/* Pairing of coordinates for paged_kv_append_rope. */
enum {
  PKV_ROPE_HALF = 1,        /* coordinate i with i + head_dim/2 (Llama, Qwen2) */
  PKV_ROPE_INTERLEAVED = 2  /* coordinate 2i with 2i + 1 */
};

/*
 * paged_kv_append_rope - paged_kv_append with rotary position embedding on K
 * (and optionally on the queries) in the same launch.
 *
 * RoPE with a configurable base theta in every forward path (TinyLoop
 * "Current Status", table "Model architecture support", row "RoPE"), fused
 * into the append so new K is read and written once.  Coordinate pair i of
 * a head vector, 0 <= i < head_dim/2, is rotated by the angle
 * positions[j] * rope_theta^(-2i/head_dim) (RoFormer's definition):
 * (a, b) -> (a cos - b sin, b cos + a sin), a the pair's first coordinate.
 * The pairing is rope_style (PKV_ROPE_HALF or PKV_ROPE_INTERLEAVED).
 *
 *   k_new, v_new, new_dtype, slot_mapping, num_tokens, k_cache, v_cache,
 *   k_scales, v_scales, cache_dtype, num_pages, num_kv_heads, head_dim,
 *   page_size      as for paged_kv_append; K is rotated, V is stored as
 *                  paged_kv_append stores it.
 *   positions      [num_tokens] int32 token positions (any value).
 *   q              NULL, or [num_tokens][num_q_heads][head_dim] of q_dtype
 *                  (F32/BF16/F16), rotated in place at the same positions,
 *                  whatever the token's slot.  Must not overlap the other
 *                  buffers.
 *   rope_theta     the base, finite and > 0 (else PKV_ERR_INVALID_ARG).
 *
 * Arithmetic: each pair frequency rope_theta^(-2i/head_dim) is evaluated in
 * double and rounded once to fp32 (the usual storage of a frequency table);
 * the angle (position times that fp32 frequency), its cosine and sine and the
 * rotation are evaluated in IEEE double (products and the sum rounded
 * separately); the rotated value
 * is rounded to fp32, then converted to the cache dtype (K) or the query
 * dtype (q) exactly as paged_kv_append converts an fp32 input.  The double
 * cosine and sine are those of the device math library, so a value lying
 * within about 1e-16 relative of an fp32 rounding boundary may round either
 * way: results agree with a correctly rounded evaluation to within one unit
 * in the last place of the stored type (one int8 code).
 */
int paged_kv_append_rope(const void* k_new, const void* v_new, int new_dtype,
                         const int64_t* slot_mapping, const int32_t* positions, int num_tokens,
                         void* q, int q_dtype, int num_q_heads, float rope_theta, int rope_style,
                         void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                         int cache_dtype, int num_pages, int num_kv_heads, int head_dim,
                         int page_size, pkv_stream_t stream);

/*
 * paged_attn_decode - one query token per sequence over its paged context.
 *
 * Batched cached decode (TinyLoop "Current Status", table "Core inference",
 * row "Generation"; mini-llm README, true batched decode) over 16-token pages
 * with GQA.  context_lens[b] counts the query token itself, whose K/V must
 * already be appended; the query attends to positions [0, context_lens[b]),
 * or with a sliding window to the `window` most recent of them.  A sequence
 * with context_lens[b] == 0 gets zeros.
 *
 *   q              [batch][num_q_heads][head_dim], dtype q_dtype (F32/BF16/F16).
 *   k_cache, v_cache, k_scales, v_scales, kv_dtype   the pool (layout above);
 *                  scales non-NULL iff kv_dtype is PKV_I8 or PKV_FP8.
 *   block_tables   [batch][max_blocks_per_seq] int32 page ids; entries past a
 *                  sequence's last page are never read.
 *   context_lens   [batch] int32, each in [0, max_context_len].
 *   max_context_len  host-side upper bound of context_lens, at most
 *                  max_blocks_per_seq*16; sizes the split of long contexts.
 *   num_pages      pool size in pages (page ids must be below it).
 *   scale          multiplies q.k before the softmax; any finite value
 *                  (negative and zero included), else PKV_ERR_INVALID_ARG.
 *   window         0 for the whole context, or a sliding window of `window`
 *                  tokens (TinyLoop "Current Status", table "KV cache modes",
 *                  row "Sliding-window cache"): the query at position
 *                  p = context_lens[b] - 1 attends to positions (p - window, p].
 *                  Block-table entries of pages wholly before the window are
 *                  never read, so a cache that bounds its storage by the
 *                  window may have recycled them.  Negative: PKV_ERR_INVALID_ARG.
 *   out            [batch][num_q_heads][head_dim], dtype out_dtype (F32/BF16/F16).
 *   workspace      device scratch of at least
 *                  paged_attn_decode_workspace_bytes(...) bytes (may be NULL
 *                  when that is 0); its contents on entry do not matter.
 *                  Calls that run concurrently must not share a workspace.
 *
 * Built for head_dim 64 and 128, page_size 16, any num_q_heads/num_kv_heads
 * ratio, keys spanning up to 262144 tokens (the whole context, or with a
 * window the window; PKV_ERR_UNSUPPORTED beyond).  Long contexts are split
 * into partitions whose softmax partials are merged with their log-sum-exp
 * weights: inside the launch, by the partition that finishes last, when the
 * plan has at most eight partitions per sequence, else by a second kernel
 * on the same stream.
 */
int paged_attn_decode(const void* q, int q_dtype,
                      const void* k_cache, const void* v_cache,
                      const float* k_scales, const float* v_scales, int kv_dtype,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* context_lens, int max_context_len,
                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                      int page_size, int num_pages, float scale, int window,
                      void* out, int out_dtype,
                      void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/*
 * paged_attn_decode_append - one decode step in one launch: each sequence's
 * new token is appended, then every sequence's query attends over its
 * context including that token.
 *
 * The cached-decode step of the pages' runtimes (TinyLoop "Current Status",
 * table "Core inference", row "Generation": the new token's K/V join the
 * paged cache, then the query attends over it) with the append fused into
 * the decode.  The result is exactly that of paged_kv_append of k_new/v_new
 * to the slot of position context_lens[b] - 1 (page
 * block_tables[b][(ctx-1)/16], offset (ctx-1)%16) followed by
 * paged_attn_decode with the same arguments: the new row is stored with
 * paged_kv_append's rounding and the attention uses the stored values.
 *
 *   k_new, v_new   [batch][num_kv_heads][head_dim], dtype new_dtype
 *                  (F32/BF16/F16); read only.
 *   k_cache, v_cache  written at the new tokens' slots, read elsewhere.
 *   k_scales, v_scales  required (non-NULL, 16-byte aligned) iff kv_dtype
 *                  is PKV_I8 or PKV_FP8, NULL otherwise; written at the new
 *                  tokens' slots (the vector's scale, exactly as
 *                  paged_kv_append stores it), read elsewhere.
 *   kv_dtype       any KV dtype.  int8 and FP8 quantise each new K and V
 *                  vector with paged_kv_append's rule, so codes and scales
 *                  are byte for byte those of paged_kv_append.
 *   other arguments as for paged_attn_decode; the workspace size is
 *                  paged_attn_decode_workspace_bytes(...).
 *
 * A sequence with context_lens[b] == 0 appends nothing and gets zeros.  A
 * new token whose page id or context length is invalid is not stored (the
 * row's output is NaN, as in paged_attn_decode).
 */
int paged_attn_decode_append(const void* q, int q_dtype,
                             const void* k_new, const void* v_new, int new_dtype,
                             void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                             int kv_dtype,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int batch, int num_q_heads, int num_kv_heads, int head_dim,
                             int page_size, int num_pages, float scale, int window,
                             void* out, int out_dtype,
                             void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/*
 * paged_attn_decode_noalloc - paged_attn_decode without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, layouts and results are those of paged_attn_decode (the same
 * kernels and split plan, so the outputs are identical bit for bit); the
 * split partials go to a static device buffer of PKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.  The
 * call allocates and frees nothing.  A call whose split partials need more
 * than that (paged_attn_decode_workspace_bytes(...) larger than
 * PKV_NOALLOC_SCRATCH_BYTES) returns PKV_ERR_SCRATCH_TOO_SMALL and launches
 * nothing.  Every call on one GPU shares that GPU's buffer: calls that may
 * overlap in time (on different streams) race and must be serialised by the
 * caller.  Nothing in the buffer needs clearing between calls: each call
 * writes every partial it reads, and its merge counters carry the call's
 * own tag.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

int paged_attn_decode_noalloc(const void* q, int q_dtype,
                              const void* k_cache, const void* v_cache,
                              const float* k_scales, const float* v_scales, int kv_dtype,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len,
                              int batch, int num_q_heads, int num_kv_heads, int head_dim,
                              int page_size, int num_pages, float scale, int window,
                              void* out, int out_dtype, pkv_stream_t stream);

/* Workspace bytes paged_attn_decode needs for these shapes (0 when the
 * contexts fit one partition, or for invalid shapes).  Pure host
 * arithmetic; touches no device. */
size_t paged_attn_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                         int head_dim, int max_context_len, int window);

/*
 * paged_attn_prefill_chunk - a causal chunk of query tokens over its paged
 * prefix.
 *
 * Chunked prefill (TinyLoop "Current Status", table "Model architecture
 * support", row "Chunked prefill"; Tiny-LLM "Project Status", supported
 * features: chunked prefill/decode scheduling with a paged KV cache).  The
 * chunk's own K/V must already be appended.  Sequence b's queries are rows
 * cu_q_lens[b] .. cu_q_lens[b+1]-1 of q; with C_b = cu_q_lens[b+1]-cu_q_lens[b]
 * and P_b = context_lens[b] - C_b (required >= 0), chunk row i sits at
 * absolute position P_b + i and attends to positions [0, P_b + i], or with
 * window > 0 to (P_b + i - window, P_b + i]; block-table entries of pages
 * wholly before the window of the chunk's first row are never read.
 *
 *   q              [num_tokens][num_q_heads][head_dim], dtype q_dtype.
 *   cu_q_lens      [batch+1] int32, cu_q_lens[0] == 0, non-decreasing,
 *                  cu_q_lens[batch] == num_tokens, each C_b <= max_q_len.
 *   context_lens   [batch] int32 = P_b + C_b, each <= max_context_len.
 *   out            [num_tokens][num_q_heads][head_dim], dtype out_dtype.
 *                  q and out may be NULL when num_tokens == 0, which is a
 *                  no-op returning PKV_OK once the other arguments check.
 *   workspace      at least paged_attn_prefill_workspace_bytes(...) bytes.
 *   other arguments as for paged_attn_decode.
 *
 * Built for head_dim 64 and 128, page_size 16 and every KV dtype (QK^T and
 * PV on MFMA with fp32 accumulation: fp32 caches on the fp32 MFMA with P in
 * fp32; 16-bit caches in their own type with P rounded to it; int8 and FP8
 * codes converted exactly to fp16, the query row scaled by a power of two
 * before it is rounded to fp16, the K scales on the scores and the V scales
 * on the probabilities).  k_scales and v_scales, when given, must be
 * 16-byte aligned (PKV_ERR_MISALIGNED).
 *
 * Non-finite cache values: a NaN or inf K or V value (int8/FP8: a NaN or
 * inf scale) at a position makes the rows that attend that position NaN or
 * inf in the query heads of its KV head.  With int8/FP8 caches rows that do
 * not attend it are unaffected.  With 16-bit caches a non-finite V value can
 * also reach chunk rows of the same sequence that do not attend it (a zero
 * probability times NaN is NaN in the PV product); a non-finite K value
 * cannot.
 */
int paged_attn_prefill_chunk(const void* q, int q_dtype,
                             const void* k_cache, const void* v_cache,
                             const float* k_scales, const float* v_scales, int kv_dtype,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* cu_q_lens,
                             int num_tokens, int max_q_len, int max_context_len,
                             int batch, int num_q_heads, int num_kv_heads, int head_dim,
                             int page_size, int num_pages, float scale, int window,
                             void* out, int out_dtype,
                             void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* Workspace bytes paged_attn_prefill_chunk needs (pure host arithmetic). */
size_t paged_attn_prefill_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                          int head_dim, int max_q_len, int max_context_len,
                                          int window);

/*
 * paged_attn_mixed - prefill chunks and decode tokens of one batch in one call.
 *
 * Chunked prefill/decode scheduling over the paged cache (Tiny-LLM "Project
 * Status", supported features: chunked prefill/decode scheduling; TinyLoop
 * "Current Status", table "Model architecture support", row "Chunked
 * prefill").  Arguments, layouts and results are exactly those of
 * paged_attn_prefill_chunk (a decode token is a chunk of one: its query row
 * cu_q_lens[b] attends to [0, context_lens[b])); the difference is how the
 * work is cut: sequences whose chunk is a single token have their context
 * split across several workgroups as in paged_attn_decode, the others run
 * the MFMA prefill row blocks, all in one launch (plus the split merge).
 *
 *   workspace      at least paged_attn_mixed_workspace_bytes(...) bytes (the
 *                  decode split partials; may be NULL when that is 0); its
 *                  contents on entry do not matter.
 *
 * Built for head_dim 64 and 128, page_size 16, every KV dtype, decode keys
 * spanning up to 262144 tokens (PKV_ERR_UNSUPPORTED otherwise);
 * `window` as for paged_attn_prefill_chunk.  A one-token
 * chunk with context_lens[b] < 1 gets NaN, like any chunk longer than its
 * context.
 */
int paged_attn_mixed(const void* q, int q_dtype,
                     const void* k_cache, const void* v_cache,
                     const float* k_scales, const float* v_scales, int kv_dtype,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* cu_q_lens,
                     int num_tokens, int max_q_len, int max_context_len,
                     int batch, int num_q_heads, int num_kv_heads, int head_dim,
                     int page_size, int num_pages, float scale, int window,
                     void* out, int out_dtype,
                     void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* Workspace bytes paged_attn_mixed needs (0 when no context is split, or for
 * invalid shapes).  The one-token rows are split across their context as in
 * paged_attn_decode when max_q_len < 128, and only as far as contexts beyond
 * 4096 tokens require otherwise.  Pure host arithmetic; touches no device. */
size_t paged_attn_mixed_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                        int head_dim, int max_q_len, int max_context_len,
                                        int window);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
