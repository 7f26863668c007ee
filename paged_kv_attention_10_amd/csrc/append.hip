// Append: new K/V tokens are written into the paged pool through a slot
// mapping and converted to the cache dtype (TinyLoop "Current Status", table
// "KV cache modes", rows "Paged attention" and "INT8 KV cache"; Tiny-LLM
// "Project Status", dtype-contract paragraph on a separate KV-cache dtype).
//
// One wave per (token, KV head): each lane converts D/64 elements, K goes to
// its token row of the page, V to column `offset` of the token-innermost V
// page.  int8 takes the absmax of the (token, head) vector with a wave
// reduction, then scale = absmax/127 (IEEE fp32 division) and
// code = clamp(rint(x/scale), -127, 127) with ties to even.
#include <math.h>

#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  float* k_scales;
  float* v_scales;
  int new_dtype, cache_dtype;
  int num_tokens, hkv;
  long num_slots;
};

// Raw 32-bit pattern of an fp32 input element (bit-exact copy path).
__device__ __forceinline__ uint32_t load_bits32(const void* base, long i) {
  return static_cast<const uint32_t*>(base)[i];
}

template <int D>
__device__ __forceinline__ void append_one(const AppendArgs& a, const void* src, void* cache,
                                           float* scales, long row, long page, int off, int g,
                                           bool is_v, int lane) {
  constexpr int PER = D / 64;
  float x[PER];
  uint32_t raw[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    long i = row * D + lane * PER + e;
    if (a.new_dtype == PKV_F32) {
      raw[e] = load_bits32(src, i);
      x[e] = __uint_as_float(raw[e]);
    } else {
      x[e] = load_as_f32(src, i, a.new_dtype);
      raw[e] = __float_as_uint(x[e]);
    }
  }
  const long head = page * a.hkv + g;
  auto dst_index = [&](int d) -> long {
    return is_v ? (head * D + d) * kPage + off : (head * kPage + off) * D + d;
  };
  if (a.cache_dtype == PKV_I8) {
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) am = fmaxf(am, fabsf(x[e]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
    const float sc = am / 127.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float code = 0.f;
      if (sc > 0.f) code = fminf(fmaxf(rintf(x[e] / sc), -127.f), 127.f);
      static_cast<int8_t*>(cache)[dst_index(lane * PER + e)] = (int8_t)(int)code;
    }
    if (lane == 0) scales[head * kPage + off] = sc;
    return;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const long di = dst_index(lane * PER + e);
    if (a.cache_dtype == PKV_F32) static_cast<uint32_t*>(cache)[di] = raw[e];
    else if (a.cache_dtype == PKV_BF16) static_cast<uint16_t*>(cache)[di] = (uint16_t)f32_to_bf16_bits(x[e]);
    else static_cast<uint16_t*>(cache)[di] = (uint16_t)f32_to_f16_bits(x[e]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long)a.num_tokens * a.hkv) return;
  const long tok = w / a.hkv;
  const int g = (int)(w - tok * a.hkv);
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= a.num_slots) return;
  const long page = slot / kPage;
  const int off = (int)(slot - page * kPage);
  const long row = tok * a.hkv + g;
  append_one<D>(a, a.k_new, a.k_cache, a.k_scales, row, page, off, g, false, lane);
  append_one<D>(a, a.v_new, a.v_cache, a.v_scales, row, page, off, g, true, lane);
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
  if ((cache_dtype == PKV_I8) != (k_scales != nullptr) || (cache_dtype == PKV_I8) != (v_scales != nullptr))
    return PKV_ERR_INVALID_ARG;
  if (page_size != PKV_PAGE_SIZE || !head_dim_built(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (k_scales && !aligned16(k_scales)) || (v_scales && !aligned16(v_scales)) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return PKV_ERR_MISALIGNED;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.new_dtype = new_dtype;
  a.cache_dtype = cache_dtype;
  a.num_tokens = num_tokens;
  a.hkv = num_kv_heads;
  a.num_slots = (long)num_pages * PKV_PAGE_SIZE;
  const long waves = (long)num_tokens * num_kv_heads;
  const long blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffffL) return PKV_ERR_INVALID_ARG;
  clear_launch_error();
  if (head_dim == 64)
    hipLaunchKernelGGL(append_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(append_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return launch_status();
}
