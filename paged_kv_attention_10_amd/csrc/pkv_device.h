// Device-side helpers for the pkv kernels (gfx950 / CDNA4, wave64).
//
// Element conversions used by the append path are written on the bit
// patterns so that they match the library's documented rounding exactly
// (nearest-even bf16 with NaN kept quiet; IEEE fp16 via the hardware
// convert, which rounds to nearest even and keeps subnormals).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/pkv.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = PKV_PAGE_SIZE;
constexpr float kLog2e = 1.4426950408889634f;

// KV dtypes stored as one-byte codes with per-(token, head) scales.
constexpr bool kv_code8(int kv) { return kv == PKV_I8 || kv == PKV_FP8; }

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// ------------------------------------------------- inputs in an io dtype
// Inputs come in fp32, bf16 or fp16, chosen at run time.  Code that loads
// several elements runs under with_io_dtype, which branches once on the
// dtype and hands the body the dtype as a compile-time constant: the loads
// then issue back to back and are converted after one wait (a per-element
// dtype branch makes each load wait inside its branch).
template <int DT>
using IoDtype = std::integral_constant<int, DT>;

template <typename F>
__device__ __forceinline__ void with_io_dtype(int dt, F&& body) {
  if (dt == PKV_F32) body(IoDtype<PKV_F32>{});
  else if (dt == PKV_BF16) body(IoDtype<PKV_BF16>{});
  else body(IoDtype<PKV_F16>{});
}

// Storage bits of element i (16-bit values zero-extended) and their value.
template <int DT>
__device__ __forceinline__ uint32_t io_bits(const void* base, long i) {
  if constexpr (DT == PKV_F32) return static_cast<const uint32_t*>(base)[i];
  else return static_cast<const uint16_t*>(base)[i];
}

template <int DT>
__device__ __forceinline__ float io_value(uint32_t bits) {
  if constexpr (DT == PKV_F32) return __uint_as_float(bits);
  else if constexpr (DT == PKV_BF16) return bf16_bits_to_f32(bits);
  else return f16_bits_to_f32(bits);
}

// The value of storage bits in the run-time dtype dt, with selects rather
// than a branch: code that loads under with_io_dtype and converts later
// keeps the conversion (and the wait for the loads) where it is written,
// since a second branch on dt would be merged with the first.
__device__ __forceinline__ float io_value_sel(uint32_t bits, int dt) {
  const float vh = f16_bits_to_f32(bits);
  const float vb = __uint_as_float(bits << 16);
  return dt == PKV_F32 ? __uint_as_float(bits) : (dt == PKV_BF16 ? vb : vh);
}

// Raw words of N (4 or 8) consecutive elements i..: N words in fp32, N/2 in
// a 16-bit dtype (element e in the low (e even) or high half of word e/2),
// with 8-, 16- or 32-byte loads (base + i must be aligned to the load's
// size).  Nothing here uses the loaded data.
template <int N, int DT>
__device__ __forceinline__ void io_words(const void* base, long i, uint32_t* w) {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint32_t*>(base) + i + 4 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * k + e] = v[e];
    }
  } else if constexpr (N == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = v[e];
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + i);
    w[0] = v[0];
    w[1] = v[1];
  }
}

// The same raw words for the run-time dtype dt, without a branch: two
// 16-byte (N = 8) or 8-byte (N = 4) loads, the second repeating the first
// in a 16-bit dtype (whose run fills only the first half of w).
template <int N>
__device__ __forceinline__ void io_words_rt(const void* base, long i, int dt, uint32_t* w) {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  const bool f32 = dt == PKV_F32;
  const char* p = static_cast<const char*>(base) + i * (f32 ? 4 : 2);
  if constexpr (N == 8) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + (f32 ? 16 : 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = lo[e];
      w[4 + e] = hi[e];
    }
  } else {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + (f32 ? 8 : 0));
    w[0] = lo[0];
    w[1] = lo[1];
    w[2] = hi[0];
    w[3] = hi[1];
  }
}

// Storage bits of element e of such words, for the run-time dtype dt.
__device__ __forceinline__ uint32_t io_word_bits(const uint32_t* w, int e, int dt) {
  return dt == PKV_F32 ? w[e] : (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

// N consecutive elements i.. as storage bits (16-bit values zero-extended).
template <int N, int DT>
__device__ __forceinline__ void io_bits_vec(const void* base, long i, uint32_t* bits) {
  uint32_t w[N];
  io_words<N, DT>(base, i, w);
#pragma unroll
  for (int e = 0; e < N; ++e) bits[e] = io_word_bits(w, e, DT);
}

__device__ __forceinline__ void store_from_f32(void* base, long i, int dt, float x) {
  if (dt == PKV_F32) static_cast<float*>(base)[i] = x;
  else if (dt == PKV_BF16) static_cast<uint16_t*>(base)[i] = (uint16_t)f32_to_bf16_bits(x);
  else static_cast<uint16_t*>(base)[i] = (uint16_t)f32_to_f16_bits(x);
}

// ------------------------------------------------------------ MFMA
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Split fp32 values into a 16-bit head and a 16-bit remainder so that
// head + remainder carries about 16 significant bits: the two MFMA products
// then keep the fp32 operand's precision well below the output tolerance.
template <typename V8>
struct Split8 { V8 hi, lo; };

__device__ __forceinline__ Split8<bf16x8> split_bf16(const float (&x)[8]) {
  Split8<bf16x8> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = (__bf16)x[e];
    r.hi[e] = h;
    r.lo[e] = (__bf16)(x[e] - (float)h);
  }
  return r;
}

__device__ __forceinline__ Split8<f16x8> split_f16(const float (&x)[8]) {
  Split8<f16x8> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 h = (_Float16)x[e];
    r.hi[e] = h;
    r.lo[e] = (_Float16)(x[e] - (float)h);
  }
  return r;
}

// Sort key of |x|: for non-negative floats the unsigned order of the bit
// patterns is the numeric order, and every NaN pattern lies above +inf, so
// the unsigned max of these keys over a vector is its absmax, or a NaN when
// any element is NaN (an fmax would skip the NaN).
__device__ __forceinline__ uint32_t abs_key(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// int8 codes (4 per dword) -> fp16, exact.  Flipping the sign bit turns a
// code x into the byte x + 128; v_perm places each such byte under the fp16
// exponent of 1024 (bits 0x64xx), which reads as 1024 + x + 128, and one
// packed fp16 subtraction of 1152 leaves x.  Every step is exact (all
// values are integers below 2048).
__device__ __forceinline__ void i8x8_to_f16x8(u32x2 w, f16x8& out) {
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t u = w[q] ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // bytes 0, 1
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // bytes 2, 3
    const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
    const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
    out[4 * q + 0] = a[0];
    out[4 * q + 1] = a[1];
    out[4 * q + 2] = b[0];
    out[4 * q + 3] = b[1];
  }
}

// OCP FP8 E4M3 codes (4 per dword) -> fp16 holding the code's value:
// gfx950's two-code convert to fp32 (v_cvt_pk_f32_fp8, which reads OCP
// E4M3 on this chip: checked over all 256 codes, NaN codes giving NaN),
// then a two-value pack to fp16, exact because every finite E4M3 value
// (2^-9 .. 448) is an fp16 normal.
__device__ __forceinline__ void fp8x8_to_f16x8_value(u32x2 w, f16x8& out) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], false);   // codes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], true);    // codes 2, 3
    const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(lo[0], lo[1]));
    const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(hi[0], hi[1]));
    out[4 * q + 0] = a[0];
    out[4 * q + 1] = a[1];
    out[4 * q + 2] = b[0];
    out[4 * q + 3] = b[1];
  }
}

// fp32 value with |r| <= 448 -> OCP FP8 E4M3 code, to the nearest E4M3 value
// with ties to even; the sign bit is r's.  With e = max(binade exponent of
// |r|, -6) the grid there is 2^(e-3), q = rint(|r| * 2^(3-e)) (an exact
// scaling) counts grid steps, and the code is ((e + 7) << 3) + (q - 8):
// q = 16 (rounded up to the next binade) carries into the exponent field,
// and for e = -6, q < 8 gives the subnormal code q.
__device__ __forceinline__ uint32_t f32_to_e4m3_bits(float r) {
  const uint32_t u = __float_as_uint(r);
  const float a = __uint_as_float(u & 0x7fffffffu);
  const int e = max((int)((u >> 23) & 0xffu) - 127, -6);
  const float q = rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
  return ((u >> 24) & 0x80u) | (uint32_t)(((e + 7) << 3) + (int)q - 8);
}

// The append's quantisation of one (token, KV head) vector, shared by every
// kernel that stores one-byte codes so that they store the same bytes.
// `am` is the vector's absmax taken as a sort key with abs_key (a NaN
// element makes it NaN); the scale is am/127 (int8) or am/448 (FP8) in IEEE
// fp32 division, and each code is clamp(rint(x/scale), -127, 127) (int8)
// or the E4M3 value nearest to clamp(x/scale, -448, 448) (FP8); a scale
// that is not positive (all-zero or NaN vector) gives codes 0.
__device__ __forceinline__ float code8_scale(float am, bool i8) { return am / (i8 ? 127.0f : 448.0f); }

__device__ __forceinline__ uint32_t code8(float x, float sc, bool i8) {
  if (!(sc > 0.f)) return 0u;
  if (i8) return (uint32_t)(int)fminf(fmaxf(rintf(x / sc), -127.f), 127.f) & 0xffu;
  return f32_to_e4m3_bits(fminf(fmaxf(x / sc, -448.f), 448.f));
}

// Cross-lane exchanges with the gfx950 lane-swap instructions (VALU, no LDS
// round trip).  v_permlane32_swap exchanges the upper 32 lanes of one
// operand with the lower 32 of the other; given x in both, the two results
// hold, in every lane l, x[l] and x[l ^ 32] (which result holds which does not
// matter to a max or a sum).  v_permlane16_swap does the same for lanes
// l and l ^ 16.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_xor_16_32(float x) { return max_xor32(max_xor16(x)); }
__device__ __forceinline__ float wave_sum_xor_16_32(float x) { return sum_xor32(sum_xor16(x)); }

}  // namespace pkv
