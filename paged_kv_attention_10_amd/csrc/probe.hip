// Streaming-read probe (measurement only; not part of the pkv library and
// not declared in include/pkv.h).  It gives the practical ceiling the
// decode's HBM rate is compared with: how fast a plain kernel on this
// part reads a buffer once, with no compute to speak of.
//
// Each thread folds (XOR) the 16-byte words base[i], base[i + S], ... with
// S the thread count of the grid, four loads in flight per step; a
// workgroup writes its value only if it equals an arbitrary constant, so
// the loads cannot be elided and the kernel writes (almost) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) at `p` once on `stream`
// with `workgroups` workgroups of 256 threads.  `out` needs `workgroups`
// uint32 slots (written only in the unlikely case above).  Returns 0, or 1
// for bad arguments, 2 if the launch failed.
extern "C" int pkv_probe_stream_read(const void* p, size_t bytes, void* out, int workgroups,
                                     void* stream) {
  if (!p || !out || workgroups <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15))
    return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(p), bytes / 16, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
