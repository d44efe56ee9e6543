// Measurement kernels (include/pace_measure.h): the fixed cost of a launch of the decode
// kernel's shape, and a read-only stream of the decode launch's byte count in that shape.
// gfx950, wave64.
#include <hip/hip_runtime.h>

#include "../../include/pace_measure.h"

namespace {

typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

__global__ void empty_kernel() {}

// Each workgroup streams its own contiguous slice; lanes take consecutive 16-byte vectors,
// so every wave instruction reads one contiguous 1 KB span.  A lane requests up to eight
// vectors at once before consuming any (a slice of up to 8 x blockDim vectors is one round
// of requests): out-of-range indices are clamped to the slice's last vector, which is
// then not counted.
__global__ void stream_kernel(const uint8_t* __restrict__ src, size_t bytes_per_wg, uint32_t* __restrict__ sink) {
  const unsigned w = blockIdx.y * gridDim.x + blockIdx.x;
  const v4u32* p = (const v4u32*)(src + (size_t)w * bytes_per_wg);
  const size_t nvec = bytes_per_wg / 16;
  const size_t step = blockDim.x;
  v4u32 acc = {0u, 0u, 0u, 0u};
  for (size_t i0 = threadIdx.x; i0 < nvec; i0 += 8 * step) {
    v4u32 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t i = i0 + u * step;
      r[u] = __builtin_nontemporal_load(p + (i < nvec ? i : nvec - 1));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * step < nvec) acc ^= r[u];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  // fold the workgroup's lanes into one word (the loads must not be dead code)
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (unsigned k = 0; k < blockDim.x / 64; ++k) y ^= part[k];
    sink[w] = y;
  }
}

bool shape_ok(int32_t gx, int32_t gy, int32_t threads) {
  return gx >= 1 && gy >= 1 && gy <= 65535 && threads >= 64 && threads <= 1024 && threads % 64 == 0;
}

}  // namespace

extern "C" int pace_measure_empty(int32_t gx, int32_t gy, int32_t threads, void* stream) {
  if (!shape_ok(gx, gy, threads)) return -1;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)gx, (unsigned)gy), dim3((unsigned)threads), 0,
                     (hipStream_t)stream);
  return (int)hipGetLastError();
}

extern "C" int pace_measure_stream(const void* src, size_t bytes_per_wg, int32_t gx, int32_t gy,
                                   int32_t threads, uint32_t* sink, void* stream) {
  if (!src || !sink || ((uintptr_t)src % 16) != 0 || bytes_per_wg == 0 || bytes_per_wg % 16 != 0 ||
      !shape_ok(gx, gy, threads))
    return -1;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)gx, (unsigned)gy), dim3((unsigned)threads), 0,
                     (hipStream_t)stream, (const uint8_t*)src, bytes_per_wg, sink);
  return (int)hipGetLastError();
}
