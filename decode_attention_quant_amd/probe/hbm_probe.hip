// hbm_probe.hip -- streaming read and copy kernels (see kvq_probe.h).
//
// Each wave reads 1 KB chunks (16 bytes per lane, lanes contiguous) and keeps
// four of them in flight; 24 waves per CU.  With plain loads this shape
// reads at the top of the measured range of plain-load streaming kernels
// (about 6.0-6.2 TB/s on MI355X) and allocates what it reads in the caches,
// which is what a cache flush needs; with the non-temporal hint on every
// load it reaches the top of all the read kernels measured (about
// 6.7-7.0 TB/s), the rate a kernel that streams data once can aim for.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace kvq_probe {

constexpr int kUnroll = 4;           // 1 KB chunks in flight per wave
constexpr int kWavesPerBlock = 4;    // 256 threads
constexpr int kBlocksPerCu = 6;      // 24 waves per CU

template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t chunks,
                                                   uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto load = [](const uint4* a) -> uint4 {
    if constexpr (NT) {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
      return make_uint4(t.x, t.y, t.z, t.w);
    } else {
      return *a;
    }
  };
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const size_t waves = (size_t)gridDim.x * kWavesPerBlock;
  const size_t groups = chunks / kUnroll;
  uint32_t acc = 0;
  for (size_t s = wave; s < groups; s += waves) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load(p + (s * kUnroll + u) * 64 + lane);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  const size_t rest = chunks - groups * kUnroll;  // < kUnroll chunks left
  if (wave < rest) {
    const uint4 v = load(p + (groups * kUnroll + wave) * 64 + lane);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

static int grid_blocks(int* blocks) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 4;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 4;
  *blocks = cus * kBlocksPerCu;
  return 0;
}

}  // namespace kvq_probe

using kvq_probe::copy_kernel;
using kvq_probe::grid_blocks;
using kvq_probe::read_kernel;

template <bool NT>
static int launch_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  if (!src || !sink || bytes % 1024 != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  if (bytes == 0) return 0;
  int blocks = 0;
  if (int st = grid_blocks(&blocks)) return st;
  hipLaunchKernelGGL(read_kernel<NT>, dim3(blocks), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     bytes / 1024, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int kvq_probe_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  return launch_read<false>(src, bytes, sink, stream);
}

extern "C" int kvq_probe_read_stream(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  return launch_read<true>(src, bytes, sink, stream);
}

extern "C" int kvq_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src || bytes % 16 != 0 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return 1;
  if (bytes == 0) return 0;
  int blocks = 0;
  if (int st = grid_blocks(&blocks)) return st;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
