// Streaming-read probe for the benchmark's roofline denominator: reads a device buffer once
// with 16-byte nontemporal loads, each workgroup a contiguous block, sixteen loads in flight
// per lane, and keeps only a per-workgroup checksum. Its GB/s is what a pure read stream reaches on this GPU; the decode kernels
// report their bandwidth as a fraction of it beside the fraction of the nominal HBM peak.
// Measurement only: not part of the KVarN library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../../include/kvarn_probe.h"

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads the contiguous block [b per, (b + 1) per) of 16-byte units; each round
// its 256 lanes load 16 consecutive units apiece (64 KB per workgroup in flight).
__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const u32x4* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  constexpr int kUnroll = 16;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = int64_t(blockIdx.x) * per;
  const int64_t e = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < e; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < e; i += kThreads) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x + a.y + a.z + a.w;
  }
  // one lane per workgroup stores (sink holds gridDim.x words); the value keeps every load
  // live and is otherwise unused
  acc = __reduce_xor_sync(~0ull, acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// VALU issue calibration: eight independent float32 FMA chains per lane, 32 v_fma_f32 per
// round; the launch's duration gives the cycles one wave64 FMA holds a SIMD.
__global__ void __launch_bounds__(kThreads) valu_fma_kernel(float* __restrict__ out, int32_t rounds) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = float(threadIdx.x) * 1e-3f + float(j);
  for (int32_t i = 0; i < rounds; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = fmaf(a[j], 0.999f, 0.25f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  out[int64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int kvarn_probe_valu_fma(void* out, int32_t grid, int32_t rounds, void* stream) {
  if (!out || grid <= 0 || grid > 65536 || rounds < 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return 1;
  hipLaunchKernelGGL(valu_fma_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<float*>(out), rounds);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int kvarn_probe_stream_read(const void* src, size_t bytes, void* sink,
                                       int32_t grid, void* stream) {
  if (!src || !sink || grid <= 0 || grid > 65536 || (bytes % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     int64_t(bytes / 16), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
