// Start-up rate measurements: the rates the layer's rooflines and the cold-expert split rest on,
// measured on the device at hand (FreeToken walk-through "深入FreeToken架构…全链路剖析", section 五:
// the engine measures the host link and memory bandwidths when it starts and derives its CPU-GPU
// split from them).
//
//   - stream_read_kernel: every thread reads 16-byte words of a buffer (four loads in flight per
//     thread, non-temporal like the GEMV's weight stream) and folds them into an xor that it stores,
//     so no load can be dropped.  Over device memory with every CU's resident blocks it gives the
//     achievable HBM read rate; over pinned host memory with the fill kernel's 8 blocks it gives the
//     host link rate that the expert cache's fill reaches.
//   - mfma_rate_kernel: each wave issues a long run of MFMAs on register operands into four
//     independent accumulators (no memory traffic inside the loop), two 4-wave blocks per CU: the
//     dense rate of v_mfma_f32_32x32x16_bf16 and of v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 x
//     e4m3 operands (the FP8-B128 prefill path) and e2m3 x e2m1 operands (the MXFP4 prefill path).
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, long long n16,
                                                          uint32_t* __restrict__ sink) {
  const long long nthr = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * nthr < n16; i += 4 * nthr) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + nthr);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * nthr);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * nthr);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += nthr) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

// KIND 0: bf16 32x32x16; 1: e4m3 x e4m3 32x32x64 (scaled); 2: e2m3 x e2m1 32x32x64 (scaled)
template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, int scale, float* __restrict__ sink) {
  const uint32_t seed = 0x3c003c00u ^ (threadIdx.x * 0x9e3779b9u);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  if constexpr (KIND == 0) {
    u32x4 ua = {seed, seed ^ 1u, seed ^ 2u, seed ^ 3u}, ub = {seed ^ 4u, seed ^ 5u, seed ^ 6u, seed ^ 7u};
    const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      a[r] = (int)(seed * (r + 1)) & 0x3f3f3f3f;  // small finite codes in every format
      b[r] = (int)(seed * (r + 9)) & 0x3f3f3f3f;
    }
    constexpr int TA = KIND == 1 ? 0 : 2, TB = KIND == 1 ? 0 : 4;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], TA, TB, 0, scale, 0, scale);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_stream_read(const void* p, long long bytes, int blocks, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)p, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t rate_launch_facts(int* stream_blocks, int* cus) {
  static LaunchCache cache;
  LaunchFacts f;
  if (cache.get((const void*)stream_read_kernel, 256, 0, &f) != hipSuccess) return hipGetLastError();
  *stream_blocks = f.per_cu * f.cus;
  *cus = f.cus;
  return hipSuccess;
}

hipError_t launch_mfma_rate(int kind, int blocks, int iters, float* sink, hipStream_t s) {
  const int scale = 127;  // E8M0 1.0 (a kernel argument: never an immediate operand)
  if (kind == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, iters, scale, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, iters, scale, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, iters, scale, sink);
  return hipGetLastError();
}

}  // namespace ftk
