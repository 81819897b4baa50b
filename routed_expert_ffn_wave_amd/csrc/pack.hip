// Bank set-up kernels: GGUF Q4_0 repack into the device layout, and the dequantisation export
// that decodes bank matrices to fp32 with the same per-format decode routine the FFN kernels use.
//
// Bank formats: FreeToken walk-through "深入FreeToken架构…全链路剖析", section 五 (per-format expert
// banks, each with its own schema).
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

// canonical block: fp16 scale (little endian) then 16 code bytes -> codes[16], scale
__global__ __launch_bounds__(256) void pack_q4_0_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales, long long nblocks) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint8_t* src = canon + b * 18;
  const uint16_t* s16 = (const uint16_t*)src;  // 18 * b is even: 2-byte aligned
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = s16[1 + 2 * i], hi = s16[2 + 2 * i];
    c[i] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  *(u32x4*)(codes + b * 16) = c;
  scales[b] = s16[0];
}

hipError_t launch_pack_q4_0(const uint8_t* canon, uint8_t* codes, uint16_t* scales, long long nblocks, hipStream_t s) {
  const long long grid = (nblocks + 255) / 256;
  hipLaunchKernelGGL(pack_q4_0_kernel, dim3((unsigned)grid), dim3(256), 0, s, canon, codes, scales, nblocks);
  return hipGetLastError();
}

// One thread per 16-byte chunk of codes.  Values are formed exactly as the GEMV kernel forms them:
// Chunk<FMT>::decode to bf16 pairs, then the chunk's scale applied in fp32.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                      int rows, int K, float* __restrict__ out) {
#pragma clang fp contract(off)
  using C = Chunk<FMT>;
  const int per_row = K / C::ELEMS;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * per_row) return;
  const int r = (int)(idx / per_row), ch = (int)(idx % per_row);
  const size_t rbytes = FMT == FMT_BF16 ? (size_t)K * 2 : FMT == FMT_FP8_B128 ? (size_t)K : (size_t)K / 2;
  const u32x4 c = *(const u32x4*)(codes + (size_t)r * rbytes + (size_t)ch * 16);
  uint32_t p[C::PAIRS];
  C::decode(c, p);
  float sc = 1.0f;
  if constexpr (FMT == FMT_Q4_0) sc = fp16_bits_to_f32(((const uint16_t*)scales)[(size_t)r * (K / 32) + ch]);
  if constexpr (FMT == FMT_MXFP4) sc = e8m0_to_f32(scales[(size_t)r * (K / 32) + ch]);
  if constexpr (FMT == FMT_FP8_B128)
    sc = ((const float*)scales)[(size_t)(r / 128) * (K / 128) + (ch * C::ELEMS) / 128];
  float* o = out + (size_t)r * K + (size_t)ch * C::ELEMS;
#pragma unroll
  for (int i = 0; i < C::PAIRS; ++i) {
    float v0 = bf16_bits_to_f32(p[i] & 0xffffu), v1 = bf16_bits_to_f32(p[i] >> 16);
    if constexpr (FMT == FMT_Q4_0) {
      v0 = v0 - 136.0f;  // decode gives 128 + q; the weight is scale * (q - 8)
      v1 = v1 - 136.0f;
    }
    if constexpr (FMT != FMT_BF16) {
      v0 = v0 * sc;
      v1 = v1 * sc;
    }
    o[C::first(i)] = v0;
    o[C::first(i) + C::SECOND] = v1;
  }
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int rows, int K, float* out,
                          hipStream_t s) {
  const int elems = fmt == FMT_BF16 ? 8 : fmt == FMT_FP8_B128 ? 16 : 32;
  const long long n = (long long)rows * (K / elems);
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (fmt) {
    case FMT_BF16: hipLaunchKernelGGL(dequant_kernel<FMT_BF16>, grid, block, 0, s, codes, scales, rows, K, out); break;
    case FMT_Q4_0: hipLaunchKernelGGL(dequant_kernel<FMT_Q4_0>, grid, block, 0, s, codes, scales, rows, K, out); break;
    case FMT_MXFP4: hipLaunchKernelGGL(dequant_kernel<FMT_MXFP4>, grid, block, 0, s, codes, scales, rows, K, out); break;
    default: hipLaunchKernelGGL(dequant_kernel<FMT_FP8_B128>, grid, block, 0, s, codes, scales, rows, K, out); break;
  }
  return hipGetLastError();
}

}  // namespace ftk
