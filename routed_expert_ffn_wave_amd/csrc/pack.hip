// Bank set-up kernels: canonical stored formats -> the row-interleaved device layout, and the
// dequantisation export that decodes device-layout bank matrices to fp32 with the same per-format
// chunk decode the GEMV kernels use.
//
// Bank formats: FreeToken walk-through "深入FreeToken架构…全链路剖析", section 五 (per-format expert
// banks, each with its own schema).  Element encodings: GGUF Q4_0, OCP MXFP4 (E8M0 scales), OCP
// e4m3fn, NVFP4 (e2m1 with e4m3 scales per 16 and an fp32 matrix scale).  All slots of a bank are treated as one matrix of n_slots * R rows: with R a multiple of
// 64, the interleave of that matrix equals the per-slot interleave with slots laid end to end.
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

// Device row of canonical row r (all slots stacked): W13 matrices (perm_I > 0) reorder the rows of
// each slot into gate/up blocks, W2 keeps the order.
__device__ __forceinline__ long long device_row(long long r, int perm_I) {
  if (perm_I == 0) return r;
  const long long per = 2LL * perm_I, s = r / per;
  return s * per + w13_device_row((int)(r % per), perm_I);
}

// 16-byte code chunks: canonical row-major [rows][nchunk][16] -> interleaved.
__global__ __launch_bounds__(256) void interleave_chunks_kernel(const u32x4* __restrict__ src, uint8_t* __restrict__ dst,
                                                                long long rows, int nchunk, int perm_I) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nchunk) return;
  const long long r = i / nchunk;
  const int c = (int)(i % nchunk);
  *(u32x4*)(dst + ilv_chunk_off((int)device_row(r, perm_I), c, nchunk)) = src[i];
}

// one scale element per (row, chunk): canonical [rows][nchunk] -> interleaved.
template <typename T>
__global__ __launch_bounds__(256) void interleave_scales_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                                long long rows, int nchunk, int perm_I) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nchunk) return;
  const long long r = i / nchunk;
  const int c = (int)(i % nchunk);
  dst[ilv_scale_idx((int)device_row(r, perm_I), c, nchunk)] = src[i];
}

// GGUF Q4_0 block (fp16 scale, then byte i = element i | element i+16 << 4) -> device chunk whose
// word w holds elements 8w+2s in bits 4s.. and 8w+2s+1 in bits 16+4s.., plus the interleaved scale.
__global__ __launch_bounds__(256) void pack_q4_0_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales, long long rows, int nchunk,
                                                        int perm_I) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nchunk) return;
  const long long r = device_row(i / nchunk, perm_I);
  const int c = (int)(i % nchunk);
  const uint8_t* blk = canon + i * 18;
  const uint16_t* s16 = (const uint16_t*)blk;  // 18 * i is even: 2-byte aligned
  uint32_t q[32];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint16_t two = s16[1 + b];  // code bytes 2b, 2b+1
    const uint32_t b0 = two & 0xffu, b1 = two >> 8;
    q[2 * b] = b0 & 15u;
    q[2 * b + 16] = b0 >> 4;
    q[2 * b + 1] = b1 & 15u;
    q[2 * b + 17] = b1 >> 4;
  }
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t v = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) v |= (q[8 * w + 2 * s] << (4 * s)) | (q[8 * w + 2 * s + 1] << (16 + 4 * s));
    o[w] = v;
  }
  *(u32x4*)(codes + ilv_chunk_off((int)r, c, nchunk)) = o;
  scales[ilv_scale_idx((int)r, c, nchunk)] = s16[0];
}

// NVFP4 scales: canonical per slot [R][K/16] e4m3 bytes then the fp32 matrix scale; device: the
// two e4m3 bytes of (row, chunk) as one 16-bit pair, interleaved over all slots' rows, then the
// n_slots matrix scales.
__global__ __launch_bounds__(256) void pack_nvfp4_scales_kernel(const uint8_t* __restrict__ canon,
                                                                uint16_t* __restrict__ dst, long long rows, int R,
                                                                int nchunk, int perm_I) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nchunk) return;
  const long long r = i / nchunk;
  const int c = (int)(i % nchunk);
  const long long slot = r / R, rr = r % R;
  const size_t stride = (size_t)R * nchunk * 2 + 4;  // canonical bytes per slot
  const uint16_t* src = (const uint16_t*)(canon + slot * stride + (size_t)rr * nchunk * 2);  // even offsets
  dst[ilv_scale_idx((int)device_row(r, perm_I), c, nchunk)] = src[c];
  if (rr == 0 && c == 0) {  // the slot's matrix scale
    float t;
    const uint8_t* ts = canon + slot * stride + (size_t)R * nchunk * 2;
    __builtin_memcpy(&t, ts, 4);
    ((float*)(dst + rows * nchunk))[slot] = t;
  }
}

static unsigned grid_for(long long n) { return (unsigned)((n + 255) / 256); }

// Pack one matrix (all slots): rows = n_slots * R, K columns.
hipError_t launch_pack_matrix(int fmt, const uint8_t* canon_codes, const uint8_t* canon_scales, uint8_t* codes,
                              uint8_t* scales, long long rows, int K, int perm_I, int R, hipStream_t s) {
  const int nchunk = K / (fmt == FMT_BF16 ? 8 : fmt == FMT_FP8_B128 ? 16 : 32);
  const long long n = rows * nchunk;
  if (n == 0) return hipSuccess;
  if (fmt == FMT_Q4_0) {
    hipLaunchKernelGGL(pack_q4_0_kernel, dim3(grid_for(n)), dim3(256), 0, s, canon_codes, codes, (uint16_t*)scales,
                       rows, nchunk, perm_I);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(interleave_chunks_kernel, dim3(grid_for(n)), dim3(256), 0, s, (const u32x4*)canon_codes, codes,
                     rows, nchunk, perm_I);
  if (fmt == FMT_MXFP4)
    hipLaunchKernelGGL(interleave_scales_kernel<uint8_t>, dim3(grid_for(n)), dim3(256), 0, s, canon_scales, scales,
                       rows, nchunk, perm_I);
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(pack_nvfp4_scales_kernel, dim3(grid_for(n)), dim3(256), 0, s, canon_scales, (uint16_t*)scales,
                       rows, R, nchunk, perm_I);
  if (fmt == FMT_FP8_B128) {
    hipError_t e = hipMemcpyAsync(scales, canon_scales, (size_t)(rows / 128) * (K / 128) * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

// One thread per 16-byte chunk: Chunk<FMT>::decode to bf16 pairs, then the chunk's scale applied
// in fp32, written row-major.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                      int rows, int K, int perm_I, const float* __restrict__ tscale,
                                                      float* __restrict__ out) {
#pragma clang fp contract(off)
  using C = Chunk<FMT>;
  const int nchunk = K / C::ELEMS;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * nchunk) return;
  const int r = (int)(idx / nchunk), c = (int)(idx % nchunk);  // logical row
  const int dr = perm_I ? w13_device_row(r, perm_I) : r;          // its device row
  const u32x4 v = *(const u32x4*)(codes + ilv_chunk_off(dr, c, nchunk));
  uint32_t p[C::PAIRS];
  C::decode(v, p);
  float sc = 1.0f;
  if constexpr (FMT == FMT_Q4_0) sc = fp16_bits_to_f32(((const uint16_t*)scales)[ilv_scale_idx(dr, c, nchunk)]);
  if constexpr (FMT == FMT_MXFP4) sc = e8m0_to_f32(scales[ilv_scale_idx(dr, c, nchunk)]);
  if constexpr (FMT == FMT_FP8_B128) sc = ((const float*)scales)[(size_t)(r / 128) * (K / 128) + (c * C::ELEMS) / 128];
  float sc_hi = sc, ts = 1.0f;
  if constexpr (FMT == FMT_NVFP4) {  // e4m3 scales of the chunk's two halves, and the matrix scale
    const uint32_t two = ((const uint16_t*)scales)[ilv_scale_idx(dr, c, nchunk)];
    sc = e4m3_to_f32(two & 0xffu);
    sc_hi = e4m3_to_f32(two >> 8);
    ts = *tscale;
  }
  float* o = out + (size_t)r * K + (size_t)c * C::ELEMS;
#pragma unroll
  for (int i = 0; i < C::PAIRS; ++i) {
    float v0 = bf16_bits_to_f32(p[i] & 0xffffu), v1 = bf16_bits_to_f32(p[i] >> 16);
    if constexpr (FMT == FMT_Q4_0) {
      v0 = v0 - 136.0f;  // decode gives 128 + q; the weight is scale * (q - 8)
      v1 = v1 - 136.0f;
    }
    if constexpr (FMT == FMT_NVFP4) {  // t * (e2m1 * e4m3): the inner product is exact
      const float s = i < C::PAIRS / 2 ? sc : sc_hi;
      v0 = ts * (v0 * s);
      v1 = ts * (v1 * s);
    } else if constexpr (FMT != FMT_BF16) {
      v0 = v0 * sc;
      v1 = v1 * sc;
    }
    o[2 * i] = v0;
    o[2 * i + 1] = v1;
  }
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int rows, int K, int perm_I,
                          const float* tscale, float* out, hipStream_t s) {
  const int elems = fmt == FMT_BF16 ? 8 : fmt == FMT_FP8_B128 ? 16 : 32;
  const long long n = (long long)rows * (K / elems);
  dim3 grid(grid_for(n)), block(256);
  switch (fmt) {
#define FT_DQ(F) hipLaunchKernelGGL(dequant_kernel<F>, grid, block, 0, s, codes, scales, rows, K, perm_I, tscale, out)
    case FMT_BF16: FT_DQ(FMT_BF16); break;
    case FMT_Q4_0: FT_DQ(FMT_Q4_0); break;
    case FMT_MXFP4: FT_DQ(FMT_MXFP4); break;
    case FMT_NVFP4: FT_DQ(FMT_NVFP4); break;
    default: FT_DQ(FMT_FP8_B128); break;
#undef FT_DQ
  }
  return hipGetLastError();
}

}  // namespace ftk
