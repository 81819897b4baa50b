// Weighted combine of expert outputs back to token order, plus the residual mask of experts that
// are not resident in the bank (FreeToken walk-through "深入FreeToken架构…全链路剖析", section 五:
// experts that are not on the GPU are handed to another path; their share is not added here and
// the weights are not renormalised).
//
// One block per token (blockDim 256); each thread owns 8 consecutive columns (one 16-byte bf16
// load per expert row), sums the k expert rows in j order in fp32, then adds the shared expert.
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_sorted,
                                                      const uint16_t* __restrict__ y_shared,
                                                      const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv,
                                                      const int32_t* __restrict__ slot_of, int n_slots, int E,
                                                      int k, int d,
                                                      void* __restrict__ out, uint32_t* __restrict__ mask) {
  const int t = blockIdx.x;
  __shared__ int s_row[32];
  __shared__ float s_w[32];
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    bool nonres = false;
    if (j < k) {
      const int e = ids[(size_t)t * k + j];
      // an invalid id, or a slot outside [0, n_slots), counts as not resident
      nonres = (unsigned)e >= (unsigned)E || (unsigned)slot_of[e] >= (unsigned)n_slots;
      s_row[j] = nonres ? -1 : inv[(size_t)t * k + j];
      s_w[j] = w[(size_t)t * k + j];
    }
    const uint64_t bits = __ballot(nonres);
    if (j == 0 && mask) mask[t] = (uint32_t)bits;
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = s_row[j];
      if (r < 0) continue;
      const u32x4 v = *(const u32x4*)(y_sorted + (size_t)r * d + c);
      const float wj = s_w[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj, bf16_bits_to_f32(v[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj, bf16_bits_to_f32(v[i] >> 16), acc[2 * i + 1]);
      }
    }
    if (y_shared) {
      const u32x4 v = *(const u32x4*)(y_shared + (size_t)t * d + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_bits_to_f32(v[i] & 0xffffu);
        acc[2 * i + 1] += bf16_bits_to_f32(v[i] >> 16);
      }
    }
    if (OUT_BF16) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i]) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16);
      *(u32x4*)((uint16_t*)out + (size_t)t * d + c) = o;
    } else {
      f32x4* o = (f32x4*)((float*)out + (size_t)t * d + c);
      o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

hipError_t launch_combine(const uint16_t* y_sorted, const uint16_t* y_shared, const int32_t* ids, const float* w,
                          const int32_t* inv, const int32_t* slot_of, int n_slots, int T, int E, int k, int d,
                          void* out, uint32_t* mask, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, y_sorted, y_shared, ids, w, inv, slot_of, n_slots,
                       E, k, d, out, mask);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, y_sorted, y_shared, ids, w, inv, slot_of,
                       n_slots, E, k, d, out, mask);
  return hipGetLastError();
}

}  // namespace ftk
