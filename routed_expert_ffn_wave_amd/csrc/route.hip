// Router top-k with renormalised softmax weights, one wave64 per token.
//
// Each token activates only k of its E experts (zuoshipin.com FreeToken article, section
// "为什么 MoE 模型适合做 CPU–GPU 协同？"; FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五).  The selection order is: larger logit first, equal logits by lower expert index.
// Softmax is strictly increasing, so choosing on the fp32 logits is choosing on the
// probabilities, without ties introduced by rounding exp().
//
// Lane l holds experts l, l+64, ... (up to 16 per lane for E <= 1024).  Each of the k rounds
// takes the lane's best remaining (logit, index) pair and reduces it across the wave with
// butterfly shuffles; every lane ends with the same winner, and the owning lane retires it.
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

struct Cand {
  float v;
  int e;  // INT_MAX: no candidate
};

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  // does (av, ae) come before (bv, be) in route order?  Missing candidates come last.
  if (ae == 0x7fffffff) return false;
  if (be == 0x7fffffff) return true;
  return av > bv || (av == bv && ae < be);
}

template <int VPL>  // values per lane
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    v[i] = (e < E) ? row[e] : 0.0f;
  }
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (lane + 64 * i < E) live |= 1u << i;

  float my_v = 0.0f;  // lane j keeps the j-th chosen logit
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      // within a lane, candidates come in ascending index, so strict '>' keeps the lowest index
      if ((live >> i) & 1u) {
        if (be == 0x7fffffff || v[i] > bv) {
          bv = v[i];
          be = lane + 64 * i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) live &= ~(1u << (be >> 6));
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  // weights: p_j = exp(v_j - v_0), w_j = p_j / sum p
  float m = __shfl(my_v, 0, 64);
  float p = (lane < k) ? expf(my_v - m) : 0.0f;
  float s = wave_sum(p);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = p / s;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace ftk
