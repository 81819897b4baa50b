// Router projection fused with route: the logits x . w_router^T on the matrix cores, then the
// top-k of each token's row, in one launch.
//
// Each token activates only k of its E experts (FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五); the router logits that choose them are the token's activation row against each
// expert's router row.  Block (token tile of 16, expert tile of 64): each of its 4 waves computes
// 16 tokens x 16 experts with v_mfma_f32_16x16x32_bf16 straight from global memory (16 bytes of a
// row per lane and K step of 32), four accumulators over K for independent MFMAs, and stores its
// logits with agent-scope stores.  The block that brings its token tile's counter to the number
// of expert tiles has every logit of those 16 tokens complete: it copies them to LDS with
// agent-scope loads, routes them with the routine of ft_moe_route, and returns the counter to zero.
#include "ft_device.h"
#include "ft_kernels.h"
#include "ft_route.h"

namespace ftk {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int RP_TT = 16;   // tokens per block
constexpr int RP_EB = 64;   // experts per block (16 per wave)
constexpr int RP_CNT = 16;  // ints between two token tiles' counters (one 64-byte line each)
constexpr int RP_EMAX = 512;

__device__ __forceinline__ void rp_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rp_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rp_wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int VPL>
__global__ __launch_bounds__(256) void route_proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                         int T, int d, int E, int k, float* logits, int32_t* ids,
                                                         float* w, int32_t* cnt) {
  __shared__ float s_log[RP_TT * RP_EMAX];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RP_TT;
  const int e0 = blockIdx.y * RP_EB + 16 * wv;
  // MFMA operands: A = 16 token rows x 32 K (lane: row lane % 16, K 8 (lane / 16) .. + 7), B = 32 K x
  // 16 expert rows (lane: expert lane % 16, same K).  Rows past T or E repeat the last one; their
  // results are not stored.
  const int ta = min(t0 + (lane & 15), T - 1);
  const int eb = min(e0 + (lane & 15), E - 1);
  const uint16_t* xa = x + (size_t)ta * d + 8 * (lane >> 4);
  const uint16_t* wb = wr + (size_t)eb * d + 8 * (lane >> 4);
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int kk = 0;
  for (; kk + 128 <= d; kk += 128) {
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = *(const bf16x8*)(xa + kk + 32 * q);
      bv[q] = *(const bf16x8*)(wb + kk + 32 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], bv[q], acc[q], 0, 0, 0);
  }
  for (; kk < d; kk += 32)
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xa + kk), *(const bf16x8*)(wb + kk), acc[0], 0, 0, 0);
  // lane holds tokens t0 + 4 (lane / 16) + i, expert e0 + lane % 16
  const int e = e0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * (lane >> 4) + i;
    const float v = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    if (t < T && e < E) rp_store(logits + (size_t)t * E + e, v);
  }
  rp_wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt + blockIdx.x * RP_CNT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (int)gridDim.y - 1;
  __syncthreads();
  if (!s_last) return;
  // every expert tile of these tokens has stored its logits (each block completed its stores
  // before its counter update)
  const int nt = min(RP_TT, T - t0);
  for (int i = threadIdx.x; i < nt * E; i += 256) s_log[i] = rp_load(logits + (size_t)t0 * E + i);
  __syncthreads();
  route_tokens<VPL>(s_log, nt, E, k, wv, 4, [&](int t, int j, int ee, float wt) {
    ids[(size_t)(t0 + t) * k + j] = ee;
    w[(size_t)(t0 + t) * k + j] = wt;
  });
  if (threadIdx.x == 0) __hip_atomic_store(cnt + blockIdx.x * RP_CNT, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t route_proj_workspace_bytes(int T) { return (size_t)((T + RP_TT - 1) / RP_TT) * RP_CNT * sizeof(int32_t); }

hipError_t launch_route_proj(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int k, float* logits,
                             int32_t* ids, float* w, void* ws, hipStream_t s) {
  dim3 grid((T + RP_TT - 1) / RP_TT, (E + RP_EB - 1) / RP_EB), block(256);
  int32_t* cnt = (int32_t*)ws;
  if (E <= 64)
    hipLaunchKernelGGL(route_proj_kernel<1>, grid, block, 0, s, x, wr, T, d, E, k, logits, ids, w, cnt);
  else if (E <= 128)
    hipLaunchKernelGGL(route_proj_kernel<2>, grid, block, 0, s, x, wr, T, d, E, k, logits, ids, w, cnt);
  else if (E <= 256)
    hipLaunchKernelGGL(route_proj_kernel<4>, grid, block, 0, s, x, wr, T, d, E, k, logits, ids, w, cnt);
  else
    hipLaunchKernelGGL(route_proj_kernel<8>, grid, block, 0, s, x, wr, T, d, E, k, logits, ids, w, cnt);
  return hipGetLastError();
}

}  // namespace ftk
