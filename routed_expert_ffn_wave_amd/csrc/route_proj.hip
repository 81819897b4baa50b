// Router projection fused with route: the logits x . w_router^T on the matrix cores, then the
// top-k of each token's row, in one launch.
//
// Each token activates only k of its E experts (FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五); the router logits that choose them are the token's activation row against each
// expert's router row.  Block = (token tile of 16, expert tile of 16), 16 waves: wave w takes the
// K steps of 32 numbered w, w + 16, ... and multiplies them with v_mfma_f32_16x16x32_bf16 straight
// from global memory (16 bytes of a row per lane and step), four accumulators for independent
// MFMAs; the 16 partial tiles are summed through LDS in a fixed order, so a logit does not depend
// on timing.  At decode the K dimension is what is long, so splitting it over the waves is what
// shortens the chain of dependent loads.  The logits are stored with agent-scope stores; the
// block that brings its token tile's counter to the number of expert tiles has every logit of
// those 16 tokens complete: it copies them to LDS with agent-scope loads, routes them with the
// routine of ft_moe_route, and returns the counter to zero.
#include "ft_device.h"
#include "ft_kernels.h"
#include "ft_route.h"

namespace ftk {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int RP_TT = 16;   // tokens per block
constexpr int RP_EB = 16;   // experts per block
constexpr int RP_W = 16;    // waves per block (K split)
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
__global__ __launch_bounds__(RP_W * 64) void route_proj_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr, int T, int d, int E,
                                                               int k, float* logits, int32_t* ids, float* w,
                                                               int32_t* cnt) {
  __shared__ float s_log[RP_TT * RP_EMAX];
  __shared__ float s_part[RP_W][256];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RP_TT;
  const int e0 = blockIdx.y * RP_EB;
  // MFMA operands: A = 16 token rows x 32 K (lane: row lane % 16, K 8 (lane / 16) .. + 7), B = 32 K x
  // 16 expert rows (lane: expert lane % 16, same K).  Rows past T or E repeat the last one; their
  // results are not stored.
  const int ta = min(t0 + (lane & 15), T - 1);
  const int eb = min(e0 + (lane & 15), E - 1);
  const uint16_t* xa = x + (size_t)ta * d + 8 * (lane >> 4);
  const uint16_t* wb = wr + (size_t)eb * d + 8 * (lane >> 4);
  const int nsteps = d / 32;
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int st = wv;
  for (; st + 3 * RP_W < nsteps; st += 4 * RP_W) {
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = *(const bf16x8*)(xa + 32 * (st + q * RP_W));
      bv[q] = *(const bf16x8*)(wb + 32 * (st + q * RP_W));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], bv[q], acc[q], 0, 0, 0);
  }
  for (; st < nsteps; st += RP_W)
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xa + 32 * st), *(const bf16x8*)(wb + 32 * st),
                                                     acc[0], 0, 0, 0);
  // lane holds tokens 4 (lane / 16) + i, expert lane % 16 of the tile
#pragma unroll
  for (int i = 0; i < 4; ++i) s_part[wv][(4 * (lane >> 4) + i) * 16 + (lane & 15)] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
  __syncthreads();
  if (threadIdx.x < 256) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < RP_W; ++q) v += s_part[q][threadIdx.x];
    const int t = t0 + (threadIdx.x >> 4), e = e0 + (threadIdx.x & 15);
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
  for (int i = threadIdx.x; i < nt * E; i += RP_W * 64) s_log[i] = rp_load(logits + (size_t)t0 * E + i);
  __syncthreads();
  route_tokens<VPL>(s_log, nt, E, k, wv, RP_W, [&](int t, int j, int ee, float wt) {
    ids[(size_t)(t0 + t) * k + j] = ee;
    w[(size_t)(t0 + t) * k + j] = wt;
  });
  if (threadIdx.x == 0) __hip_atomic_store(cnt + blockIdx.x * RP_CNT, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t route_proj_workspace_bytes(int T) { return (size_t)((T + RP_TT - 1) / RP_TT) * RP_CNT * sizeof(int32_t); }

hipError_t launch_route_proj(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int k, float* logits,
                             int32_t* ids, float* w, void* ws, hipStream_t s) {
  dim3 grid((T + RP_TT - 1) / RP_TT, (E + RP_EB - 1) / RP_EB), block(RP_W * 64);
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
