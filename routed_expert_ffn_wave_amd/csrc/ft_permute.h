// Stable token -> expert ranking pieces shared by the permutation kernels and the fused decode
// kernel (FreeToken walk-through "深入FreeToken架构…全链路剖析", section 一: expert dispatch).
// Positions come from ballots over the expert-id bits in flat (token, slot) order, never from the
// order in which atomics happen to land, so the permutation is deterministic.
#pragma once
#include "ft_device.h"

namespace ftk {

constexpr int SEG = 1024;  // flat entries per wave segment
constexpr int SEG_STEPS = SEG / 64;

// The segment's expert ids, lane l holding entries seg_begin + 64 i + l: every load is issued before
// the first is used, so the segment costs one memory latency, not one per step.
__device__ __forceinline__ void load_segment(const int32_t* __restrict__ ids, int seg_begin, int seg_end,
                                             int (&ev)[SEG_STEPS]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < SEG_STEPS; ++i) {
    const int f = seg_begin + 64 * i + lane;
    ev[i] = f < seg_end ? ids[f] : -1;
  }
}

__device__ __forceinline__ uint64_t peers_of(int e, bool active, int id_bits) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < id_bits; ++b) {
    uint64_t bal = __ballot(active && ((e >> b) & 1));
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return m;
}

// Walk one segment in order and scatter; `base` (LDS, length E) holds this segment's next sorted
// position per expert and is advanced in place.  Only this wave touches `base`.
__device__ __forceinline__ void scatter_segment(const int32_t* __restrict__ ids, int n, int E, int seg_begin,
                                                int id_bits, int* base, int32_t* __restrict__ gather,
                                                int32_t* __restrict__ inv) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int seg_end = min(seg_begin + SEG, n);
  int ev[SEG_STEPS];
  load_segment(ids, seg_begin, seg_end, ev);
#pragma unroll
  for (int i = 0; i < SEG_STEPS; ++i) {
    const int f0 = seg_begin + 64 * i;
    if (f0 >= seg_end) break;
    const int f = f0 + lane;
    const int e_raw = ev[i];
    const bool active = f < seg_end && (unsigned)e_raw < (unsigned)E;  // invalid ids get no position
    const int e = active ? e_raw : 0;
    const uint64_t peers = peers_of(e, active, id_bits);
    int pos = 0;
    if (active) {
      pos = base[e] + __popcll(peers & lt);
      gather[pos] = f;
      inv[f] = pos;
    }
    __builtin_amdgcn_wave_barrier();
    // the highest lane of each peer set advances the running base
    if (active && (peers >> lane) == 1ull) base[e] = pos + 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

__device__ __forceinline__ void count_segment(const int32_t* __restrict__ ids, int n, int E, int seg_begin,
                                              int* hist) {
  const int seg_end = min(seg_begin + SEG, n);
  int ev[SEG_STEPS];
  load_segment(ids, seg_begin, seg_end, ev);
#pragma unroll
  for (int i = 0; i < SEG_STEPS; ++i) {
    const int e = ev[i];  // -1 past the end; ids outside [0, E) are skipped
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
}

// Exclusive prefix sum of a[0..n) into out[0..n] (out[n] = total) by one wave; a and out may be LDS.
__device__ __forceinline__ void wave_exclusive_scan(const int* a, int n, int* out) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int b = lane * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) loc += a[b + i];
  int x = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  int run = x - loc;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int c = a[b + i];
      out[b + i] = run;
      run += c;
    }
  if (lane == 63) out[n] = x;
}

}  // namespace ftk
