// Router top-k of one token by one wave64, shared by the router kernel and the fused decode
// prologue.
//
// Each token activates only k of its E experts (zuoshipin.com FreeToken article, section
// "为什么 MoE 模型适合做 CPU–GPU 协同？"; FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五).  The selection order is: larger logit first, equal logits by lower expert index.
// Softmax is strictly increasing, so choosing on the fp32 logits is choosing on the
// probabilities, without ties introduced by rounding exp().
//
// Lane l holds experts l, l+64, ... (VPL values per lane, E <= 64 * VPL).  Each of the k rounds
// finds the largest remaining logit with DPP row exchanges (no LDS round trips) and its lowest
// index with one ballot per value group; every lane ends with the same winner.
#pragma once
#include <climits>
#include <type_traits>

#include "ft_device.h"

namespace ftk {

// Maximum of v over the wave, returned to every lane: DPP exchanges inside each row of 16 lanes,
// then the four row maxima read as scalars.
__device__ __forceinline__ float wave_max_dpp(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                  0xf, 0xf, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Lane j < k returns the j-th chosen expert in `e_out` and its renormalised weight
// p_j / sum_i p_i, p_j = exp(logit_j - logit_0), in `w_out`.  All 64 lanes must call it.
// Round j: the largest remaining logit m (retired candidates count as -inf), then the lowest
// expert index among the remaining candidates equal to m (ballots in index order); its lane
// retires it.  Equal values, -0.0 and +0.0 included, therefore go in ascending index order.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int& e_out, float& w_out) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? row[e] : 0.0f;
  }
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (lane + 64 * i < E) live |= 1u << i;

  float my_v = 0.0f;  // lane j keeps the j-th chosen logit
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float best = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if ((live >> i) & 1u) best = fmaxf(best, v[i]);
    const float m = wave_max_dpp(best);
    int e = 0x7fffffff;
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i) {  // lowest index wins: scan from the last group down
      const uint64_t bal = __ballot(((live >> i) & 1u) && v[i] == m);
      if (bal) e = 64 * i + (int)__builtin_ctzll(bal);
    }
    if ((e & 63) == lane) live &= ~(1u << (e >> 6));
    if (lane == j) {
      my_v = m;
      my_e = e;
    }
  }
  const float m0 = __shfl(my_v, 0, 64);
  const float p = (lane < k) ? expf(my_v - m0) : 0.0f;
  const float s = wave_sum(p);
  e_out = my_e;
  w_out = p / s;
}


// ---------------------------------------------------------------------------------------------
// Four tokens per wave, one per row of 16 lanes (E <= 16 * VPR, k <= 16).  Logits become integer
// keys whose signed order is the IEEE order with -0.0 folded onto +0.0, so each round is an
// integer max over the row (4 DPP steps) and an integer min over the indices holding it (4 more):
// no cross-row traffic at all.  Lane l16 of row r holds experts l16, l16 + 16, ... of token
// t_base + r; missing and retired candidates hold INT_MIN, below every real key (-inf included).

__device__ __forceinline__ int float_key(float f) {
  const int b = __builtin_bit_cast(int, f + 0.0f);  // -0.0 + 0.0 = +0.0
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_float(int key) { return __builtin_bit_cast(float, key ^ ((key >> 31) & 0x7fffffff)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
// all-reduce over the 16 lanes of each row: quad swaps, then the mirrors pair quads and halves
__device__ __forceinline__ int row_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  return max(v, dpp_i<0x140>(v));
}
__device__ __forceinline__ int row_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  return min(v, dpp_i<0x140>(v));
}
__device__ __forceinline__ float row_sum_f(float v) {
  v += __builtin_bit_cast(float, dpp_i<0xB1>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i<0x4E>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i<0x141>(__builtin_bit_cast(int, v)));
  return v + __builtin_bit_cast(float, dpp_i<0x140>(__builtin_bit_cast(int, v)));
}

// Lane l16 < k of a row whose token exists returns the l16-th chosen expert and its renormalised
// weight; `ok` tells the lane whether it holds a result.  All 64 lanes must call it.
template <int VPR>
__device__ __forceinline__ void route_rows(const float* __restrict__ logits, int T, int E, int k, int t_base,
                                           int& e_out, float& w_out, bool& ok) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int t = t_base + (lane >> 4);
  const bool tok = t < T;
  const float* row = logits + (size_t)(tok ? t : 0) * E;
  int key[VPR];
#pragma unroll
  for (int i = 0; i < VPR; ++i) {
    const int e = 16 * i + l16;
    key[i] = (tok && e < E) ? float_key(row[e]) : INT_MIN;
  }
  int my_key = INT_MIN, my_e = 0, key0 = INT_MIN;
  for (int j = 0; j < k; ++j) {
    int best = key[0];
#pragma unroll
    for (int i = 1; i < VPR; ++i) best = max(best, key[i]);
    const int m = row_max_i(best);
    if (j == 0) key0 = m;  // the row's largest logit, in every lane
    // lowest index holding m in this lane: a min over independent selects, not a chain
    int cand = INT_MAX;
#pragma unroll
    for (int i = 0; i < VPR; ++i) cand = min(cand, key[i] == m ? 16 * i + l16 : INT_MAX);
    if (m == INT_MIN) cand = INT_MAX;  // nothing left (a missing token)
    const int e = row_min_i(cand);
#pragma unroll
    for (int i = 0; i < VPR; ++i)
      if (e == 16 * i + l16) key[i] = INT_MIN;  // retire
    if (l16 == j) {
      my_key = m;
      my_e = e;
    }
  }
  // p_j = exp(v_j - v_0) over the row's k chosen logits, w_j = p_j / sum p
  const float p = (l16 < k) ? expf(key_float(my_key) - key_float(key0)) : 0.0f;
  const float s = row_sum_f(p);
  ok = tok && l16 < k;
  e_out = my_e;
  w_out = p / s;
}

// Route tokens 0..T-1 with the waves wave, wave + nwaves, ... (wave-uniform arguments): four tokens
// per wave with route_rows when E <= 256 and k <= 16, else one per wave with route_token.
// store(t, j, e, w) receives the j-th choice of token t.
inline __host__ __device__ bool route_by_rows(int E, int k) { return E <= 256 && k <= 16; }

template <int VPL, class Store>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int T, int E, int k, int wave,
                                             int nwaves, Store store) {
  const int lane = threadIdx.x & 63;
  if constexpr (VPL <= 4) {
    if (route_by_rows(E, k)) {
      for (int tb = 4 * wave; tb < T; tb += 4 * nwaves) {
        int e;
        float wt;
        bool ok;
        route_rows<4 * VPL>(logits, T, E, k, tb, e, wt, ok);
        if (ok) store(tb + (lane >> 4), lane & 15, e, wt);
      }
      return;
    }
  }
  for (int t = wave; t < T; t += nwaves) {
    int e;
    float wt;
    route_token<VPL>(logits + (size_t)t * E, E, k, e, wt);
    if (lane < k) store(t, lane, e, wt);
  }
}

}  // namespace ftk
