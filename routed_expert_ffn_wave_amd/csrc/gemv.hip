// Streaming grouped GEMV for expert groups with few tokens (decode).
//
// Expert FFNs are read from per-format quantised banks (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", section 五).  With a handful of tokens per expert the work is one
// pass over the expert's weights, so the kernel is bound by HBM bandwidth: every byte of a touched
// expert's weights is read exactly once per token chunk, straight from HBM into registers with one
// 16-byte load per row per lane, decoded in registers to bf16 pairs, and multiplied against the
// activations with v_dot2_f32_bf16 (fp32 accumulate).  Block scales multiply the fp32 partial sum
// of their block, so every weight value is used exactly as the format defines it.
//
// Work item = (group, chunk of up to GEMV_NT tokens, tile of output columns); each wave takes items
// in turn.  A wave spreads K over its 64 lanes, each lane owning whole 16-byte chunks, and reduces
// the per-lane partial sums across the wave at the end of the item.
//   gate/up: tile = 2 intermediate columns i -> weight rows {i, i+1} (gate) and {I+i, I+i+1} (up);
//            h = SiLU(g) * u is rounded to bf16 and written to the h workspace.
//   down:    tile = 4 output columns -> 4 rows of W2; y is rounded to bf16.
#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"

namespace ftk {

template <int FMT>
__device__ __forceinline__ size_t code_row_bytes(int K) {
  return FMT == FMT_BF16 ? (size_t)K * 2 : FMT == FMT_FP8_B128 ? (size_t)K : (size_t)K / 2;
}

// Build the activation bf16 pairs that match Chunk<FMT>::decode's code order.
template <int FMT>
__device__ __forceinline__ void x_pairs(const uint16_t* xrow_chunk, uint32_t* xp) {
  using C = Chunk<FMT>;
  const u32x4* p = (const u32x4*)xrow_chunk;
  uint32_t X[C::ELEMS / 2];
#pragma unroll
  for (int i = 0; i < C::ELEMS / 8; ++i) {
    u32x4 v = p[i];
    X[4 * i] = v[0];
    X[4 * i + 1] = v[1];
    X[4 * i + 2] = v[2];
    X[4 * i + 3] = v[3];
  }
  if constexpr (FMT == FMT_Q4_0) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int m = 2 * w + 8 * (s & 1);
        xp[4 * w + s] = __builtin_amdgcn_perm(X[m + 1], X[m], (s >> 1) ? 0x07060302u : 0x05040100u);
      }
  } else {
#pragma unroll
    for (int i = 0; i < C::PAIRS; ++i) xp[i] = X[i];
  }
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void gemv_kernel(FfnArgs a) {
  using C = Chunk<FMT>;
  constexpr int NT = GEMV_NT;
  constexpr int NR = 4;                  // weight rows per item
  constexpr int NCOL = GATEUP ? 2 : 4;   // output columns per item
  __shared__ int s_slot[1025], s_row0[1025], s_cnt[1025], s_item0[1026], s_tmp[4];

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? a.I : a.d;
  const int tiles = ncols / NCOL;
  const int nrows_mat = GATEUP ? 2 * a.I : a.d;  // rows of the weight matrix
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + NT - 1) / NT) * tiles; });

  const int lane = threadIdx.x & 63;
  const int nitems = s_item0[gl.n];
  const int nwaves = gridDim.x * 4;
  const int nchunk = K / C::ELEMS;
  const size_t rbytes = code_row_bytes<FMT>(K);
  const uint8_t* codes = GATEUP ? a.w13 : a.w2;
  const uint8_t* scales = GATEUP ? a.s13 : a.s2;
  const int TK = a.T * a.k;

  for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += nwaves) {
    const int g = find_group(s_item0, gl.n, it);
    const int local = it - s_item0[g];
    const int tchunk = local / tiles, tile = local % tiles;
    const int slot = s_slot[g], row0 = s_row0[g], cnt = s_cnt[g];
    const bool shared = row0 >= TK;
    const int t0 = tchunk * NT;
    const int nt = min(NT, cnt - t0);

    // activation row of local token `lane` (lanes >= nt unused)
    const uint16_t* my_in = nullptr;
    if (lane < nt) {
      if (GATEUP) {
        const int tok = shared ? (t0 + lane) : (a.gather[row0 + t0 + lane] / a.k);
        my_in = a.x + (size_t)tok * a.d;
      } else {
        my_in = a.h + (size_t)(row0 + t0 + lane) * a.I;
      }
    }

    // per-token input rows, broadcast while the whole wave is active
    const uint16_t* xin[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xin[t] = (const uint16_t*)__shfl((long long)(uintptr_t)my_in, t, 64);

    int wrow[NR];
    if (GATEUP) {
      const int i0 = tile * 2;
      wrow[0] = i0;
      wrow[1] = i0 + 1;
      wrow[2] = a.I + i0;
      wrow[3] = a.I + i0 + 1;
    } else {
#pragma unroll
      for (int r = 0; r < NR; ++r) wrow[r] = tile * 4 + r;
    }
    const uint8_t* rowp[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) rowp[r] = codes + ((size_t)slot * nrows_mat + wrow[r]) * rbytes;

    float acc[NR][NT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = 0.0f;

    for (int ch = lane; ch < nchunk; ch += 64) {
      uint32_t wp[NR][C::PAIRS];
      float sc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 c = *(const u32x4*)(rowp[r] + (size_t)ch * 16);
        C::decode(c, wp[r]);
        if constexpr (FMT == FMT_Q4_0) {
          const uint16_t* s16 = (const uint16_t*)scales;
          sc[r] = fp16_bits_to_f32(s16[((size_t)slot * nrows_mat + wrow[r]) * (K / 32) + ch]);
        } else if constexpr (FMT == FMT_MXFP4) {
          sc[r] = e8m0_to_f32(scales[((size_t)slot * nrows_mat + wrow[r]) * (K / 32) + ch]);
        } else if constexpr (FMT == FMT_FP8_B128) {
          const float* s32 = (const float*)scales;
          sc[r] = s32[((size_t)slot * (nrows_mat / 128) + wrow[r] / 128) * (K / 128) + (ch * 16) / 128];
        } else {
          sc[r] = 1.0f;
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nt) {
          uint32_t xp[C::PAIRS];
          x_pairs<FMT>(xin[t] + (size_t)ch * C::ELEMS, xp);
          float xsum = 0.0f;
          if constexpr (FMT == FMT_Q4_0) {
#pragma unroll
            for (int i = 0; i < C::PAIRS; ++i) xsum = dot2_bf16(xp[i], 0x3F803F80u, xsum);
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < C::PAIRS; ++i) part = dot2_bf16(wp[r][i], xp[i], part);
            if constexpr (FMT == FMT_Q4_0)
              acc[r][t] = fmaf(sc[r], fmaf(-136.0f, xsum, part), acc[r][t]);
            else if constexpr (FMT == FMT_BF16)
              acc[r][t] += part;
            else
              acc[r][t] = fmaf(part, sc[r], acc[r][t]);
          }
        }
      }
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        float v[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = wave_sum(acc[r][t]);
        const int orow = row0 + t0 + t;  // h row, or y_sorted row
        if (GATEUP) {
          if (lane < 2) {
            const float gte = lane ? v[1] : v[0];
            const float up = lane ? v[3] : v[2];
            const float hv = gte / (1.0f + expf(-gte)) * up;
            a.h[(size_t)orow * a.I + tile * 2 + lane] = f32_to_bf16_bits(hv);
          }
        } else {
          if (lane < 4) {
            const float yv = lane == 0 ? v[0] : lane == 1 ? v[1] : lane == 2 ? v[2] : v[3];
            uint16_t* yrow = shared ? a.y_shared + (size_t)(t0 + t) * a.d : a.y_sorted + (size_t)orow * a.d;
            yrow[tile * 4 + lane] = f32_to_bf16_bits(yv);
          }
        }
      }
    }
  }
}

template <bool GATEUP>
static hipError_t launch_gemv(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  const int tiles = GATEUP ? a.I / 2 : a.d / 4;
  long long items = (long long)chunks_upper * tiles;
  long long blocks = (items + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(256);
  switch (a.fmt) {
    case FMT_BF16: hipLaunchKernelGGL((gemv_kernel<FMT_BF16, GATEUP>), grid, block, 0, s, a); break;
    case FMT_Q4_0: hipLaunchKernelGGL((gemv_kernel<FMT_Q4_0, GATEUP>), grid, block, 0, s, a); break;
    case FMT_MXFP4: hipLaunchKernelGGL((gemv_kernel<FMT_MXFP4, GATEUP>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<FMT_FP8_B128, GATEUP>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_gateup(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  return launch_gemv<true>(a, chunks_upper, s);
}
hipError_t launch_gemv_down(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  return launch_gemv<false>(a, chunks_upper, s);
}

}  // namespace ftk
