// Streaming grouped GEMV for expert groups with few tokens (decode).
//
// Expert FFNs are read from per-format quantised banks (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", section 五).  With a handful of tokens per expert the work is one
// pass over the expert's weights, so the kernel is bound by HBM bandwidth: every byte of a touched
// expert's weights is read once per chunk of up to NT tokens, decoded in registers to bf16 pairs
// and multiplied against the activations with v_dot2_f32_bf16 (fp32 accumulate).  Block scales
// multiply the fp32 partial sum of their block, so every weight is used exactly as its format
// defines it.
//
// Mapping onto the row-interleaved bank layout (chunk c of 64 consecutive rows = 1 KiB contiguous):
//   - lane l of every wave owns row l of the item's row block, so one 16-byte load per lane reads
//     1 KiB of contiguous weights and each lane accumulates a whole row: no cross-lane reduction;
//   - the WPB waves of a block split K: wave w takes chunks w, w+WPB, ...; their partial sums meet
//     in LDS and are added in wave order (deterministic);
//   - the item's activation rows and its rows' block scales are staged once in LDS; all lanes of a
//     wave read the same chunk, so every activation read is an LDS broadcast on the LDS counter,
//     and the vector-load counter carries nothing but the weight codes, which run PF chunks ahead
//     of the arithmetic.
// Block work item = (group, chunk of up to NT tokens, 64-row device block cb):
//   gate/up: a W13 device block holds gate rows 32cb.. (lanes 0-31) and the matching up rows
//            (lanes 32-63) -> h = SiLU(g) * u for 32 columns, rounded to bf16 into the h workspace;
//   down:    W2 rows 64cb..64cb+63 -> 64 output columns of y, rounded to bf16.
// The grid is sized to the blocks the device holds at once; blocks walk the item list with a stride.
#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"

namespace ftk {

constexpr int GV_RPL = 1;  // row blocks per item (one row of each per lane)
constexpr int GV_PF = 6;   // chunks of weights in flight per lane (prefetch ring)

typedef const __attribute__((address_space(4))) uint32_t* scalar_u32p;  // read through the scalar cache

template <int FMT>
__device__ __forceinline__ size_t mat_bytes(int rows, int K) {
  return FMT == FMT_BF16 ? (size_t)rows * K * 2 : FMT == FMT_FP8_B128 ? (size_t)rows * K : (size_t)rows * K / 2;
}

// dynamic LDS: [groups: 4 x (E+2) ints][tmp: 4 ints][x rows NT x K bf16, item scales | partial sums]
__host__ __device__ inline size_t gv_group_bytes(int E) { return ((size_t)4 * (E + 2) * 4 + 16 + 15) & ~(size_t)15; }
// per-(row, chunk) scale bytes of one 64-row block (Q4_0: fp16, MXFP4: E8M0; none otherwise)
__host__ __device__ inline size_t gv_scale_bytes(int fmt, int K) {
  return fmt == FMT_Q4_0 ? (size_t)64 * (K / 32) * 2 : fmt == FMT_MXFP4 ? (size_t)64 * (K / 32) : 0;
}
// Q4_0: per-(token, 32-element block) activation sums, fp32
__host__ __device__ inline size_t gv_xsum_bytes(int fmt, int K, int NT) {
  return fmt == FMT_Q4_0 ? (size_t)NT * (K / 32) * 4 : 0;
}
__host__ __device__ inline size_t gv_union_bytes(int fmt, int K, int NT, int WPB) {
  const size_t xb = (size_t)NT * K * 2 + gv_scale_bytes(fmt, K) + gv_xsum_bytes(fmt, K, NT);
  const size_t rb = (size_t)WPB * GV_RPL * NT * 64 * 4;
  return xb > rb ? xb : rb;
}

template <int FMT, bool GATEUP, int WPB, int NT>
__global__ __launch_bounds__(WPB * 64) void gemv_kernel(FfnArgs a) {
  using C = Chunk<FMT>;
  constexpr int RPL = GV_RPL, PF = GV_PF, NTHR = WPB * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint8_t* s_union = lds + gv_group_bytes(a.E);
  uint16_t* s_x = (uint16_t*)s_union;  // [NT][K] activation rows of the item
  uint8_t* s_sc = s_union + (size_t)NT * (GATEUP ? a.d : a.I) * 2;  // [nchunk][64] scales of the item's rows
  float* s_xsum = (float*)(s_sc + gv_scale_bytes(FMT, GATEUP ? a.d : a.I));  // [NT][K/32] (Q4_0)
  float* s_red = (float*)s_union;      // [WPB][RPL][NT][64] partial sums (after the K loop)

  const int K = GATEUP ? a.d : a.I;
  const int nrows = GATEUP ? 2 * a.I : a.d;
  const int ncb = nrows / 64;  // 64-row device blocks
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + NT - 1) / NT) * ncb; });

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nitems = s_item0[gl.n];
  const int nchunk = K / C::ELEMS;
  const int niter = (nchunk - w + WPB - 1) / WPB;  // chunks w, w+WPB, ... of this wave
  const int jlast = niter > 0 ? niter - 1 : 0;
  const size_t mbytes = mat_bytes<FMT>(nrows, K);
  const uint8_t* codes = GATEUP ? a.w13 : a.w2;
  const uint8_t* scales = GATEUP ? a.s13 : a.s2;
  const int TK = a.T * a.k;
  constexpr size_t CSTRIDE = 64 * 16;  // consecutive chunks of one row block are 1 KiB apart

  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    const int g = find_group(s_item0, gl.n, it);
    const int local = it - s_item0[g];
    const int tchunk = local / ncb, cb = local % ncb;
    const int slot = s_slot[g], row0 = s_row0[g], cnt = s_cnt[g];
    const bool shared = row0 >= TK;
    const int t0 = tchunk * NT;
    const int nt = min(NT, cnt - t0);

    // the RPL rows of this lane
    int rowq[RPL];
    rowq[0] = 64 * cb + lane;  // device row (gate/up: lanes 0-31 gate 32cb+l, lanes 32-63 up 32cb+l-32)
    auto chunk_of = [&](int j) { return WPB * j + w; };  // this wave's j-th chunk
    const uint8_t* mat = codes + (size_t)slot * mbytes;
    const uint8_t* rowp[RPL];
#pragma unroll
    for (int q = 0; q < RPL; ++q) rowp[q] = mat + ilv_chunk_off(rowq[q], 0, nchunk);

    // ---- stage the item's activation rows in LDS before the weight prefetch is issued, so waiting
    // for the rows never waits for weights (the vector-load counter is in order).  Token indices
    // come through the scalar cache.
    for (int t = 0; t < nt; ++t) {
      const uint16_t* xr;
      if (GATEUP) {
        const int tok = shared ? t0 + t : (int)((scalar_u32p)(uintptr_t)a.gather)[row0 + t0 + t] / a.k;
        xr = a.x + (size_t)tok * a.d;
      } else {
        xr = a.h + (size_t)(row0 + t0 + t) * a.I;
      }
      for (int e8 = threadIdx.x; e8 < K / 8; e8 += NTHR) {
        const u32x4 v = *(const u32x4*)(xr + 8 * e8);
        *(u32x4*)(s_x + (size_t)t * K + 8 * e8) = v;
        if constexpr (FMT == FMT_Q4_0) {
          // Q4_0 weights are decoded as 128 + q, so each block needs the sum of its 32 activations;
          // four consecutive threads hold one block (K/8 is a multiple of 4, so they stay together)
          float sum = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) sum = dot2_bf16(v[i], 0x3F803F80u, sum);
          sum += __shfl_xor(sum, 1, 64);
          sum += __shfl_xor(sum, 2, 64);
          if ((e8 & 3) == 0) s_xsum[t * (K / 32) + (e8 >> 2)] = sum;
        }
      }
    }
    // the row block's per-(row, chunk) scales are one contiguous run in the bank: stage them too,
    // so the weight stream carries codes only
    if constexpr (FMT == FMT_Q4_0 || FMT == FMT_MXFP4) {
      constexpr int SB = FMT == FMT_Q4_0 ? 2 : 1;
      const uint8_t* src = scales + ((size_t)slot * nrows * nchunk + (size_t)cb * nchunk * 64) * SB;
      for (int i = threadIdx.x; i < nchunk * 64 * SB / 16; i += NTHR)
        *(u32x4*)(s_sc + 16 * (size_t)i) = *(const u32x4*)(src + 16 * (size_t)i);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads below the waits for the rows

    // ---- prefetch ring of PF chunks of codes.  Loads are issued unconditionally, with indices past
    // the wave's last chunk clamped to it, so every path keeps the same loads in flight.
    u32x4 buf[PF][RPL];
    auto issue = [&](u32x4* b, int j) {
      const int c = chunk_of(j);
#pragma unroll
      for (int q = 0; q < RPL; ++q) b[q] = *(const u32x4*)(rowp[q] + (size_t)c * CSTRIDE);
    };
    if (niter > 0) {
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) issue(buf[p], min(p, jlast));
    }

    __syncthreads();

    float acc[RPL][NT];
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = 0.0f;

    for (int j0 = 0; j0 < niter; j0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int j = j0 + p;
        issue(buf[(p + PF - 1) % PF], min(j + PF - 1, jlast));
        if (j < niter) {
          const int c = chunk_of(j);
          float fsc[RPL];
#pragma unroll
          for (int q = 0; q < RPL; ++q) {
            if constexpr (FMT == FMT_FP8_B128) {
              // one fp32 scale per 128x128 block of logical rows (a gate/up device block holds 32 gate
              // rows in lanes 0-31 and the matching 32 up rows in lanes 32-63)
              const float* s32 = (const float*)scales + (size_t)slot * (size_t)(nrows / 128) * (K / 128);
              const int rb = (GATEUP ? 32 * cb + (lane >= 32 ? a.I : 0) : 64 * cb) / 128;
              fsc[q] = s32[(size_t)rb * (K / 128) + (c * 16) / 128];
            } else if constexpr (FMT == FMT_Q4_0) {
              fsc[q] = fp16_bits_to_f32(((const uint16_t*)s_sc)[c * 64 + lane]);
            } else if constexpr (FMT == FMT_MXFP4) {
              fsc[q] = e8m0_to_f32(s_sc[c * 64 + lane]);
            } else {
              fsc[q] = 1.0f;
            }
          }
          uint32_t wp[RPL][C::PAIRS];  // decoded once, used for every token
#pragma unroll
          for (int q = 0; q < RPL; ++q) C::decode(buf[p][q], wp[q]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nt) {
              uint32_t xw[C::PAIRS];
              const u32x4* xs = (const u32x4*)(s_x + (size_t)t * K + (size_t)c * C::ELEMS);
#pragma unroll
              for (int i = 0; i < C::PAIRS / 4; ++i) {
                const u32x4 v = xs[i];
                xw[4 * i] = v[0];
                xw[4 * i + 1] = v[1];
                xw[4 * i + 2] = v[2];
                xw[4 * i + 3] = v[3];
              }
              float xsum = 0.0f;
              if constexpr (FMT == FMT_Q4_0) xsum = s_xsum[t * (K / 32) + c];
#pragma unroll
              for (int q = 0; q < RPL; ++q) {
                float part = 0.0f;
#pragma unroll
                for (int i = 0; i < C::PAIRS; ++i) part = dot2_bf16(wp[q][i], xw[i], part);
                if constexpr (FMT == FMT_Q4_0)
                  acc[q][t] = fmaf(fsc[q], fmaf(-136.0f, xsum, part), acc[q][t]);  // decoded as 128 + q
                else if constexpr (FMT == FMT_BF16)
                  acc[q][t] += part;
                else
                  acc[q][t] = fmaf(part, fsc[q], acc[q][t]);
              }
            }
          }
        }
      }
    }

    // ---- add the waves' partial sums in wave order and write (the x rows are no longer needed)
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt) s_red[((w * RPL + q) * NT + t) * 64 + lane] = acc[q][t];
    __syncthreads();
    for (int t = w; t < nt; t += WPB) {
      const int orow = row0 + t0 + t;  // h row, or y_sorted row
      if (GATEUP) {
        if (lane < 32) {
          float g = 0.0f, u = 0.0f;
#pragma unroll
          for (int ww = 0; ww < WPB; ++ww) {
            g += s_red[(ww * NT + t) * 64 + lane];
            u += s_red[(ww * NT + t) * 64 + lane + 32];
          }
          a.h[(size_t)orow * a.I + 32 * cb + lane] = f32_to_bf16_bits(g / (1.0f + expf(-g)) * u);
        }
      } else {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WPB; ++ww) v += s_red[(ww * NT + t) * 64 + lane];
        uint16_t* yrow = shared ? a.y_shared + (size_t)(t0 + t) * a.d : a.y_sorted + (size_t)orow * a.d;
        yrow[64 * cb + lane] = f32_to_bf16_bits(v);
      }
    }
    __syncthreads();
  }
}

// Tokens per pass and waves per block: all NT activation rows of an item sit in LDS, so long rows
// get fewer tokens per pass and more waves per block (to keep enough loads in flight per CU).
template <int FMT, bool GATEUP, int WPB, int NT>
static hipError_t launch_cfg(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  auto kern = gemv_kernel<FMT, GATEUP, WPB, NT>;
  const int K = GATEUP ? a.d : a.I;
  const size_t lds = gv_group_bytes(a.E) + gv_union_bytes(FMT, K, NT, WPB);
  static int resident_per_cu = -1;  // blocks of this kernel per CU, for the largest LDS request seen
  static size_t resident_lds = 0;
  if (resident_per_cu < 0 || lds > resident_lds) {
    int per_cu = 0;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipGetLastError();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WPB * 64, lds) != hipSuccess)
      return hipGetLastError();
    resident_per_cu = per_cu > 0 ? per_cu : 1;
    resident_lds = lds;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return hipGetLastError();
  const int ncb = (GATEUP ? 2 * a.I : a.d) / 64;
  const long long chunks = (rows_upper + NT - 1) / NT + groups_upper;
  long long blocks = chunks * ncb;
  const long long cap = (long long)resident_per_cu * cus;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WPB * 64), lds, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP>
static hipError_t launch_fmt(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  const int K = GATEUP ? a.d : a.I;
  if (K <= 2048) return launch_cfg<FMT, GATEUP, 4, 4>(a, groups_upper, rows_upper, s);
  return launch_cfg<FMT, GATEUP, 8, 4>(a, groups_upper, rows_upper, s);
}

template <bool GATEUP>
static hipError_t launch_gemv(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  switch (a.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16, GATEUP>(a, groups_upper, rows_upper, s);
    case FMT_Q4_0: return launch_fmt<FMT_Q4_0, GATEUP>(a, groups_upper, rows_upper, s);
    case FMT_MXFP4: return launch_fmt<FMT_MXFP4, GATEUP>(a, groups_upper, rows_upper, s);
    default: return launch_fmt<FMT_FP8_B128, GATEUP>(a, groups_upper, rows_upper, s);
  }
}

hipError_t launch_gemv_gateup(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  return launch_gemv<true>(a, groups_upper, rows_upper, s);
}
hipError_t launch_gemv_down(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  return launch_gemv<false>(a, groups_upper, rows_upper, s);
}

}  // namespace ftk
