// Streaming grouped GEMV for expert groups with few tokens (decode).
//
// Expert FFNs are read from per-format quantised banks (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", section 五).  With a handful of tokens per expert the work is one
// pass over the expert's weights, so the kernel is bound by HBM bandwidth: every byte of a touched
// expert's weights is read once per chunk of up to GEMV_NT tokens, decoded in registers to bf16
// pairs and multiplied against the activations with v_dot2_f32_bf16 (fp32 accumulate).  Block
// scales multiply the fp32 partial sum of their block, so every weight is used exactly as its
// format defines it.
//
// Mapping onto the row-interleaved bank layout (chunk c of 64 consecutive rows = 1 KiB contiguous):
//   - lane l of every wave owns row l of each of RPL row blocks, so one 16-byte load per lane reads
//     1 KiB of contiguous weights and each lane accumulates whole rows: no cross-lane reduction;
//   - the 4 waves of a block split K: wave w takes chunks w, w+4, ..., so a block streams 4 KiB
//     contiguous per step; the 4 partial sums meet in LDS and are added in wave order;
//   - every lane of a wave works on the same chunk, so the activations of a chunk are wave-uniform
//     and arrive through scalar loads (their own counter), never stalling the vector-load stream of
//     weights, which runs PF chunks ahead of the arithmetic.
// Block work item = (group, chunk of up to GEMV_NT tokens, column block):
//   gate/up: the gate rows 64cb.. and the up rows I+64cb.. -> h = SiLU(g) * u for 64 columns,
//            rounded to bf16 into the h workspace;
//   down:    W2 rows 128cb..128cb+127 -> 128 output columns of y, rounded to bf16.
// The grid is sized to the blocks the device holds at once; blocks walk the item list with a stride.
#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"

namespace ftk {

constexpr int GV_RPL = 2;  // row blocks per item (one row of each per lane)
constexpr int GV_PF = 3;   // chunks of weights in flight per lane (prefetch ring)

typedef const __attribute__((address_space(4))) uint32_t* scalar_u32p;  // read through the scalar cache

template <int FMT>
__device__ __forceinline__ size_t mat_bytes(int rows, int K) {
  return FMT == FMT_BF16 ? (size_t)rows * K * 2 : FMT == FMT_FP8_B128 ? (size_t)rows * K : (size_t)rows * K / 2;
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void gemv_kernel(FfnArgs a) {
  using C = Chunk<FMT>;
  constexpr int NT = GEMV_NT, RPL = GV_RPL, PF = GV_PF;
  __shared__ int s_slot[1025], s_row0[1025], s_cnt[1025], s_item0[1026], s_tmp[4];
  __shared__ float s_red[4][RPL][NT][64];

  const int K = GATEUP ? a.d : a.I;
  const int nrows = GATEUP ? 2 * a.I : a.d;
  const int ncb = GATEUP ? a.I / 64 : a.d / 128;  // column blocks
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + NT - 1) / NT) * ncb; });

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nitems = s_item0[gl.n];
  const int nchunk = K / C::ELEMS;
  const int niter = (nchunk - w + 3) / 4;  // chunks w, w+4, ... of this wave
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
    if (GATEUP) {
      rowq[0] = 64 * cb + lane;          // gate row i
      rowq[1] = a.I + 64 * cb + lane;    // up row I + i
    } else {
      rowq[0] = 128 * cb + lane;
      rowq[1] = 128 * cb + 64 + lane;
    }
    const uint8_t* mat = codes + (size_t)slot * mbytes;
    const uint8_t* rowp[RPL];
#pragma unroll
    for (int q = 0; q < RPL; ++q) rowp[q] = mat + ilv_chunk_off(rowq[q], 0, nchunk);

    // ---- prefetch ring of PF chunks (codes and, for Q4_0 / MXFP4, the per-row chunk scales)
    // (raw scale bits are kept in the ring and converted at use, so no load is waited for early)
    u32x4 buf[PF][RPL];
    uint32_t sbuf[PF][RPL];
    auto issue = [&](u32x4* b, uint32_t* sb, int j) {
      const int c = 4 * j + w;
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        b[q] = *(const u32x4*)(rowp[q] + (size_t)c * CSTRIDE);
        if constexpr (FMT == FMT_Q4_0) {
          const uint16_t* s16 = (const uint16_t*)scales + (size_t)slot * ((size_t)nrows * nchunk);
          sb[q] = s16[ilv_scale_idx(rowq[q], c, nchunk)];
        } else if constexpr (FMT == FMT_MXFP4) {
          const uint8_t* s8 = scales + (size_t)slot * ((size_t)nrows * nchunk);
          sb[q] = s8[ilv_scale_idx(rowq[q], c, nchunk)];
        } else {
          sb[q] = 0;
        }
      }
    };
    // Loads are issued unconditionally (indices past the wave's last chunk are clamped to it and
    // the values ignored) so every path has the same number of loads in flight and the wait before
    // each use only covers the chunk being used.
    const int jlast = niter > 0 ? niter - 1 : 0;
    if (niter > 0) {
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) issue(buf[p], sbuf[p], min(p, jlast));
    }

    // wave-uniform activation rows of the item's tokens, through scalar loads (no vector-load wait);
    // slots t >= nt repeat the last real row so every address stays inside its buffer
    const uint16_t* xin[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tt = min(t, nt - 1);
      if (GATEUP) {
        const int tok = shared ? t0 + tt : (int)((scalar_u32p)(uintptr_t)a.gather)[row0 + t0 + tt] / a.k;
        xin[t] = a.x + (size_t)tok * a.d;
      } else {
        xin[t] = a.h + (size_t)(row0 + t0 + tt) * a.I;
      }
    }

    float acc[RPL][NT];
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = 0.0f;

    for (int j0 = 0; j0 < niter; j0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int j = j0 + p;
        issue(buf[(p + PF - 1) % PF], sbuf[(p + PF - 1) % PF], min(j + PF - 1, jlast));
        if (j < niter) {
          const int c = 4 * j + w;
          float fsc[RPL];
#pragma unroll
          for (int q = 0; q < RPL; ++q) {
            if constexpr (FMT == FMT_FP8_B128) {
              // one fp32 scale per 128x128 block: uniform across the wave's 64 rows
              const scalar_u32p s32 =
                  (scalar_u32p)(uintptr_t)(scales + (size_t)slot * (size_t)(nrows / 128) * (K / 128) * 4);
              const int rb = (GATEUP ? (q == 0 ? 64 * cb : a.I + 64 * cb) : 128 * cb + 64 * q) / 128;
              fsc[q] = __uint_as_float(s32[(size_t)rb * (K / 128) + (c * 16) / 128]);
            } else if constexpr (FMT == FMT_Q4_0) {
              fsc[q] = fp16_bits_to_f32((uint16_t)sbuf[p][q]);
            } else if constexpr (FMT == FMT_MXFP4) {
              fsc[q] = e8m0_to_f32(sbuf[p][q]);
            } else {
              fsc[q] = 1.0f;
            }
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nt) {
              const scalar_u32p xs = (scalar_u32p)(uintptr_t)(xin[t] + (size_t)c * C::ELEMS);
              uint32_t xw[C::PAIRS];
#pragma unroll
              for (int i = 0; i < C::PAIRS; ++i) xw[i] = xs[i];
              float xsum = 0.0f;
              if constexpr (FMT == FMT_Q4_0) {
#pragma unroll
                for (int i = 0; i < C::PAIRS; ++i) xsum = dot2_bf16(xw[i], 0x3F803F80u, xsum);
              }
#pragma unroll
              for (int q = 0; q < RPL; ++q) {
                uint32_t wp[C::PAIRS];
                C::decode(buf[p][q], wp);
                float part = 0.0f;
#pragma unroll
                for (int i = 0; i < C::PAIRS; ++i) part = dot2_bf16(wp[i], xw[i], part);
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

    // ---- add the 4 waves' partial sums in wave order and write
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt) s_red[w][q][t][lane] = acc[q][t];
    __syncthreads();
    for (int t = w; t < nt; t += 4) {
      float v[RPL];
#pragma unroll
      for (int q = 0; q < RPL; ++q)
        v[q] = ((s_red[0][q][t][lane] + s_red[1][q][t][lane]) + s_red[2][q][t][lane]) + s_red[3][q][t][lane];
      const int orow = row0 + t0 + t;  // h row, or y_sorted row
      if (GATEUP) {
        a.h[(size_t)orow * a.I + 64 * cb + lane] = f32_to_bf16_bits(v[0] / (1.0f + expf(-v[0])) * v[1]);
      } else {
        uint16_t* yrow = shared ? a.y_shared + (size_t)(t0 + t) * a.d : a.y_sorted + (size_t)orow * a.d;
#pragma unroll
        for (int q = 0; q < RPL; ++q) yrow[128 * cb + 64 * q + lane] = f32_to_bf16_bits(v[q]);
      }
    }
    __syncthreads();
  }
}

template <int FMT, bool GATEUP>
static hipError_t launch_fmt(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  auto kern = gemv_kernel<FMT, GATEUP>;
  static int resident_blocks = 0;  // blocks of this kernel the device holds at once
  if (resident_blocks == 0) {
    int dev = 0, per_cu = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipGetLastError();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess) return hipGetLastError();
    resident_blocks = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  }
  const int ncb = GATEUP ? a.I / 64 : a.d / 128;
  long long blocks = (long long)chunks_upper * ncb;
  if (blocks > resident_blocks) blocks = resident_blocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool GATEUP>
static hipError_t launch_gemv(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  switch (a.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16, GATEUP>(a, chunks_upper, s);
    case FMT_Q4_0: return launch_fmt<FMT_Q4_0, GATEUP>(a, chunks_upper, s);
    case FMT_MXFP4: return launch_fmt<FMT_MXFP4, GATEUP>(a, chunks_upper, s);
    default: return launch_fmt<FMT_FP8_B128, GATEUP>(a, chunks_upper, s);
  }
}

hipError_t launch_gemv_gateup(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  return launch_gemv<true>(a, chunks_upper, s);
}
hipError_t launch_gemv_down(const FfnArgs& a, int chunks_upper, hipStream_t s) {
  return launch_gemv<false>(a, chunks_upper, s);
}

}  // namespace ftk
