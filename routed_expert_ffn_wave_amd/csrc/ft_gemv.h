// The streaming GEMV work item shared by the grouped-FFN GEMV kernels and the fused decode layer
// kernel.
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
#pragma once
#include <type_traits>

#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

constexpr int GV_PF = 6;   // chunks of weights in flight per lane (prefetch ring)

typedef const __attribute__((address_space(4))) uint32_t* scalar_u32p;  // read through the scalar cache

template <int FMT>
__device__ __forceinline__ size_t mat_bytes(int rows, int K) {
  return FMT == FMT_BF16 ? (size_t)rows * K * 2 : FMT == FMT_FP8_B128 ? (size_t)rows * K : (size_t)rows * K / 2;
}

// dynamic LDS: [groups: 4 x (E+2) ints][tmp: 4 ints][x rows NT x K bf16, item scales | partial sums]
__host__ __device__ inline size_t gv_group_bytes(int E) { return ((size_t)4 * (E + 2) * 4 + 16 + 15) & ~(size_t)15; }
// per-(row, chunk) scale bytes of one 64-row block (Q4_0: fp16, MXFP4: E8M0, NVFP4: two e4m3), or
// for FP8-B128 the fp32 block scales of the 128-row blocks the 64 rows lie in: two (a gate/up
// device block holds gate and up rows) of K/128 each
__host__ __device__ inline size_t gv_scale_bytes(int fmt, int K) {
  return (fmt == FMT_Q4_0 || fmt == FMT_NVFP4) ? (size_t)64 * (K / 32) * 2
         : fmt == FMT_MXFP4                   ? (size_t)64 * (K / 32)
         : fmt == FMT_FP8_B128                ? (size_t)2 * (K / 128) * 4
                                              : 0;
}
// Q4_0: per-(token, 32-element block) activation sums, fp32
__host__ __device__ inline size_t gv_xsum_bytes(int fmt, int K, int NT) {
  return fmt == FMT_Q4_0 ? (size_t)NT * (K / 32) * 4 : 0;
}
__host__ __device__ inline size_t gv_union_bytes(int fmt, int K, int NT, int WPB, int RPL = 1) {
  const size_t xb = (size_t)NT * K * 2 + RPL * gv_scale_bytes(fmt, K) + gv_xsum_bytes(fmt, K, NT);
  const size_t rb = (size_t)WPB * RPL * NT * 64 * 4;
  return xb > rb ? xb : rb;
}

// Accesses of h and y rows that other blocks of the same launch read: single-copy atomic at agent
// scope (the sc1 loads and stores of gfx950), so they need no cache write-back or invalidation.
__device__ __forceinline__ void store_u32_agent(uint16_t* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_u32_agent(const uint16_t* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 load_u32x4_agent(const uint16_t* p) {
  const uint64_t lo = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load((const uint64_t*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
// Wait until this wave's stores have completed (a compiler barrier too).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// No block-wide step between the weight prefetch and the activation rows (see gemv_item).
struct NoPre {
  __device__ void operator()() const {}
};

// One work item: the RPL 64-row device blocks RPL*cb .. RPL*cb+RPL-1 of bank slot `slot` against the
// nt (<= NT) token rows t0.. of a group whose sorted rows start at row0 (`shared`: the shared
// expert's group).  Writes 32 columns of h per row block (gate/up) or 64 columns of y (down).  All threads of the block call it;
// it ends with a block barrier, after which the LDS union may be reused.  COH: h rows are read and
// h / y rows written with agent-scope atomic accesses (other blocks of the launch use them).
// s_tok: token of each sorted row in LDS, or null to read a.gather through the scalar cache.
// `pre`: a block-wide step that the activation rows depend on (a dependency wait): when given, the
// item's first PF - 1 weight chunks are issued before it (the weights do not depend on it) and the
// rows and scales after it; otherwise the rows and scales are issued first.
template <int FMT, bool GATEUP, int WPB, int NT, bool COH = false, int RPL = 1, class Pre = NoPre>
__device__ __forceinline__ void gemv_item(const FfnArgs& a, uint8_t* s_union, int slot, int row0, int t0, int nt,
                                          int cb, bool shared, const int* s_tok = nullptr, Pre pre = Pre{}) {
  constexpr bool WEIGHTS_FIRST = !std::is_same<Pre, NoPre>::value;
  static_assert(!GATEUP || RPL == 1, "gate/up items cover one 64-row block");
  using C = Chunk<FMT>;
  constexpr int PF = GV_PF / RPL, NTHR = WPB * 64;  // the same bytes in flight for any RPL
  const int K = GATEUP ? a.d : a.I;
  const int nrows = GATEUP ? 2 * a.I : a.d;
  uint16_t* s_x = (uint16_t*)s_union;                                // [NT][K] activation rows of the item
  uint8_t* s_sc = s_union + (size_t)NT * K * 2;                      // [RPL][nchunk][64] scales of the item's rows
  float* s_xsum = (float*)(s_sc + RPL * gv_scale_bytes(FMT, K));     // [NT][K/32] (Q4_0)
  float* s_red = (float*)s_union;                                    // [WPB][RPL][NT][64] partial sums

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = K / C::ELEMS;
  const int niter = (nchunk - w + WPB - 1) / WPB;  // chunks w, w+WPB, ... of this wave
  const int jlast = niter > 0 ? niter - 1 : 0;
  const size_t mbytes = mat_bytes<FMT>(nrows, K);
  const uint8_t* codes = GATEUP ? a.w13 : a.w2;
  const uint8_t* scales = GATEUP ? a.s13 : a.s2;
  constexpr size_t CSTRIDE = 64 * 16;  // consecutive chunks of one row block are 1 KiB apart
  // the RPL rows of this lane
  // row block RPL*cb + q of the matrix for each q: device row (gate/up: lanes 0-31 gate rows,
  // lanes 32-63 the matching up rows)
  int rowq[RPL];
#pragma unroll
  for (int q = 0; q < RPL; ++q) rowq[q] = 64 * (RPL * cb + q) + lane;
  auto chunk_of = [&](int j) { return WPB * j + w; };  // this wave's j-th chunk
  const uint8_t* mat = codes + (size_t)slot * mbytes;
  const uint8_t* rowp[RPL];
#pragma unroll
  for (int q = 0; q < RPL; ++q) rowp[q] = mat + ilv_chunk_off(rowq[q], 0, nchunk);

  // ---- one round trip before the K loop: the item's activation rows (all tokens at once) and its
  // rows' block scales are loaded first, then the first PF-1 chunks of weights; waiting for the
  // rows and scales leaves the weights in flight (the vector-load counter is in order), and the
  // rows, their Q4_0 block sums and the scales go to LDS while the weights arrive.  Token indices
  // come through the scalar cache.
  constexpr int XMAX = WPB <= 4 ? 1 : 2;  // 16-byte activation loads per thread and token in the batch
  constexpr int SMAX = WPB <= 4 ? 2 : 4;  // 16-byte scale loads per thread in the batch
  // With more than 4 tokens per item the rows are staged as one flat list of 16-byte pieces
  // (piece v = token v / (K/8), column piece v % (K/8)), XB pieces per thread and batch.
  constexpr bool FLAT = NT > 4;
  constexpr int XB = 4;
  constexpr int SB = (FMT == FMT_Q4_0 || FMT == FMT_NVFP4) ? 2 : 1;
  constexpr bool STAGE_SCALES = FMT == FMT_Q4_0 || FMT == FMT_MXFP4 || FMT == FMT_NVFP4;
  const int nx8 = K / 8;
  // FP8-B128: the fp32 scales of the item's NSEL 128-row blocks (gate/up: the gate rows' and the up
  // rows'; down: one per 64-row block), staged as s_scf[sel][K/128] with the activation rows, so
  // that the K loop issues nothing but weight loads (a scale load there would have to wait for
  // every weight load in flight before it: the vector-load counter is in order)
  constexpr int NSEL = GATEUP ? 2 : RPL;
  const int nsb = FMT == FMT_FP8_B128 ? K / 128 : 0;
  float* s_scf = (float*)s_sc;
  auto fp8_scale_src = [&](int v) -> const float* {  // v = sel * nsb + column block
    const int sel = v / nsb, b = v % nsb;
    const int rb = GATEUP ? (32 * cb + (sel ? a.I : 0)) / 128 : (64 * (RPL * cb + sel)) / 128;
    return (const float*)scales + ((size_t)slot * (nrows / 128) + rb) * nsb + b;
  };
  const int nsv = STAGE_SCALES ? RPL * nchunk * 64 * SB / 16 : 0;  // the RPL row blocks' scales are one run
  const uint8_t* ssrc = scales + ((size_t)slot * nrows * nchunk + (size_t)RPL * cb * nchunk * 64) * SB;
  auto row_of = [&](int tt) -> const uint16_t* {  // activation row of the item's token tt
    if (GATEUP) {
      const int tok = shared ? t0 + tt
                      : s_tok ? s_tok[row0 + t0 + tt]
                              : (int)((scalar_u32p)(uintptr_t)a.gather)[row0 + t0 + tt] / a.k;
      return a.x + (size_t)tok * a.d;
    }
    return a.h + (size_t)(row0 + t0 + tt) * a.I;
  };
  constexpr int NXR = FLAT ? 1 : NT;
  const uint16_t* xr[NXR];
  if constexpr (!FLAT) {
#pragma unroll
    for (int t = 0; t < NT; ++t) xr[t] = row_of(t < nt ? t : nt - 1);
  }
  auto load_x = [&](const uint16_t* p) -> u32x4 {
    return (COH && !GATEUP) ? load_u32x4_agent(p) : *(const u32x4*)p;
  };
  const int nx = nt * nx8;
  auto load_piece = [&](int v) { return load_x(row_of(v / nx8) + 8 * (v % nx8)); };
  // ---- prefetch ring of PF chunks of codes.  Loads are issued unconditionally, with indices past
  // the wave's last chunk clamped to it, so every path keeps the same loads in flight.
  u32x4 buf[PF][RPL];
  auto issue = [&](u32x4* b, int j) {
    const int c = chunk_of(j);
#pragma unroll
    for (int q = 0; q < RPL; ++q)  // streamed once: non-temporal, so they do not evict what is reused
      b[q] = __builtin_nontemporal_load((const u32x4*)(rowp[q] + (size_t)c * CSTRIDE));
  };
  auto issue_ring = [&]() {
    if (niter > 0) {
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) issue(buf[p], min(p, jlast));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (WEIGHTS_FIRST) {
    issue_ring();
    pre();
  }
  u32x4 xv[FLAT ? 1 : XMAX][NXR];
  u32x4 xf[FLAT ? XB : 1];
  if constexpr (FLAT) {
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int v = threadIdx.x + i * NTHR;
      if (v < nx) xf[i] = load_piece(v);
    }
  } else {
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
      const int e8 = threadIdx.x + i * NTHR;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt && e8 < nx8) xv[i][t] = load_x(xr[t] + 8 * e8);
    }
  }
  u32x4 sv[SMAX];
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const int v = threadIdx.x + i * NTHR;
    if (v < nsv) sv[i] = *(const u32x4*)(ssrc + 16 * (size_t)v);
  }
  float f8s = 0.0f;  // one scale per thread here, the rest (rows longer than NTHR * 64) further down
  if constexpr (FMT == FMT_FP8_B128) {
    if ((int)threadIdx.x < NSEL * nsb) f8s = *fp8_scale_src(threadIdx.x);
  }
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (!WEIGHTS_FIRST) issue_ring();

  // Q4_0 weights are decoded as 128 + q, so each block needs the sum of its 32 activations; four
  // consecutive threads hold one block (K/8 is a multiple of 4, so they stay together)
  auto put_x = [&](int t, int e8, const u32x4& v) {
    *(u32x4*)(s_x + (size_t)t * K + 8 * e8) = v;
    if constexpr (FMT == FMT_Q4_0) {
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) sum = dot2_bf16(v[i], 0x3F803F80u, sum);
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      if ((e8 & 3) == 0) s_xsum[t * (K / 32) + (e8 >> 2)] = sum;
    }
  };
  if constexpr (FLAT) {
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int v = threadIdx.x + i * NTHR;
      if (v < nx) put_x(v / nx8, v % nx8, xf[i]);
    }
    for (int v0 = XB * NTHR; v0 < nx; v0 += XB * NTHR) {  // further batches (the weights are in flight)
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int v = v0 + threadIdx.x + i * NTHR;
        if (v < nx) xf[i] = load_piece(v);
      }
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int v = v0 + threadIdx.x + i * NTHR;
        if (v < nx) put_x(v / nx8, v % nx8, xf[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
      const int e8 = threadIdx.x + i * NTHR;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt && e8 < nx8) put_x(t, e8, xv[i][t]);
    }
  }
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const int v = threadIdx.x + i * NTHR;
    if (v < nsv) *(u32x4*)(s_sc + 16 * (size_t)v) = sv[i];
  }
  // rows longer than the batch (not reached by the shapes the launch pairs with WPB)
  if constexpr (!FLAT) {
    for (int e8 = threadIdx.x + XMAX * NTHR; e8 < nx8; e8 += NTHR)
      for (int t = 0; t < nt; ++t) put_x(t, e8, load_x(xr[t] + 8 * e8));
  }
  for (int v = threadIdx.x + SMAX * NTHR; v < nsv; v += NTHR)
    *(u32x4*)(s_sc + 16 * (size_t)v) = *(const u32x4*)(ssrc + 16 * (size_t)v);
  if constexpr (FMT == FMT_FP8_B128) {
    if ((int)threadIdx.x < NSEL * nsb) s_scf[threadIdx.x] = f8s;
    for (int v = threadIdx.x + NTHR; v < NSEL * nsb; v += NTHR) s_scf[v] = *fp8_scale_src(v);
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
        float fsc[RPL], fsc_hi[RPL];
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          fsc_hi[q] = 1.0f;
          if constexpr (FMT == FMT_FP8_B128) {
            // one fp32 scale per 128x128 block of logical rows (a gate/up device block holds 32 gate
            // rows in lanes 0-31 and the matching 32 up rows in lanes 32-63), staged above
            const int sel = GATEUP ? (lane >= 32 ? 1 : 0) : q;
            fsc[q] = s_scf[sel * nsb + (c * C::ELEMS) / 128];
          } else if constexpr (FMT == FMT_Q4_0) {
            fsc[q] = fp16_bits_to_f32(((const uint16_t*)s_sc)[(q * nchunk + c) * 64 + lane]);
          } else if constexpr (FMT == FMT_MXFP4) {
            fsc[q] = e8m0_to_f32(s_sc[(q * nchunk + c) * 64 + lane]);
          } else if constexpr (FMT == FMT_NVFP4) {  // e4m3 scales of the chunk's two 16-element halves
            const uint32_t two = ((const uint16_t*)s_sc)[(q * nchunk + c) * 64 + lane];
            fsc[q] = e4m3_to_f32(two & 0xffu);
            fsc_hi[q] = e4m3_to_f32(two >> 8);
          } else {
            fsc[q] = 1.0f;
          }
        }
        // one row block at a time: its chunk is decoded once and used for every token (the token
        // rows are read again from LDS for the next row block rather than held in registers)
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          uint32_t wp[C::PAIRS];
          C::decode(buf[p][q], wp);
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
              if constexpr (FMT == FMT_NVFP4) {  // each half's scale on its own fp32 partial sum
                float lo = 0.0f, hi = 0.0f;
#pragma unroll
                for (int i = 0; i < C::PAIRS / 2; ++i) lo = dot2_bf16(wp[i], xw[i], lo);
#pragma unroll
                for (int i = C::PAIRS / 2; i < C::PAIRS; ++i) hi = dot2_bf16(wp[i], xw[i], hi);
                acc[q][t] = fmaf(hi, fsc_hi[q], fmaf(lo, fsc[q], acc[q][t]));
                continue;
              }
              float part = 0.0f;
#pragma unroll
              for (int i = 0; i < C::PAIRS; ++i) part = dot2_bf16(wp[i], xw[i], part);
              if constexpr (FMT == FMT_Q4_0)
                acc[q][t] = fmaf(fsc[q], fmaf(-136.0f, s_xsum[t * (K / 32) + c], part), acc[q][t]);  // 128 + q
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
  // NVFP4: the matrix's fp32 scale, stored after every slot's block scales
  float tsc = 1.0f;
  if constexpr (FMT == FMT_NVFP4)
    tsc = ((const float*)(scales + (size_t)a.n_slots * nrows * nchunk * 2))[slot];
  for (int tq = w; tq < nt * RPL; tq += WPB) {
    const int t = tq / RPL, q = tq % RPL, cbq = RPL * cb + q;
    const int orow = row0 + t0 + t;  // h row, or y_sorted row
    if (GATEUP) {
      float g = 0.0f, u = 0.0f;
      if (lane < 32) {
#pragma unroll
        for (int ww = 0; ww < WPB; ++ww) {
          g += s_red[((ww * RPL + q) * NT + t) * 64 + lane];
          u += s_red[((ww * RPL + q) * NT + t) * 64 + lane + 32];
        }
      }
      if constexpr (FMT == FMT_NVFP4) {
        g *= tsc;
        u *= tsc;
      }
      const uint32_t hb = f32_to_bf16_bits(g / (1.0f + expf(-g)) * u);
      uint16_t* hp = a.h + (size_t)orow * a.I + 32 * cbq + lane;
      if constexpr (COH) {
        const uint32_t nb = __shfl_down(hb, 1, 64);  // pairs of columns as one 32-bit store
        if (lane < 32 && (lane & 1) == 0) store_u32_agent(hp, hb | (nb << 16));
      } else {
        if (lane < 32) *hp = (uint16_t)hb;
      }
    } else {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < WPB; ++ww) v += s_red[((ww * RPL + q) * NT + t) * 64 + lane];
      if constexpr (FMT == FMT_NVFP4) v *= tsc;
      uint16_t* yrow = shared ? a.y_shared + (size_t)(t0 + t) * a.d : a.y_sorted + (size_t)orow * a.d;
      const uint32_t yb = f32_to_bf16_bits(v);
      if constexpr (COH) {
        const uint32_t nb = __shfl_down(yb, 1, 64);
        if ((lane & 1) == 0) store_u32_agent(yrow + 64 * cbq + lane, yb | (nb << 16));
      } else {
        yrow[64 * cbq + lane] = (uint16_t)yb;
      }
    }
  }
  __syncthreads();
}

}  // namespace ftk
