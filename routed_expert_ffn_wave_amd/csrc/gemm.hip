// Grouped expert GEMM on MFMA for expert groups with many tokens (prefill).
//
// Expert FFNs are read from per-format quantised banks (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", section 五).  With many tokens per expert the FFN is a dense
// contraction per expert, so it runs on the matrix cores: v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Weights are decoded to bf16 on their way into LDS; every format's element values
// are exact in bf16 (e4m3, e2m1 * 2^k, q - 8), and the block scales that are not exactly
// representable in bf16 (Q4_0's fp16 per 32, FP8's fp32 per 128x128) multiply fp32 partial sums of
// their K block, so each weight is used exactly as its format defines it.
//
// Work item = (group, tile of BM=128 tokens, tile of 128 weight rows), one block of 4 waves each;
// wave (wm, wn) computes 64x64 of the output as 2x2 MFMA tiles of 32x32.
//   gate/up: the 128 weight rows of a tile are 64 intermediate columns i, laid out as
//            [gate i0..i0+31 | up i0..i0+31 | gate i0+32.. | up i0+32..], so each wave holds the gate
//            and up sums of the same (token, i) in the same lane and applies SiLU(g)*u in registers.
//   down:    128 rows of W2 = 128 output columns.
#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"

namespace ftk {

constexpr int BM = GEMM_BM, BN = 128, BK = 32, LDK = BK + 8;  // LDS row stride in bf16 (padded)

template <int FMT>
__device__ __forceinline__ size_t gemm_mat_bytes(int rows, int K) {
  return FMT == FMT_BF16 ? (size_t)rows * K * 2 : FMT == FMT_FP8_B128 ? (size_t)rows * K : (size_t)rows * K / 2;
}

// Decode this thread's 16 K-consecutive weights of K step `ks` (half `hf` = elements 16hf..16hf+15
// of the 32-wide step) of weight row `r` in a row-interleaved matrix (base `mat`, nchunk chunks
// per row) into 8 dwords of bf16 pairs in K order.  All element values are exact in bf16; MXFP4's
// power-of-two scale is folded into the conversion (exact while the product is a normal bf16).
template <int FMT>
__device__ __forceinline__ void load_b_half(const uint8_t* mat, int r, int nchunk, int ks, int hf,
                                            const uint8_t* mx_scales, uint32_t* out) {
  if constexpr (FMT == FMT_BF16) {  // 8 elements per chunk: chunks 4ks + 2hf, +1
    const u32x4 a = *(const u32x4*)(mat + ilv_chunk_off(r, 4 * ks + 2 * hf, nchunk));
    const u32x4 b = *(const u32x4*)(mat + ilv_chunk_off(r, 4 * ks + 2 * hf + 1, nchunk));
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
  } else if constexpr (FMT == FMT_FP8_B128) {  // 16 elements per chunk: chunk 2ks + hf
    const u32x4 c = *(const u32x4*)(mat + ilv_chunk_off(r, 2 * ks + hf, nchunk));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
      out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
    }
  } else if constexpr (FMT == FMT_MXFP4) {  // 32 elements per chunk: half hf = bytes 8hf..8hf+7
    const u32x2 c = *(const u32x2*)(mat + ilv_chunk_off(r, ks, nchunk) + hf * 8);
    const float sc = e8m0_to_f32(mx_scales[ilv_scale_idx(r, ks, nchunk)]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      out[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 0));
      out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 1));
      out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 2));
      out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 3));
    }
  } else {  // Q4_0: words 2hf, 2hf+1 of the chunk; nibble pair s of word w = elements 8w+2s, 8w+2s+1
    const u32x2 c = *(const u32x2*)(mat + ilv_chunk_off(r, ks, nchunk) + hf * 8);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t v = (c[i] >> (4 * s)) & 0x000F000Fu;
        const float lo = (float)(int)(v & 0xffffu) - 8.0f, hi = (float)(int)(v >> 16) - 8.0f;  // q - 8, exact
        out[4 * i + s] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      }
    }
  }
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void gemm_kernel(FfnArgs a) {
  constexpr bool PARTIAL = (FMT == FMT_Q4_0 || FMT == FMT_FP8_B128);
  constexpr int SCALE_STEPS = (FMT == FMT_FP8_B128) ? 4 : 1;  // K steps per scale block
  __shared__ int s_slot[1025], s_row0[1025], s_cnt[1025], s_item0[1026], s_tmp[4];
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];
  __shared__ float s_bscale[BN];   // per weight row scale of the current scale block
  __shared__ const uint16_t* s_arow[BM];

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;  // weight rows
  const int ntiles = ncols / BN;
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + BM - 1) / BM) * ntiles; });
  const int it = blockIdx.x;
  if (it >= s_item0[gl.n]) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int g = find_group(s_item0, gl.n, it);
  const int local = it - s_item0[g];
  const int mt = local / ntiles, nt = local % ntiles;
  const int slot = s_slot[g], row0 = s_row0[g], cnt = s_cnt[g];
  const int TK = a.T * a.k;
  const bool shared = row0 >= TK;
  const int m0 = mt * BM;
  const int mrows = min(BM, cnt - m0);

  // activation row pointers of the tile (null past the group's end)
  if (tid < BM) {
    const uint16_t* p = nullptr;
    if (tid < mrows) {
      if (GATEUP) {
        const int tok = shared ? (m0 + tid) : (a.gather[row0 + m0 + tid] / a.k);
        p = a.x + (size_t)tok * a.d;
      } else {
        p = a.h + (size_t)(row0 + m0 + tid) * a.I;
      }
    }
    s_arow[tid] = p;
  }

  // weight row of local column n
  const int half_id = tid & 1;
  const int ln = tid >> 1;  // 0..127: the A row and the B row this thread stages
  // device row of the B-tile row ln (W13 device blocks already hold 32 gate then 32 up rows, so
  // tile nt's 128 device rows are gate i0..i0+31, up i0.., gate i0+32.., up i0+32.. with i0 = 64nt)
  // and its logical row (for the FP8 scale grid, which is indexed by logical rows)
  const int drow = nt * BN + ln;
  const int wrow = GATEUP ? w13_logical_row(drow, a.I) : drow;
  const uint8_t* codes = GATEUP ? a.w13 : a.w2;
  const uint8_t* scales = GATEUP ? a.s13 : a.s2;
  const int nchunk = K / chunk_elems<FMT>();
  const uint8_t* bmat = codes + (size_t)slot * gemm_mat_bytes<FMT>(ncols, K);
  const uint8_t* bscales = nullptr;  // per-(row, chunk) scales of this slot (Q4_0, MXFP4)
  if constexpr (FMT == FMT_Q4_0) bscales = scales + (size_t)slot * ncols * (size_t)nchunk * 2;
  if constexpr (FMT == FMT_MXFP4) bscales = scales + (size_t)slot * ncols * (size_t)nchunk;
  __syncthreads();
  const uint16_t* arow = s_arow[ln];

  f32x16 acc[2][2], part[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[i][j][r] = 0.0f;
        part[i][j][r] = 0.0f;
      }

  const int nsteps = K / BK;
  for (int ks = 0; ks < nsteps; ++ks) {
    // ---- stage A (16 bf16 per thread) and B (16 decoded weights per thread) into LDS
    u32x4 av0 = {0, 0, 0, 0}, av1 = {0, 0, 0, 0};
    if (arow) {
      const u32x4* p = (const u32x4*)(arow + (size_t)ks * BK + half_id * 16);
      av0 = p[0];
      av1 = p[1];
    }
    uint32_t bw[8];
    load_b_half<FMT>(bmat, drow, nchunk, ks, half_id, bscales, bw);
    float bsc = 1.0f;
    if constexpr (PARTIAL) {
      if ((ks % SCALE_STEPS) == 0) {
        if constexpr (FMT == FMT_Q4_0) {
          bsc = fp16_bits_to_f32(((const uint16_t*)bscales)[ilv_scale_idx(drow, ks, nchunk)]);
        } else {
          const float* s32 = (const float*)scales;
          bsc = s32[((size_t)slot * (ncols / 128) + wrow / 128) * (K / 128) + ks / 4];
        }
      }
    }
    __syncthreads();  // every wave is done with the previous step's As, Bs and s_bscale
    if constexpr (PARTIAL) {
      if (half_id == 0 && (ks % SCALE_STEPS) == 0) s_bscale[ln] = bsc;
    }
    *(u32x4*)&As[ln * LDK + half_id * 16] = av0;
    *(u32x4*)&As[ln * LDK + half_id * 16 + 8] = av1;
    *(u32x4*)&Bs[ln * LDK + half_id * 16] = u32x4{bw[0], bw[1], bw[2], bw[3]};
    *(u32x4*)&Bs[ln * LDK + half_id * 16 + 8] = u32x4{bw[4], bw[5], bw[6], bw[7]};
    __syncthreads();

    // ---- MFMA: two K sub-steps of 16
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = *(const bf16x8*)&As[r * LDK + kk + 8 * (lane >> 5)];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + j * 32 + (lane & 31);
        bf[j] = *(const bf16x8*)&Bs[c * LDK + kk + 8 * (lane >> 5)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (PARTIAL)
            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], part[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (PARTIAL) {
      if ((ks % SCALE_STEPS) == SCALE_STEPS - 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float sc = s_bscale[wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[i][j][r] = fmaf(part[i][j][r], sc, acc[i][j][r]);
              part[i][j][r] = 0.0f;
            }
        }
      }
    }
  }

  // ---- epilogue.  Lane holds, for tile (i, j), rows wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4 and
  // column wn*64 + j*32 + lane%32.
  const int col = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (m >= mrows) continue;
      if (GATEUP) {
        const float gte = acc[i][0][r], up = acc[i][1][r];
        const float hv = gte / (1.0f + expf(-gte)) * up;
        const int icol = nt * 64 + wn * 32 + col;
        a.h[(size_t)(row0 + m0 + m) * a.I + icol] = f32_to_bf16_bits(hv);
      } else {
        uint16_t* yrow = shared ? a.y_shared + (size_t)(m0 + m) * a.d : a.y_sorted + (size_t)(row0 + m0 + m) * a.d;
#pragma unroll
        for (int j = 0; j < 2; ++j) yrow[nt * BN + wn * 64 + j * 32 + col] = f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

template <bool GATEUP>
static hipError_t launch_gemm(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  const int ntiles = GATEUP ? (2 * a.I) / BN : a.d / BN;
  long long blocks = (long long)tiles_upper * ntiles;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks), block(256);
  switch (a.fmt) {
    case FMT_BF16: hipLaunchKernelGGL((gemm_kernel<FMT_BF16, GATEUP>), grid, block, 0, s, a); break;
    case FMT_Q4_0: hipLaunchKernelGGL((gemm_kernel<FMT_Q4_0, GATEUP>), grid, block, 0, s, a); break;
    case FMT_MXFP4: hipLaunchKernelGGL((gemm_kernel<FMT_MXFP4, GATEUP>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_kernel<FMT_FP8_B128, GATEUP>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  return launch_gemm<true>(a, tiles_upper, s);
}
hipError_t launch_gemm_down(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  return launch_gemm<false>(a, tiles_upper, s);
}

}  // namespace ftk
