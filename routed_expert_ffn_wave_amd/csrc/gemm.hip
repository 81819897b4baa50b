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
// Tile = (group, BM=128 tokens, BN weight rows), K in steps of BK=64; one block of 4 waves, wave
// (wm, wn) computes 64 x (BN/2) of the tile as 2 x WN MFMA tiles of 32x32.  BN = 256 (WN = 4) for
// bf16 and MXFP4 banks; Q4_0 and FP8 banks, which also keep per-scale-block partial sums, use
// BN = 128 (WN = 2).  The step s+1 operands are loaded into registers while the MFMAs of step s run
// from LDS, then written to LDS (decoded) between two barriers.  Blocks are persistent: the grid
// is what the device holds at once and blocks stride over the tile list, which is built on the
// device (groups from the permutation, row chunk major), so skewed groups need no host round trip.
//   gate/up: W13 device blocks of 64 rows hold 32 gate rows then the matching 32 up rows, so MFMA
//            column tiles 2p and 2p+1 of a wave are the gate and up sums of the same (token, i) in
//            the same lane, and SiLU(g)*u is applied in registers.
//   down:    BN rows of W2 = BN output columns.
#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"

namespace ftk {

constexpr int BM = GEMM_BM, BK = 64, LDK = BK + 8;  // LDS row stride in bf16 (padded)

template <int FMT>
__device__ __forceinline__ size_t gemm_mat_bytes(int rows, int K) {
  return FMT == FMT_BF16 ? (size_t)rows * K * 2 : FMT == FMT_FP8_B128 ? (size_t)rows * K : (size_t)rows * K / 2;
}
template <int FMT, int WN_>
struct GemmCfg {
  static constexpr int WN = WN_;                                            // MFMA column tiles per wave
  static constexpr int BN = 64 * WN;                                        // weight rows per tile
  static constexpr bool PARTIAL = FMT == FMT_Q4_0 || FMT == FMT_FP8_B128;   // scale per K block
  // raw 16-byte code chunks per thread and step (B tile: BN rows x BK; 256 threads)
  static constexpr int BCH = (BN * BK / chunk_elems<FMT>()) / 256;
};

// dynamic LDS: [groups 4 x (E+2) ints + tmp][A: BM x LDK][B: BN x LDK][row pointers BM][scales BN]
__host__ __device__ inline size_t gemm_lds_bytes(int E, int BN) {
  return group_lds_bytes(E) + (size_t)(BM + BN) * LDK * 2 + (size_t)BM * 8 + (size_t)BN * 4 * 2;
}

// Decode one raw chunk of the B tile into bf16 pairs in K order (pairs per chunk: 4 bf16, 8 e4m3,
// 16 four-bit); MXFP4's power-of-two scale is folded into the conversion (exact while the product
// is a normal bf16), Q4_0 gives q - 8.
template <int FMT>
__device__ __forceinline__ void decode_b(const u32x4& c, float mx_scale, uint32_t* out, float nv_lo = 1.0f,
                                         float nv_hi = 1.0f) {
  if constexpr (FMT == FMT_BF16) {
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
  } else if constexpr (FMT == FMT_FP8_B128) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
      out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
    }
  } else if constexpr (FMT == FMT_NVFP4) {  // exact e2m1, then each value times its half's e4m3 scale
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = i < 2 ? nv_lo : nv_hi;
      uint32_t p[4];
      p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 0));
      p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 1));
      p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 2));
      p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 3));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float lo = bf16_bits_to_f32(p[b] & 0xffffu) * s, hi = bf16_bits_to_f32(p[b] >> 16) * s;
        out[4 * i + b] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      }
    }
  } else if constexpr (FMT == FMT_MXFP4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], mx_scale, 0));
      out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], mx_scale, 1));
      out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], mx_scale, 2));
      out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], mx_scale, 3));
    }
  } else {  // Q4_0: nibble pair s of word w = elements 8w+2s, 8w+2s+1 -> bf16 (q - 8), exact
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t v = (c[w] >> (4 * s)) & 0x000F000Fu;
        const float lo = (float)(int)(v & 0xffffu) - 8.0f, hi = (float)(int)(v >> 16) - 8.0f;
        out[4 * w + s] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      }
    }
  }
}

template <int FMT, bool GATEUP, int WN_>
__global__ __launch_bounds__(256, 2) void gemm_kernel(FfnArgs a) {
  using G = GemmCfg<FMT, WN_>;
  constexpr int WN = G::WN, BN = G::BN, BCH = G::BCH;
  constexpr int EPC = chunk_elems<FMT>();          // K elements per 16-byte chunk
  constexpr int CPR = BK / EPC;                     // chunks per B row and step
  constexpr int SCALE_STEPS = FMT == FMT_FP8_B128 ? 2 : 1;  // K steps per scale block (FP8: 128 = 2 x 64)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint16_t* As = (uint16_t*)(lds + group_lds_bytes(a.E));
  uint16_t* Bs = As + BM * LDK;
  const uint16_t** s_arow = (const uint16_t**)(Bs + BN * LDK);
  float* s_bscale = (float*)(s_arow + BM);  // [2][BN]: Q4_0 scales of the step's two 32-blocks, or FP8's

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;  // weight rows
  const int ntiles = ncols / BN;
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + BM - 1) / BM) * ntiles; });
  const int nitems = s_item0[gl.n];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int TK = a.T * a.k;
  const int nchunk = K / EPC;
  const uint8_t* codes = GATEUP ? a.w13 : a.w2;
  const uint8_t* scales = GATEUP ? a.s13 : a.s2;
  const int nsteps = K / BK;
  // A staging: thread -> row tid/2, K half (tid&1)*32 of the step: 4 x 16 bytes
  const int ar = tid >> 1, ah = tid & 1;

  // Blocks are placed on the 8 XCDs round-robin (block b on XCD b % 8).  Give each XCD a contiguous
  // run of each round's tiles, so that the tiles running at once on one XCD share their activation
  // rows (same token tile, neighbouring weight tiles) and weight tiles through its L2.
  const int NB = gridDim.x;
  const int lb = (NB % 8 == 0) ? (blockIdx.x % 8) * (NB / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int it = lb; it < nitems; it += NB) {
    const int g = find_group(s_item0, gl.n, it);
    const int local = it - s_item0[g];
    const int mt = local / ntiles, nt = local % ntiles;
    const int slot = s_slot[g], row0 = s_row0[g], cnt = s_cnt[g];
    const bool shared = row0 >= TK;
    const int m0 = mt * BM;
    const int mrows = min(BM, cnt - m0);
    if (tid < BM) {  // activation rows of the tile (null past the group's end)
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
    __syncthreads();
    const uint16_t* arow = s_arow[ar];
    const uint8_t* bmat = codes + (size_t)slot * gemm_mat_bytes<FMT>(ncols, K);
    // B staging: thread -> (row, chunk) pairs of the BN x BK tile, rows fastest so that 64 lanes
    // read one 1 KiB run of the row-interleaved layout
    auto b_row = [&](int i) { return (tid + 256 * i) % BN; };
    auto b_chk = [&](int i) { return (tid + 256 * i) / BN; };

    u32x4 ra[4], rb[BCH];
    float rsc[2] = {1.0f, 1.0f};  // this thread's B-row scales for the step (Q4_0: two 32-blocks)
    float rmx[BCH];               // MXFP4 scale of each staged chunk (NVFP4: scale of its low half)
    float rnv[BCH];               // NVFP4: scale of the chunk's high half
    auto load_step = [&](int s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = arow ? *(const u32x4*)(arow + (size_t)s * BK + ah * 32 + 8 * i) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int r = nt * BN + b_row(i), c = s * CPR + b_chk(i);
        rb[i] = *(const u32x4*)(bmat + ilv_chunk_off(r, c, nchunk));
        if constexpr (FMT == FMT_MXFP4)
          rmx[i] = e8m0_to_f32(scales[(size_t)slot * ncols * nchunk + ilv_scale_idx(r, c, nchunk)]);
        if constexpr (FMT == FMT_NVFP4) {
          const uint32_t two = ((const uint16_t*)scales)[(size_t)slot * ncols * nchunk + ilv_scale_idx(r, c, nchunk)];
          rmx[i] = e4m3_to_f32(two & 0xffu);
          rnv[i] = e4m3_to_f32(two >> 8);
        }
      }
      if constexpr (FMT == FMT_Q4_0) {  // rows tid < BN: the scales of the step's two 32-blocks
        if (tid < BN) {
          const int r = nt * BN + tid;
          const uint16_t* s16 = (const uint16_t*)scales + (size_t)slot * ncols * nchunk;
          rsc[0] = fp16_bits_to_f32(s16[ilv_scale_idx(r, 2 * s, nchunk)]);
          rsc[1] = fp16_bits_to_f32(s16[ilv_scale_idx(r, 2 * s + 1, nchunk)]);
        }
      }
      if constexpr (FMT == FMT_FP8_B128) {
        if (tid < BN && (s % SCALE_STEPS) == 0) {
          const int r = nt * BN + tid;
          const int lr = GATEUP ? w13_logical_row(r, a.I) : r;
          rsc[0] = ((const float*)scales)[((size_t)slot * (ncols / 128) + lr / 128) * (K / 128) + s / SCALE_STEPS];
        }
      }
    };
    auto store_step = [&](int s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)&As[ar * LDK + ah * 32 + 8 * i] = ra[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        uint32_t w[EPC / 2];
        if constexpr (FMT == FMT_NVFP4)
          decode_b<FMT>(rb[i], 1.0f, w, rmx[i], rnv[i]);
        else
          decode_b<FMT>(rb[i], FMT == FMT_MXFP4 ? rmx[i] : 1.0f, w);
        uint32_t* dst = (uint32_t*)&Bs[b_row(i) * LDK + b_chk(i) * EPC];
#pragma unroll
        for (int q = 0; q < EPC / 8; ++q)
          *(u32x4*)(dst + 4 * q) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
      }
      if constexpr (FMT == FMT_Q4_0) {
        if (tid < BN) {
          s_bscale[tid] = rsc[0];
          s_bscale[BN + tid] = rsc[1];
        }
      }
      if constexpr (FMT == FMT_FP8_B128) {
        if (tid < BN && (s % SCALE_STEPS) == 0) s_bscale[tid] = rsc[0];
      }
    };

    f32x16 acc[2][WN], part[2][G::PARTIAL ? WN : 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll
      for (int j = 0; j < (G::PARTIAL ? WN : 1); ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
    }

    load_step(0);
    for (int s = 0; s < nsteps; ++s) {
      __syncthreads();  // every wave is done with the previous step's LDS tiles
      store_step(s);
      __syncthreads();
      if (s + 1 < nsteps) load_step(s + 1);  // in flight during this step's MFMAs
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        bf16x8 af[2], bf[WN];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + (lane & 31);
          af[i] = *(const bf16x8*)&As[r * LDK + kk + 8 * (lane >> 5)];
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int c = wn * (BN / 2) + j * 32 + (lane & 31);
          bf[j] = *(const bf16x8*)&Bs[c * LDK + kk + 8 * (lane >> 5)];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            if constexpr (G::PARTIAL)
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], part[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
          }
        if constexpr (FMT == FMT_Q4_0) {  // a 32-block ends every second K sub-step
          if ((kk & 16) != 0) {
#pragma unroll
            for (int j = 0; j < WN; ++j) {
              const float sc = s_bscale[(kk >> 5) * BN + wn * (BN / 2) + j * 32 + (lane & 31)];
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
      if constexpr (FMT == FMT_FP8_B128) {  // a 128-block ends every second step
        if ((s % SCALE_STEPS) == SCALE_STEPS - 1) {
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const float sc = s_bscale[wn * (BN / 2) + j * 32 + (lane & 31)];
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

    // ---- epilogue.  Lane holds, for tile (i, j), rows wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4
    // and column wn*(BN/2) + j*32 + lane%32.
    const int col = lane & 31;
    float tsc = 1.0f;  // NVFP4: the matrix's fp32 scale, stored after every slot's block scales
    if constexpr (FMT == FMT_NVFP4) tsc = ((const float*)(scales + (size_t)a.n_slots * ncols * nchunk * 2))[slot];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m >= mrows) continue;
        if (GATEUP) {
#pragma unroll
          for (int p = 0; p < WN / 2; ++p) {
            const float gte = acc[i][2 * p][r] * tsc, up = acc[i][2 * p + 1][r] * tsc;
            const float hv = gte / (1.0f + expf(-gte)) * up;
            // device block (nt*BN + wn*BN/2)/64 + p holds intermediate columns 32 * that + 0..31
            const int icol = 32 * ((nt * BN + wn * (BN / 2)) / 64 + p) + col;
            a.h[(size_t)(row0 + m0 + m) * a.I + icol] = f32_to_bf16_bits(hv);
          }
        } else {
          uint16_t* yrow = shared ? a.y_shared + (size_t)(m0 + m) * a.d : a.y_sorted + (size_t)(row0 + m0 + m) * a.d;
#pragma unroll
          for (int j = 0; j < WN; ++j)
            yrow[nt * BN + wn * (BN / 2) + j * 32 + col] = f32_to_bf16_bits(acc[i][j][r] * tsc);
        }
      }
    }
    __syncthreads();  // s_arow and the LDS tiles are rewritten by the next tile
  }
}

template <int FMT, bool GATEUP, int WN>
static hipError_t launch_gemm_cfg(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  auto kern = gemm_kernel<FMT, GATEUP, WN>;
  const size_t lds = gemm_lds_bytes(a.E, 64 * WN);
  static LaunchCache cache;
  LaunchFacts f;
  if (cache.get((const void*)kern, 256, lds, &f) != hipSuccess) return hipGetLastError();
  const int ntiles = (GATEUP ? 2 * a.I : a.d) / (64 * WN);
  long long blocks = (long long)tiles_upper * ntiles;
  const long long cap = (long long)f.per_cu * f.cus;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

// 256-row weight tiles for bf16 and MXFP4 when the matrix divides into them; 128-row tiles otherwise
// and for the formats that keep per-scale-block partial sums
template <int FMT, bool GATEUP>
static hipError_t launch_gemm_fmt(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  const int rows = GATEUP ? 2 * a.I : a.d;
  if (gemm_wide_fits(FMT, rows, GATEUP ? a.d : a.I, a.E)) return launch_gemm_wide(a, GATEUP, tiles_upper, s);
  if constexpr (FMT == FMT_BF16 || FMT == FMT_MXFP4 || FMT == FMT_NVFP4)
    if (rows % 256 == 0) return launch_gemm_cfg<FMT, GATEUP, 4>(a, tiles_upper, s);
  return launch_gemm_cfg<FMT, GATEUP, 2>(a, tiles_upper, s);
}

template <bool GATEUP>
static hipError_t launch_gemm(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  switch (a.fmt) {
    case FMT_BF16: return launch_gemm_fmt<FMT_BF16, GATEUP>(a, tiles_upper, s);
    case FMT_Q4_0: return launch_gemm_fmt<FMT_Q4_0, GATEUP>(a, tiles_upper, s);
    case FMT_MXFP4: return launch_gemm_fmt<FMT_MXFP4, GATEUP>(a, tiles_upper, s);
    case FMT_NVFP4: return launch_gemm_fmt<FMT_NVFP4, GATEUP>(a, tiles_upper, s);
    default: return launch_gemm_fmt<FMT_FP8_B128, GATEUP>(a, tiles_upper, s);
  }
}

hipError_t launch_gemm_gateup(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  return launch_gemm<true>(a, tiles_upper, s);
}
hipError_t launch_gemm_down(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  return launch_gemm<false>(a, tiles_upper, s);
}

}  // namespace ftk
