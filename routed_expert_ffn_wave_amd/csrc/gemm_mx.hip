// Grouped expert GEMM for MXFP4 and FP8-B128 banks on the scaled low-precision MFMA of gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4), with the weights used in their stored format.
//
// Expert FFNs are read from per-format banks (FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五); at prefill each expert group is a dense contraction.  The weights enter the matrix
// cores as stored: MXFP4 as e2m1 codes with their E8M0 scale per 32 K (the instruction's own block
// scale), FP8-B128 as e4m3 codes (unit block scale), whose fp32 scale per 128 x 128 block multiplies
// the fp32 partial sum of each 128-K block.
//
// Activations in one low-precision term would miss the fp32 reference by ~4e-2 (rel-L2), so each
// activation is carried as two terms of the operand format, hi + lo, each with an E8M0 scale per
// 32 K: hi is the nearest code of x / 2^e1, lo the nearest code of the residual x - hi, and every
// product is issued twice (once per term) into the same fp32 accumulators.  MXFP4 banks take e2m3
// (fp6) terms: fp6 x fp4 issues at the fp4 rate, so the two passes cost what one fp8 pass would.
// FP8 banks take e4m3 terms.  A prepass (quant_act_kernel) writes the terms of every activation row
// once: x before gate/up, h before down.
//
// Tile = 128 token rows x BN weight rows, one block of 4 waves per CU, K steps of 64 (one MFMA).
//   MXFP4: BN = 512, each wave 128 x 128 = 4 x 4 MFMA tiles (two device row blocks);
//   FP8:   BN = 256, each wave 128 x 64 = 4 x 2 MFMA tiles (one device row block: 32 gate rows and
//          the 32 matching up rows, or 64 rows of W2) plus a second accumulator set for the
//          running 128-K block.
// A wave's weight rows are used by that wave only: each lane loads its own B operands (16 or 32
// bytes per fragment and step) straight into one of RING register sets, 3 steps ahead.  The
// activation terms, which all four waves read, go through a two-stage LDS buffer: each step
// stores the next step's rows (loaded a step earlier) and reads its own.
//
// Operand layouts of the 32x32x64 instruction (checked on the device): lane l holds row l % 32 of
// its operand; fp4 and fp6 lanes hold the 32 K values 32 (l / 32) .. + 31 as consecutive 4- or
// 6-bit fields, fp8 lanes hold K 16 (l / 32) .. + 15 in bytes 0-15 and K 32 + 16 (l / 32) .. + 15
// in bytes 16-31; the lane's scale byte covers K block l / 32 of its row.
#include <type_traits>

#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"
#include "ft_queue.h"
#include "ft_tile.h"

namespace ftk {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int MX_BM = GEMM_BM;  // token rows per tile
constexpr int MX_RING = 4;      // weight register sets (loads run 3 steps ahead)
constexpr int MX_DEEP = 8;      // the same for tiles of at most 32 rows (loads run 7 steps ahead)

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void constexpr_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    constexpr_for<B + 1, E>(f);
  }
}

template <bool FP8>
struct MxCfg;
template <>
struct MxCfg<false> {                   // MXFP4 weights, e2m3 activation terms
  static constexpr int CB = 48;         // code bytes of one activation block of 32: hi 24, lo 24
  static constexpr int WN = 4;          // 32-row weight fragments per wave
  static constexpr int BN = 512;        // weight rows per tile
  static constexpr int ATYPE = 2, BTYPE = 4;  // operand formats of the instruction: e2m3, e2m1
  static constexpr int PITCH = 112;     // LDS bytes per activation row and step (96 codes, 4 scales)
};
template <>
struct MxCfg<true> {                    // FP8-B128 weights, e4m3 activation terms
  static constexpr int CB = 64;         // hi 32, lo 32
  static constexpr int WN = 2;
  static constexpr int BN = 256;
  static constexpr int ATYPE = 0, BTYPE = 0;  // e4m3, e4m3
  static constexpr int PITCH = 144;     // 128 codes, 4 scales
};
template <bool FP8>
constexpr int a_units() { return 2 * MxCfg<FP8>::CB / 16; }  // 16-byte pieces of codes per row and step

constexpr int MX_KBMAX = 256;   // FP8: 128-K blocks per weight row held in LDS (K <= 32768)

// LDS: the group list, each group's first short-tile item ([E + 2] ints), then the buffers
__host__ __device__ inline size_t mx_buf_off(int E) {
  return (group_lds_bytes(E) + (size_t)(E + 2) * 4 + 255) & ~(size_t)255;
}
// FP8: each wave's block scales ([wave][fragment][K / 128] fp32) follow the activation buffers
template <bool FP8>
__host__ __device__ inline size_t mx_bsc_off(int E) {
  const size_t abuf = (size_t)2 * MX_BM * MxCfg<FP8>::PITCH;
  const size_t stg = FP8 ? (size_t)4 * 64 * (64 * 2 + 16) : (size_t)STG_BYTES;
  return mx_buf_off(E) + (abuf > stg ? abuf : stg);
}
template <bool FP8>
__host__ __device__ inline size_t mx_lds_bytes(int E) {
  return mx_bsc_off<FP8>(E) + (FP8 ? (size_t)4 * MxCfg<FP8>::WN * MX_KBMAX * 4 : 0);
}

// ---------------------------------------------------------------------------------------------
// Activation terms.  Block b of 32 values of a row: e1 = the smallest exponent with
// max|x| / 2^e1 <= the format's largest value (7.5 for e2m3, 448 for e4m3), hi = nearest code of
// x / 2^e1 (ties to even), r = x - hi * 2^e1 (exact in fp32), e2 and lo the same for r.  E8M0
// bytes are e + 127, clamped to [0, 254]; an all-zero block gets byte 0 and zero codes.

template <bool FP8>
__device__ __forceinline__ int term_exp(float amax) {
  constexpr int EMAX = FP8 ? 8 : 2;
  constexpr float VMAX = FP8 ? 448.0f : 7.5f;
  if (!(amax > 0.0f)) return -127;
  int e = __builtin_amdgcn_frexp_expf(amax) - 1 - EMAX;
  if (__builtin_ldexpf(amax, -e) > VMAX) ++e;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// e2m3 code of v (|v| clamped to 7.5), nearest with ties to even, and its value
__device__ __forceinline__ uint32_t e2m3_code(float v, float& val) {
  const float a = fminf(fabsf(v), 7.5f);
  const int E = a >= 4.0f ? 2 : (a >= 2.0f ? 1 : 0);  // binade (0 also holds the subnormals)
  const float q = rintf(__builtin_ldexpf(a, 3 - E));   // 0..16 steps of 2^(E-3)
  val = __builtin_copysignf(__builtin_ldexpf(q, E - 3), v);
  return ((uint32_t)(E << 3) + (uint32_t)q) | (v < 0.0f ? 32u : 0u);
}

template <bool FP8>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ src, long long nrows, int K,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int CB = MxCfg<FP8>::CB;
  const int nblk = K / 32;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nrows * nblk) return;
  const long long row = gid / nblk;
  const int b = (int)(gid - row * nblk);
  const u32x4* p = (const u32x4*)(src + row * K + (long long)b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = p[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[8 * q + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e1 = term_exp<FP8>(amax);
  uint32_t hi[FP8 ? 8 : 6], lo[FP8 ? 8 : 6];
#pragma unroll
  for (int i = 0; i < (FP8 ? 8 : 6); ++i) hi[i] = lo[i] = 0u;
  float r[32];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      int w = 0;
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v[i], -e1), __builtin_ldexpf(v[i + 1], -e1), w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v[i + 2], -e1), __builtin_ldexpf(v[i + 3], -e1), w, true);
      hi[i / 4] = (uint32_t)w;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r[i + j] = v[i + j] - __builtin_ldexpf(e4m3_to_f32(((uint32_t)w >> (8 * j)) & 0xffu), e1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float hv;
      const uint32_t c = e2m3_code(__builtin_ldexpf(v[i], -e1), hv);
      r[i] = v[i] - __builtin_ldexpf(hv, e1);
      const int bit = 6 * i, wd = bit >> 5, sh = bit & 31;
      hi[wd] |= c << sh;
      if (sh > 26) hi[wd + 1] |= c >> (32 - sh);
    }
  }
  float rmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) rmax = fmaxf(rmax, fabsf(r[i]));
  const int e2 = term_exp<FP8>(rmax);
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      int w = 0;
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(r[i], -e2), __builtin_ldexpf(r[i + 1], -e2), w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(r[i + 2], -e2), __builtin_ldexpf(r[i + 3], -e2), w, true);
      lo[i / 4] = (uint32_t)w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float lv;
      const uint32_t c = e2m3_code(__builtin_ldexpf(r[i], -e2), lv);
      const int bit = 6 * i, wd = bit >> 5, sh = bit & 31;
      lo[wd] |= c << sh;
      if (sh > 26) lo[wd + 1] |= c >> (32 - sh);
    }
  }
  uint8_t* o = codes + (size_t)gid * CB;  // [row][block][CB]: hi terms, then lo terms
  if constexpr (FP8) {
    *(u32x4*)(o) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4*)(o + 16) = u32x4{hi[4], hi[5], hi[6], hi[7]};
    *(u32x4*)(o + 32) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *(u32x4*)(o + 48) = u32x4{lo[4], lo[5], lo[6], lo[7]};
  } else {
    *(u32x4*)(o) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4*)(o + 16) = u32x4{hi[4], hi[5], lo[0], lo[1]};
    *(u32x4*)(o + 32) = u32x4{lo[2], lo[3], lo[4], lo[5]};
  }
  ((uint16_t*)scales)[gid] = (uint16_t)((uint32_t)(e1 + 127) | ((uint32_t)(e2 + 127) << 8));
}

// ---------------------------------------------------------------------------------------------
// The GEMM.  qcodes / qscales: the activation terms of the A rows ([row][K/32][CB] and
// [row][K/32][2]): gate/up rows are tokens (gathered), down rows are h rows in sorted order.
template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_mx_kernel(FfnArgs a, const uint8_t* __restrict__ qcodes,
                                                         const uint8_t* __restrict__ qscales) {
  using C = MxCfg<FP8>;
  constexpr int WN = C::WN, PITCH = C::PITCH, UPR = a_units<FP8>();
  constexpr int QN = MX_BM * UPR / 256;  // 16-byte pieces per thread and step
  static_assert(MX_BM * UPR % 256 == 0, "pieces per thread");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  int* s_pitem0 = (int*)(lds + group_lds_bytes(a.E));
  uint8_t* abuf = lds + mx_buf_off(a.E);

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;
  const int ntiles = ncols / C::BN;
  const int nsteps = K / 64;
  const int nblk = K / 32;
  const size_t qpitch = (size_t)nblk * C::CB;
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  // Items in two parts: the long tiles of every group (more than MX_BM / 2 rows: every full m-tile,
  // and the last one if it holds more than half a tile; s_item0 prefix), then the short tile (the
  // group's last m-tile with 1 .. MX_BM / 2 rows) of every group that has one (s_pitem0 prefix).  A
  // long tile takes about twice as long as a short one, so each queue hands out its long tiles
  // first and the launch ends on short ones.
  build_groups(src, gl, s_tmp, [&](int cnt) { return (cnt / MX_BM + (cnt % MX_BM > MX_BM / 2)) * ntiles; });
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int carry = 0;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int i0 = 0; i0 < gl.n; i0 += 64) {
      const int i = i0 + lane;
      const int rem = i < gl.n ? s_cnt[i] % MX_BM : 0;
      const uint64_t b = __ballot(rem > 0 && rem <= MX_BM / 2);
      if (i < gl.n) s_pitem0[i] = (carry + __popcll(b & below)) * ntiles;
      carry += __popcll(b);
    }
    if (lane == 0) s_pitem0[gl.n] = carry * ntiles;
  }
  __syncthreads();
  const int nlong = s_item0[gl.n], nshort = s_pitem0[gl.n];
  const int nitems = nlong + nshort;

  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int TK = a.T * a.k;
  // the weights' unit block scale (E8M0 127) for FP8, kept in a register: a literal would be read
  // as an fp32 constant by the instruction
  int unit_scale = 127;
  asm volatile("" : "+v"(unit_scale));

  // tiles from the launch's work queues: block b serves the run of XCD b % 8 first (blocks go to
  // the XCDs round-robin, so tiles that share activation rows or weights share an L2), then the
  // others, long tiles before short ones; a block that starts late takes fewer tiles (each is
  // claimed as the previous one's K loop ends)
  int* s_claim = s_tmp + 1;
  int qoff = 0;
  if (tid == 0) s_claim[0] = queue_claim2(a.qctr, nlong, nshort, qoff);
  __syncthreads();
  int it = s_claim[0];
  __syncthreads();
  for (; it >= 0 && it < nitems;) {
    int nxt = -1;  // the next tile, claimed as this one's K loop ends
    const bool lng = it < nlong;  // a long tile
    const int* pre = lng ? s_item0 : s_pitem0;
    const int v = lng ? it : it - nlong;
    const int g = find_group(pre, gl.n, v);
    const int local = __builtin_amdgcn_readfirstlane(v - pre[g]);
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[g]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_row0[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[g]);
    const int mt = lng ? local / ntiles : cnt / MX_BM, nt = lng ? local % ntiles : local;
    const bool shared = row0 >= TK;
    const int m0 = mt * MX_BM;
    const int mrows = min(MX_BM, cnt - m0);

    // A tile whose group has at most 32 or 64 rows left (a partial tile) skips the MFMAs and LDS
    // reads of its empty 32-row tiles; it loads what a full tile loads (rows past the group repeat
    // its last row), and its empty tiles' accumulators stay zero.  The variants are separate copies
    // of the whole tile, epilogue included, so none carries another's registers.
    auto tile = [&](auto mi, auto rg) {
      constexpr int MI = decltype(mi)::value;    // 32-row tiles computed
      constexpr int RING = decltype(rg)::value;  // weight register sets: loads run RING - 1 steps ahead
      // A deep ring (more than MX_RING sets) also gives the activation terms one register set per
      // step in flight, issued with the step's weights, so that waiting for a step's activations
      // never waits for weights issued after them; such a tile stages only its MI row tiles.
      constexpr bool DEEP = RING > MX_RING;
      constexpr int AR = DEEP ? 32 * MI : MX_BM;  // activation rows staged per step
      constexpr int NPC = AR * UPR;               // their 16-byte pieces per step
      constexpr int QA = DEEP ? (NPC + 255) / 256 : QN;
      constexpr int NSET = DEEP ? RING : 2;       // activation register sets
      static_assert(DEEP || NPC == 256 * QN, "a full tile's pieces cover the threads exactly");
      // ---- this thread's share of the activation rows (rows past the group's end repeat its last
      // row; their results are never stored): QA code pieces and a scale word (threads past the
      // staged rows repeat the first ones: the same words to the same places).  32-bit offsets from
      // the terms base.
      auto src_row = [&](int r) -> uint32_t {
        const int m = min(r, mrows - 1);
        if (GATEUP) return shared ? (uint32_t)(m0 + m) : (uint32_t)(a.gather[row0 + m0 + m] / a.k);
        return (uint32_t)(row0 + m0 + m);
      };
      uint32_t aoff[QA];
      uint32_t adst[QA];
#pragma unroll
      for (int q = 0; q < QA; ++q) {
        const int u = (tid + 256 * q) % NPC, r = u / UPR, pc = u % UPR;
        aoff[q] = src_row(r) * (uint32_t)qpitch + (uint32_t)(pc * 16);
        adst[q] = (uint32_t)(r * PITCH + pc * 16);
      }
      const uint32_t soff = src_row(tid % AR) * (uint32_t)(nblk * 2);
      const uint32_t sdst = (uint32_t)((tid % AR) * PITCH + 2 * C::CB);
      // register sets of staged activations: by step parity (a step's rows are loaded two steps
      // before they are stored), or one per ring slot (DEEP)
      u32x4 areg[NSET][QA];
      uint32_t sreg[NSET];
      auto load_a = [&](int set, int s) {  // step s's codes and scales (s clamped to the last step)
        s = min(s, nsteps - 1);
        const uint8_t* cb = qcodes + (size_t)s * 2 * C::CB;   // uniform
        const uint8_t* sb = qscales + (size_t)s * 4;
#pragma unroll
        for (int q = 0; q < QA; ++q) areg[set][q] = *(const u32x4*)(cb + aoff[q]);
        sreg[set] = *(const uint32_t*)(sb + soff);
      };
      auto store_a = [&](int set, int buf) {
        uint8_t* b = abuf + buf * (MX_BM * PITCH);
#pragma unroll
        for (int q = 0; q < QA; ++q) *(u32x4*)(b + adst[q]) = areg[set][q];
        *(uint32_t*)(b + sdst) = sreg[set];
      };

      // ---- this wave's weight rows: a uniform base per fragment, one 32-bit lane offset
      const int nchunk = FP8 ? K / 16 : K / 32;  // 16-byte code chunks per weight row
      const size_t mat_bytes = (size_t)ncols * nchunk * 16;
      const uint8_t* wmat = (GATEUP ? a.w13 : a.w2) + (size_t)slot * mat_bytes;
      const int blk0 = FP8 ? 4 * nt + wv : 8 * nt + 2 * wv;  // the wave's first 64-row device block
      const uint8_t* wbase = wmat + (size_t)blk0 * nchunk * 1024;
      const uint8_t* sbase = FP8 ? nullptr
                                 : (GATEUP ? a.s13 : a.s2) + (size_t)slot * ncols * nchunk + (size_t)blk0 * nchunk * 64;
      const uint32_t blane = (uint32_t)(hi * 1024 + l32 * 16);  // chunk parity and row of this lane
      const uint32_t slane = (uint32_t)(hi * 64 + l32);
      // fragment j: rows 32 (j % 2) of device block blk0 + j / 2 (MXFP4); rows 32 j of blk0 (FP8)
      auto frag_off = [&](int j) -> size_t {
        return FP8 ? (size_t)j * 512 : (size_t)(j >> 1) * nchunk * 1024 + (size_t)(j & 1) * 512;
      };
      auto frag_soff = [&](int j) -> size_t { return (size_t)(j >> 1) * nchunk * 64 + (size_t)(j & 1) * 32; };
      float bsc[WN];  // FP8: the current 128-K block's scale of each fragment's rows
      int rb[WN];     // FP8: 128-row scale block of each fragment
      // FP8: this wave's block scales in LDS ([fragment][K / 128]), read a block at a time, so that
      // no scale load in the K loop waits for the weights issued before it
      float* s_bs = (float*)(lds + mx_bsc_off<FP8>(a.E)) + wv * WN * MX_KBMAX;
      const float* s32 = FP8 ? (const float*)(GATEUP ? a.s13 : a.s2) + (size_t)slot * (size_t)(ncols / 128) * (K / 128)
                             : nullptr;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        rb[j] = GATEUP ? (32 * blk0 + (j ? a.I : 0)) / 128 : (64 * blk0 + 32 * j) / 128;
        bsc[j] = 1.0f;
      }
      u32x4 bq[RING][WN][FP8 ? 2 : 1];
      int bs[RING][WN];
      // FP8: the wave's block scales, loaded before the prologue's loads and written to LDS after
      // them (the wait for them leaves the prologue's loads in flight)
      constexpr int BSN = FP8 ? MX_KBMAX / 64 : 1;
      float bsl[WN][BSN];
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int q = 0; q < BSN; ++q) {
            const int kb = lane + 64 * q;
            bsl[j][q] = kb < K / 128 ? s32[(size_t)rb[j] * (K / 128) + kb] : 0.0f;
          }
      }
      auto load_b = [&](auto SL, int s) {  // step s's weight operands into register set SL
        constexpr int sl = decltype(SL)::value;
        s = min(s, nsteps - 1);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          if constexpr (FP8) {
            const uint8_t* p0 = wbase + frag_off(j) + (size_t)(4 * s) * 1024;   // uniform
            bq[sl][j][0] = *(const u32x4*)(p0 + blane);
            bq[sl][j][FP8 ? 1 : 0] = *(const u32x4*)(p0 + 2048 + blane);
            bs[sl][j] = unit_scale;
          } else {
            const uint8_t* p0 = wbase + frag_off(j) + (size_t)(2 * s) * 1024;
            bq[sl][j][0] = *(const u32x4*)(p0 + blane);
            bs[sl][j] = (int)*(sbase + frag_soff(j) + (size_t)(2 * s) * 64 + slane);
          }
        }
      };

      f32x16 acc[4][WN], part[4][WN];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = part[i][j][r] = 0.0f;
        }

      // ---- prologue: step 0's activations in buffer 0; weights of steps 0 .. RING - 2, and the
      // activations of steps 1 and 2 (DEEP: 1 .. RING - 2, each with its weights) in registers
      if constexpr (DEEP) {
        load_a(0, 0);
        load_b(std::integral_constant<int, 0>{}, 0);
        constexpr_for<1, RING - 1>([&](auto S) {
          load_b(S, S);
          load_a(S, S);
        });
        store_a(0, 0);
      } else {
        load_a(0, 0);
        store_a(0, 0);
        load_a(1, 1);
        load_a(0, 2);
        load_b(std::integral_constant<int, 0>{}, 0);
        load_b(std::integral_constant<int, 1>{}, 1);
        load_b(std::integral_constant<int, 2>{}, 2);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int q = 0; q < BSN; ++q)
            if (lane + 64 * q < K / 128) s_bs[j * MX_KBMAX + lane + 64 * q] = bsl[j][q];
      }
      __syncthreads();

      // A fragment i of the buffer at `ab`: both terms and their scale bytes
      struct AFrag {
        i32x8 h, l;
        int sh, sl;
      };
      auto read_a = [&](const uint8_t* ab, int i) -> AFrag {
        const uint8_t* rp = ab + (32 * i + l32) * PITCH;
        AFrag f;
        if constexpr (FP8) {
          const u32x4 h0 = *(const u32x4*)(rp + 16 * hi), h1 = *(const u32x4*)(rp + 64 + 16 * hi);
          const u32x4 q0 = *(const u32x4*)(rp + 32 + 16 * hi), q1 = *(const u32x4*)(rp + 96 + 16 * hi);
          f.h = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
          f.l = i32x8{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3], (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
        } else {
          const u32x4 h0 = *(const u32x4*)(rp + 48 * hi);
          const u32x2 h1 = *(const u32x2*)(rp + 48 * hi + 16);
          const u32x2 q0 = *(const u32x2*)(rp + 48 * hi + 24);
          const u32x4 q1 = *(const u32x4*)(rp + 48 * hi + 32);
          f.h = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], 0, 0};
          f.l = i32x8{(int)q0[0], (int)q0[1], (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3], 0, 0};
        }
        const uint32_t sw = *(const uint16_t*)(rp + 2 * C::CB + 2 * hi);
        f.sh = (int)(sw & 0xffu);
        f.sl = (int)(sw >> 8);
        return f;
      };

      auto step = [&](auto SL, int s) {
        constexpr int sl = decltype(SL)::value;
        load_b(std::integral_constant<int, (sl + RING - 1) % RING>{}, s + RING - 1);
        if constexpr (DEEP) load_a((sl + RING - 1) % RING, s + RING - 1);
        const uint8_t* ab = abuf + (sl & 1) * (MX_BM * PITCH);  // s and sl have the same parity
        if constexpr (FP8) {
          if constexpr ((sl & 1) == 0) {  // a new 128-K block: its scales
#pragma unroll
            for (int j = 0; j < WN; ++j) bsc[j] = s_bs[j * MX_KBMAX + s / 2];
          }
        }
        i32x8 bv[WN];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const u32x4 c0 = bq[sl][j][0], c1 = bq[sl][j][FP8 ? 1 : 0];
          bv[j] = FP8 ? i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]}
                      : i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], 0, 0, 0, 0};
        }
        AFrag cur = read_a(ab, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          AFrag nxt;
          if (i < 3 && i + 1 < MI) nxt = read_a(ab, i + 1);  // the next row tile's reads go out before these MFMAs
          __builtin_amdgcn_sched_barrier(0);
          // the hi terms of every fragment, then the lo terms: products into one accumulator are WN
          // instructions apart
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (i >= MI) break;
#pragma unroll
            for (int j = 0; j < WN; ++j) {
              const i32x8& av = t ? cur.l : cur.h;
              const int as = t ? cur.sl : cur.sh;
              if constexpr (FP8) {
                f32x16 p = part[i][j];
                if (t == 0 && (sl & 1) == 0) p = f32x16{};  // the block's first product starts from zero
                part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[j], p, C::ATYPE, C::BTYPE, 0, as, 0,
                                                                             bs[sl][j]);
              } else {
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[j], acc[i][j], C::ATYPE, C::BTYPE, 0,
                                                                            as, 0, bs[sl][j]);
              }
            }
          }
          // FP8, last step of a 128-K block: row tile i - 1's block is complete (its MFMAs were
          // issued a tile earlier): scale its partial sums into acc while tile i's MFMAs run
          if constexpr (FP8) {
            if ((sl & 1) == 1 && i > 0 && i - 1 < MI) {
#pragma unroll
              for (int j = 0; j < WN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i - 1][j][r] = fmaf(part[i - 1][j][r], bsc[j], acc[i - 1][j][r]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (i < 3) cur = nxt;
        }
        if constexpr (FP8 && MI == 4) {
          if ((sl & 1) == 1) {
#pragma unroll
            for (int j = 0; j < WN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[3][j][r] = fmaf(part[3][j][r], bsc[j], acc[3][j][r]);
          }
        }
        // the next step's activations into the other buffer: DEEP, from the set loaded with its
        // weights; else from the parity set loaded two steps ago, which then takes step s + 3's
        if constexpr (DEEP) {
          store_a((sl + 1) % RING, (sl + 1) & 1);
        } else {
          store_a((sl + 1) & 1, (sl + 1) & 1);
          load_a((sl + 1) & 1, s + 3);
        }
        __syncthreads();
      };
      for (int s = 0; s < nsteps; s += RING)
        constexpr_for<0, RING>([&](auto S) { step(S, s + S); });

      // ---- epilogue: staging slices over the activation buffers (every step has been read)
      const int dev_blk = FP8 ? 4 * nt + wv : 8 * nt + 2 * wv;
      // the next tile is claimed only now (its latency hides behind the epilogue): claimed at the
      // start of this tile, it would be bound to this block however late this block ends, and a
      // block that drew a long tile would take a short one behind it while others sit idle
      if (tid == 0) nxt = queue_claim2(a.qctr, nlong, nshort, qoff);
      store_tile<GATEUP, WN>(acc, abuf, a, lane, wv, dev_blk, shared, row0, m0, mrows);
    };
    // An FP8 tile of at most 32 rows is bound by its weight stream, not its MFMAs: it keeps
    // MX_DEEP - 1 steps of loads in flight where the step count allows.  (The MXFP4 kernel has no
    // registers to spare for it.)
    bool deep = false;
    if constexpr (FP8) {
      if (mrows <= MX_BM / 4 && nsteps % MX_DEEP == 0) {
        tile(std::integral_constant<int, 1>{}, std::integral_constant<int, MX_DEEP>{});
        deep = true;
      }
    }
    if (deep) {
    } else if (mrows <= MX_BM / 4)
      tile(std::integral_constant<int, 1>{}, std::integral_constant<int, MX_RING>{});
    else if (mrows <= MX_BM / 2)
      tile(std::integral_constant<int, 2>{}, std::integral_constant<int, MX_RING>{});
    else
      tile(std::integral_constant<int, 4>{}, std::integral_constant<int, MX_RING>{});
    __syncthreads();  // the next tile's activations overwrite the staging slices
    if (tid == 0) s_claim[0] = nxt;
    __syncthreads();
    it = s_claim[0];
    __syncthreads();
  }
}

template <bool FP8, bool GATEUP>
hipError_t launch_mx_cfg(const FfnArgs& a, const uint8_t* qcodes, const uint8_t* qscales, int tiles_upper,
                         hipStream_t s) {
  auto kern = gemm_mx_kernel<FP8, GATEUP>;
  static LaunchCache cache;  // the LDS limit is set once for the largest E (512)
  LaunchFacts f;
  if (cache.get((const void*)kern, 256, mx_lds_bytes<FP8>(512), &f) != hipSuccess) return hipGetLastError();
  const int ntiles = (GATEUP ? 2 * a.I : a.d) / MxCfg<FP8>::BN;
  long long blocks = (long long)tiles_upper * ntiles;
  if (blocks > f.cus) blocks = f.cus;  // one block per CU
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), mx_lds_bytes<FP8>(a.E), s, a, qcodes, qscales);
  return hipGetLastError();
}

}  // namespace

bool gemm_mx_fits(int fmt, int rows, int K, int E) {
  if (E > 512 || K % 256 != 0 || K < 256) return false;
  if (fmt == FMT_MXFP4) return rows % MxCfg<false>::BN == 0 && mx_lds_bytes<false>(E) <= 160 * 1024;
  if (fmt == FMT_FP8_B128)
    return rows % MxCfg<true>::BN == 0 && K / 128 <= MX_KBMAX && mx_lds_bytes<true>(E) <= 160 * 1024;
  return false;
}

size_t mx_term_bytes(int fmt, long long rows, int K) {
  const int cb = fmt == FMT_FP8_B128 ? MxCfg<true>::CB : MxCfg<false>::CB;
  const size_t codes = (size_t)rows * (K / 32) * cb, scales = (size_t)rows * (K / 32) * 2;
  return ((codes + 255) & ~(size_t)255) + ((scales + 255) & ~(size_t)255);
}

hipError_t launch_quant_act(int fmt, const uint16_t* src, long long rows, int K, uint8_t* terms, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int cb = fmt == FMT_FP8_B128 ? MxCfg<true>::CB : MxCfg<false>::CB;
  const size_t codes = (size_t)rows * (K / 32) * cb;
  uint8_t* sc = terms + ((codes + 255) & ~(size_t)255);
  const long long n = rows * (K / 32);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (fmt == FMT_FP8_B128)
    hipLaunchKernelGGL(quant_act_kernel<true>, dim3(grid), dim3(256), 0, s, src, rows, K, terms, sc);
  else
    hipLaunchKernelGGL(quant_act_kernel<false>, dim3(grid), dim3(256), 0, s, src, rows, K, terms, sc);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const FfnArgs& a, bool gateup, const uint8_t* terms, long long term_rows,
                          int tiles_upper, hipStream_t s) {
  const int K = gateup ? a.d : a.I;
  const int cb = a.fmt == FMT_FP8_B128 ? MxCfg<true>::CB : MxCfg<false>::CB;
  const size_t codes = (size_t)term_rows * (K / 32) * cb;
  const uint8_t* sc = terms + ((codes + 255) & ~(size_t)255);
  if (a.fmt == FMT_FP8_B128)
    return gateup ? launch_mx_cfg<true, true>(a, terms, sc, tiles_upper, s)
                  : launch_mx_cfg<true, false>(a, terms, sc, tiles_upper, s);
  return gateup ? launch_mx_cfg<false, true>(a, terms, sc, tiles_upper, s)
                : launch_mx_cfg<false, false>(a, terms, sc, tiles_upper, s);
}

}  // namespace ftk
