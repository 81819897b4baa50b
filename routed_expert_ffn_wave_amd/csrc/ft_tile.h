// Epilogue shared by the MFMA GEMM kernels with 128-row token tiles: one wave's finished 32 x 32
// fp32 tiles (the v_mfma 32x32 result layout) go to the h workspace (gate/up: SiLU(g) * u, rounded
// to bf16) or to y (down: rounded to bf16), staged through LDS so that every lane stores whole
// 16-byte row segments.
#pragma once
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {

// Store one finished tile.
// WJ: 32-column fragments per wave (4: 128 weight rows, 2: 64); dev_blk: the wave's first 64-row
// device block of the matrix.
template <bool GATEUP, int WJ>
__device__ __forceinline__ void store_tile(f32x16 (&acc)[4][WJ], uint8_t* stg_base, const FfnArgs& a, int lane, int wv,
                                           int dev_blk, bool shared, int row0, int m0, int mrows) {
  // Lane holds, for tile (i, j), rows 32 i + (r/4)*8 + hi*4 + r%4 and weight
  // row 128 wv + 32 j + l32 of the tile.  Each wave stages its bf16 results for 64 rows at a time
  // in its own slice of `stg_base` (4 x 64 x PITCH bytes), two columns per dword:
  // lanes 2c and 2c + 1 swap one value of rows (a, a + 1), so lane 2c holds row a and lane 2c + 1
  // row a + 1, each for columns 2c, 2c + 1.  The slice is then stored as whole row segments.
  //   gate/up: SiLU(g) * u; device row block dev_blk + p holds 32 gate rows, then the 32 up rows
  //            of intermediate columns 32 * (dev_blk + p) + 0..31: 16 WJ columns per wave.
  //   down:    32 WJ output columns per wave, from column 64 dev_blk.
  constexpr int OCOLS = GATEUP ? 16 * WJ : 32 * WJ;  // bf16 output columns per wave
  constexpr int PITCH = OCOLS * 2 + 16;         // staging row pitch in bytes
  constexpr int LPR = OCOLS * 2 / 16;           // lanes per row segment (16 bytes each)
  constexpr int RPI = 64 / LPR;                 // rows per store instruction
  uint8_t* stg = stg_base + wv * (64 * PITCH);
  // lane index laundered through an empty asm, so that the epilogue's per-lane offsets are
  // computed here and not hoisted out of the tile loop (where they would only take registers)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int el32 = ln & 31, ehi = ln >> 5;
  const bool odd = ln & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // byte selectors of the pair swap
  uint16_t* ocol0 = GATEUP ? a.h + 32 * dev_blk : (shared ? a.y_shared : a.y_sorted) + 64 * dev_blk;
  const size_t opitch = GATEUP ? (size_t)a.I : (size_t)a.d;
  const int orow0 = (GATEUP || !shared) ? row0 + m0 : m0;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (hh == 1 && mrows <= 64) break;  // rows 64.. of the tile hold nothing to store
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hh + ii;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = 32 * ii + (r >> 2) * 8 + ehi * 4 + (r & 3) + (odd ? 1 : 0);  // in the half
#pragma unroll
        for (int jj = 0; jj < OCOLS / 32; ++jj) {
          float v0, v1;  // rows r, r + 1 of this lane's column
          if (GATEUP) {
            // SiLU(g) * u with the hardware exp and reciprocal (about 1 ulp each, far below the
            // bf16 rounding of h)
            const float g0 = acc[i][2 * jj][r], u0 = acc[i][2 * jj + 1][r];
            const float g1 = acc[i][2 * jj][r + 1], u1 = acc[i][2 * jj + 1][r + 1];
            v0 = g0 * __builtin_amdgcn_rcpf(1.0f + __expf(-g0)) * u0;
            v1 = g1 * __builtin_amdgcn_rcpf(1.0f + __expf(-g1)) * u1;
          } else {
            v0 = acc[i][jj][r];
            v1 = acc[i][jj][r + 1];
          }
          const bf16x2 pv = {(__bf16)v0, (__bf16)v1};
          const uint32_t pk = __builtin_bit_cast(uint32_t, pv);
          const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pk, 0xB1, 0xf, 0xf, false);
          // even lane: (own row r, partner row r); odd lane: (partner row r + 1, own row r + 1)
          const uint32_t word = __builtin_amdgcn_perm(other, pk, sel);
          *(uint32_t*)(stg + row * PITCH + (32 * jj + (el32 & ~1)) * 2) = word;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 64 / RPI; ++q) {
      const int row = q * RPI + ln / LPR, seg = ln % LPR;
      const u32x4 v = *(const u32x4*)(stg + row * PITCH + seg * 16);
      const int m = 64 * hh + row;
      if (m < mrows) *(u32x4*)(ocol0 + (size_t)(orow0 + m) * opitch + seg * 8) = v;
    }
  }
}

// Staging bytes of store_tile: 4 waves x 64 rows x the down kernel's pitch (128 columns).
constexpr int STG_BYTES = 4 * 64 * (128 * 2 + 16);

}  // namespace ftk
