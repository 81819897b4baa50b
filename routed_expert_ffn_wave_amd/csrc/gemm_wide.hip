// Grouped expert GEMM on MFMA with wide wave tiles and a direct-to-LDS operand ring (bf16 and MXFP4
// banks).
//
// Expert FFNs are read from per-format banks (FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 五); with many tokens per expert, each group is a dense contraction on the matrix cores.
//
// Tile = 128 token rows x 512 weight rows, one block of 4 waves per CU.  Wave w computes the 128
// rows times weight rows 128w .. 128w+127 as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32
// accumulators per lane), so each K step of 16 reads 8 fragments from LDS for 16 MFMAs: half the LDS
// traffic per flop of a 64 x 128 wave tile.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4: 64 lanes x 16 bytes
// to consecutive LDS bytes) through a ring of NS stages of 32 K columns.  The stage for step s + NS
// is issued at step s, once every wave has finished reading step s, so each load has NS - 1 steps
// of MFMA work to arrive.  The loads are issued from inline assembly: the compiler then puts no
// full vmcnt wait in front of the LDS reads; the kernel waits for exactly the stage it needs (vmcnt
// counts one wave's own loads, which complete in issue order) and meets the other waves at a
// barrier that does not drain the memory counters.
//
// LDS stage layout:
//   A: 128 rows x 64 bytes; row r keeps its 16-byte K chunk c in slot c ^ f(r), with
//      f(r) = ((r >> 1) ^ (r >> 2)) & 3, so the fragment reads (32 rows at one chunk) touch each
//      bank once per 8 lanes (32 banks) or per 16 lanes (64 banks).
//   B: the bank's row-interleaved layout keeps one chunk of 64 rows in 1 KiB; a stage holds the 8
//      row blocks of the tile, [block][chunk][64 rows][16 bytes]: 4 chunks of 8 bf16, or one chunk
//      of 32 MXFP4 codes, whose E8M0 scales follow (256 bytes per wave: its two blocks' 64-byte
//      runs).  MXFP4 fragments are decoded to bf16 in registers (e2m1 times a power of two is exact
//      in bf16), so every format runs the bf16 MFMA.
#include <type_traits>

#include "ft_device.h"
#include "ft_groups.h"
#include "ft_kernels.h"
#include "ft_queue.h"
#include "ft_tile.h"

namespace ftk {
namespace {

constexpr int WBM = GEMM_BM;                 // token rows per tile
constexpr int WBN = 512;                     // weight rows per tile (4 waves x 128)
constexpr int WBK = 32;                      // K columns per ring stage
constexpr int A_BYTES = WBM * WBK * 2;       // 8 KiB of activations per stage
constexpr int DMA_A = A_BYTES / 1024 / 4;    // A loads (1 KiB) per wave and stage
static_assert(WBM == 128 && DMA_A == 2, "stage shape");

template <int FMT>
struct WideCfg;
template <>
struct WideCfg<FMT_BF16> {
  static constexpr int NS = 3;                   // ring stages
  static constexpr int B_BYTES = WBN * WBK * 2;  // 4 chunks of 8 bf16 per row
  static constexpr int S_BYTES = 0;
  static constexpr int DMA = DMA_A + 8;          // loads per wave and stage
};
template <>
struct WideCfg<FMT_MXFP4> {
  static constexpr int NS = 5;
  static constexpr int B_BYTES = WBN * 16;       // one chunk of 32 codes per row
  static constexpr int S_BYTES = 4 * 256;        // E8M0 scales, 256 bytes per wave
  static constexpr int DMA = DMA_A + 3;
};
template <int FMT>
constexpr int stage_bytes() { return A_BYTES + WideCfg<FMT>::B_BYTES + WideCfg<FMT>::S_BYTES; }

__host__ __device__ inline size_t wide_ring_off(int E) { return (group_lds_bytes(E) + 1023) & ~(size_t)1023; }
template <int FMT>
__host__ __device__ inline size_t wide_lds_bytes(int E) { return wide_ring_off(E) + (size_t)WideCfg<FMT>::NS * stage_bytes<FMT>(); }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave: lane l's 16 bytes at base + voff are written to LDS bytes lds + 16 l .. + 15.  M0
// carries the LDS address (one wait state after writing it) and gets its old value back.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}
// Four loads of 1 KiB: global base + voff + 1024 t to LDS lds + 1024 t (t = 0..3; the immediate
// offset applies to both addresses).
__device__ __forceinline__ void dma16x4(const uint8_t* base, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}
// One wave: lane l's 4 bytes at base + voff are written to LDS bytes lds + 4 l .. + 3.
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}
// Wait until this wave's loads of a stage have landed, `newer` (0..4, wave-uniform) stages of U
// loads each having been issued after it.
template <int U>
__device__ __forceinline__ void wait_newer(int newer) {
  static_assert(4 * U <= 63, "vmcnt range");
  if (newer >= 4)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * U) : "memory");
  else if (newer == 3)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * U) : "memory");
  else if (newer == 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * U) : "memory");
  else if (newer == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(U) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Own LDS reads complete, then the block barrier; memory operations do not move across it.
__device__ __forceinline__ void lds_reads_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(FfnArgs a) {
  using C = WideCfg<FMT>;
  constexpr bool MX = FMT == FMT_MXFP4;
  constexpr int NS = C::NS, STAGE = stage_bytes<FMT>();
  static_assert(STG_BYTES <= NS * STAGE, "epilogue staging fits in the ring");
  constexpr int EPC = MX ? 32 : 8;  // K elements per 16-byte chunk
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint8_t* ring = lds + wide_ring_off(a.E);
  const uint32_t ring_m0 = lds_u32(ring);

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;  // weight rows
  const int ntiles = ncols / WBN;
  const int nchunk = K / EPC;                // 16-byte chunks per weight row
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + WBM - 1) / WBM) * ntiles; });
  const int nitems = s_item0[gl.n];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int TK = a.T * a.k;
  const int nsteps = K / WBK;
  const uint8_t* abase = GATEUP ? (const uint8_t*)a.x : (const uint8_t*)a.h;
  const uint32_t arow_bytes = (uint32_t)K * 2;

  // Fragment reads, byte offsets inside a stage.  A fragment i of substep u: rows 32 i + l32, chunk
  // 2 u + hi.  B fragment j of substep u: row block 2 wv + j / 2, rows 32 (j % 2) + l32, chunk 2 u + hi.
  const int xo = ((l32 >> 1) ^ (l32 >> 2)) & 3;
  // (MXFP4 pairs substep u and half hi with chunk 2 hi + u instead of 2 u + hi: any order of the
  // K sum is the same contraction, and this one gives each lane both substeps' B codes as one
  // 8-byte read, dwords 2 hi and 2 hi + 1 of the row's 16-byte chunk.)
  const int a_rd0 = l32 * 64 + (((MX ? 2 * hi : hi) ^ xo) << 4);
  const int a_rd1 = l32 * 64 + (((MX ? 2 * hi + 1 : 2 + hi) ^ xo) << 4);
  const int b_rd = A_BYTES + (8 * wv + hi) * 1024 + l32 * 16;
  // MXFP4: this lane's 8 code bytes of B row 32 (j % 2) + l32 of block 2 wv + j / 2 (both
  // substeps), and the row's scale byte in this wave's scale run
  const int bx_rd = A_BYTES + (2 * wv * 64 + l32) * 16 + 8 * hi;
  const int sx_rd = A_BYTES + C::B_BYTES + wv * 256 + l32;

  // Blocks are placed on the 8 XCDs round-robin: give each XCD a contiguous run of the tile list so
  // that tiles running at once on one XCD share activation rows and weight tiles through its L2.
  const int NB = gridDim.x;
  const int lb = (NB % 8 == 0) ? (blockIdx.x % 8) * (NB / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int it = lb; it < nitems; it += NB) {
    const int g = find_group(s_item0, gl.n, it);
    const int local = __builtin_amdgcn_readfirstlane(it - s_item0[g]);
    const int mt = local / ntiles, nt = local % ntiles;
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[g]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_row0[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[g]);
    const bool shared = row0 >= TK;
    const int m0 = mt * WBM;
    const int mrows = min(WBM, cnt - m0);

    // This lane's two A rows (rows past the group's end repeat its last row; their results are
    // never stored) and the chunk its LDS slot holds.
    uint32_t aoff[DMA_A];
#pragma unroll
    for (int q = 0; q < DMA_A; ++q) {
      const int r = 16 * (DMA_A * wv + q) + (lane >> 2);
      const int m = min(r, mrows - 1);
      int src_row;
      if (GATEUP)
        src_row = shared ? (m0 + m) : a.gather[row0 + m0 + m] / a.k;
      else
        src_row = row0 + m0 + m;
      const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
      aoff[q] = (uint32_t)src_row * arow_bytes + (uint32_t)(c << 4);
    }
    // this wave's two 64-row blocks of the weight tile (and their scale runs)
    const size_t mat_bytes = (size_t)ncols * nchunk * 16;
    const uint8_t* bt = (GATEUP ? a.w13 : a.w2) + (size_t)slot * mat_bytes + (size_t)(8 * nt + 2 * wv) * nchunk * 1024;
    const uint8_t* st_sc = MX ? (GATEUP ? a.s13 : a.s2) + (size_t)slot * ncols * nchunk + (size_t)(8 * nt + 2 * wv) * nchunk * 64
                              : nullptr;
    // Load unit q of this wave's share of stage s into the ring buffer at LDS byte `buf`:
    //   q = 0, 1: 16 A rows each;
    //   bf16:  q = 2, 3: one 64-row block of the weight tile, its 4 chunks;
    //   MXFP4: q = 2, 3: one 64-row block's chunk; q = 4: both blocks' 64 scale bytes (lanes 0-15
    //          and 16-31; lanes 32-63 repeat them into the unused half of the wave's 256 bytes).
    const uint32_t bvoff = (uint32_t)lane * 16;
    const uint32_t svoff = (uint32_t)(((lane >> 4) & 1) * nchunk * 64 + (lane & 15) * 4);
    auto issue_unit = [&](uint32_t buf, int s, int q) {
      if (q < DMA_A) {
        dma16(abase + (size_t)s * (WBK * 2), aoff[q], buf + (DMA_A * wv + q) * 1024);
      } else if constexpr (!MX) {
        const int rb = q - DMA_A;
        dma16x4(bt + ((size_t)rb * nchunk + 4 * s) * 1024, bvoff, buf + A_BYTES + (2 * wv + rb) * 4096);
      } else {
        if (q < DMA_A + 2) {
          const int rb = q - DMA_A;
          dma16(bt + ((size_t)rb * nchunk + s) * 1024, bvoff, buf + A_BYTES + (2 * wv + rb) * 1024);
        } else {
          dma4(st_sc + (size_t)s * 64, svoff, buf + A_BYTES + C::B_BYTES + wv * 256);
        }
      }
    };
    constexpr int UNITS = MX ? 5 : 4;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    bf16x8 f0[8], f1[8];  // fragments of substeps 0 and 1: A rows 0..3, then B columns 0..3
    uint2 braw[4];        // MXFP4: codes of the 4 B fragments (substep 0 in .x, 1 in .y)
    uint32_t bsb[4];      // MXFP4: their E8M0 scale bytes, as read
    float bsc[4];         // MXFP4: the scales as fp32 (converted when substep 0 is decoded)
    // fragment n of substep u of the stage at `st` (bf16 B fragments, or A)
    auto frag = [&](const uint8_t* st, int u, int n) -> bf16x8 {
      if (n < 4) return *(const bf16x8*)(st + (u ? a_rd1 : a_rd0) + n * 2048);
      return *(const bf16x8*)(st + b_rd + u * 2048 + ((n - 4) >> 1) * 4096 + ((n - 4) & 1) * 512);
    };
    auto read_raw = [&](const uint8_t* st, int j) {  // MXFP4 B fragment j: codes and scale
      braw[j] = *(const uint2*)(st + bx_rd + (j >> 1) * 1024 + (j & 1) * 512);
      bsb[j] = st[sx_rd + (j >> 1) * 64 + (j & 1) * 32];
    };
    // MXFP4 B fragment j of substep u: codes 16 hi + 8 u .. + 7 of the chunk (dword 2 hi + u)
    auto decode = [&](int j, int u) -> bf16x8 {
      if (u == 0) bsc[j] = e8m0_to_f32(bsb[j]);  // the read was issued a phase earlier
      const uint32_t w = u ? braw[j].y : braw[j].x;
      u32x4 o;
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bsc[j], 0));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bsc[j], 1));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bsc[j], 2));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bsc[j], 3));
      return __builtin_bit_cast(bf16x8, o);
    };
    auto mfma = [&](int i, int j, const bf16x8& av, const bf16x8& bv) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i][j], 0, 0, 0);
    };

    const int pre = min(NS, nsteps);
    for (int s = 0; s < pre; ++s)
#pragma unroll
      for (int q = 0; q < UNITS; ++q) issue_unit(ring_m0 + (uint32_t)s * STAGE, s, q);
    wait_newer<C::DMA>(pre - 1);
    lds_reads_done_barrier();
#pragma unroll
    for (int n = 0; n < 4; ++n) f0[n] = frag(ring, 0, n);
    if constexpr (MX) {
#pragma unroll
      for (int j = 0; j < 4; ++j) read_raw(ring, j);
#pragma unroll
      for (int j = 0; j < 4; ++j) f0[4 + j] = decode(j, 0);
    } else {
#pragma unroll
      for (int n = 4; n < 8; ++n) f0[n] = frag(ring, 0, n);
    }
    int cb = 0;  // ring buffer of step s
    // One step: 16 MFMAs on substep 0 with substep 1's fragment reads (MXFP4: A reads and B decodes)
    // between them; the wait for stage s + 1 and the barrier; 16 MFMAs on substep 1 with the next
    // stage's substep-0 reads (MXFP4: A reads, raw B reads, then the B decodes of its substep 0)
    // and (while stages remain) this wave's loads of stage s + NS, into the buffer just released,
    // between them.  The scheduling barriers keep that order, so reads, decodes and loads issue in
    // the MFMAs' shadow.
    auto step = [&](int s, auto load_ahead) {
      const uint8_t* st = ring + cb * STAGE;
      const int nb = (cb + 1 == NS) ? 0 : cb + 1;
      const uint8_t* nst = ring + nb * STAGE;  // past the last step: read but unused
      const uint32_t dbuf = ring_m0 + (uint32_t)cb * STAGE;
      if constexpr (MX) {
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          mfma(n >> 2, n & 3, f0[n >> 2], f0[4 + (n & 3)]);
          if (n < 4) f1[n] = frag(st, 1, n);
          else if (n < 8) f1[n] = decode(n - 4, 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          mfma(n >> 2, n & 3, f0[n >> 2], f0[4 + (n & 3)]);
          if (n < 8) f1[n] = frag(st, 1, n);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // every wave is done reading stage s and has stage s + 1 in LDS
      if (s + 1 < nsteps) wait_newer<C::DMA>(min(NS - 2, nsteps - 2 - s));
      lds_reads_done_barrier();
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        mfma(n >> 2, n & 3, f1[n >> 2], f1[4 + (n & 3)]);
        if constexpr (MX) {  // the next stage: A reads, raw B reads, then its substep-0 decode
          if (n < 4) f0[n] = frag(nst, 0, n);
          else if (n < 8) read_raw(nst, n - 4);
          else if (n >= 12) f0[n - 8] = decode(n - 12, 0);
        } else {
          if (n < 8) f0[n] = frag(nst, 0, n);
        }
        if constexpr (decltype(load_ahead)::value) {
          if (n >= 2 && n < 2 + 2 * UNITS && (n & 1) == 0) issue_unit(dbuf, s + NS, (n - 2) >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      cb = nb;
    };
    int s = 0;
    for (; s < nsteps - NS; ++s) step(s, std::true_type{});
    for (; s < nsteps; ++s) step(s, std::false_type{});

    // ---- epilogue (staging slices in the ring: every stage has been read)
    store_tile<GATEUP, 4>(acc, ring, a, lane, wv, 8 * nt + 2 * wv, shared, row0, m0, mrows);
    lds_reads_done_barrier();  // the next tile's loads overwrite the staging slices
  }
}


// ---------------------------------------------------------------------------------------------
// bf16 banks: weights straight from global memory into registers, activations through the ring.
//
// A wave's weight rows are used by that wave alone, so they need not pass through LDS: each lane
// loads its own B fragments (16 bytes of one row per fragment and substep: 512-byte runs per half
// wave) into one of 4 register sets, 3.5 steps ahead of their MFMAs.  Only the activation rows,
// which all 4 waves read, go through the LDS ring (BD_NS stages of 128 rows x 32 K).  Per step that
// leaves 8 KiB of LDS writes and 32 KiB of LDS reads per CU, against 40 + 64 KiB when the weights
// also pass through LDS.
//
// Issue order per step s (every step issues the same loads; past the end of the tile they repeat
// its last step, into registers or ring buffers nobody reads again):
//   phase 0: 16 MFMAs on substep 0; between them the substep-1 A reads and the 4 B loads of
//            substep 1 of step s + 3 (into the set whose substep-1 registers step s - 1 used);
//   wait for A stage s + 1, barrier;
//   phase 1: 16 MFMAs on substep 1; between them the next stage's substep-0 A reads, this wave's
//            2 loads of A stage s + BD_NS, then the 4 B loads of substep 0 of step s + 4.
// vmcnt counts every one of these loads in issue order, so "A stage s + 1 has landed" is "at most
// C(s) loads outstanding", C(s) = the loads issued after it (capped at the counter's 63).
constexpr int BD_NS = 7;       // A ring stages
constexpr int BD_PRO_B = 28;   // B loads of the prologue: steps 0..2 whole, substep 0 of step 3

__host__ __device__ inline size_t bd_lds_bytes(int E) { return wide_ring_off(E) + (size_t)BD_NS * A_BYTES + STG_BYTES; }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Loads issued after A stage s + 1 by the time step s waits for it (see above), for BD_NS = 7.
__device__ __forceinline__ void bd_wait_stage(int s) {
  static_assert(BD_NS == 7, "counts below");
  // s + 1 >= BD_NS: 4 + 10 (BD_NS - 2) + 4 = 58; else 2 BD_NS + BD_PRO_B + 8 s = 42 + 8 s
  if (s >= BD_NS - 1) wait_vm<58>();
  else if (s == 0) wait_vm<42>();
  else if (s == 1) wait_vm<50>();
  else if (s == 2) wait_vm<58>();
  else wait_vm<63>();
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_bd_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint8_t* ring = lds + wide_ring_off(a.E);
  uint8_t* stg = ring + BD_NS * A_BYTES;
  const uint32_t ring_m0 = lds_u32(ring);

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;
  const int ntiles = ncols / WBN;
  const int nchunk = K / 8;
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + WBM - 1) / WBM) * ntiles; });
  const int nitems = s_item0[gl.n];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int TK = a.T * a.k;
  const int nsteps = K / WBK;  // a multiple of 4 (K % 128 == 0)
  const uint8_t* abase = GATEUP ? (const uint8_t*)a.x : (const uint8_t*)a.h;
  const uint32_t arow_bytes = (uint32_t)K * 2;
  const int xo = ((l32 >> 1) ^ (l32 >> 2)) & 3;
  const int a_rd0 = l32 * 64 + ((hi ^ xo) << 4);
  const int a_rd1 = l32 * 64 + (((2 + hi) ^ xo) << 4);

  // Tiles come from the launch's work queues (each claimed as the previous one's K loop ends): a
  // tile takes ~60 us at K = 2048, so a fixed stride over the tile list leaves the whole device
  // waiting on the few blocks that drew one tile more than the rest, while queues let every block
  // take the next tile as soon as it is free, which with tiles of unequal cost (the partial tiles
  // below) evens out the finish.
  int* s_claim = s_tmp + 1;
  int qoff = 0;
  if (tid == 0) s_claim[0] = queue_claim(a.qctr, nitems, qoff);
  __syncthreads();
  int it = s_claim[0];
  __syncthreads();
  while (it >= 0 && it < nitems) {
    int nxt = -1;  // the next tile, claimed as this one's K loop ends
    const int g = find_group(s_item0, gl.n, it);
    const int local = __builtin_amdgcn_readfirstlane(it - s_item0[g]);
    const int mt = local / ntiles, nt = local % ntiles;
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[g]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_row0[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[g]);
    const bool shared = row0 >= TK;
    const int m0 = mt * WBM;
    const int mrows = min(WBM, cnt - m0);

    // A tile whose group has at most 32 or 64 rows left (a partial tile) skips the MFMAs and LDS
    // reads of its empty 32-row fragments; its loads are the same as a full tile's (rows past the
    // group repeat its last row), so the load counts the waits rely on do not change.  The variants
    // are separate copies of the whole tile, epilogue included, so none carries another's registers.
    auto tile = [&](auto mi) {
      constexpr int MI = decltype(mi)::value;  // 32-row fragments computed
      uint32_t aoff[DMA_A];
#pragma unroll
      for (int q = 0; q < DMA_A; ++q) {
        const int r = 16 * (DMA_A * wv + q) + (lane >> 2);
        const int m = min(r, mrows - 1);
        int src_row;
        if (GATEUP)
          src_row = shared ? (m0 + m) : a.gather[row0 + m0 + m] / a.k;
        else
          src_row = row0 + m0 + m;
        const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
        aoff[q] = (uint32_t)src_row * arow_bytes + (uint32_t)(c << 4);
      }
      // A stage s (clamped to the last) into ring buffer `b`
      auto issue_a = [&](int b, int s, int q) {
        const int sc = min(s, nsteps - 1);
        dma16(abase + (size_t)sc * (WBK * 2), aoff[q], ring_m0 + (uint32_t)b * A_BYTES + (DMA_A * wv + q) * 1024);
      };
      // This lane's B fragment j of substep u of step s (clamped): row 32 (j % 2) + l32 of block
      // 8 nt + 2 wv + j / 2, chunk 4 s + 2 u + hi.
      const uint8_t* bl = (GATEUP ? a.w13 : a.w2) + (size_t)slot * ncols * K * 2 + (size_t)(8 * nt + 2 * wv) * nchunk * 1024 +
                          (size_t)(hi * 1024 + l32 * 16);
      auto load_b = [&](int s, int u, int j) -> bf16x8 {
        const int sc = min(s, nsteps - 1);
        return *(const bf16x8*)(bl + ((size_t)(j >> 1) * nchunk + 4 * sc + 2 * u) * 1024 + (j & 1) * 512);
      };

      f32x16 acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
      bf16x8 fa0[4], fa1[4];   // A fragments of substeps 0 and 1
      bf16x8 bq[4][2][4];      // B register sets: [step % 4][substep][fragment]
      auto frag_a = [&](const uint8_t* st, int u, int i) -> bf16x8 {
        return *(const bf16x8*)(st + (u ? a_rd1 : a_rd0) + i * 2048);
      };

      // prologue: A stages 0..BD_NS-1, then B of steps 0..2 and substep 0 of step 3
      for (int s = 0; s < BD_NS; ++s)
#pragma unroll
        for (int q = 0; q < DMA_A; ++q) issue_a(s, s, q);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (st < 3 || u == 0) bq[st][u][j] = load_b(st, u, j);
      wait_vm<2 * (BD_NS - 1) + BD_PRO_B>();  // A stage 0
      lds_reads_done_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) fa0[i] = frag_a(ring, 0, i);

      int cb = 0;  // ring buffer of step s
      auto step = [&](int s, auto kset) {
        constexpr int k = decltype(kset)::value;
        const uint8_t* st = ring + cb * A_BYTES;
        const int nb = (cb + 1 == BD_NS) ? 0 : cb + 1;
        const uint8_t* nst = ring + nb * A_BYTES;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          if ((n >> 2) < MI)
            acc[n >> 2][n & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[n >> 2], bq[k][0][n & 3], acc[n >> 2][n & 3], 0, 0, 0);
          if (n < 4) {
            if (n < MI) fa1[n] = frag_a(st, 1, n);
          } else if (n < 8) bq[(k + 3) & 3][1][n - 4] = load_b(s + 3, 1, n - 4);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 1 < nsteps) bd_wait_stage(s);
        lds_reads_done_barrier();
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          if ((n >> 2) < MI)
            acc[n >> 2][n & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[n >> 2], bq[k][1][n & 3], acc[n >> 2][n & 3], 0, 0, 0);
          if (n < 4) {
            if (n < MI) fa0[n] = frag_a(nst, 0, n);  // past the last step: read but unused
          } else if (n < 6) issue_a(cb, s + BD_NS, n - 4);
          else if (n < 10) bq[k][0][n - 6] = load_b(s + 4, 0, n - 6);
          __builtin_amdgcn_sched_barrier(0);
        }
        cb = nb;
      };
      for (int s = 0; s < nsteps; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
      }
      // The clamped loads past the end are still in flight: they land in ring buffers and registers
      // that nothing reads, but the staging area is separate and the next tile's prologue loads
      // complete after them (issue order), so no wait is needed here.  The next tile is claimed
      // only now (its latency hides behind the epilogue), so that a block that ends late does not
      // hold a tile that another block could have started.
      if (tid == 0) nxt = queue_claim(a.qctr, nitems, qoff);
      store_tile<GATEUP, 4>(acc, stg, a, lane, wv, 8 * nt + 2 * wv, shared, row0, m0, mrows);
    };
    if (mrows <= WBM / 4)
      tile(std::integral_constant<int, 1>{});
    else if (mrows <= WBM / 2)
      tile(std::integral_constant<int, 2>{});
    else
      tile(std::integral_constant<int, 4>{});
    if (tid == 0) s_claim[0] = nxt;
    lds_reads_done_barrier();  // staging slices and ring buffers are rewritten by the next tile
    it = s_claim[0];
    __syncthreads();  // every thread has read the claim before thread 0 writes the next one
  }
}


// ---------------------------------------------------------------------------------------------
// FP8-B128 banks: e4m3 weights straight into registers, an fp32 scale per 128 x 128 block.
//
// The block scale must multiply the sum over its 128 K columns, so each wave keeps two sets of
// accumulators in the AGPRs: `part` collects one 128-K block (4 steps, the first MFMA of a block
// starting from zero) and is then scaled into `acc`.  That makes the wave tile 128 x 64 (4 x 2
// MFMA tiles, 128 + 128 fp32 per lane) and the block tile 128 x 256; the wave's 64 rows are one
// device row block, whose rows lie in one 128-row scale block for each half (gate and up rows of
// W13, or the 64 rows of W2), so a wave needs two scales per K block.
//
// Each lane loads the 16 e4m3 of its row's chunk 2 s + hi for step s (one 16-byte load per
// fragment and step, covering both substeps: the same K permutation as MXFP4, chunk 2 hi + u of A)
// into one of 4 register sets, 4 steps ahead, and decodes them exactly to bf16 with
// v_cvt_scalef32_pk_bf16_fp8 at scale 1.  The activations go through the same 7-stage ring.
// Per step: phase 0 = 8 MFMAs on substep 0 (A substep-1 reads and the substep-1 decodes between
// them), the wait and barrier, phase 1 = 8 MFMAs on substep 1 (next stage's A reads, this wave's 2
// A loads of stage s + F8_NS, then its 2 weight loads of step s + 4).
constexpr int F8_NS = 7;
constexpr int F8_BN = 256;      // weight rows per tile
constexpr int F8_SETS = 4;      // weight register sets
constexpr int F8_STG = 4 * 64 * (64 * 2 + 16);

__host__ __device__ inline size_t f8_lds_bytes(int E) { return wide_ring_off(E) + (size_t)F8_NS * A_BYTES + F8_STG; }

// Loads issued after A stage s + 1 when step s waits for it: 2 + 4 (F8_NS - 2) = 22 once the ring
// is in its steady state; in the first F8_NS - 1 steps of a tile the prologue's loads count
// (2 (F8_NS - 2 - s) + 2 F8_SETS + 4 s = 18 + 2 s).
__device__ __forceinline__ void f8_wait_stage(int s) {
  static_assert(F8_NS == 7 && F8_SETS == 4, "counts below");
  if (s >= F8_NS - 1) wait_vm<22>();
  else if (s == 0) wait_vm<18>();
  else if (s == 1) wait_vm<20>();
  else if (s == 2) wait_vm<22>();
  else if (s == 3) wait_vm<24>();
  else if (s == 4) wait_vm<26>();
  else wait_vm<28>();
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void gemm_f8_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint8_t* ring = lds + wide_ring_off(a.E);
  uint8_t* stg = ring + F8_NS * A_BYTES;
  const uint32_t ring_m0 = lds_u32(ring);

  const int K = GATEUP ? a.d : a.I;
  const int ncols = GATEUP ? 2 * a.I : a.d;
  const int ntiles = ncols / F8_BN;
  const int nchunk = K / 16;   // 16-byte chunks (16 e4m3) per weight row
  const int kblocks = K / 128;
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + WBM - 1) / WBM) * ntiles; });
  const int nitems = s_item0[gl.n];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int TK = a.T * a.k;
  const int nsteps = K / WBK;  // a multiple of 8 (K % 256 == 0)
  const uint8_t* abase = GATEUP ? (const uint8_t*)a.x : (const uint8_t*)a.h;
  const uint32_t arow_bytes = (uint32_t)K * 2;
  const int xo = ((l32 >> 1) ^ (l32 >> 2)) & 3;
  const int a_rd0 = l32 * 64 + (((2 * hi) ^ xo) << 4);
  const int a_rd1 = l32 * 64 + (((2 * hi + 1) ^ xo) << 4);

  const int NB = gridDim.x;
  const int lb = (NB % 8 == 0) ? (blockIdx.x % 8) * (NB / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int it = lb; it < nitems; it += NB) {
    const int g = find_group(s_item0, gl.n, it);
    const int local = __builtin_amdgcn_readfirstlane(it - s_item0[g]);
    const int mt = local / ntiles, nt = local % ntiles;
    const int slot = __builtin_amdgcn_readfirstlane(s_slot[g]);
    const int row0 = __builtin_amdgcn_readfirstlane(s_row0[g]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[g]);
    const bool shared = row0 >= TK;
    const int m0 = mt * WBM;
    const int mrows = min(WBM, cnt - m0);
    const int blk = 4 * nt + wv;  // this wave's device row block

    uint32_t aoff[DMA_A];
#pragma unroll
    for (int q = 0; q < DMA_A; ++q) {
      const int r = 16 * (DMA_A * wv + q) + (lane >> 2);
      const int m = min(r, mrows - 1);
      int src_row;
      if (GATEUP)
        src_row = shared ? (m0 + m) : a.gather[row0 + m0 + m] / a.k;
      else
        src_row = row0 + m0 + m;
      const int c = (lane & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
      aoff[q] = (uint32_t)src_row * arow_bytes + (uint32_t)(c << 4);
    }
    auto issue_a = [&](int b, int s, int q) {
      const int sc = min(s, nsteps - 1);
      dma16(abase + (size_t)sc * (WBK * 2), aoff[q], ring_m0 + (uint32_t)b * A_BYTES + (DMA_A * wv + q) * 1024);
    };
    // weight bytes of fragment j (rows 32 j + l32 of the block), chunk 2 s + hi
    const uint8_t* bl = (GATEUP ? a.w13 : a.w2) + (size_t)slot * ncols * K + (size_t)blk * nchunk * 1024 +
                        (size_t)(hi * 1024 + l32 * 16);
    auto load_b = [&](int s, int j) -> u32x4 {
      const int sc = min(s, nsteps - 1);
      return *(const u32x4*)(bl + (size_t)(2 * sc) * 1024 + j * 512);
    };
    // the two scales of a K block: gate and up rows of W13 (logical rows 32 blk, I + 32 blk), or
    // the block's rows of W2 (64 blk)
    const float* sbase = (const float*)(GATEUP ? a.s13 : a.s2) + (size_t)slot * (ncols / 128) * kblocks;
    const int sr0 = GATEUP ? (32 * blk) / 128 : (64 * blk) / 128;
    const int sr1 = GATEUP ? (a.I + 32 * blk) / 128 : sr0;

    f32x16 acc[4][2], part[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    f32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0.0f;
    bf16x8 fa0[4], fa1[4], fb0[2], fb1[2];
    u32x4 braw[F8_SETS][2];
    auto frag_a = [&](const uint8_t* st, int u, int i) -> bf16x8 {
      return *(const bf16x8*)(st + (u ? a_rd1 : a_rd0) + i * 2048);
    };
    // substep u of raw fragment w: its 8 e4m3 (dwords 2 u, 2 u + 1) exactly as bf16
    auto decode = [&](const u32x4& w, int u) -> bf16x8 {
      u32x4 o;
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * u], 1.0f, false));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * u], 1.0f, true));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * u + 1], 1.0f, false));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * u + 1], 1.0f, true));
      return __builtin_bit_cast(bf16x8, o);
    };

    for (int s = 0; s < F8_NS; ++s)
#pragma unroll
      for (int q = 0; q < DMA_A; ++q) issue_a(s, s, q);
#pragma unroll
    for (int t = 0; t < F8_SETS; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) braw[t][j] = load_b(t, j);
    wait_vm<2 * (F8_NS - 1) + 2 * F8_SETS>();  // A stage 0
    lds_reads_done_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) fa0[i] = frag_a(ring, 0, i);

    int cb = 0;
    float sc0 = 0.0f, sc1 = 0.0f;  // the current K block's scales
    auto step = [&](int s, auto kset) {
      constexpr int k = decltype(kset)::value;
      constexpr bool kb_first = (k & 3) == 0, kb_last = (k & 3) == 3;
      const uint8_t* st = ring + cb * A_BYTES;
      const int nb = (cb + 1 == F8_NS) ? 0 : cb + 1;
      const uint8_t* nst = ring + nb * A_BYTES;
      if (kb_first) {  // this K block's scales (scalar loads, used 4 steps later)
        sc0 = sbase[(size_t)sr0 * kblocks + (s >> 2)];
        sc1 = sbase[(size_t)sr1 * kblocks + (s >> 2)];
      }
      fb0[0] = decode(braw[k][0], 0);
      fb0[1] = decode(braw[k][1], 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int i = n >> 1, j = n & 1;
        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[i], fb0[j], kb_first ? zero : part[i][j], 0, 0, 0);
        if (n < 4) fa1[n] = frag_a(st, 1, n);
        else if (n < 6) fb1[n - 4] = decode(braw[k][n - 4], 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s + 1 < nsteps) {
        if (s < F8_NS - 1)
          f8_wait_stage(s);
        else
          wait_vm<22>();
      }
      lds_reads_done_barrier();
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int i = n >> 1, j = n & 1;
        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1[j], part[i][j], 0, 0, 0);
        if (n < 4) fa0[n] = frag_a(nst, 0, n);
        else if (n < 6) issue_a(cb, s + F8_NS, n - 4);
        else braw[k][n - 6] = load_b(s + F8_SETS, n - 6);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kb_last) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[i][0][r] = fmaf(part[i][0][r], sc0, acc[i][0][r]);
            acc[i][1][r] = fmaf(part[i][1][r], sc1, acc[i][1][r]);
          }
      }
      cb = nb;
    };
    for (int s = 0; s < nsteps; s += 4) {
      step(s, std::integral_constant<int, 0>{});
      step(s + 1, std::integral_constant<int, 1>{});
      step(s + 2, std::integral_constant<int, 2>{});
      step(s + 3, std::integral_constant<int, 3>{});
    }
    store_tile<GATEUP, 2>(acc, stg, a, lane, wv, blk, shared, row0, m0, mrows);
    // every load of this tile has landed (the repeated ones past its end included) before the next
    // tile's prologue reuses the ring and the registers
    wait_vm<0>();
    lds_reads_done_barrier();
  }
}

template <int FMT, bool GATEUP>
hipError_t launch_wide(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  auto kern = gemm_wide_kernel<FMT, GATEUP>;
  static LaunchCache cache;  // the LDS limit is set once for the largest E (512)
  LaunchFacts f;
  if (cache.get((const void*)kern, 256, wide_lds_bytes<FMT>(512), &f) != hipSuccess) return hipGetLastError();
  const int cus = f.cus;
  const int ntiles = (GATEUP ? 2 * a.I : a.d) / WBN;
  long long blocks = (long long)tiles_upper * ntiles;
  if (blocks > cus) blocks = cus;  // one block per CU (the ring takes most of its LDS)
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), wide_lds_bytes<FMT>(a.E), s, a);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_bd(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  auto kern = gemm_bd_kernel<GATEUP>;
  static LaunchCache cache;  // the LDS limit is set once for the largest E (512)
  LaunchFacts f;
  if (cache.get((const void*)kern, 256, bd_lds_bytes(512), &f) != hipSuccess) return hipGetLastError();
  const int cus = f.cus;
  const int ntiles = (GATEUP ? 2 * a.I : a.d) / WBN;
  long long blocks = (long long)tiles_upper * ntiles;
  if (blocks > cus) blocks = cus;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), bd_lds_bytes(a.E), s, a);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_f8(const FfnArgs& a, int tiles_upper, hipStream_t s) {
  auto kern = gemm_f8_kernel<GATEUP>;
  static LaunchCache cache;  // the LDS limit is set once for the largest E (512)
  LaunchFacts f;
  if (cache.get((const void*)kern, 256, f8_lds_bytes(512), &f) != hipSuccess) return hipGetLastError();
  const int cus = f.cus;
  const int ntiles = (GATEUP ? 2 * a.I : a.d) / F8_BN;
  long long blocks = (long long)tiles_upper * ntiles;
  if (blocks > cus) blocks = cus;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), f8_lds_bytes(a.E), s, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_f8_fits(int rows, int K, int E) {
  return rows % F8_BN == 0 && K % 256 == 0 && E <= 512 && f8_lds_bytes(E) <= 160 * 1024;
}

// The wide kernels need 512-row weight tiles and enough K steps of 32 to fill their rings.
bool gemm_wide_fits(int fmt, int rows, int K, int E) {
  if (fmt == FMT_FP8_B128) return gemm_f8_fits(rows, K, E);
  if (rows % WBN != 0 || E > 512) return false;
  if (fmt == FMT_BF16) return K % 128 == 0 && K >= 128 && bd_lds_bytes(E) <= 160 * 1024;
  if (fmt == FMT_MXFP4) return K >= WideCfg<FMT_MXFP4>::NS * WBK && wide_lds_bytes<FMT_MXFP4>(E) <= 160 * 1024;
  return false;
}

hipError_t launch_gemm_wide(const FfnArgs& a, bool gateup, int tiles_upper, hipStream_t s) {
  if (a.fmt == FMT_FP8_B128) return gateup ? launch_f8<true>(a, tiles_upper, s) : launch_f8<false>(a, tiles_upper, s);
  if (a.fmt == FMT_MXFP4)
    return gateup ? launch_wide<FMT_MXFP4, true>(a, tiles_upper, s) : launch_wide<FMT_MXFP4, false>(a, tiles_upper, s);
  return gateup ? launch_bd<true>(a, tiles_upper, s) : launch_bd<false>(a, tiles_upper, s);
}

}  // namespace ftk
