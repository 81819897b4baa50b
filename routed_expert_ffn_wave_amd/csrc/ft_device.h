// Device-side helpers shared by the gfx950 kernels of the MoE layer: vector types, bf16
// conversion, per-format weight decode to bf16 pairs, wave reductions.
//
// Weight formats are the expert-bank formats of the FreeToken walk-through
// ("深入FreeToken架构：从HTTP API到CUDA内核的本地MoE推理引擎全链路剖析", section 五); the element
// encodings are the public definitions (GGUF Q4_0, OCP MXFP4 / E8M0, OCP e4m3fn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftk {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

enum { FMT_BF16 = 0, FMT_Q4_0 = 1, FMT_MXFP4 = 2, FMT_FP8_B128 = 3, FMT_NVFP4 = 4 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// OCP e4m3fn byte as fp32 (exact): bias 7, subnormal below exponent 1, S.1111.111 is NaN, no inf.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u, sign = (b & 0x80u) << 24;
  if (e == 15u && m == 7u) return __uint_as_float(0x7fc00000u | sign);
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// E8M0 scale 2^(s-127) as fp32 (s = 255 is NaN).  2^-127 is an fp32 subnormal and is kept exactly.
// Plain integer arithmetic (no compare, no branch): s << 23 is 2^(s-127) for s = 1..254; the max
// turns s = 0 into the subnormal 0x00400000, and (s + 1) >> 8 sets the quiet-NaN bit for s = 255.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  const uint32_t b = max(s << 23, 0x00400000u) | (((s + 1u) >> 8) << 22);
  return __uint_as_float(b);
}

// (v & m) | o in one instruction: m is uniform (an SGPR), o is kept in a VGPR
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(m), "v"(o));
  return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------------------------------------
// Per-format decode of one 16-byte code chunk (8 bf16, 16 e4m3 or 32 four-bit codes) into bf16
// pairs; pair i holds K elements (2i, 2i+1) of the chunk, low half first, so it lines up with the
// i-th 32-bit word of the matching bf16 activations.  Chunks are in the device layout of the
// public header (Q4_0 words already hold (2i, 2i+1) pairs in matching nibble positions).
// Values are exact in bf16: bf16 as stored, e4m3 (3 mantissa bits), e2m1 with unit scale, and for
// Q4_0 the value 128 + q (bf16 128.0 has ulp 1), from which the caller removes 136 = 128 + 8
// through the block's activation sum.  Block scales are applied by the caller in fp32.

template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_BF16> {
  static constexpr int ELEMS = 8;  // K elements per 16-byte chunk
  static constexpr int PAIRS = 4;
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = c[i];
  }
};

template <>
struct Chunk<FMT_FP8_B128> {
  static constexpr int ELEMS = 16;
  static constexpr int PAIRS = 8;
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false));
      p[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true));
    }
  }
};

template <>
struct Chunk<FMT_MXFP4> {
  static constexpr int ELEMS = 32;
  static constexpr int PAIRS = 16;
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 0));
      p[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 1));
      p[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 2));
      p[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 3));
    }
  }
};

template <>
struct Chunk<FMT_Q4_0> {
  static constexpr int ELEMS = 32;
  static constexpr int PAIRS = 16;
  // word w, shift 4s: nibbles s (low half) and s+4 (high half) = elements 8w+2s and 8w+2s+1
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) decode_word(c[w], p + 4 * w);
  }
  // (v >> 4s) & 0x000F000F | 0x43004300 as one shift and one v_and_or_b32 (the compiler would
  // otherwise emit an AND and an OR, each with a literal operand)
  __device__ static void decode_word(uint32_t v, uint32_t* p) {
#pragma unroll
    for (int s = 0; s < 4; ++s) p[s] = and_or(s == 0 ? v : v >> (4 * s), 0x000F000Fu, 0x43004300u);
  }
};

// NVFP4: codes as MXFP4; the two 16-element halves of a chunk (words 0-1 and 2-3) have their own
// e4m3 scales, which the caller applies to fp32 partial sums (or, for the MFMA tiles, to each
// decoded value: e2m1 * e4m3 has at most 6 significant bits, so that bf16 product is exact).  The
// conversion instruction's scale operand contributes only its power of two (checked on the
// device), so it is given 1.0 here.
template <>
struct Chunk<FMT_NVFP4> {
  static constexpr int ELEMS = 32;
  static constexpr int PAIRS = 16;
  __device__ static void decode(const u32x4& c, uint32_t* p) { Chunk<FMT_MXFP4>::decode(c, p); }
};

template <int FMT>
__host__ __device__ constexpr int chunk_elems() {
  return FMT == FMT_BF16 ? 8 : FMT == FMT_FP8_B128 ? 16 : 32;  // four-bit formats: 32
}

// W13 device row order: each 64-row block holds 32 gate rows then the 32 matching up rows, so one
// block produces 32 columns of h.  Logical row L (gate 0..I-1, up I..2I-1) <-> device row.
__host__ __device__ __forceinline__ int w13_device_row(int L, int I) {
  return L < I ? 64 * (L >> 5) + (L & 31) : 64 * ((L - I) >> 5) + 32 + ((L - I) & 31);
}
__host__ __device__ __forceinline__ int w13_logical_row(int r, int I) {
  return (r & 63) < 32 ? 32 * (r >> 6) + (r & 31) : I + 32 * (r >> 6) + (r & 31);
}

// Byte offset of chunk c of row r in a row-interleaved matrix with nchunk chunks per row.
__device__ __forceinline__ size_t ilv_chunk_off(int r, int c, int nchunk) {
  return (((size_t)(r >> 6) * nchunk + c) * 64 + (r & 63)) * 16;
}
// Element index of the per-(row, chunk) scale of row r, chunk c (Q4_0, MXFP4).
__device__ __forceinline__ size_t ilv_scale_idx(int r, int c, int nchunk) {
  return ((size_t)(r >> 6) * nchunk + c) * 64 + (r & 63);
}

// ---------------------------------------------------------------------------------------------
// wave64 reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Inclusive prefix sum over the 64 lanes with DPP (gfx9): shifts within each row of 16 lanes, then
// the row totals broadcast to the rows above.  Lanes whose source is outside the pattern add 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_or_zero<0x111>(x);        // row_shr:1
  x += dpp_or_zero<0x112>(x);        // row_shr:2
  x += dpp_or_zero<0x114>(x);        // row_shr:4
  x += dpp_or_zero<0x118>(x);        // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

}  // namespace ftk
