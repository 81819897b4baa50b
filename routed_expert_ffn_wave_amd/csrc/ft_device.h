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

enum { FMT_BF16 = 0, FMT_Q4_0 = 1, FMT_MXFP4 = 2, FMT_FP8_B128 = 3 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// E8M0 scale 2^(s-127) as fp32 (s = 255 is NaN).  2^-127 is an fp32 subnormal and is kept exactly.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  if (s == 255u) return __uint_as_float(0x7fc00000u);
  if (s == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(s << 23);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------------------------------------
// Per-format decode of one lane's code chunk into bf16 pairs.
//
// Each format is read as one 16-byte load per row per lane ("chunk"): 8 bf16, 16 e4m3, or 32
// 4-bit codes (one Q4_0 / MXFP4 block).  decode_chunk() returns the chunk's weights as bf16
// pairs in "code order"; x_pair_index() gives, for pair p of code order, the index in K order
// (relative to the chunk start) of its first element; the second element is first + stride.
//   BF16 / FP8: code order = K order, pairs (2p, 2p+1).
//   MXFP4: byte i holds elements 2i (low) and 2i+1 (high) -> pairs (2p, 2p+1).
//   Q4_0 (GGUF): byte i holds element i (low nibble) and element i+16 (high nibble); we form
//   pairs from the low nibbles of bytes (4w+2c, 4w+2c+1)...  see q4_pairs below.
// For Q4_0 the decoded bf16 values are (128 + q) (exact; the caller subtracts 136 * sum(x) per block).

template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_BF16> {
  static constexpr int ELEMS = 8;    // K elements per 16-byte chunk
  static constexpr int PAIRS = 4;
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = c[i];
  }
  // pair i covers K elements (2i, 2i+1)
  __device__ static int first(int i) { return 2 * i; }
  static constexpr int SECOND = 1;
};

template <>
struct Chunk<FMT_FP8_B128> {
  static constexpr int ELEMS = 16;
  static constexpr int PAIRS = 8;
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // e4m3 -> bf16 is exact (3 mantissa bits, exponent range inside bf16's).
      bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false);
      bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true);
      p[2 * i] = __builtin_bit_cast(uint32_t, lo);
      p[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
    }
  }
  __device__ static int first(int i) { return 2 * i; }
  static constexpr int SECOND = 1;
};

template <>
struct Chunk<FMT_MXFP4> {
  static constexpr int ELEMS = 32;
  static constexpr int PAIRS = 16;
  // Decodes e2m1 with unit scale (exact in bf16); the block's E8M0 scale is applied to the
  // fp32 partial sum.
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 0));
      p[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 1));
      p[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 2));
      p[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], 1.0f, 3));
    }
  }
  __device__ static int first(int i) { return 2 * i; }
  static constexpr int SECOND = 1;
};

template <>
struct Chunk<FMT_Q4_0> {
  static constexpr int ELEMS = 32;
  static constexpr int PAIRS = 16;
  // Dword w (bytes 4w..4w+3) of a block holds, nibble by nibble from bit 0:
  //   e(4w) e(4w+16) e(4w+1) e(4w+17) e(4w+2) e(4w+18) e(4w+3) e(4w+19).
  // (d >> 4s) & 0x000F000F picks nibbles s and s+4: elements (4w + s/2 + 16*(s&1)) and
  // (4w + 2 + s/2 + 16*(s&1)); OR-ing 0x4300 (bf16 128.0, ulp 1) makes each half 128 + q exactly.
  __device__ static void decode(const u32x4& c, uint32_t* p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int s = 0; s < 4; ++s) p[4 * w + s] = ((c[w] >> (4 * s)) & 0x000F000Fu) | 0x43004300u;
    }
  }
  // pair 4w+s: first element index (K order inside the block), second = first + 2
  __device__ static int first(int i) {
    int w = i >> 2, s = i & 3;
    return 4 * w + (s >> 1) + 16 * (s & 1);
  }
  static constexpr int SECOND = 2;
};

// ---------------------------------------------------------------------------------------------
// wave64 reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

}  // namespace ftk
