// Residual path for the cold experts, on the host cores: the (token, expert) pairs whose expert is
// not resident on the device, computed from the bank of every expert in host memory.
//
// The engine of the pages keeps cold experts in host memory and runs them on the CPU beside the GPU
// (FreeToken walk-through section 五: bandwidth-adaptive CPU-GPU execution, the CPU side a GEMV over
// cold experts; zuoshipin.com FreeToken article, mechanism two).  The device layer leaves exactly
// those pairs out and sets their bits in the residual mask; this routine computes them with the
// device layer's numerics (fp32 sums; h and y rounded to bf16) and sums them per token in slot order
// j, from the same device-layout bank bytes the expert cache copies to the GPU.
//
// Plain C++ (no device code): the inner loops are compiled for AVX-512, AVX2 + FMA and the baseline,
// and the loader picks the widest the host supports.  Element codes are decoded through tables built
// once from the formats' definitions.
#include <immintrin.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <thread>
#include <vector>

// A build may define FT_HOST_CLONES empty (one baseline version of each loop): the thread-sanitizer
// build of the tests does, since its runtime cannot start beside the clones' load-time resolvers.
#ifndef FT_HOST_CLONES
#define FT_HOST_CLONES __attribute__((target_clones("avx512f", "arch=haswell", "default")))
#endif

namespace ftk {

// Bank format codes of the public header (FT_W_*).
enum { RF_BF16 = 0, RF_Q4_0 = 1, RF_MXFP4 = 2, RF_FP8_B128 = 3, RF_NVFP4 = 4 };

int residual_host(int fmt, int n_experts, int d, int I, const uint8_t* w13, const uint8_t* w2, const uint8_t* s13,
                  const uint8_t* s2, const uint16_t* x, const int32_t* ids, const float* w, const uint32_t* mask,
                  const int32_t* slot_of_expert, int T, int E, int k, float* out, int threads);

namespace {

inline float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
inline uint32_t to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
inline float round_bf16(float f) {  // to the nearest bf16, ties to even (NaN kept quiet)
  uint32_t u = to_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return from_bits((u | 0x00400000u) & 0xffff0000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return from_bits(u & 0xffff0000u);
}

// OCP e4m3fn: exponent bias 7, subnormals m * 2^-9, S.1111.111 is NaN, no infinities.
inline float decode_e4m3(uint32_t v) {
  const uint32_t s = (v & 0x80u) << 24, e = (v >> 3) & 15u, m = v & 7u;
  if (e == 15u && m == 7u) return NAN;
  return from_bits(s | (e ? (((e + 120u) << 23) | (m << 20)) : to_bits((float)m * 0.001953125f)));
}
// OCP e2m1: exponent bias 1, values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives.
inline float e2m1(uint32_t q) {
  const uint32_t s = (q & 8u) << 28, e = (q >> 1) & 3u, m = q & 1u;
  return from_bits(s | (e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u)));
}
// OCP E8M0: 2^(s - 127), s = 255 is NaN.
inline float e8m0(uint32_t s) {
  if (s == 255u) return NAN;
  return s ? from_bits(s << 23) : from_bits(0x00400000u);
}
// Decode tables: every e4m3 byte, and every byte of two e2m1 codes (low nibble first).
struct Tables {
  float e4m3[256];
  float fp4_pair[256][2];
  Tables() {
    for (uint32_t v = 0; v < 256; ++v) {
      e4m3[v] = decode_e4m3(v);
      fp4_pair[v][0] = e2m1(v & 15u);
      fp4_pair[v][1] = e2m1(v >> 4);
    }
  }
};
const Tables& tables() {
  static const Tables t;
  return t;
}
// 16 e4m3 codes times s, with AVX-512: the same values as the table (normal: exponent e + 120 and
// mantissa m << 20 in the fp32 bits; subnormal: m * 2^-9; S.1111.111: NaN).
__attribute__((target("avx512f"))) void decode_e4m3x16_avx512(const uint8_t* ch, float s, float* out) {
  const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)ch));
  const __m512i sign = _mm512_slli_epi32(_mm512_and_si512(v, _mm512_set1_epi32(0x80)), 24);
  const __m512i e = _mm512_and_si512(_mm512_srli_epi32(v, 3), _mm512_set1_epi32(15));
  const __m512i m = _mm512_and_si512(v, _mm512_set1_epi32(7));
  const __m512i normal =
      _mm512_or_si512(_mm512_slli_epi32(_mm512_add_epi32(e, _mm512_set1_epi32(120)), 23), _mm512_slli_epi32(m, 20));
  const __m512i sub = _mm512_castps_si512(_mm512_mul_ps(_mm512_cvtepi32_ps(m), _mm512_set1_ps(0.001953125f)));
  const __mmask16 is_sub = _mm512_cmpeq_epi32_mask(e, _mm512_setzero_si512());
  __m512 val = _mm512_castsi512_ps(_mm512_or_si512(_mm512_mask_blend_epi32(is_sub, normal, sub), sign));
  const __mmask16 is_nan = _mm512_cmpeq_epi32_mask(_mm512_and_si512(v, _mm512_set1_epi32(0x7f)), _mm512_set1_epi32(0x7f));
  val = _mm512_mask_blend_ps(is_nan, val, _mm512_set1_ps(NAN));
  _mm512_storeu_ps(out, _mm512_mul_ps(val, _mm512_set1_ps(s)));
}
bool host_has_avx512() {
  static const bool has = __builtin_cpu_supports("avx512f");
  return has;
}

// IEEE binary16.
inline float half_value(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  const float x = e == 0 ? ldexpf((float)m, -24) : e == 31 ? (m ? NAN : INFINITY) : ldexpf((float)(1024 + m), e - 25);
  return s ? -x : x;
}

// Device row of logical W13 row L (gate rows 0..I-1, then up rows): 64-row block b holds gate rows
// 32b..32b+31, then the matching up rows (the bank's documented device layout).
inline int w13_row(int L, int I) { return L < I ? 64 * (L >> 5) + (L & 31) : 64 * ((L - I) >> 5) + 32 + ((L - I) & 31); }

// One bank matrix of one slot in the device layout: 16-byte code chunks interleaved in 64-row blocks,
// per-(row, chunk) scales interleaved the same way (Q4_0, MXFP4, NVFP4), FP8 scales on the
// [rows / 128][K / 128] grid of logical rows, NVFP4 matrix scales after every slot's block scales.
struct MatView {
  int fmt, K, nchunk, perm_I;  // perm_I = I for W13 (gate/up block order), 0 for W2
  long long row0;              // first (stacked) row of the slot
  long long rows_all;          // rows of all slots
  int slot;
  const uint8_t* codes;
  const uint8_t* scales;
};

// Logical row L of the slot to fp32 values out[0..K).
FT_HOST_CLONES void decode_row(const MatView& m, int L, float* __restrict__ out) {
  const Tables& tb = tables();
  const long long g = m.row0 + (m.perm_I ? w13_row(L, m.perm_I) : L);
  const size_t blk = (size_t)(g >> 6) * m.nchunk, lane = (size_t)(g & 63);
  switch (m.fmt) {
    case RF_BF16:
      for (int c = 0; c < m.nchunk; ++c) {
        const uint16_t* ch = (const uint16_t*)(m.codes + ((blk + c) * 64 + lane) * 16);
        for (int i = 0; i < 8; ++i) out[8 * c + i] = from_bits((uint32_t)ch[i] << 16);
      }
      break;
    case RF_FP8_B128: {
      const float* sc = (const float*)m.scales + (size_t)((m.row0 + L) / 128) * (m.K / 128);
      if (host_has_avx512()) {
        for (int c = 0; c < m.nchunk; ++c)
          decode_e4m3x16_avx512(m.codes + ((blk + c) * 64 + lane) * 16, sc[(16 * c) / 128], out + 16 * c);
        break;
      }
      for (int c = 0; c < m.nchunk; ++c) {
        const uint8_t* ch = m.codes + ((blk + c) * 64 + lane) * 16;
        const float s = sc[(16 * c) / 128];
        for (int i = 0; i < 16; ++i) out[16 * c + i] = s * tb.e4m3[ch[i]];
      }
      break;
    }
    case RF_MXFP4:
      for (int c = 0; c < m.nchunk; ++c) {
        const size_t idx = (blk + c) * 64 + lane;
        const uint8_t* ch = m.codes + idx * 16;
        const float s = e8m0(m.scales[idx]);
        for (int i = 0; i < 16; ++i) {
          out[32 * c + 2 * i] = s * tb.fp4_pair[ch[i]][0];
          out[32 * c + 2 * i + 1] = s * tb.fp4_pair[ch[i]][1];
        }
      }
      break;
    case RF_NVFP4: {
      const float t = ((const float*)(m.scales + 2 * (size_t)m.rows_all * m.nchunk))[m.slot];
      for (int c = 0; c < m.nchunk; ++c) {
        const size_t idx = (blk + c) * 64 + lane;
        const uint8_t* ch = m.codes + idx * 16;
        const uint16_t pair = ((const uint16_t*)m.scales)[idx];
        const float s0 = tb.e4m3[pair & 255u], s1 = tb.e4m3[pair >> 8];
        for (int i = 0; i < 16; ++i) {
          const float s = i < 8 ? s0 : s1;
          out[32 * c + 2 * i] = t * (tb.fp4_pair[ch[i]][0] * s);
          out[32 * c + 2 * i + 1] = t * (tb.fp4_pair[ch[i]][1] * s);
        }
      }
      break;
    }
    default:  // Q4_0: word w holds element 8w+2s in bits 4s and 8w+2s+1 in bits 16+4s; value d (q - 8)
      for (int c = 0; c < m.nchunk; ++c) {
        const size_t idx = (blk + c) * 64 + lane;
        const uint8_t* ch = m.codes + idx * 16;
        const float dsc = half_value(((const uint16_t*)m.scales)[idx]);
        for (int wd = 0; wd < 4; ++wd) {
          uint32_t word;
          memcpy(&word, ch + 4 * wd, 4);
          for (int s = 0; s < 4; ++s) {
            out[32 * c + 8 * wd + 2 * s] = dsc * (float)((int)((word >> (4 * s)) & 15u) - 8);
            out[32 * c + 8 * wd + 2 * s + 1] = dsc * (float)((int)((word >> (16 + 4 * s)) & 15u) - 8);
          }
        }
      }
  }
}

// 64 partial sums (four independent vector chains at AVX-512 width), then a fixed tree.
FT_HOST_CLONES float dot(const float* __restrict__ a, const float* __restrict__ b, int n) {
  float acc[64];
  for (int l = 0; l < 64; ++l) acc[l] = 0.0f;
  int i = 0;
  for (; i + 64 <= n; i += 64)
    for (int l = 0; l < 64; ++l) acc[l] += a[i + l] * b[i + l];
  for (; i < n; ++i) acc[i & 63] += a[i] * b[i];
  for (int h = 32; h > 0; h >>= 1)
    for (int l = 0; l < h; ++l) acc[l] += acc[l + h];
  return acc[0];
}

// Four dot products against one row: the row is loaded once per four multiply-adds; 16 partial sums
// per product (one vector chain each), then the same fixed tree as dot.
FT_HOST_CLONES void dot4(const float* __restrict__ wr, const float* __restrict__ x0, const float* __restrict__ x1,
                         const float* __restrict__ x2, const float* __restrict__ x3, int n, float* __restrict__ r) {
  float a0[16], a1[16], a2[16], a3[16];
  for (int l = 0; l < 16; ++l) a0[l] = a1[l] = a2[l] = a3[l] = 0.0f;
  int i = 0;
  for (; i + 16 <= n; i += 16)
    for (int l = 0; l < 16; ++l) {
      const float v = wr[i + l];
      a0[l] += v * x0[i + l];
      a1[l] += v * x1[i + l];
      a2[l] += v * x2[i + l];
      a3[l] += v * x3[i + l];
    }
  for (; i < n; ++i) {
    a0[i & 15] += wr[i] * x0[i];
    a1[i & 15] += wr[i] * x1[i];
    a2[i & 15] += wr[i] * x2[i];
    a3[i & 15] += wr[i] * x3[i];
  }
  for (int h = 8; h > 0; h >>= 1)
    for (int l = 0; l < h; ++l) {
      a0[l] += a0[l + h];
      a1[l] += a1[l + h];
      a2[l] += a2[l + h];
      a3[l] += a3[l + h];
    }
  r[0] = a0[0];
  r[1] = a1[0];
  r[2] = a2[0];
  r[3] = a3[0];
}

// Dot products of one row with the rows p0..p1-1 of xs (stride n) into out[p - p0].
inline void dots(const float* wr, const float* xs, int p0, int p1, int n, float* out) {
  int p = p0;
  for (; p + 4 <= p1; p += 4)
    dot4(wr, xs + (size_t)p * n, xs + (size_t)(p + 1) * n, xs + (size_t)(p + 2) * n, xs + (size_t)(p + 3) * n, n,
         out + (p - p0));
  for (; p < p1; ++p) out[p - p0] = dot(wr, xs + (size_t)p * n, n);
}

template <class F>
void run_parallel(int items, int threads, F&& f) {
  std::atomic<int> next{0};
  auto worker = [&]() {
    std::vector<float> buf;
    for (int it = next.fetch_add(1); it < items; it = next.fetch_add(1)) f(it, buf);
  };
  const int n = threads < items ? threads : items;
  std::vector<std::thread> pool;
  for (int i = 1; i < n; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

int residual_host(int fmt, int n_experts, int d, int I, const uint8_t* w13, const uint8_t* w2, const uint8_t* s13,
                  const uint8_t* s2, const uint16_t* x, const int32_t* ids, const float* w, const uint32_t* mask,
                  const int32_t* slot_of_expert, int T, int E, int k, float* out, int threads) {
  // the cold pairs (mask bit set, or the expert's slot negative), grouped by expert (flat pair
  // index ascending inside a group)
  auto take = [&](int t, int j) {
    const int e = ids[(size_t)t * k + j];
    if (e < 0 || e >= E || e >= n_experts) return false;
    return mask ? ((mask[t] >> j) & 1u) != 0 : slot_of_expert[e] < 0;
  };
  std::vector<int> cnt(E + 1, 0);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j)
      if (take(t, j)) ++cnt[ids[(size_t)t * k + j] + 1];
  for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
  const int npairs = cnt[E];
  std::vector<int> pair_flat(npairs), fill(cnt.begin(), cnt.end() - 1);
  std::vector<int> pos_of_flat((size_t)T * k, -1);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j)
      if (take(t, j)) {
        const int e = ids[(size_t)t * k + j];
        pair_flat[fill[e]] = t * k + j;
        pos_of_flat[(size_t)t * k + j] = fill[e]++;
      }
  memset(out, 0, sizeof(float) * (size_t)T * d);
  if (npairs == 0) return 0;
  std::vector<int> groups;
  for (int e = 0; e < E; ++e)
    if (cnt[e + 1] > cnt[e]) groups.push_back(e);
  const int ng = (int)groups.size();
  std::vector<float> xf((size_t)npairs * d), h((size_t)npairs * I), y((size_t)npairs * d);
  for (int p = 0; p < npairs; ++p) {
    const int t = pair_flat[p] / k;
    for (int c = 0; c < d; ++c) xf[(size_t)p * d + c] = from_bits((uint32_t)x[(size_t)t * d + c] << 16);
  }
  const int per_chunk = fmt == RF_BF16 ? 8 : fmt == RF_FP8_B128 ? 16 : 32;
  auto view = [&](int e, bool gateup) {
    MatView m;
    m.fmt = fmt;
    m.K = gateup ? d : I;
    m.nchunk = m.K / per_chunk;
    m.perm_I = gateup ? I : 0;
    const int R = gateup ? 2 * I : d;
    m.row0 = (long long)e * R;
    m.rows_all = (long long)n_experts * R;
    m.slot = e;
    m.codes = gateup ? w13 : w2;
    m.scales = gateup ? s13 : s2;
    return m;
  };
  // gate/up: items of 32 h columns of one expert
  const int hb = (I + 31) / 32;
  run_parallel(ng * hb, threads, [&](int it, std::vector<float>& buf) {
    const int e = groups[it / hb], i0 = (it % hb) * 32;
    const MatView m = view(e, true);
    const int np = cnt[e + 1] - cnt[e];
    buf.resize(2 * (size_t)d + 2 * (size_t)np);
    float* gs = buf.data() + 2 * (size_t)d;
    float* us = gs + np;
    for (int i = i0; i < i0 + 32 && i < I; ++i) {
      decode_row(m, i, buf.data());
      decode_row(m, I + i, buf.data() + d);
      dots(buf.data(), xf.data(), cnt[e], cnt[e + 1], d, gs);
      dots(buf.data() + d, xf.data(), cnt[e], cnt[e + 1], d, us);
      for (int q = 0; q < np; ++q) {
        const float gv = gs[q], uv = us[q];
        h[(size_t)(cnt[e] + q) * I + i] = round_bf16(gv / (1.0f + expf(-gv)) * uv);
      }
    }
  });
  // down: items of 64 output columns of one expert
  const int yb = (d + 63) / 64;
  run_parallel(ng * yb, threads, [&](int it, std::vector<float>& buf) {
    const int e = groups[it / yb], r0 = (it % yb) * 64;
    const MatView m = view(e, false);
    const int np = cnt[e + 1] - cnt[e];
    buf.resize((size_t)I + (size_t)np);
    float* ys = buf.data() + I;
    for (int r = r0; r < r0 + 64 && r < d; ++r) {
      decode_row(m, r, buf.data());
      dots(buf.data(), h.data(), cnt[e], cnt[e + 1], I, ys);
      for (int q = 0; q < np; ++q) y[(size_t)(cnt[e] + q) * d + r] = round_bf16(ys[q]);
    }
  });
  // per token, the masked slots in order j
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int p = pos_of_flat[(size_t)t * k + j];
      if (p < 0) continue;
      const float wj = w[(size_t)t * k + j];
      float* o = out + (size_t)t * d;
      const float* yr = y.data() + (size_t)p * d;
      for (int c = 0; c < d; ++c) o[c] += wj * yr[c];
    }
  return npairs;
}

}  // namespace ftk
