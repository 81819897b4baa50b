// Residual path for the cold experts: the (token, expert) pairs whose expert is not resident on the
// device, computed on the host cores from the bank of every expert in host memory, and the kernel
// that adds their sum into the layer output.
//
// The engine of the pages keeps cold experts in host memory and runs them on the CPU beside the GPU
// (FreeToken walk-through section 五: bandwidth-adaptive CPU-GPU execution, the CPU side a GEMV over
// cold experts; zuoshipin.com FreeToken article, mechanism two).  The device layer leaves exactly
// those pairs out and sets their bits in the residual mask; this routine computes them with the
// device layer's numerics (fp32 sums; h and y rounded to bf16) and sums them per token in slot order
// j, from the same device-layout bank bytes the expert cache copies to the GPU.
#include <math.h>
#include <string.h>

#include <atomic>
#include <thread>
#include <vector>

#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {
namespace {

inline float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
inline float bf16_to_f(uint16_t b) { return from_bits((uint32_t)b << 16); }
inline float round_bf16(float f) {  // to the nearest bf16, ties to even (NaN kept quiet)
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return from_bits((u | 0x00400000u) & 0xffff0000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return from_bits(u & 0xffff0000u);
}

// Element decoders (IEEE binary16; OCP e4m3fn, e2m1, E8M0).
struct Tables {
  float e4m3[256], e2m1[16], e8m0[256];
  Tables() {
    for (int v = 0; v < 256; ++v) {
      const int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
      float x = (e == 15 && m == 7) ? NAN : e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
      e4m3[v] = s ? -x : x;
      e8m0[v] = v == 255 ? NAN : ldexpf(1.0f, v - 127);
    }
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    for (int q = 0; q < 16; ++q) e2m1[q] = (q & 8) ? -mag[q & 7] : mag[q & 7];
  }
};
const Tables& tables() {
  static const Tables t;
  return t;
}
inline float half_to_f(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  float x = e == 0 ? ldexpf((float)m, -24) : e == 31 ? (m ? NAN : INFINITY) : ldexpf((float)(1024 + m), e - 25);
  return s ? -x : x;
}

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

// Logical row L of the slot (W13: gate rows 0..I-1, then up rows) to fp32 values out[0..K).
void decode_row(const MatView& m, int L, float* out) {
  const Tables& tb = tables();
  const long long g = m.row0 + (m.perm_I ? w13_device_row(L, m.perm_I) : L);
  for (int c = 0; c < m.nchunk; ++c) {
    const size_t idx = ((size_t)(g >> 6) * m.nchunk + c) * 64 + (size_t)(g & 63);
    const uint8_t* ch = m.codes + idx * 16;
    switch (m.fmt) {
      case FMT_BF16: {
        for (int i = 0; i < 8; ++i) out[8 * c + i] = bf16_to_f((uint16_t)(ch[2 * i] | ch[2 * i + 1] << 8));
        break;
      }
      case FMT_FP8_B128: {
        const float* sc = (const float*)m.scales;
        const float s = sc[(size_t)((m.row0 + L) / 128) * (m.K / 128) + (16 * c) / 128];
        for (int i = 0; i < 16; ++i) out[16 * c + i] = s * tb.e4m3[ch[i]];
        break;
      }
      case FMT_MXFP4: {
        const float s = tb.e8m0[m.scales[idx]];
        for (int i = 0; i < 16; ++i) {
          out[32 * c + 2 * i] = s * tb.e2m1[ch[i] & 15];
          out[32 * c + 2 * i + 1] = s * tb.e2m1[ch[i] >> 4];
        }
        break;
      }
      case FMT_NVFP4: {
        const uint16_t pair = ((const uint16_t*)m.scales)[idx];
        const float s0 = tb.e4m3[pair & 255], s1 = tb.e4m3[pair >> 8];
        const float t = ((const float*)(m.scales + 2 * (size_t)m.rows_all * m.nchunk))[m.slot];
        for (int i = 0; i < 16; ++i) {
          const float s = i < 8 ? s0 : s1;
          out[32 * c + 2 * i] = t * (tb.e2m1[ch[i] & 15] * s);
          out[32 * c + 2 * i + 1] = t * (tb.e2m1[ch[i] >> 4] * s);
        }
        break;
      }
      default: {  // Q4_0: word w holds element 8w+2s in bits 4s and 8w+2s+1 in bits 16+4s
        const float dsc = half_to_f(((const uint16_t*)m.scales)[idx]);
        for (int w = 0; w < 4; ++w) {
          uint32_t word;
          memcpy(&word, ch + 4 * w, 4);
          for (int s = 0; s < 4; ++s) {
            out[32 * c + 8 * w + 2 * s] = dsc * (float)((int)((word >> (4 * s)) & 15u) - 8);
            out[32 * c + 8 * w + 2 * s + 1] = dsc * (float)((int)((word >> (16 + 4 * s)) & 15u) - 8);
          }
        }
      }
    }
  }
}

inline float dot(const float* a, const float* b, int n) {  // 8 partial sums, then a fixed tree
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int i = 0;
  for (; i + 8 <= n; i += 8)
    for (int l = 0; l < 8; ++l) acc[l] += a[i + l] * b[i + l];
  for (; i < n; ++i) acc[i & 7] += a[i] * b[i];
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
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

__global__ __launch_bounds__(256) void residual_add_kernel(void* out, const float* __restrict__ res, long long n,
                                                           bool out_bf16) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    if (out_bf16) {
      uint16_t* o = (uint16_t*)out;
      const float v = __uint_as_float((uint32_t)o[i] << 16) + res[i];
      uint32_t u = __float_as_uint(v);
      u = ((u & 0x7fffffffu) > 0x7f800000u) ? (u | 0x00400000u) : u + 0x7fffu + ((u >> 16) & 1u);
      o[i] = (uint16_t)(u >> 16);
    } else {
      ((float*)out)[i] += res[i];
    }
  }
}

}  // namespace

int residual_host(int fmt, int n_experts, int d, int I, const uint8_t* w13, const uint8_t* w2, const uint8_t* s13,
                  const uint8_t* s2, const uint16_t* x, const int32_t* ids, const float* w, const uint32_t* mask,
                  int T, int E, int k, float* out, int threads) {
  // the masked pairs, grouped by expert (flat pair index ascending inside a group)
  std::vector<int> cnt(E + 1, 0);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if (((mask[t] >> j) & 1u) && e >= 0 && e < E && e < n_experts) ++cnt[e + 1];
    }
  for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
  const int npairs = cnt[E];
  std::vector<int> pair_flat(npairs), fill(cnt.begin(), cnt.end() - 1);
  std::vector<int> pos_of_flat((size_t)T * k, -1);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if (((mask[t] >> j) & 1u) && e >= 0 && e < E && e < n_experts) {
        pair_flat[fill[e]] = t * k + j;
        pos_of_flat[(size_t)t * k + j] = fill[e]++;
      }
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
    for (int c = 0; c < d; ++c) xf[(size_t)p * d + c] = bf16_to_f(x[(size_t)t * d + c]);
  }
  const int per13 = fmt == FMT_BF16 ? 8 : fmt == FMT_FP8_B128 ? 16 : 32;
  auto view = [&](int e, bool gateup) {
    MatView m;
    m.fmt = fmt;
    m.K = gateup ? d : I;
    m.nchunk = m.K / per13;
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
    buf.resize(2 * (size_t)d);
    for (int i = i0; i < i0 + 32 && i < I; ++i) {
      decode_row(m, i, buf.data());
      decode_row(m, I + i, buf.data() + d);
      for (int p = cnt[e]; p < cnt[e + 1]; ++p) {
        const float* xr = xf.data() + (size_t)p * d;
        const float gv = dot(xr, buf.data(), d), uv = dot(xr, buf.data() + d, d);
        h[(size_t)p * I + i] = round_bf16(gv / (1.0f + expf(-gv)) * uv);
      }
    }
  });
  // down: items of 64 output columns of one expert
  const int yb = (d + 63) / 64;
  run_parallel(ng * yb, threads, [&](int it, std::vector<float>& buf) {
    const int e = groups[it / yb], r0 = (it % yb) * 64;
    const MatView m = view(e, false);
    buf.resize((size_t)I);
    for (int r = r0; r < r0 + 64 && r < d; ++r) {
      decode_row(m, r, buf.data());
      for (int p = cnt[e]; p < cnt[e + 1]; ++p) y[(size_t)p * d + r] = round_bf16(dot(h.data() + (size_t)p * I, buf.data(), I));
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

hipError_t launch_residual_add(void* out, const float* res, long long n, bool out_bf16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, res, n, out_bf16);
  return hipGetLastError();
}

}  // namespace ftk
