/*
 * Scalar CPU oracle of one Mixture-of-Experts layer.  TEST INFRASTRUCTURE ONLY:
 * only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * may load it.  It shares no code with the HIP library.
 *
 * What it computes.  The FreeToken architecture walk-through ("深入FreeToken架构
 * …全链路剖析", section 五 "MoE 引擎") fixes the structure: expert FFNs live in
 * per-format quantised banks (BF16, FP8 block, NVFP4, MXFP4, GGUF Q4_0), GPU-resident
 * ("hot") experts are found by lookup, and cold experts are computed elsewhere.
 * Section 一 names "MoE 专家调度" (expert dispatch) as a stage of the request
 * path.  The pages give no formula for the gate, the top-k rule, the FFN or the
 * combine; the layer written here is the standard routed-expert layer:
 *
 *   route   : softmax over the E router logits, top-k (descending, ties to the
 *             lowest expert index), renormalise the k probabilities;
 *   permute : expert histogram, exclusive prefix sum, gather index stable by
 *             flat (token, slot) index, and its inverse;
 *   dequant : the format's decode of stored codes to fp32;
 *   ffn     : per (token, expert): h = SiLU(x Wg^T) * (x Wu^T), y = h Wd^T, fp32;
 *   combine : out[t] = sum_j w[t][j] * y[t][j] over resident experts j, plus the
 *             shared expert's output; bit j of mask[t] is set when expert j of
 *             token t is not resident (its share is left to another path, as the
 *             walk-through's section 五 leaves cold experts to the CPU).
 *
 * Numbers are fp32 with sequential sums; build with -ffp-contract=off and no
 * vectorisation so every sum is evaluated in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORA_BF16 = 0, ORA_Q4_0 = 1, ORA_MXFP4 = 2, ORA_FP8_B128 = 3, ORA_NVFP4 = 4 };

int ora_version(void) { return 1; }

/* ---------------------------------------------------------------- element decoders */

/* bf16 is the upper half of an IEEE binary32. */
float ora_bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float ora_fp16_value(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -24); /* subnormal: m * 2^-10 * 2^-14 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexpf((float)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* OCP e2m1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal. */
float ora_e2m1_value(unsigned code) {
  int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  float v = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return sign ? -v : v;
}

/* OCP e4m3fn (FP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN; no inf. */
float ora_e4m3_value(unsigned code) {
  int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  float v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexpf((float)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

/* OCP E8M0 scale: 2^(s-127); 0xFF is NaN. */
float ora_e8m0_value(unsigned s) { return s == 255 ? NAN : ldexpf(1.0f, (int)s - 127); }

/* ---------------------------------------------------------------- dequant
 * Decode rows [row0, row0+nrows) of one stored [rows][K] matrix to fp32, out[nrows][K].
 * Canonical stored layouts:
 *   BF16     codes uint16 [rows][K]
 *   Q4_0     codes uint8 [rows][K/32][18]: fp16 scale (little endian), then 16 bytes; byte i
 *            holds element i (low nibble) and element i+16 (high nibble); v = scale * (q - 8)
 *   MXFP4    codes uint8 [rows][K/2] (element 2i low nibble, 2i+1 high), scales uint8 [rows][K/32];
 *            v = e2m1(q) * 2^(s-127)
 *   FP8_B128 codes uint8 [rows][K], scales fp32 [rows/128][K/128]; v = fl32(scale * e4m3(q))
 *   NVFP4    codes uint8 [rows][K/2] as MXFP4; scales uint8 [rows][K/16] e4m3 (one per 16 along K)
 *            followed by one fp32 tensor scale t (little endian, 4-byte aligned);
 *            v = fl32(t * (e2m1(q) * e4m3(s)))  (the inner product is exact in fp32)
 * Returns 0, or -1 for a bad format or shape.
 */
int ora_dequant(int fmt, const void* codes, const void* scales, int rows, int K, int row0, int nrows,
                float* out) {
  if (row0 < 0 || nrows < 0 || row0 + nrows > rows || K <= 0) return -1;
  for (int r = row0; r < row0 + nrows; ++r) {
    float* o = out + (size_t)(r - row0) * K;
    if (fmt == ORA_BF16) {
      const uint16_t* c = (const uint16_t*)codes + (size_t)r * K;
      for (int j = 0; j < K; ++j) o[j] = ora_bf16_value(c[j]);
    } else if (fmt == ORA_Q4_0) {
      if (K % 32) return -1;
      for (int b = 0; b < K / 32; ++b) {
        const uint8_t* blk = (const uint8_t*)codes + ((size_t)r * (K / 32) + b) * 18;
        float scale = ora_fp16_value((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int i = 0; i < 16; ++i) {
          int lo = blk[2 + i] & 15, hi = blk[2 + i] >> 4;
          o[32 * b + i] = scale * (float)(lo - 8);
          o[32 * b + i + 16] = scale * (float)(hi - 8);
        }
      }
    } else if (fmt == ORA_MXFP4) {
      if (K % 32) return -1;
      const uint8_t* c = (const uint8_t*)codes + (size_t)r * (K / 2);
      const uint8_t* s = (const uint8_t*)scales + (size_t)r * (K / 32);
      for (int j = 0; j < K; ++j) {
        unsigned q = (j & 1) ? (c[j / 2] >> 4) : (c[j / 2] & 15);
        o[j] = ora_e2m1_value(q) * ora_e8m0_value(s[j / 32]);
      }
    } else if (fmt == ORA_NVFP4) {
      if (K % 32) return -1;
      const uint8_t* c = (const uint8_t*)codes + (size_t)r * (K / 2);
      const uint8_t* s = (const uint8_t*)scales + (size_t)r * (K / 16);
      float t;
      memcpy(&t, (const uint8_t*)scales + (size_t)rows * (K / 16), 4);
      for (int j = 0; j < K; ++j) {
        const unsigned q = (c[j >> 1] >> (4 * (j & 1))) & 15u; /* element 2i low nibble, 2i+1 high */
        o[j] = t * (ora_e2m1_value(q) * ora_e4m3_value(s[j / 16]));
      }
    } else if (fmt == ORA_FP8_B128) {
      if (K % 128 || rows % 128) return -1;
      const uint8_t* c = (const uint8_t*)codes + (size_t)r * K;
      const float* s = (const float*)scales + (size_t)(r / 128) * (K / 128);
      for (int j = 0; j < K; ++j) o[j] = s[j / 128] * ora_e4m3_value(c[j]);
    } else {
      return -1;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- route
 * logits fp32 [T][E] -> ids int32 [T][k] (descending logit, ties to the lowest index) and
 * w fp32 [T][k]: P = softmax over all E logits, w_j = P[ids_j] / sum_i P[ids_i].
 */
int ora_route(const float* logits, int T, int E, int k, int32_t* ids, float* w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  float* p = (float*)malloc(sizeof(float) * (size_t)E);
  if (!taken || !p) { free(taken); free(p); return -1; }
  for (int t = 0; t < T; ++t) {
    const float* L = logits + (size_t)t * E;
    int32_t* id = ids + (size_t)t * k;
    float* wt = w + (size_t)t * k;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || L[e] > L[best]) best = e; /* strict: an equal later logit never wins */
      }
      id[j] = best;
      taken[best] = 1;
    }
    float m = L[id[0]];
    float Z = 0.0f;
    for (int e = 0; e < E; ++e) {
      p[e] = expf(L[e] - m);
      Z = Z + p[e];
    }
    float S = 0.0f;
    for (int j = 0; j < k; ++j) S = S + p[id[j]] / Z;
    for (int j = 0; j < k; ++j) wt[j] = (p[id[j]] / Z) / S;
  }
  free(taken);
  free(p);
  return 0;
}

/* ---------------------------------------------------------------- router projection
 * The step before route: each token's router logits are its activation row against each
 * expert's router row (the gate that picks k of the E experts, FreeToken walk-through section 五).
 * x bf16 [T][d], wr bf16 [E][d] -> out fp64 [T][E], out[t][e] = sum_c x[t][c] * wr[e][c] with c
 * ascending in double precision (each bf16 product is exact in fp64; only the sum rounds).
 */
int ora_router_logits(const uint16_t* x, const uint16_t* wr, int T, int d, int E, double* out) {
  if (T < 0 || d <= 0 || E <= 0) return -1;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c)
        acc += (double)ora_bf16_value(x[(size_t)t * d + c]) * (double)ora_bf16_value(wr[(size_t)e * d + c]);
      out[(size_t)t * E + e] = acc;
    }
  return 0;
}

/* ---------------------------------------------------------------- permute
 * ids int32 [T][k] (flat index f = t*k + j) -> counts[E], offsets[E+1] (exclusive prefix sum),
 * gather[T*k] (sorted position -> f; grouped by expert id, ascending f inside a group) and
 * inv[T*k] (f -> sorted position).
 */
int ora_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* gather, int32_t* inv) {
  if (T < 0 || E <= 0 || k <= 0) return -1;
  int n = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int f = 0; f < n; ++f) {
    if (ids[f] < 0 || ids[f] >= E) return -1;
    counts[ids[f]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int pos = 0;
  for (int e = 0; e < E; ++e)
    for (int f = 0; f < n; ++f)
      if (ids[f] == e) {
        gather[pos] = f;
        inv[f] = pos;
        pos += 1;
      }
  return 0;
}

/* ---------------------------------------------------------------- expert FFN
 * SwiGLU expert on n input rows: x fp32 [n][d], w13 fp32 [2I][d] (gate rows 0..I-1, then up rows),
 * w2 fp32 [d][I].  h[n][I] = SiLU(g) * u with g = x.Wg_i, u = x.Wu_i; y[n][d] = h . W2_c.
 * SiLU(g) = g / (1 + exp(-g)).  h may be NULL.
 */
int ora_swiglu_ffn(const float* x, int n, int d, int I, const float* w13, const float* w2, float* h,
                   float* y) {
  if (n < 0 || d <= 0 || I <= 0) return -1;
  float* hr = (float*)malloc(sizeof(float) * (size_t)I);
  if (!hr) return -1;
  for (int r = 0; r < n; ++r) {
    const float* xr = x + (size_t)r * d;
    for (int i = 0; i < I; ++i) {
      const float* wg = w13 + (size_t)i * d;
      const float* wu = w13 + (size_t)(I + i) * d;
      float g = 0.0f, u = 0.0f;
      for (int c = 0; c < d; ++c) g = g + xr[c] * wg[c];
      for (int c = 0; c < d; ++c) u = u + xr[c] * wu[c];
      hr[i] = g / (1.0f + expf(-g)) * u;
    }
    if (h) memcpy(h + (size_t)r * I, hr, sizeof(float) * (size_t)I);
    float* yr = y + (size_t)r * d;
    for (int c = 0; c < d; ++c) {
      const float* wd = w2 + (size_t)c * I;
      float acc = 0.0f;
      for (int i = 0; i < I; ++i) acc = acc + hr[i] * wd[i];
      yr[c] = acc;
    }
  }
  free(hr);
  return 0;
}

/* ---------------------------------------------------------------- combine
 * out fp32 [T][d]: for each token, in j order, add w[t][j] * y_sorted[inv[t*k+j]] when expert
 * ids[t][j] is resident (slot_of[e] >= 0), then add y_shared[t] when given.
 * mask[t] bit j = 1 when expert ids[t][j] is not resident.  y_sorted fp32 [T*k][d].
 * Only tokens listed in `tokens` (ntok of them; NULL = all T) are written; out and mask are
 * indexed by token.
 */
int ora_combine(const float* y_sorted, const float* y_shared, const int32_t* ids, const float* w,
                const int32_t* inv, const int32_t* slot_of, int T, int E, int k, int d,
                const int32_t* tokens, int ntok, float* out, uint32_t* mask) {
  if (T < 0 || E <= 0 || k <= 0 || k > 32 || d <= 0) return -1;
  int n = tokens ? ntok : T;
  for (int q = 0; q < n; ++q) {
    int t = tokens ? tokens[q] : q;
    if (t < 0 || t >= T) return -1;
    float* o = out + (size_t)t * d;
    uint32_t bits = 0;
    for (int c = 0; c < d; ++c) o[c] = 0.0f;
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      if (slot_of[e] < 0) {
        bits |= 1u << j;
        continue;
      }
      const float* yr = y_sorted + (size_t)inv[(size_t)t * k + j] * d;
      float wj = w[(size_t)t * k + j];
      for (int c = 0; c < d; ++c) o[c] = o[c] + wj * yr[c];
    }
    if (y_shared) {
      const float* ys = y_shared + (size_t)t * d;
      for (int c = 0; c < d; ++c) o[c] = o[c] + ys[c];
    }
    if (mask) mask[t] = bits;
  }
  return 0;
}

/* ---------------------------------------------------------------- expert cache step
 * The GPU keeps the most used experts in a fixed set of S bank slots under one global
 * least-recently-used policy (zuoshipin.com FreeToken article, mechanism four; walk-through
 * section 五: hot experts resident on the GPU, cold ones in pinned host memory, a global LRU
 * expert cache, copies overlapped with compute; the paper summary's key insights: the LRU is
 * CUDA-Graph compatible).  The pages fix no order of choice, so one step reads:
 *
 *   - the step's clock is tick + 1; an expert is demanded when counts[e] > 0;
 *   - a demanded expert that is resident marks its slot used at this step;
 *   - at most max_loads loads, and when load_fraction > 0 at most ceil(load_fraction * m) of them
 *     (fp32 product), m being the number of demanded absent experts: the share of the cold experts
 *     that is copied to the GPU, the rest being computed on the host (the bandwidth-adaptive split
 *     of the walk-through's section 五 and the article's mechanism two);
 *   - repeatedly, while fewer loads than that are chosen: take the demanded absent expert
 *     with the most tokens (ties to the lowest index) and the slot to reuse: empty slots before
 *     occupied ones, then the least recently used, ties to the lowest slot index; a slot whose
 *     expert is demanded at this step is never taken.  Stop when either is missing.  The slot's
 *     old expert becomes absent; the new one is resident there and its slot used at this step;
 *   - compute_slot[e] is e's slot if e was resident before the step and still is, else -1: the
 *     experts that were already on the device; load_slot[e] is e's slot if it was loaded in this
 *     step, else -1 (a caller may compute those once their copy is done, or from the next step on).
 *
 * State: slot_of_expert[E] and expert_of_slot[S] (-1 = none, a bijection on the resident set),
 * last_use[S] and *tick; all updated in place.  loads[2n], loads[2n+1] = (expert, slot) of the
 * n-th load.  Returns the number of loads, or -1 on bad arguments.
 */
int ora_cache_update(const int32_t* counts, int E, int S, int max_loads, float load_fraction,
                     int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use, uint32_t* tick,
                     int32_t* compute_slot, int32_t* load_slot, int32_t* loads) {
  if (E <= 0 || S <= 0 || max_loads < 0) return -1;
  const uint32_t now = *tick + 1u;
  int32_t* before = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!before) return -1;
  for (int e = 0; e < E; ++e) before[e] = slot_of_expert[e];
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0 && slot_of_expert[e] >= 0) last_use[slot_of_expert[e]] = now;
  int limit = max_loads;
  if (load_fraction > 0.0f) {
    int m = 0;
    for (int e = 0; e < E; ++e) m += counts[e] > 0 && slot_of_expert[e] < 0;
    const int share = (int)ceilf(load_fraction * (float)m);
    if (share < limit) limit = share;
  }
  int n = 0;
  while (n < limit) {
    int want = -1;
    for (int e = 0; e < E; ++e)
      if (counts[e] > 0 && slot_of_expert[e] < 0 && (want < 0 || counts[e] > counts[want])) want = e;
    if (want < 0) break;
    int slot = -1;
    for (int s = 0; s < S; ++s) {
      const int v = expert_of_slot[s];
      if (v >= 0 && counts[v] > 0) continue;
      if (slot < 0) {
        slot = s;
        continue;
      }
      const int occ = v >= 0, occ_best = expert_of_slot[slot] >= 0;
      if (occ < occ_best || (occ == occ_best && last_use[s] < last_use[slot])) slot = s;
    }
    if (slot < 0) break;
    const int old = expert_of_slot[slot];
    if (old >= 0) slot_of_expert[old] = -1;
    slot_of_expert[want] = slot;
    expert_of_slot[slot] = want;
    last_use[slot] = now;
    loads[2 * n] = want;
    loads[2 * n + 1] = slot;
    ++n;
  }
  for (int e = 0; e < E; ++e) {
    compute_slot[e] = (before[e] >= 0 && slot_of_expert[e] == before[e]) ? before[e] : -1;
    load_slot[e] = (before[e] < 0 && slot_of_expert[e] >= 0) ? slot_of_expert[e] : -1;
  }
  *tick = now;
  free(before);
  return n;
}
