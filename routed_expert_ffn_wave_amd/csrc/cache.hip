// Global LRU expert cache: one step of its bookkeeping, and the copy of the chosen experts from the
// pinned host bank into their device slots.
//
// The GPU keeps the experts it uses most in a fixed set of bank slots under one global
// least-recently-used policy; cold experts stay in pinned host memory and are copied in beside the
// compute (zuoshipin.com FreeToken article, mechanism four; FreeToken walk-through section 五: hot
// experts on the GPU, cold ones in pinned host memory, copies overlapped with compute).  Both
// kernels read their work from device memory (the step's expert counts, the tables, the load
// list), so a step needs no host round trip and a stream capture can hold it (the paper summary's
// key insights: the LRU is CUDA-Graph compatible).
//
// Policy of one step (the pages fix no order of choice):
//   - the clock is tick + 1; an expert with tokens in this step is demanded;
//   - a demanded resident expert marks its slot used now;
//   - loads pair the demanded absent experts, by token count descending then expert index, with
//     the slots whose experts are idle in this step, empty slots first, then by last use
//     ascending, then slot index; as many as the shorter list and max_loads allow, and with a load
//     fraction q > 0 at most ceil(q m) of the m demanded absent experts (the share of the cold
//     experts copied to the GPU, the rest being left to the host: the bandwidth-adaptive split);
//   - compute_slot keeps an expert's slot only if it was resident before the step and still is;
//     load_slot names the slots loaded in this step (usable once their copy is done).
#include "ft_device.h"
#include "ft_kernels.h"

namespace ftk {
namespace {

constexpr int CACHE_THREADS = 1024;  // one block; E and the slot count are at most this

// Position of this thread among the block's threads with `pred` set (thread order) and their total.
__device__ __forceinline__ int block_compact(bool pred, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t m = __ballot(pred);
  if (lane == 0) wave_tot[wv] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < CACHE_THREADS / 64; ++i) {
    const int c = wave_tot[i];
    base += i < wv ? c : 0;
    tot += c;
  }
  total = tot;
  __syncthreads();
  return base + __popcll(m & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(CACHE_THREADS) void cache_update_kernel(const int32_t* __restrict__ counts, int E,
                                                                       int S, int max_loads, float load_fraction,
                                                                       int32_t* __restrict__ soe_g,
                                                                       int32_t* __restrict__ eos_g,
                                                                       uint32_t* __restrict__ lu_g,
                                                                       uint32_t* __restrict__ tick,
                                                                       int32_t* __restrict__ compute_slot,
                                                                       int32_t* __restrict__ load_slot,
                                                                       int32_t* __restrict__ loads,
                                                                       int32_t* __restrict__ n_loads) {
  __shared__ int cnt[CACHE_THREADS], soe[CACHE_THREADS], eos[CACHE_THREADS];
  __shared__ uint32_t lu[CACHE_THREADS];
  // ordering keys of the misses, later of the idle slots, compacted in index order; a smaller key
  // ranks first and no two keys are equal, so a key's rank is the number of smaller keys
  __shared__ unsigned long long keys[CACHE_THREADS];
  __shared__ int miss_by_rank[CACHE_THREADS], slot_by_rank[CACHE_THREADS];
  __shared__ int wave_tot[CACHE_THREADS / 64];
  const int t = threadIdx.x;
  const uint32_t now = tick[0] + 1u;
  int before = -1;
  if (t < E) {
    cnt[t] = counts[t];
    const int s = soe_g[t];
    before = (s >= 0 && s < S) ? s : -1;
    soe[t] = before;
  }
  if (t < S) {
    const int v = eos_g[t];
    eos[t] = (v >= 0 && v < E) ? v : -1;
    lu[t] = lu_g[t];
  }
  __syncthreads();
  if (t < E && cnt[t] > 0 && before >= 0) lu[before] = now;

  int nmiss = 0;
  const bool is_miss = t < E && cnt[t] > 0 && before < 0;
  const int pm = block_compact(is_miss, wave_tot, nmiss);
  // more tokens first, then the lower expert index
  const unsigned long long mkey = ((unsigned long long)(uint32_t)(0x7fffffff - (is_miss ? cnt[t] : 0)) << 32) | t;
  if (is_miss) keys[pm] = mkey;
  __syncthreads();
  if (is_miss) {
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < nmiss; ++j) r += keys[j] < mkey;
    miss_by_rank[r] = t;
  }
  __syncthreads();

  int nidle = 0;
  const int v = t < S ? eos[t] : -1;
  const bool is_idle = t < S && (v < 0 || cnt[v] == 0);
  const int pi = block_compact(is_idle, wave_tot, nidle);
  // empty first, then the earlier last use, then the lower slot (slot < 1024: 10 bits)
  const unsigned long long ikey =
      ((unsigned long long)(v >= 0) << 42) | ((unsigned long long)(t < S ? lu[t] : 0u) << 10) | t;
  if (is_idle) keys[pi] = ikey;
  __syncthreads();
  if (is_idle) {
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < nidle; ++j) r += keys[j] < ikey;
    slot_by_rank[r] = t;
  }
  __syncthreads();

  int nl = min(min(nmiss, nidle), max_loads);
  if (load_fraction > 0.0f) nl = min(nl, (int)ceilf(load_fraction * (float)nmiss));
  if (t < nl) {  // distinct experts and slots per thread: no two threads touch the same entry
    const int e = miss_by_rank[t], s = slot_by_rank[t], old = eos[s];
    if (old >= 0) soe[old] = -1;
    soe[e] = s;
    eos[s] = e;
    lu[s] = now;
    loads[2 * t] = e;
    loads[2 * t + 1] = s;
  }
  __syncthreads();
  if (t < E) {
    soe_g[t] = soe[t];
    compute_slot[t] = (before >= 0 && soe[t] == before) ? before : -1;
    if (load_slot) load_slot[t] = (before < 0 && soe[t] >= 0) ? soe[t] : -1;
  }
  if (t < S) {
    eos_g[t] = eos[t];
    lu_g[t] = lu[t];
  }
  if (t == 0) {
    tick[0] = now;
    n_loads[0] = nl;
  }
}

constexpr long long FILL_CHUNK = 64 * 1024;  // bytes one block copies per work unit

// Work unit u = (load r, segment g, chunk c) with units of one load numbered segment by segment.
__global__ __launch_bounds__(256) void cache_fill_kernel(CacheFillArgs a) {
  const int nl = min(a.n_loads[0], a.max_loads);
  long long per_load = 0;
  for (int g = 0; g < a.nseg; ++g) per_load += (a.seg[g].bytes + FILL_CHUNK - 1) / FILL_CHUNK;
  const long long units = per_load * nl;
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const int r = (int)(u / per_load);
    long long c = u - (long long)r * per_load;
    int g = 0;
    for (;; ++g) {
      const long long ng = (a.seg[g].bytes + FILL_CHUNK - 1) / FILL_CHUNK;
      if (c < ng) break;
      c -= ng;
    }
    const int e = a.loads[2 * r], s = a.loads[2 * r + 1];
    if (e < 0 || e >= a.n_src || s < 0 || s >= a.n_dst) continue;
    const long long bytes = a.seg[g].bytes, off = c * FILL_CHUNK;
    const long long len = min(FILL_CHUNK, bytes - off);
    const uint8_t* src = a.seg[g].src + (size_t)e * bytes + off;
    uint8_t* dst = a.seg[g].dst + (size_t)s * bytes + off;
    if ((bytes & 15) == 0) {  // 16-byte words, four in flight per thread
      const uint4* s4 = (const uint4*)src;
      uint4* d4 = (uint4*)dst;
      const int n = (int)(len >> 4);
      int i = threadIdx.x;
      for (; i + 3 * 256 < n; i += 4 * 256) {
        const uint4 w0 = s4[i], w1 = s4[i + 256], w2 = s4[i + 512], w3 = s4[i + 768];
        d4[i] = w0;
        d4[i + 256] = w1;
        d4[i + 512] = w2;
        d4[i + 768] = w3;
      }
      for (; i < n; i += 256) d4[i] = s4[i];
    } else {  // every segment size is a multiple of 4 bytes
      const uint32_t* s1 = (const uint32_t*)src;
      uint32_t* d1 = (uint32_t*)dst;
      for (int i = threadIdx.x; i < (int)(len >> 2); i += 256) d1[i] = s1[i];
    }
  }
}

}  // namespace

hipError_t launch_cache_update(const int32_t* counts, int E, int S, int max_loads, float load_fraction,
                               int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use, uint32_t* tick,
                               int32_t* compute_slot, int32_t* load_slot, int32_t* loads, int32_t* n_loads,
                               hipStream_t s) {
  hipLaunchKernelGGL(cache_update_kernel, dim3(1), dim3(CACHE_THREADS), 0, s, counts, E, S, max_loads, load_fraction,
                     slot_of_expert, expert_of_slot, last_use, tick, compute_slot, load_slot, loads, n_loads);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheFillArgs& a, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(cache_fill_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ftk
