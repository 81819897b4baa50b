// The whole MoE layer for decode batches (T <= LAYER_MAX_T tokens) in one kernel launch: routing,
// permutation, grouped SwiGLU expert FFN and combine (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", sections 一 and 五: expert dispatch, per-format expert banks, hot
// experts resident on the GPU, the others left to another path).
//
// With a handful of tokens the routing and the permutation are a few hundred entries, so every
// block computes them itself in LDS (no launch, no global round trip before the weights start to
// stream).  Block 0 also writes them out.  The work is then the GEMV items of ft_gemv.h: all
// gate/up items (row chunk major), then all down items, dealt over LAYER_NQ queues (one counter
// each, on its own 256-byte line; block b uses queue b % nq, and blocks are placed on the XCDs
// round-robin).  A block's first position is fixed by its index; it claims each later one while it
// works on the current item.
//
// Dependencies, and why every wait ends:
//   - a down item of row chunk rc needs the h columns of all ncb13 gate/up items of rc.  Those
//     items come before it in every queue, so each has been claimed by a running block that
//     finishes it without waiting on anything, or will be claimed by a running block of its queue
//     (a queue hands out down items only after all of its gate/up items).  Waits are bounded
//     anyway: one that gives up raises the sticky error word, and later waits give up at once.
//   - the down item that completes the last contribution to a (token, 64-column block) combines
//     those 64 output columns: the same fp32 sum in the same order as the combine kernel.
// h and y rows cross blocks (and XCDs, whose L2 caches are not coherent with each other) only
// through agent-scope atomic loads and stores, completed (s_waitcnt) before the counter update that
// publishes them.  Every counter starts the launch at zero; the last block to finish puts the ones
// it used back to zero for the next launch (the workspace is zero-filled once by the caller).
#include "ft_device.h"
#include "ft_gemv.h"
#include "ft_groups.h"
#include "ft_kernels.h"
#include "ft_permute.h"
#include "ft_route.h"

namespace ftk {

constexpr int SPIN_LIMIT = 1 << 20;

__device__ __forceinline__ int atomic_add_agent(int32_t* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_load_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_zero_agent(int32_t* p) {
  __hip_atomic_store(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS of the routing / permutation / group part, in ints (the GEMV union follows, 16-aligned)
__host__ __device__ inline size_t layer_meta_ints(int T, int E, int k, int NT) {
  const int n = T * k;
  return (size_t)E                 // slot table
         + 5 * (size_t)n           // ids, w, gather, inv, crow
         + 3 * (size_t)E + 1       // counts, offsets (E+1), running bases
         + (size_t)T               // contributions expected per token
         + 4 * (size_t)(E + 2) + 4 // groups
         + 2 + NT * LAYER_RPL2;    // control
}

// LDS of the GEMV items: gate/up items over d, down items (LAYER_RPL2 row blocks) over I
__host__ __device__ inline size_t layer_union_bytes(int fmt, int d, int I, int NT, int WPB) {
  const size_t u13 = gv_union_bytes(fmt, d, NT, WPB, 1), u2 = gv_union_bytes(fmt, I, NT, WPB, LAYER_RPL2);
  return u13 > u2 ? u13 : u2;
}

template <int FMT, int WPB, int NT, int VPL, bool OUT_BF16>
__global__ __launch_bounds__(WPB * 64) void layer_decode_kernel(LayerArgs L) {
  const FfnArgs& a = L.f;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int T = a.T, E = a.E, k = a.k, n = T * k;
  int* s_slot = (int*)lds;        // [E]
  int* s_ids = s_slot + E;        // [n]
  float* s_w = (float*)(s_ids + n);  // [n]
  int* s_gather = (int*)(s_w + n);   // [n] sorted position -> flat index; then -> token
  int* s_inv = s_gather + n;      // [n]
  int* s_crow = s_inv + n;        // [n] sorted row a (token, slot) pair's y sits in, -1 if not computed
  int* s_cnt = s_crow + n;        // [E]
  int* s_off = s_cnt + E;         // [E+1]
  int* s_base = s_off + E + 1;    // [E]
  int* s_tgt = s_base + E;        // [T]
  int* g_slot = s_tgt + T;        // groups: [E+2] each
  int* g_row0 = g_slot + E + 2;
  int* g_cnt = g_row0 + E + 2;
  int* g_rc0 = g_cnt + E + 2;
  int* g_tmp = g_rc0 + E + 2;     // [4]
  int* s_ctl = g_tmp + 4;         // [0]: claimed position, [1]: last block, [2..): (token, column block)s to combine
  uint8_t* s_union = lds + ((layer_meta_ints(T, E, k, NT) * 4 + 15) & ~(size_t)15);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // Queue qx is served by blocks qx, qx + nq, ...: each takes its first position statically (no
  // burst of atomics on one counter at launch) and claims the later ones, after the first nb_q.
  const int nq = min((int)gridDim.x, LAYER_NQ), qx = blockIdx.x % nq;
  const int nb_q = ((int)gridDim.x - qx + nq - 1) / nq;
  int32_t* queue = L.ctl + CTL_QUEUE + qx * CNT_STRIDE;
  for (int i = tid; i < E; i += WPB * 64) {
    s_slot[i] = a.slot_of[i];
    s_cnt[i] = 0;
  }

  // ---- route (the same routine as the router kernel, so both give the same bits)
  route_tokens<VPL>(L.logits, T, E, k, w, WPB, [&](int t, int j, int e, float wt) {
    s_ids[t * k + j] = e;
    s_w[t * k + j] = wt;
  });
  __syncthreads();

  // ---- permute (wave 0): histogram, offsets, stable positions
  if (w == 0) {
    count_segment(s_ids, n, E, 0, s_cnt);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    wave_exclusive_scan(s_cnt, E, s_off);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < E; i += 64) s_base[i] = s_off[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    scatter_segment(s_ids, n, E, 0, L.id_bits, s_base, s_gather, s_inv);
  }
  __syncthreads();

  // ---- per pair: the row its y will be in (or -1: expert not resident); per token: the mask and
  // the number of contributions its combine waits for
  const bool shared_on = a.shared_slot >= 0;
  for (int f = tid; f < n; f += WPB * 64) {
    const int slot = s_slot[s_ids[f]];
    s_crow[f] = (slot >= 0 && slot < a.n_slots) ? s_inv[f] : -1;
  }
  if (tid < T) {
    uint32_t bits = 0;
    int cnt = 0;
    for (int j = 0; j < k; ++j) {
      const int slot = s_slot[s_ids[tid * k + j]];
      if (slot >= 0 && slot < a.n_slots)
        ++cnt;
      else
        bits |= 1u << j;
    }
    s_tgt[tid] = cnt + (shared_on ? 1 : 0);
    if (blockIdx.x == 0 && L.mask) L.mask[tid] = bits;
  }
  __syncthreads();
  if (blockIdx.x == 0) {  // the routing and permutation outputs of the call
    for (int f = tid; f < n; f += WPB * 64) {
      L.ids[f] = s_ids[f];
      L.w[f] = s_w[f];
      L.gather[f] = s_gather[f];
      L.inv[f] = s_inv[f];
    }
    for (int e = tid; e < E; e += WPB * 64) L.counts[e] = s_cnt[e];
    for (int e = tid; e <= E; e += WPB * 64) L.offsets[e] = s_off[e];
    for (int t = 0; t < T; ++t) {  // tokens with nothing to combine
      if (s_tgt[t] != 0) continue;
      for (int c = tid; c < a.d; c += WPB * 64) {
        if (OUT_BF16)
          ((uint16_t*)L.out)[(size_t)t * a.d + c] = 0;
        else
          ((float*)L.out)[(size_t)t * a.d + c] = 0.0f;
      }
    }
  }
  // sorted row -> token, in place (block 0's thread stored the flat index above, same element)
  for (int p = tid; p < n; p += WPB * 64) s_gather[p] = s_gather[p] / k;

  // ---- groups, then the items
  GroupSrc src{s_slot, s_off, E, T, k, a.shared_slot, 1, 0x7fffffff, a.n_slots};
  GroupList gl{g_slot, g_row0, g_cnt, g_rc0, 0};
  build_groups(src, gl, g_tmp, [&](int cnt) { return (cnt + NT - 1) / NT; });  // ends with a barrier
  constexpr int RPL2 = LAYER_RPL2;
  const int ncb13 = 2 * a.I / 64, ncb2 = a.d / 64, nit2 = ncb2 / RPL2;  // down items: RPL2 row blocks each
  const int nrc = g_rc0[gl.n];
  const int n13 = nrc * ncb13, total = n13 + nrc * nit2;

  int pos = blockIdx.x / nq;
  for (int it = pos * nq + qx; it < total; it = pos * nq + qx) {
    int next = 0;
    if (tid == 0) next = nb_q + atomic_add_agent(queue, 1);  // claim ahead
    const bool gateup = it < n13;
    const int local = gateup ? it : it - n13;
    const int ncb = gateup ? ncb13 : nit2;
    const int rc = local / ncb, cb = local % ncb;
    const int g = find_group(g_rc0, gl.n, rc);
    const int row0 = g_row0[g], slot = g_slot[g];
    const int t0 = (rc - g_rc0[g]) * NT;
    const int nt = min(NT, g_cnt[g] - t0);
    const bool shared = row0 >= n;
    if (gateup) {
      gemv_item<FMT, true, WPB, NT, true>(a, s_union, slot, row0, t0, nt, cb, shared, s_gather);
      wait_stores();  // this wave's h stores have completed before the count moves
      __syncthreads();
      if (tid == 0) atomic_add_agent(L.done13 + rc * CNT_STRIDE, 1);
    } else {
      if (tid == 0) {
        int spins = 0;
        while (atomic_load_agent(L.done13 + rc * CNT_STRIDE) < ncb13) {
          __builtin_amdgcn_s_sleep(8);
          if (++spins >= SPIN_LIMIT) {
            atomic_add_agent(L.ctl + CTL_ERR, 1);
            break;
          }
          // after one wait has given up, later waits give up at once
          if ((spins & 63) == 0 && atomic_load_agent(L.ctl + CTL_ERR) != 0) break;
        }
      }
      __syncthreads();  // the row chunk's h is complete: read it below with agent-scope loads
      gemv_item<FMT, false, WPB, NT, true, RPL2>(a, s_union, slot, row0, t0, nt, cb, shared, s_gather);
      wait_stores();  // this wave's y stores have completed before the counts move
      __syncthreads();
      if (tid < nt * RPL2) {  // one contribution per (token, 64-column block) of the item
        const int t = tid / RPL2, cbq = RPL2 * cb + tid % RPL2;
        const int tok = shared ? t0 + t : s_gather[row0 + t0 + t];
        const int done = atomic_add_agent(L.cdone + (tok * ncb2 + cbq) * CNT_STRIDE, 1);
        s_ctl[2 + tid] = done + 1 == s_tgt[tok] ? tok * ncb2 + cbq : -1;  // the last one: combine here
      }
      __syncthreads();
      for (int i = w; i < nt * RPL2; i += WPB) {
        const int v = s_ctl[2 + i];
        if (v < 0) continue;
        const int tok = v / ncb2, cbq = v % ncb2;
        // every contribution's y rows are complete: agent-scope loads of column pairs
        const int col = 64 * cbq + lane, pcol = col & ~1, hi = (lane & 1) * 16;
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
          const int r = s_crow[tok * k + j];
          if (r < 0) continue;
          const uint32_t pr = load_u32_agent(a.y_sorted + (size_t)r * a.d + pcol);
          acc = fmaf(s_w[tok * k + j], bf16_bits_to_f32((pr >> hi) & 0xffffu), acc);
        }
        if (a.y_shared) {
          const uint32_t pr = load_u32_agent(a.y_shared + (size_t)tok * a.d + pcol);
          acc += bf16_bits_to_f32((pr >> hi) & 0xffffu);
        }
        if (OUT_BF16)
          ((uint16_t*)L.out)[(size_t)tok * a.d + col] = f32_to_bf16_bits(acc);
        else
          ((float*)L.out)[(size_t)tok * a.d + col] = acc;
      }
    }
    if (tid == 0) s_ctl[0] = next;
    __syncthreads();
    pos = s_ctl[0];
  }

  // ---- the last block to finish returns the counters to zero
  if (tid == 0) {
    wait_stores();  // this block's counter updates have landed before it reports its exit
    s_ctl[1] = atomic_add_agent(L.ctl + CTL_EXIT, 1) == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (s_ctl[1]) {
    for (int q = tid; q < nq; q += WPB * 64) atomic_zero_agent(L.ctl + CTL_QUEUE + q * CNT_STRIDE);
    for (int i = tid; i < nrc; i += WPB * 64) atomic_zero_agent(L.done13 + i * CNT_STRIDE);
    for (int i = tid; i < T * ncb2; i += WPB * 64) atomic_zero_agent(L.cdone + i * CNT_STRIDE);
    if (tid == 0) atomic_zero_agent(L.ctl + CTL_EXIT);
  }
}

template <int FMT, int WPB, int VPL, bool OUT_BF16>
static hipError_t launch_layer_cfg(const LayerArgs& L, hipStream_t s) {
  constexpr int NT = LAYER_NT;
  auto kern = layer_decode_kernel<FMT, WPB, NT, VPL, OUT_BF16>;
  const FfnArgs& a = L.f;
  const int K = a.d > a.I ? a.d : a.I;
  const size_t lds = ((layer_meta_ints(a.T, a.E, a.k, NT) * 4 + 15) & ~(size_t)15) +
                     layer_union_bytes(FMT, a.d, a.I, NT, WPB);
  static int resident_per_cu = -1;
  static size_t resident_lds = 0;
  if (resident_per_cu < 0 || lds > resident_lds) {
    int per_cu = 0;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return hipGetLastError();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WPB * 64, lds) != hipSuccess)
      return hipGetLastError();
    resident_per_cu = per_cu > 0 ? per_cu : 1;
    resident_lds = lds;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return hipGetLastError();
  // at most the blocks the device holds at once (every block runs, so every queue advances)
  const long long items = (long long)L.n_rc * (2 * a.I / 64 + a.d / (64 * LAYER_RPL2));
  long long blocks = (long long)resident_per_cu * cus;
  if (blocks > items) blocks = items;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WPB * 64), lds, s, L);
  return hipGetLastError();
}

template <int FMT, int WPB, bool OUT_BF16>
static hipError_t launch_layer_vpl(const LayerArgs& L, hipStream_t s) {
  const int E = L.f.E;
  if (E <= 64) return launch_layer_cfg<FMT, WPB, 1, OUT_BF16>(L, s);
  if (E <= 128) return launch_layer_cfg<FMT, WPB, 2, OUT_BF16>(L, s);
  if (E <= 256) return launch_layer_cfg<FMT, WPB, 4, OUT_BF16>(L, s);
  if (E <= 512) return launch_layer_cfg<FMT, WPB, 8, OUT_BF16>(L, s);
  return launch_layer_cfg<FMT, WPB, 16, OUT_BF16>(L, s);
}

template <int FMT>
static hipError_t launch_layer_fmt(const LayerArgs& L, hipStream_t s) {
  const int K = L.f.d > L.f.I ? L.f.d : L.f.I;
  if (K <= 2048) {
    if (L.out_bf16) return launch_layer_vpl<FMT, 4, true>(L, s);
    return launch_layer_vpl<FMT, 4, false>(L, s);
  }
  if (L.out_bf16) return launch_layer_vpl<FMT, 8, true>(L, s);
  return launch_layer_vpl<FMT, 8, false>(L, s);
}

bool layer_decode_fits(int fmt, int T, int E, int k, int d, int I) {
  const int WPB = (d > I ? d : I) <= 2048 ? 4 : 8;
  const size_t lds = ((layer_meta_ints(T, E, k, LAYER_NT) * 4 + 15) & ~(size_t)15) +
                     layer_union_bytes(fmt, d, I, LAYER_NT, WPB);
  return lds <= 160 * 1024;
}

hipError_t launch_layer_decode(const LayerArgs& L, hipStream_t s) {
  switch (L.f.fmt) {
    case FMT_BF16: return launch_layer_fmt<FMT_BF16>(L, s);
    case FMT_Q4_0: return launch_layer_fmt<FMT_Q4_0>(L, s);
    case FMT_MXFP4: return launch_layer_fmt<FMT_MXFP4>(L, s);
    default: return launch_layer_fmt<FMT_FP8_B128>(L, s);
  }
}

}  // namespace ftk
