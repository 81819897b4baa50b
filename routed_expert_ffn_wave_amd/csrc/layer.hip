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

// Groups a fused call can have: one per routed (token, slot) pair at most, one per expert at
// most, plus the shared expert.
__host__ __device__ inline int layer_group_cap(int T, int E, int k) { return (T * k < E ? T * k : E) + 1; }

// LDS of the routing / permutation / group part, in ints (the GEMV union follows, 16-aligned)
__host__ __device__ inline size_t layer_meta_ints(int T, int E, int k, int NT) {
  const int n = T * k;
  return (size_t)E                                // slot table
         + 4 * (size_t)n                          // ids, w, gather, crow
         + (size_t)T                              // contributions expected per token
         + 4 * (size_t)(layer_group_cap(T, E, k) + 1) + 4  // groups
         + 1 + 16                                 // resident ballots (8 x 64 bits, 8-aligned)
         + 2 + NT * LAYER_RPL2;                   // control
}

// LDS of the GEMV items: gate/up items over d, down items (LAYER_RPL2 row blocks) over I
__host__ __device__ inline size_t layer_union_bytes(int fmt, int d, int I, int NT, int WPB) {
  const size_t u13 = gv_union_bytes(fmt, d, NT, WPB, 1), u2 = gv_union_bytes(fmt, I, NT, WPB, LAYER_RPL2);
  return u13 > u2 ? u13 : u2;
}

// Permutation, group list and per-pair / per-token bookkeeping of a decode layer, by one wave and
// without LDS round trips between the steps (FreeToken walk-through "深入FreeToken架构…全链路剖析",
// section 一: expert dispatch).  Pair f = t*k + j with expert e_f takes sorted position
//   pos(f) = #{g : e_g < e_f} + #{g < f : e_g == e_f},
// which is the stable order by expert; both counts come from ballots of the experts' bits in
// segments of 64 pairs (an MSB-first comparison of every lane's value against all 64 at once), and
// the same comparison against expert index e gives offsets[e] = #{g : e_g < e} and counts[e].
// Writes: s_gtok[pos] = token, s_crow[f] = pos or -1 (expert not resident), s_tgt[t] = number of
// contributions token t's combine waits for, the groups (resident experts with tokens in
// ascending expert order, then the shared expert) with their first row chunk, g_tmp[0] = number
// of groups; block 0 also writes gather, inv, counts, offsets and the residual mask.
// PART 0 (one wave): the per-pair positions and rows, then the per-token counts and mask; PART 1
// (another wave, at the same time): counts, offsets and the group list.
template <int NT, int VPL, int PART>
__device__ __forceinline__ void decode_bookkeeping(const LayerArgs& L, const int* s_slot, const int* s_ids, int* s_gtok,
                                                   int* s_crow, int* s_tgt, int* g_slot, int* g_row0, int* g_cnt,
                                                   int* g_rc0, int* g_tmp, uint64_t* s_resb) {
  const FfnArgs& a = L.f;
  const int T = a.T, E = a.E, k = a.k, n = T * k, nseg = (n + 63) / 64;
  // expert ids are below E <= 64 * VPL, so IDB bits order them
  constexpr int IDB = VPL <= 1 ? 6 : VPL <= 2 ? 7 : VPL <= 4 ? 8 : VPL <= 8 ? 9 : 10;
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const bool out = blockIdx.x == 0;
  auto resident = [&](int slot) { return slot >= 0 && slot < a.n_slots; };

  // ballots of the expert-id bits of segment s (pairs 64s .. 64s+63); returns the valid lanes
  uint64_t bits[IDB];
  auto segment = [&](int s) {
    const int f = lane + 64 * s;
    const int e = f < n ? s_ids[f] : -1;
    const bool ok = f < n && (unsigned)e < (unsigned)E;
#pragma unroll
    for (int b = 0; b < IDB; ++b) bits[b] = __ballot(ok && ((e >> b) & 1));
    return __ballot(ok);
  };
  // lanes of the current segment with expert < x (returned) and == x (eq), most significant bit
  // first, without branches: sel is all ones where bit b of x is set
  auto compare = [&](int x, uint64_t valid, uint64_t& eq) {
    uint64_t lt = 0;
    eq = valid;
#pragma unroll
    for (int b = IDB - 1; b >= 0; --b) {
      const uint64_t m = bits[b];
      const uint64_t sel = 0ull - (uint64_t)((x >> b) & 1);
      lt |= eq & ~m & sel;
      eq &= ~(m ^ sel);
    }
    return lt;
  };

  if constexpr (PART == 0) {
    // per pair: sorted position -> token, and the row its y will be in; s_resb[r]: which pairs of
    // segment r have a resident expert
    for (int r = 0; r < nseg; ++r) {
      const int f = lane + 64 * r;
      const int e = f < n ? s_ids[f] : -1;
      const bool ok = f < n && (unsigned)e < (unsigned)E;
      int p = 0;
      for (int s = 0; s < nseg; ++s) {
        const uint64_t valid = segment(s);
        uint64_t eq;
        const uint64_t lt = compare(ok ? e : 0, valid, eq);
        p += __popcll(lt) + (s < r ? __popcll(eq) : s == r ? __popcll(eq & below) : 0);
      }
      const bool res = ok && resident(s_slot[e]);
      const uint64_t rb = __ballot(res);
      if (lane == 0) s_resb[r] = rb;
      if (ok) {
        s_gtok[p] = f / k;
        s_crow[f] = res ? p : -1;
        if (out) {
          L.gather[p] = f;
          L.inv[f] = p;
        }
      } else if (f < n) {
        s_crow[f] = -1;  // an id outside [0, E) (a row of NaN logits): no y row, as in the combine kernel
      }
    }
    // per token: the residual mask and the contributions its combine waits for, from the resident
    // ballots (token t's k <= 32 pairs start at bit t*k and span at most two segments)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < T) {
      const int b0 = lane * k, s0 = b0 >> 6, sh = b0 & 63;
      uint64_t v = s_resb[s0] >> sh;
      if (sh + k > 64) v |= s_resb[s0 + 1] << (64 - sh);
      const uint32_t kmask = k == 32 ? 0xffffffffu : (1u << k) - 1u;
      const uint32_t res = (uint32_t)v & kmask;
      s_tgt[lane] = __popc(res) + (a.shared_slot >= 0 ? 1 : 0);
      if (out && L.mask) L.mask[lane] = ~res & kmask;
    }
  } else {
    int ex_lt[VPL], ex_eq[VPL];
#pragma unroll
    for (int u = 0; u < VPL; ++u) ex_lt[u] = ex_eq[u] = 0;
    int total = 0;
    for (int s = 0; s < nseg; ++s) {
      const uint64_t valid = segment(s);
      total += __popcll(valid);
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        uint64_t eq;
        const uint64_t lt = compare(lane + 64 * u, valid, eq);
        ex_lt[u] += __popcll(lt);
        ex_eq[u] += __popcll(eq);
      }
    }
    // per expert: counts, offsets; groups in ascending expert order with their first row chunk
    int ng = 0, nrc = 0;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int e = lane + 64 * u;
      if (64 * u >= E) break;
      const int cnt = ex_eq[u], off = ex_lt[u];
      if (out && e < E) {
        L.counts[e] = cnt;
        L.offsets[e] = off;
      }
      const int slot = e < E ? s_slot[e] : -1;
      const bool keep = e < E && cnt > 0 && resident(slot);
      const int items = keep ? (cnt + NT - 1) / NT : 0;
      const uint64_t kb = __ballot(keep);
      const int incl = wave_incl_scan(items);
      if (keep) {
        const int gi = ng + __popcll(kb & below);
        g_slot[gi] = slot;
        g_row0[gi] = off;
        g_cnt[gi] = cnt;
        g_rc0[gi] = nrc + incl - items;
      }
      ng += __popcll(kb);
      nrc += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
      if (out) L.offsets[E] = total;
      if (resident(a.shared_slot)) {  // the shared expert: every token, rows T*k.. of h
        g_slot[ng] = a.shared_slot;
        g_row0[ng] = n;
        g_cnt[ng] = T;
        g_rc0[ng] = nrc;
        nrc += (T + NT - 1) / NT;
        ++ng;
      }
      g_rc0[ng] = nrc;
      g_tmp[0] = ng;
    }
  }
}

// The MXFP4 and NVFP4 instances, and Q4_0 with 8-wave blocks, are held to 128 VGPRs (four waves per
// SIMD): they would otherwise take a few more, which leaves room for only one 8-wave block per CU
// at d = 7168 (measured on mxfp4_shared at T = 16: 452 against 551 us per layer; nvfp4_decode 3 %
// faster too).  The other instances fit four waves per SIMD as they are.
template <int FMT, int WPB, int NT, int VPL, bool OUT_BF16, bool PROJ>
__global__ __launch_bounds__(WPB * 64)
__attribute__((amdgpu_waves_per_eu(FMT == FMT_MXFP4 || FMT == FMT_NVFP4 || (FMT == FMT_Q4_0 && WPB == 8) ? 4 : 1)))
void layer_decode_kernel(LayerArgs L) {
  const FfnArgs& a = L.f;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int T = a.T, E = a.E, k = a.k, n = T * k;
  int* s_slot = (int*)lds;           // [E]
  int* s_ids = s_slot + E;           // [n]
  float* s_w = (float*)(s_ids + n);  // [n]
  int* s_gather = (int*)(s_w + n);   // [n] sorted position -> token
  int* s_crow = s_gather + n;        // [n] sorted row a (token, slot) pair's y sits in, -1 if not computed
  int* s_tgt = s_crow + n;           // [T]
  const int gcap = layer_group_cap(T, E, k);
  int* g_slot = s_tgt + T;           // groups: [gcap + 1] each
  int* g_row0 = g_slot + gcap + 1;
  int* g_cnt = g_row0 + gcap + 1;
  int* g_rc0 = g_cnt + gcap + 1;
  int* g_tmp = g_rc0 + gcap + 1;     // [4]
  // [8] resident-pair ballots per segment of 64 pairs, at an even int offset (8-byte aligned)
  uint64_t* s_resb = (uint64_t*)(s_slot + (((int)(g_tmp + 4 - s_slot) + 1) & ~1));
  int* s_ctl = (int*)(s_resb + 8);         // [0]: claimed position, [1]: last block, [2..): (token, column block)s to combine
  uint8_t* s_union = lds + ((layer_meta_ints(T, E, k, NT) * 4 + 15) & ~(size_t)15);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // Queue qx is served by blocks qx, qx + nq, ...: each takes its first position statically (no
  // burst of atomics on one counter at launch) and claims the later ones, after the first nb_q.
  const int nq = min((int)gridDim.x, LAYER_NQ), qx = blockIdx.x % nq;
  const int nb_q = ((int)gridDim.x - qx + nq - 1) / nq;
  int32_t* queue = L.ctl + CTL_QUEUE + qx * CNT_STRIDE;
  // the slot table is loaded into registers first, so that its round trip overlaps the logits'
  constexpr int SLOTS_PER_THREAD = (64 * VPL + WPB * 64 - 1) / (WPB * 64);  // E <= 64 * VPL
  int slot_reg[SLOTS_PER_THREAD];
#pragma unroll
  for (int i = 0; i < SLOTS_PER_THREAD; ++i) {
    const int e = tid + i * WPB * 64;
    slot_reg[i] = e < E ? a.slot_of[e] : -1;
  }

  // ---- the router projection (ft_moe_layer_proj): blocks LAYER_PG t .. LAYER_PG t + LAYER_PG - 1
  // compute token t's logits.  Each wave takes experts (its block's rank in the token's group,
  // its own index) plus multiples of LAYER_PG * WPB, four at a time with all their loads issued
  // together: lane l takes the 16-byte pieces l, l + 64, ... of the row, and a butterfly over the
  // wave adds the lanes' sums, the same order every run.  The logits go out with agent-scope
  // stores, then each block adds one to the token's flag.  Every block waits until each of the T
  // flags reaches LAYER_PG and copies the logits into LDS with agent-scope loads (another XCD's L2
  // may hold stale lines of the array from an earlier call).  The computing blocks never wait
  // before publishing and every block of the grid is resident, so every wait ends (bounded anyway,
  // like the dependency waits).
  const float* route_src = L.logits;
  if constexpr (PROJ) {
    const int d = a.d, npc = d / 8;
    if ((int)blockIdx.x < T * LAYER_PG) {
      const int t = blockIdx.x / LAYER_PG, gb = blockIdx.x % LAYER_PG;
      const int stride = LAYER_PG * WPB;
      const u32x4* xr = (const u32x4*)(a.x + (size_t)t * d);
      for (int e0 = gb * WPB + w; e0 < E; e0 += 4 * stride) {
        float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const u32x4* wr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) wr[u] = (const u32x4*)(L.w_router + (size_t)min(e0 + u * stride, E - 1) * d);
        for (int pc = lane; pc < npc; pc += 64) {
          const u32x4 xv = xr[pc];
          u32x4 rv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) rv[u] = wr[u][pc];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[u] = dot2_bf16(xv[i], rv[u][i], sum[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) sum[u] += __shfl_xor(sum[u], o, 64);
          const int e = e0 + u * stride;
          if (lane == 0 && e < E)
            __hip_atomic_store(L.proj_logits + (size_t)t * E + e, sum[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      wait_stores();  // this wave's logits have landed before the flag moves
      __syncthreads();
      if (tid == 0) atomic_add_agent(L.pflag + t, 1);
    }
    if (w == 0 && lane < T) {
      int spins = 0;
      while (atomic_load_agent(L.pflag + lane) < LAYER_PG) {
        __builtin_amdgcn_s_sleep(8);
        if (++spins >= SPIN_LIMIT) {
          atomic_add_agent(L.ctl + CTL_ERR, 1);
          break;
        }
        if ((spins & 63) == 0 && atomic_load_agent(L.ctl + CTL_ERR) != 0) break;
      }
    }
    __syncthreads();
    float* s_lg = (float*)s_union;  // free until the first work item
    for (int i = tid; i < T * E; i += WPB * 64)
      s_lg[i] = __hip_atomic_load(L.proj_logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    route_src = s_lg;
  }

  // ---- route (the same routine as the router kernel, so both give the same bits)
  route_tokens<VPL>(route_src, T, E, k, w, WPB, [&](int t, int j, int e, float wt) {
    s_ids[t * k + j] = e;
    s_w[t * k + j] = wt;
  });
#pragma unroll
  for (int i = 0; i < SLOTS_PER_THREAD; ++i) {
    const int e = tid + i * WPB * 64;
    if (e < E) s_slot[e] = slot_reg[i];
  }
  __syncthreads();

  // ---- permutation, per-pair rows and per-token counts (wave 0) and, at the same time, counts,
  // offsets and the group list (wave 1), in registers
  if (w == 0)
    decode_bookkeeping<NT, VPL, 0>(L, s_slot, s_ids, s_gather, s_crow, s_tgt, g_slot, g_row0, g_cnt, g_rc0, g_tmp,
                                   s_resb);
  else if (w == 1)
    decode_bookkeeping<NT, VPL, 1>(L, s_slot, s_ids, s_gather, s_crow, s_tgt, g_slot, g_row0, g_cnt, g_rc0, g_tmp,
                                   s_resb);
  __syncthreads();
  if (blockIdx.x == 0) {  // the routing outputs of the call, and zero rows for tokens with nothing to combine
    for (int f = tid; f < n; f += WPB * 64) {
      L.ids[f] = s_ids[f];
      L.w[f] = s_w[f];
    }
    for (int t = 0; t < T; ++t) {
      if (s_tgt[t] != 0) continue;
      for (int c = tid; c < a.d; c += WPB * 64) {
        if (OUT_BF16)
          ((uint16_t*)L.out)[(size_t)t * a.d + c] = 0;
        else
          ((float*)L.out)[(size_t)t * a.d + c] = 0.0f;
      }
    }
  }
  GroupList gl{g_slot, g_row0, g_cnt, g_rc0, g_tmp[0]};
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
      // the wait for the row chunk's h runs after the item's first weight chunks are issued (W2 does
      // not depend on h); after it, h is read with agent-scope loads
      auto dep_wait = [&]() {
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
        __syncthreads();
      };
      gemv_item<FMT, false, WPB, NT, true, RPL2>(a, s_union, slot, row0, t0, nt, cb, shared, s_gather, dep_wait);
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
    if (PROJ && tid < T) atomic_zero_agent(L.pflag + tid);
    for (int i = tid; i < T * ncb2; i += WPB * 64) atomic_zero_agent(L.cdone + i * CNT_STRIDE);
    if (tid == 0) atomic_zero_agent(L.ctl + CTL_EXIT);
  }
}

// LDS of a fused launch: the bookkeeping, then the union of the GEMV items (which also holds the
// router projection's logits before the first item)
inline size_t layer_lds_bytes(int fmt, int T, int E, int k, int d, int I, int NT, int WPB, bool proj) {
  size_t u = layer_union_bytes(fmt, d, I, NT, WPB);
  if (proj && (size_t)T * E * 4 > u) u = (size_t)T * E * 4;
  return ((layer_meta_ints(T, E, k, NT) * 4 + 15) & ~(size_t)15) + u;
}

template <int FMT, int WPB, int VPL, bool OUT_BF16, bool PROJ>
static hipError_t launch_layer_cfg(const LayerArgs& L, hipStream_t s) {
  constexpr int NT = LAYER_NT;
  auto kern = layer_decode_kernel<FMT, WPB, NT, VPL, OUT_BF16, PROJ>;
  const FfnArgs& a = L.f;
  const size_t lds = layer_lds_bytes(FMT, a.T, a.E, a.k, a.d, a.I, NT, WPB, PROJ);
  static LaunchCache cache;
  LaunchFacts f;
  if (cache.get((const void*)kern, WPB * 64, lds, &f) != hipSuccess) return hipGetLastError();
  // at most the blocks the device holds at once (every block runs, so every queue advances)
  const long long items = (long long)L.n_rc * (2 * a.I / 64 + a.d / (64 * LAYER_RPL2));
  long long blocks = (long long)f.per_cu * f.cus;
  if (blocks > items) blocks = items;
  if (PROJ && blocks < (long long)a.T * LAYER_PG) blocks = (long long)a.T * LAYER_PG;  // the projection's blocks
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WPB * 64), lds, s, L);
  return hipGetLastError();
}

template <int FMT, int WPB, bool OUT_BF16, bool PROJ>
static hipError_t launch_layer_vpl(const LayerArgs& L, hipStream_t s) {
  const int E = L.f.E;
  if (E <= 64) return launch_layer_cfg<FMT, WPB, 1, OUT_BF16, PROJ>(L, s);
  if (E <= 128) return launch_layer_cfg<FMT, WPB, 2, OUT_BF16, PROJ>(L, s);
  if (E <= 256) return launch_layer_cfg<FMT, WPB, 4, OUT_BF16, PROJ>(L, s);
  if (E <= 512) return launch_layer_cfg<FMT, WPB, 8, OUT_BF16, PROJ>(L, s);
  if constexpr (PROJ)
    return hipErrorInvalidValue;  // the router projection takes E <= 512
  else
    return launch_layer_cfg<FMT, WPB, 16, OUT_BF16, PROJ>(L, s);
}

template <int FMT, bool PROJ>
static hipError_t launch_layer_proj(const LayerArgs& L, hipStream_t s) {
  const int K = L.f.d > L.f.I ? L.f.d : L.f.I;
  if (K <= 2048) {
    if (L.out_bf16) return launch_layer_vpl<FMT, 4, true, PROJ>(L, s);
    return launch_layer_vpl<FMT, 4, false, PROJ>(L, s);
  }
  if (L.out_bf16) return launch_layer_vpl<FMT, 8, true, PROJ>(L, s);
  return launch_layer_vpl<FMT, 8, false, PROJ>(L, s);
}

template <int FMT>
static hipError_t launch_layer_fmt(const LayerArgs& L, hipStream_t s) {
  if (L.w_router) return launch_layer_proj<FMT, true>(L, s);
  return launch_layer_proj<FMT, false>(L, s);
}

bool layer_decode_fits(int fmt, int T, int E, int k, int d, int I, bool proj) {
  const int WPB = (d > I ? d : I) <= 2048 ? 4 : 8;
  return layer_lds_bytes(fmt, T, E, k, d, I, LAYER_NT, WPB, proj) <= 160 * 1024;
}

hipError_t launch_layer_decode(const LayerArgs& L, hipStream_t s) {
  switch (L.f.fmt) {
    case FMT_BF16: return launch_layer_fmt<FMT_BF16>(L, s);
    case FMT_Q4_0: return launch_layer_fmt<FMT_Q4_0>(L, s);
    case FMT_MXFP4: return launch_layer_fmt<FMT_MXFP4>(L, s);
    case FMT_NVFP4: return launch_layer_fmt<FMT_NVFP4>(L, s);
    default: return launch_layer_fmt<FMT_FP8_B128>(L, s);
  }
}

}  // namespace ftk
