// Streaming grouped GEMV for expert groups with few tokens (decode).
//
// Expert FFNs are read from per-format quantised banks (FreeToken walk-through
// "深入FreeToken架构…全链路剖析", section 五).  With a handful of tokens per expert the work is one
// pass over the expert's weights, so the kernel is bound by HBM bandwidth: every byte of a touched
// expert's weights is read once per chunk of up to NT tokens, decoded in registers to bf16 pairs
// and multiplied against the activations with v_dot2_f32_bf16 (fp32 accumulate).  Block scales
// multiply the fp32 partial sum of their block, so every weight is used exactly as its format
// defines it.
//
// Mapping onto the row-interleaved bank layout (chunk c of 64 consecutive rows = 1 KiB contiguous):
//   - lane l of every wave owns row l of the item's row block, so one 16-byte load per lane reads
//     1 KiB of contiguous weights and each lane accumulates a whole row: no cross-lane reduction;
//   - the WPB waves of a block split K: wave w takes chunks w, w+WPB, ...; their partial sums meet
//     in LDS and are added in wave order (deterministic);
//   - the item's activation rows and its rows' block scales are staged once in LDS; all lanes of a
//     wave read the same chunk, so every activation read is an LDS broadcast on the LDS counter,
//     and the vector-load counter carries nothing but the weight codes, which run PF chunks ahead
//     of the arithmetic.
// Block work item = (group, chunk of up to NT tokens, 64-row device block cb):
//   gate/up: a W13 device block holds gate rows 32cb.. (lanes 0-31) and the matching up rows
//            (lanes 32-63) -> h = SiLU(g) * u for 32 columns, rounded to bf16 into the h workspace;
//   down:    W2 rows 64cb..64cb+63 -> 64 output columns of y, rounded to bf16.
// The grid is sized to the blocks the device holds at once; blocks take items from per-XCD work
// queues (ft_queue.h), so a block that starts late takes fewer items.
#include "ft_device.h"
#include "ft_gemv.h"
#include "ft_groups.h"
#include "ft_kernels.h"
#include "ft_queue.h"

namespace ftk {

__global__ void zero_ints_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_zero_ints(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <int FMT, bool GATEUP, int WPB, int NT>
__global__ __launch_bounds__(WPB * 64, 4) void gemv_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int E2 = a.E + 2;
  int* s_slot = (int*)lds;
  int* s_row0 = s_slot + E2;
  int* s_cnt = s_row0 + E2;
  int* s_item0 = s_cnt + E2;
  int* s_tmp = s_item0 + E2;
  uint8_t* s_union = lds + gv_group_bytes(a.E);
  const int ncb = (GATEUP ? 2 * a.I : a.d) / 64;  // 64-row device blocks
  GroupSrc src{a.slot_of, a.offsets, a.E, a.T, a.k, a.shared_slot, a.min_cnt, a.max_cnt, a.n_slots};
  GroupList gl{s_slot, s_row0, s_cnt, s_item0, 0};
  build_groups(src, gl, s_tmp, [&](int cnt) { return ((cnt + NT - 1) / NT) * ncb; });
  const int nitems = s_item0[gl.n];
  const int TK = a.T * a.k;
  // items from the launch's work queues (claimed one item ahead), or a fixed stride without them
  int* s_claim = s_tmp + 1;
  const bool queued = a.qctr != nullptr;
  int qoff = 0;
  int it = blockIdx.x;
  if (queued) {
    if (threadIdx.x == 0) s_claim[0] = queue_claim(a.qctr, nitems, qoff);
    __syncthreads();
    it = s_claim[0];
    __syncthreads();
  }
  while (it >= 0 && it < nitems) {
    int nxt = -1;
    if (queued && threadIdx.x == 0) nxt = queue_claim(a.qctr, nitems, qoff);
    const int g = find_group(s_item0, gl.n, it);
    const int local = it - s_item0[g];
    const int tchunk = local / ncb, cb = local % ncb;
    const int row0 = s_row0[g], cnt = s_cnt[g];
    const int t0 = tchunk * NT;
    gemv_item<FMT, GATEUP, WPB, NT>(a, s_union, s_slot[g], row0, t0, min(NT, cnt - t0), cb, row0 >= TK);
    if (queued) {
      if (threadIdx.x == 0) s_claim[0] = nxt;
      __syncthreads();
      it = s_claim[0];
      __syncthreads();
    } else {
      it += gridDim.x;
    }
  }
}

// Tokens per pass and waves per block: all NT activation rows of an item sit in LDS, so long rows
// get fewer tokens per pass and more waves per block (to keep enough loads in flight per CU).
template <int FMT, bool GATEUP, int WPB, int NT>
static hipError_t launch_cfg(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  auto kern = gemv_kernel<FMT, GATEUP, WPB, NT>;
  const int K = GATEUP ? a.d : a.I;
  const size_t lds = gv_group_bytes(a.E) + gv_union_bytes(FMT, K, NT, WPB);
  static LaunchCache cache;
  LaunchFacts f;
  if (cache.get((const void*)kern, WPB * 64, lds, &f) != hipSuccess) return hipGetLastError();
  const int ncb = (GATEUP ? 2 * a.I : a.d) / 64;
  const long long chunks = (rows_upper + NT - 1) / NT + groups_upper;
  long long blocks = chunks * ncb;
  const long long cap = (long long)f.per_cu * f.cus;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WPB * 64), lds, s, a);
  return hipGetLastError();
}

// Groups reach this kernel with up to GEMV_MAX_ROWS tokens; an item carries up to NT of them, and
// every further row chunk of a group reads the expert's weights again.  So short rows take 16
// tokens per item (one pass over the weights per group), longer rows 8 or 4 (their activation rows
// must fit in LDS); eight waves per block keep enough loads in flight with two blocks per CU.
template <int FMT, bool GATEUP>
static hipError_t launch_fmt(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  const int K = GATEUP ? a.d : a.I;
  if (K <= 2048) return launch_cfg<FMT, GATEUP, 8, 16>(a, groups_upper, rows_upper, s);
  if (K <= 4096) return launch_cfg<FMT, GATEUP, 8, 8>(a, groups_upper, rows_upper, s);
  return launch_cfg<FMT, GATEUP, 8, 4>(a, groups_upper, rows_upper, s);
}

template <bool GATEUP>
static hipError_t launch_gemv(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  switch (a.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16, GATEUP>(a, groups_upper, rows_upper, s);
    case FMT_Q4_0: return launch_fmt<FMT_Q4_0, GATEUP>(a, groups_upper, rows_upper, s);
    case FMT_MXFP4: return launch_fmt<FMT_MXFP4, GATEUP>(a, groups_upper, rows_upper, s);
    case FMT_NVFP4: return launch_fmt<FMT_NVFP4, GATEUP>(a, groups_upper, rows_upper, s);
    default: return launch_fmt<FMT_FP8_B128, GATEUP>(a, groups_upper, rows_upper, s);
  }
}

hipError_t launch_gemv_gateup(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  return launch_gemv<true>(a, groups_upper, rows_upper, s);
}
hipError_t launch_gemv_down(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s) {
  return launch_gemv<false>(a, groups_upper, rows_upper, s);
}

}  // namespace ftk
