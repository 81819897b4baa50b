// Token -> expert permutation: expert histogram (LDS atomics), exclusive prefix sum, and a gather
// index stable by flat (token, slot) index, plus its inverse.  This is the expert-dispatch stage
// of the FreeToken request path (walk-through "深入FreeToken架构…全链路剖析", section 一).
//
// The flat index range is cut into segments of SEG = 1024 entries, one per wave.
//   1. histogram: each wave counts its segment into its own LDS row with LDS atomics
//      (counts do not depend on the order of the atomics);
//   2. scan: per expert, an exclusive prefix over segments gives each segment's base inside the
//      expert's group; an exclusive prefix over experts gives the offsets;
//   3. scatter: each wave walks its segment in order, 64 entries at a time.  Lanes holding the same
//      expert find each other with ballots over the id bits; a lane's rank among its lower-numbered
//      peers plus the segment's running base is its sorted position, so positions follow flat
//      order exactly and never depend on the order atomics happen to take.
// Up to 16 segments (T*k <= 16384) run as one block of 16 waves; larger inputs use three kernels
// and a workspace of per-(expert, segment) counts.
#include "ft_device.h"
#include "ft_kernels.h"
#include "ft_permute.h"

namespace ftk {


// dynamic LDS above the default 64 KiB has to be granted per kernel
static hipError_t allow_lds(const void* kern, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}


// Block-wide exclusive scan, in place, of a[0..E) in LDS (E <= 16 * blockDim.x).  tmp: LDS, >= 32 ints.
// Returns the total to every thread.  All threads of the block must call it.
__device__ int block_exclusive_scan(int* a, int E, int* tmp) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, nw = nt >> 6;
  const int per = (E + nt - 1) / nt;
  const int b = tid * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < E) loc += a[b + i];
  int x = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int s = (lane < nw) ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < 16) tmp[16 + lane] = s;  // inclusive prefix of wave totals
  }
  __syncthreads();
  int run = x - loc + (wv > 0 ? tmp[16 + wv - 1] : 0);
  for (int i = 0; i < per; ++i)
    if (b + i < E) {
      int c = a[b + i];
      a[b + i] = run;
      run += c;
    }
  const int total = tmp[16 + nw - 1];
  __syncthreads();
  return total;
}

// One block of 1024 threads (16 waves), n <= 16 * SEG; ids may live in LDS or global memory.
// lds: at least 17 * E + 32 ints.
__device__ void permute_block(const int32_t* ids, int n, int E, int id_bits, int* lds, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ gather,
                              int32_t* __restrict__ inv) {
  int* hist = lds;            // [16][E]: per-wave counts, then per-wave bases
  int* off = lds + 16 * E;    // [E]
  int* tmp = off + E;         // [32]
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int i = tid; i < 17 * E; i += 1024) lds[i] = 0;
  __syncthreads();
  count_segment(ids, n, E, wv * SEG, hist + wv * E);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int s = 0; s < 16; ++s) {
      int c = hist[s * E + e];
      hist[s * E + e] = run;
      run += c;
    }
    off[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(off, E, tmp);
  for (int e = tid; e < E; e += 1024) offsets[e] = off[e];
  if (tid == 0) offsets[E] = total;
  for (int i = tid; i < 16 * E; i += 1024) hist[i] += off[i % E];
  __syncthreads();
  scatter_segment(ids, n, E, wv * SEG, id_bits, hist + wv * E, gather, inv);
}

__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                              int id_bits, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ gather,
                                                              int32_t* __restrict__ inv) {
  extern __shared__ int lds[];
  permute_block(ids, n, E, id_bits, lds, counts, offsets, gather, inv);
}

// ---- large path: blocks of 256 threads (4 waves), one segment per wave.
// seg_cnt layout [E][nseg] (expert major).

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids, int n, int E, int nseg,
                                                            int32_t* __restrict__ seg_cnt) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int i = tid; i < 4 * E; i += 256) lds[i] = 0;
  __syncthreads();
  const int seg = blockIdx.x * 4 + wv;
  count_segment(ids, n, E, seg * SEG, lds + wv * E);
  __syncthreads();
  for (int i = tid; i < 4 * E; i += 256) {
    int s = blockIdx.x * 4 + i / E;
    if (s < nseg) seg_cnt[(size_t)(i % E) * nseg + s] = lds[i];
  }
}

// One wave per expert: exclusive prefix over segments in place; counts[e] = total.
__global__ __launch_bounds__(256) void permute_segscan_kernel(int32_t* __restrict__ seg_cnt, int nseg, int E,
                                                               int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t* row = seg_cnt + (size_t)e * nseg;
  int carry = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    int s = s0 + lane;
    int v = (s < nseg) ? row[s] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (s < nseg) row[s] = carry + x - v;
    carry += __shfl(x, 63, 64);
  }
  if (lane == 0) counts[e] = carry;
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ ids, int n, int E, int nseg,
                                                               int id_bits, const int32_t* __restrict__ seg_base,
                                                               const int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ gather,
                                                               int32_t* __restrict__ inv) {
  extern __shared__ int lds[];
  int* off = lds;              // [E]
  int* base = lds + E;         // [4][E]
  int* tmp = base + 4 * E;     // [32]
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int e = tid; e < E; e += 256) off[e] = counts[e];
  __syncthreads();
  const int total = block_exclusive_scan(off, E, tmp);
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) offsets[e] = off[e];
    if (tid == 0) offsets[E] = total;
  }
  for (int i = tid; i < 4 * E; i += 256) {
    int s = blockIdx.x * 4 + i / E, e = i % E;
    base[i] = (s < nseg) ? off[e] + seg_base[(size_t)e * nseg + s] : 0;
  }
  __syncthreads();
  const int seg = blockIdx.x * 4 + wv;
  if (seg < nseg) scatter_segment(ids, n, E, seg * SEG, id_bits, base + wv * E, gather, inv);
}

size_t permute_workspace_bytes(int T, int E, int k) {
  long long n = (long long)T * k;
  if (n <= 16LL * SEG) return 0;
  long long nseg = (n + SEG - 1) / SEG;
  return (size_t)(nseg * E * 4);
}

static int id_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* gather, int32_t* inv, void* ws, hipStream_t s) {
  const int n = T * k;
  const int bits = id_bits_for(E);
  if (n <= 16 * SEG) {
    size_t lds = (size_t)(17 * E + 32) * sizeof(int);
    hipError_t e = allow_lds((const void*)permute_small_kernel, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), lds, s, ids, n, E, bits, counts, offsets,
                       gather, inv);
    return hipGetLastError();
  }
  const int nseg = (n + SEG - 1) / SEG;
  const int nblk = (nseg + 3) / 4;
  int32_t* seg = (int32_t*)ws;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(256), (size_t)4 * E * sizeof(int), s, ids, n, E, nseg,
                     seg);
  hipLaunchKernelGGL(permute_segscan_kernel, dim3((E + 3) / 4), dim3(256), 0, s, seg, nseg, E, counts);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(256), (size_t)(5 * E + 32) * sizeof(int), s, ids,
                     n, E, nseg, bits, seg, counts, offsets, gather, inv);
  return hipGetLastError();
}

}  // namespace ftk
