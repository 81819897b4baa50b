// Work queues of one kernel launch over its item list (GEMV items or GEMM tiles).
//
// The items are cut into QN contiguous runs, one per XCD; block b serves run b % QN first (blocks
// are placed on the XCDs round-robin, so a run's items share that XCD's L2) and then the other
// runs in turn.  Each run hands out its items through a counter, so a block that starts late (its
// compute unit held by a kernel on another stream, such as the expert-cache fill) takes fewer
// items instead of holding the launch until it has worked through a fixed share.  The counters
// start every launch at zero (the grouped FFN call clears them first).
#pragma once
#include "ft_device.h"

namespace ftk {

constexpr int QN = 8;          // runs (one per XCD)
constexpr int Q_STRIDE = 16;   // ints between two run counters (64 bytes)
constexpr int Q_INTS = QN * Q_STRIDE;

// Claims the block's next item (thread 0 only): -1 when every run is exhausted.  `qoff` is the
// block's position in its cycle over the runs, kept by the caller (starts at 0).
__device__ __forceinline__ int queue_claim(int32_t* ctr, int nitems, int& qoff) {
  const int run = (nitems + QN - 1) / QN;
  for (; qoff < QN; ++qoff) {
    const int q = (int)((blockIdx.x + qoff) % QN);
    const int lo = q * run, hi = min(nitems, lo + run);
    if (lo >= hi) continue;
    const int i = __hip_atomic_fetch_add(ctr + q * Q_STRIDE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lo + i < hi) return lo + i;
  }
  return -1;
}

// The same over an item list in two parts, [0, nA) and then [nA, nA + nB): each part is cut into
// QN contiguous runs, and run q hands out its share of the first part before its share of the
// second, so that every XCD takes its long items (tiles of many rows) before its short ones.
__device__ __forceinline__ int queue_claim2(int32_t* ctr, int nA, int nB, int& qoff) {
  const int runA = (nA + QN - 1) / QN, runB = (nB + QN - 1) / QN;
  for (; qoff < QN; ++qoff) {
    const int q = (int)((blockIdx.x + qoff) % QN);
    const int loA = q * runA, lenA = max(0, min(nA, loA + runA) - loA);
    const int loB = q * runB, lenB = max(0, min(nB, loB + runB) - loB);
    if (lenA + lenB == 0) continue;
    const int i = __hip_atomic_fetch_add(ctr + q * Q_STRIDE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < lenA) return loA + i;
    if (i < lenA + lenB) return nA + loB + (i - lenA);
  }
  return -1;
}

}  // namespace ftk
