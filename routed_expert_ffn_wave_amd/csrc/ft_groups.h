// Expert groups of the grouped FFN, built on the device from the permutation so that no host
// synchronisation is needed between the permute and the FFN kernels.
//
// A group is one resident expert with at least one routed token (rows offsets[e]..offsets[e+1]
// of the sorted order), or the always-on shared expert (all T tokens).  Experts whose
// slot_of_expert entry is -1 are not resident: the FreeToken walk-through ("深入FreeToken架构…
// 全链路剖析", section 五) keeps only hot experts on the GPU and hands the others to another path.
#pragma once
#include "ft_device.h"

namespace ftk {

struct GroupSrc {
  const int32_t* slot_of;  // [E]
  const int32_t* offsets;  // [E+1]
  int E, T, k;
  int shared_slot;         // -1: none
  int min_cnt, max_cnt;    // keep groups with min_cnt <= count <= max_cnt
  int n_slots;             // table entries outside [0, n_slots) are skipped (never dereferenced)
};

struct GroupList {
  int* slot;   // bank slot
  int* row0;   // first row of the group in the h / y_sorted order (T*k + 0 for the shared group)
  int* cnt;    // rows (tokens) in the group
  int* item0;  // exclusive prefix of work items; item0[n] = total
  int n;
};

// LDS bytes of a group list for E experts: slot, row0, cnt and item0 arrays of E + 2 ints each, and
// a few ints of scratch, rounded up to 16 bytes.
__host__ __device__ inline size_t group_lds_bytes(int E) { return (((size_t)4 * (E + 2) + 4) * 4 + 15) & ~(size_t)15; }

// Build the group list in LDS with wave 0 (ascending expert order, shared group last).
// items_of(cnt) gives the number of work items of a group with `cnt` rows.  Every thread of the
// block must call this; it ends with a block barrier.
template <class ItemsOf>
__device__ __forceinline__ void build_groups(const GroupSrc& s, GroupList& g, int* tmp, ItemsOf items_of) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int n = 0;
    const int last = s.E + (s.shared_slot >= 0 ? 1 : 0);
    for (int e0 = 0; e0 < last; e0 += 64) {
      const int e = e0 + lane;
      int slot = -1, row0 = 0, cnt = 0;
      if (e < s.E) {
        slot = s.slot_of[e];
        row0 = s.offsets[e];
        cnt = s.offsets[e + 1] - row0;
      } else if (e == s.E && s.shared_slot >= 0) {
        slot = s.shared_slot;
        row0 = s.T * s.k;
        cnt = s.T;
      }
      const bool keep = slot >= 0 && slot < s.n_slots && cnt > 0 && cnt >= s.min_cnt && cnt <= s.max_cnt;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int at = n + __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        g.slot[at] = slot;
        g.row0[at] = row0;
        g.cnt[at] = cnt;
      }
      n += __popcll(bal);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int carry = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const int v = (i < n) ? items_of(g.cnt[i]) : 0;
      int x = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (i < n) g.item0[i] = carry + x - v;
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) {
      g.item0[n] = carry;
      tmp[0] = n;
    }
  }
  __syncthreads();
  g.n = tmp[0];
}

// Group holding work item `it` (item0 ascending): largest g with item0[g] <= it.
__device__ __forceinline__ int find_group(const int* item0, int n, int it) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (item0[mid] <= it)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace ftk
