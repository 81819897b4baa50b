// Internal launch interface between the C ABI (api.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace ftk {

// What a kernel's launch code reuses from call to call: the device's CU count and the blocks of the
// kernel one CU holds at the largest dynamic-LDS size it has been given on that device (so the count
// never exceeds what a smaller request allows).  One instance per kernel; every read and update is
// under its mutex, so host threads may launch concurrently on any devices.
struct LaunchFacts {
  int per_cu;  // blocks per CU
  int cus;     // compute units of the current device
};
class LaunchCache {
 public:
  // Sets the kernel's dynamic-LDS limit to at least `lds` on the current device (once per larger
  // size) and returns the facts above for `threads` threads per block.
  hipError_t get(const void* kern, int threads, size_t lds, LaunchFacts* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu_);
    if (cus_[dev] == 0 &&
        hipDeviceGetAttribute(&cus_[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      cus_[dev] = 0;
      return hipGetLastError();
    }
    if (per_cu_[dev] == 0 || lds > lds_[dev]) {
      int per_cu = 0;
      if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipGetLastError();
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess)
        return hipGetLastError();
      per_cu_[dev] = per_cu > 0 ? per_cu : 1;
      lds_[dev] = lds;
    }
    *out = LaunchFacts{per_cu_[dev], cus_[dev]};
    return hipSuccess;
  }

 private:
  static constexpr int MAXDEV = 64;
  std::mutex mu_;
  size_t lds_[MAXDEV] = {};
  int per_cu_[MAXDEV] = {};
  int cus_[MAXDEV] = {};
};

// Everything the grouped FFN kernels read or write, in device memory.
struct FfnArgs {
  int fmt, d, I, n_slots;
  const uint8_t* w13;  // bank arrays (device layout of the public header)
  const uint8_t* w2;
  const uint8_t* s13;
  const uint8_t* s2;
  const int32_t* slot_of;
  int shared_slot;
  const uint16_t* x;   // bf16 [T][d]
  int T, E, k;
  const int32_t* offsets;
  const int32_t* gather;
  uint16_t* h;         // bf16 [T*k + T][I] workspace (rows T*k.. for the shared expert)
  uint16_t* y_sorted;  // bf16 [T*k][d]
  uint16_t* y_shared;  // bf16 [T][d] or null
  int min_cnt, max_cnt;  // groups this launch handles, by routed-row count
  int32_t* qctr;         // work-queue counters of this launch ([QN][Q_STRIDE], zero at launch), or null:
                         // the kernels that take items from queues (GEMV, scaled-MFMA GEMM) need them
};
// Grouped FFN launches: every launch's queue counters ([4][QN * Q_STRIDE] ints) cleared in one kernel
constexpr int FFN_QCTR_INTS = 4 * 8 * 16;
hipError_t launch_zero_ints(int32_t* p, int n, hipStream_t s);

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);

// router projection fused with route (x bf16 [T][d], w_router bf16 [E][d], d % 32 == 0, E <= 512)
size_t route_proj_workspace_bytes(int T);
hipError_t launch_route_proj(const uint16_t* x, const uint16_t* wr, int T, int d, int E, int k, float* logits,
                             int32_t* ids, float* w, void* ws, hipStream_t s);

// global LRU expert cache: one bookkeeping step (E, S <= 1024) and the copy of the chosen experts
hipError_t launch_cache_update(const int32_t* counts, int E, int S, int max_loads, float load_fraction,
                               int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use, uint32_t* tick,
                               int32_t* compute_slot, int32_t* load_slot, int32_t* loads, int32_t* n_loads,
                               hipStream_t s);
struct CacheFillSeg {
  const uint8_t* src;  // expert e's bytes at src + e * bytes (device-visible address of pinned host memory)
  uint8_t* dst;        // slot s's bytes at dst + s * bytes
  long long bytes;     // a multiple of 4
};
struct CacheFillArgs {
  CacheFillSeg seg[6];
  int nseg, n_src, n_dst, max_loads;
  const int32_t* loads;    // [max_loads][2] (expert, slot)
  const int32_t* n_loads;  // [1]
};
hipError_t launch_cache_fill(const CacheFillArgs& a, int blocks, hipStream_t s);

// residual path of the cold experts: host compute of the masked pairs (returns the pair count) and
// the device add of its result into the layer output
int residual_host(int fmt, int n_experts, int d, int I, const uint8_t* w13, const uint8_t* w2, const uint8_t* s13,
                  const uint8_t* s2, const uint16_t* x, const int32_t* ids, const float* w, const uint32_t* mask,
                  const int32_t* slot_of_expert, int T, int E, int k, float* out, int threads);
hipError_t launch_residual_add(void* out, const float* res, long long n, bool out_bf16, hipStream_t s);

// ---- start-up rate measurements (rates.hip)
// every resident 256-thread block of the streaming-read kernel (per CU x CUs) and the CU count
hipError_t rate_launch_facts(int* stream_blocks, int* cus);
// reads `bytes` (a multiple of 16) at p with `blocks` blocks; sink: 4 words per block
hipError_t launch_stream_read(const void* p, long long bytes, int blocks, uint32_t* sink, hipStream_t s);
// kind 0: bf16 32x32x16, 1: e4m3 x e4m3 32x32x64, 2: e2m3 x e2m1 32x32x64; each of the `blocks`
// 4-wave blocks issues iters x 4 MFMAs per wave; sink: 256 floats per block
hipError_t launch_mfma_rate(int kind, int blocks, int iters, float* sink, hipStream_t s);

size_t permute_workspace_bytes(int T, int E, int k);
// zero (optional): nzero ints the permutation also sets to zero, in its own kernel when it runs as
// one block (so a caller can clear the next call's counters without a launch of their own)
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* gather, int32_t* inv, void* ws, hipStream_t s, int32_t* zero = nullptr,
                          int nzero = 0);

hipError_t launch_combine(const uint16_t* y_sorted, const uint16_t* y_shared, const int32_t* ids, const float* w,
                          const int32_t* inv, const int32_t* slot_of, int n_slots, int T, int E, int k, int d,
                          void* out, uint32_t* mask, bool out_bf16, hipStream_t s);

// Streaming GEMV path (few rows per group).  groups_upper / rows_upper: host-side bounds on the
// number of groups and of rows (tokens) the launch may see, used to size the grid.
hipError_t launch_gemv_gateup(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s);
hipError_t launch_gemv_down(const FfnArgs& a, int groups_upper, long long rows_upper, hipStream_t s);
constexpr int GEMV_MAX_ROWS = 16;  // largest group the automatic path sends to the GEMV kernels

// MFMA GEMM path.
hipError_t launch_gemm_gateup(const FfnArgs& a, int tiles_upper, hipStream_t s);
hipError_t launch_gemm_down(const FfnArgs& a, int tiles_upper, hipStream_t s);
constexpr int GEMM_BM = 128;  // token rows per tile
// bf16 and MXFP4 banks whose weight rows divide into 512-row tiles (128 x 512 tiles, 128 x 128 per
// wave) and FP8-B128 banks whose rows divide into 256-row tiles (128 x 256, 128 x 64 per wave),
// activations loaded straight into an LDS ring
bool gemm_wide_fits(int fmt, int rows, int K, int E);
hipError_t launch_gemm_wide(const FfnArgs& a, bool gateup, int tiles_upper, hipStream_t s);

// Grouped GEMM on the scaled low-precision MFMA with the weights in their stored format (MXFP4:
// e2m3 x e2m1, FP8-B128: e4m3 x e4m3), activations carried as two terms of the operand format.
// launch_quant_act writes the terms of `rows` bf16 rows of K values into `terms` (mx_term_bytes);
// launch_gemm_mx reads the A rows' terms from there (term_rows: rows the terms array holds).
bool gemm_mx_fits(int fmt, int rows, int K, int E);
size_t mx_term_bytes(int fmt, long long rows, int K);
hipError_t launch_quant_act(int fmt, const uint16_t* src, long long rows, int K, uint8_t* terms, hipStream_t s);
hipError_t launch_gemm_mx(const FfnArgs& a, bool gateup, const uint8_t* terms, long long term_rows, int tiles_upper,
                          hipStream_t s);

// ---- fused decode layer: one kernel whose blocks each route and permute the (few) tokens in LDS,
// then share one list of gate/up and down items through per-XCD work queues, and combine.  Its
// counters start at zero and the last block to finish returns them to zero.
constexpr int LAYER_MAX_T = 16;   // tokens per call on the fused path (one routing wave per token)
constexpr int LAYER_NT = 4;       // tokens per GEMV pass on the fused path
constexpr int LAYER_RPL2 = 2;     // 64-row blocks per down item on the fused path (d % 128 == 0)
constexpr int CNT_STRIDE = 64;    // ints between two counters: one 256-byte line each, so polls and
                                  // updates of different counters never share a line
constexpr int LAYER_NQ = 8;       // work queues of the fused FFN kernel (one per XCD)
constexpr int LAYER_PG = 8;       // blocks that compute one token's router logits (ft_moe_layer_proj)
constexpr int CTL_ERR = 0;        // control word: non-zero when a dependency wait gave up
constexpr int CTL_QUEUE = CNT_STRIDE;  // queue q's next position at CTL_QUEUE + q * CNT_STRIDE
constexpr int CTL_EXIT = CTL_QUEUE + LAYER_NQ * CNT_STRIDE;  // blocks that have finished
constexpr int CTL_INTS = CNT_STRIDE * (2 + LAYER_NQ);

struct LayerArgs {
  FfnArgs f;                 // the grouped FFN (offsets/gather from the prologue)
  const float* logits;       // fp32 [T][E]
  int32_t* ids;              // [T][k]
  float* w;                  // [T][k]
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* gather;           // [T*k]
  int32_t* inv;              // [T*k]
  uint32_t* mask;            // [T] or null
  void* out;                 // fp32 or bf16 [T][d]
  int out_bf16;
  int id_bits;
  int32_t* ctl;              // [CTL_INTS] control words
  int32_t* done13;           // [n_rc][CNT_STRIDE] finished gate/up items per row chunk
  int n_rc;                  // upper bound on row chunks (groups x token chunks)
  int32_t* cdone;            // [T][d/64][CNT_STRIDE] contributions made per (token, 64-column block)
  // the router projection inside the launch (ft_moe_layer_proj), or w_router null: logits are an input
  const uint16_t* w_router;  // bf16 [E][d]
  float* proj_logits;        // fp32 [T][E]: the logits the launch computes (the same array as logits)
  int32_t* pflag;            // [T]: tokens whose logits are published (zero at start, returned to zero)
};
hipError_t launch_layer_decode(const LayerArgs& L, hipStream_t s);
// its LDS fits one CU (proj: with the router projection's logits staged in LDS)
bool layer_decode_fits(int fmt, int T, int E, int k, int d, int I, bool proj = false);
// upper bound on the row chunks (groups x chunks of LAYER_NT tokens) of a fused call
inline int layer_decode_rowchunks_upper(int T, int E, int k, bool shared) {
  const int groups = (E < T * k ? E : T * k) + (shared ? 1 : 0);
  return groups + (T * k + (shared ? T : 0)) / LAYER_NT;
}

// canonical -> row-interleaved device layout for one matrix of `rows` rows (all slots) and K columns
// (perm_I > 0: W13 of expert intermediate size perm_I, whose rows are reordered into gate/up blocks;
// R: rows per slot)
hipError_t launch_pack_matrix(int fmt, const uint8_t* canon_codes, const uint8_t* canon_scales, uint8_t* codes,
                              uint8_t* scales, long long rows, int K, int perm_I, int R, hipStream_t s);
// tscale: the matrix scale of an NVFP4 matrix (device pointer), else unused
hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int rows, int K, int perm_I,
                          const float* tscale, float* out, hipStream_t s);

}  // namespace ftk
