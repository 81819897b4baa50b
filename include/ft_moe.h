/*
 * ft_moe.h -- C ABI of a Mixture-of-Experts layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer is the hot path of an edge MoE inference engine as described by the FreeToken
 * pages:
 *   [walk-through]  "深入FreeToken架构：从HTTP API到CUDA内核的本地MoE推理引擎全链路剖析"
 *                   (yfxerp.com), sections 一 (request path: ... -> MoE expert dispatch ->
 *                   kernels) and 五 "MoE 引擎" (expert FFNs held in per-format banks -- BF16,
 *                   FP8 block, NVFP4, MXFP4, GGUF Q4_0 -- hot experts resident on the GPU,
 *                   cold ones in host memory, run by a CPU path).
 *   [article]       zuoshipin.com FreeToken article, sections "一句话看懂 FreeToken" (frequently
 *                   used expert weights stay in GPU memory) and "为什么 MoE 模型适合做 CPU–GPU
 *                   协同？" (each token activates only a few experts).
 *   [summary]       "FreeToken：高效的边缘原生 MoE 服务与带宽自适应执行" (ai-feeds.com), section
 *                   "方法" (decode-time expert caching, GPU/CPU placement per expert).
 * The pages give no formulas; the layer computed here is the standard routed-expert layer:
 * softmax router with top-k and renormalisation, token->expert permutation, SwiGLU expert FFN,
 * weighted combine.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless the argument says "host".  The caller owns every
 *     buffer (inputs, outputs and workspace); the library allocates nothing and keeps no device
 *     state between calls.
 *   - Calls validate their arguments on the host, then enqueue kernels on `stream` and return
 *     without waiting: results are valid once the stream reaches that point.  No call
 *     synchronises the device, so sequences of calls can be captured into a hipGraph.
 *   - Status: FT_OK (0) or an FT_E_* code.  A non-OK call enqueues nothing and records a message
 *     readable with ft_moe_last_error() on the same host thread.  No C++ exception crosses the ABI.
 *   - Every device pointer must be 16-byte aligned; all arrays are dense and row-major.
 *   - Limits: T >= 0 (T == 0 enqueues nothing), 1 <= E <= 1024, 1 <= k <= min(E, 32).
 *   - Calls are reentrant: host threads may call concurrently, and independent calls may run on
 *     different streams concurrently (ft_moe_layer's one-kernel path expects the device to itself:
 *     see there).
 */
#ifndef FT_MOE_H
#define FT_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FT_MOE_ABI_VERSION 1

enum ft_status {
  FT_OK = 0,
  FT_E_INVAL = 1,        /* bad argument (null pointer, size out of range, misalignment) */
  FT_E_UNSUPPORTED = 2,  /* valid request the library does not implement (format, shape) */
  FT_E_WORKSPACE = 3,    /* workspace pointer missing or smaller than the size query asked */
  FT_E_HIP = 4,          /* a HIP call or kernel launch failed; message has hipGetErrorString */
  FT_E_INTERNAL = 5      /* unexpected internal failure */
};

/* Expert-bank formats ([walk-through] section 五 lists the bank formats). */
enum ft_weight_format {
  FT_W_BF16 = 0,      /* bf16 weights */
  FT_W_Q4_0 = 1,      /* GGUF Q4_0: blocks of 32 int4 codes along K with one fp16 scale, v = s*(q-8) */
  FT_W_MXFP4 = 2,     /* OCP MXFP4: e2m1 codes with one E8M0 scale per 32 along K, v = e2m1*2^(s-127) */
  FT_W_FP8_B128 = 3,  /* OCP e4m3fn codes with one fp32 scale per 128x128 (row, K) block, v = s*e4m3 */
  FT_W_NVFP4 = 4      /* NVFP4: e2m1 codes, one e4m3fn scale per 16 along K and one fp32 scale t per
                         matrix, v = t * (e2m1 * e4m3) */
};

/* ft_moe_grouped_ffn flags */
#define FT_PATH_AUTO 0x0  /* per expert group: few tokens -> streaming GEMV, many -> MFMA GEMM */
#define FT_PATH_GEMV 0x1  /* every group through the streaming GEMV kernels */
#define FT_PATH_GEMM 0x2  /* every group through the MFMA GEMM kernels */
#define FT_PATH_MASK 0x3
#define FT_GEMM_WIDEN 0x10  /* MXFP4 and FP8-B128 GEMM groups decode their weights to bf16 in registers and
                               run the bf16 MFMA, instead of the scaled MFMA on the stored fp4 / fp8
                               codes with two-term activations (the default where the shape fits) */

/* ft_moe_combine / ft_moe_layer flags */
#define FT_OUT_BF16 0x4   /* write `out` as bf16 instead of fp32 */

/* ft_moe_layer flags */
#define FT_LAYER_UNFUSED 0x8  /* always run the four calls' kernels, never the fused decode kernels */

/*
 * Expert bank in DEVICE layout (passed by host pointer; the struct itself is read on the host).
 * Slot s holds one expert: W13 = [gate rows 0..I-1 ; up rows I..2I-1] of shape [2I][d] and
 * W2 of shape [d][I].  ft_moe_pack_bank builds this layout from the canonical stored formats.
 *
 * Each matrix of R rows and K columns is cut into 16-byte code chunks along K (8 bf16, 16 e4m3 or
 * 32 four-bit codes; nchunk = K / elements-per-chunk) and stored row-interleaved in blocks of 64
 * rows: chunk c of row r sits at byte ((r/64 * nchunk + c) * 64 + r%64) * 16 of the matrix, so the
 * same chunk of 64 consecutive rows is 1 KiB of contiguous memory.  Slots are consecutive.
 * W13 rows are stored in gate/up blocks: device row 64b + j is gate row 32b + j for j < 32 and up
 * row I + 32b + (j - 32) for j >= 32, so every 64-row block yields 32 columns of SiLU(g) * u.
 * W2 rows keep their order.
 *   FT_W_BF16     codes = bf16 in K order; s13 = s2 = NULL
 *   FT_W_Q4_0     32 codes of one GGUF block per chunk; 32-bit word w of a chunk holds elements
 *                 8w..8w+7, element 8w+2s in bits 4s..4s+3 and element 8w+2s+1 in bits 16+4s..19+4s;
 *                 value = scale * (q - 8); scales fp16, one per (row, chunk), same interleave:
 *                 scale of (r, c) is element (r/64 * nchunk + c) * 64 + r%64
 *   FT_W_MXFP4    32 e2m1 codes per chunk in K order (element 2i low nibble of byte i, 2i+1 high);
 *                 E8M0 scales, one byte per (row, chunk), interleaved as for Q4_0
 *   FT_W_FP8_B128 16 e4m3fn codes per chunk in K order; scales fp32 [rows/128][K/128] per matrix,
 *                 row-major over logical rows (not interleaved, not reordered)
 *   FT_W_NVFP4    codes as FT_W_MXFP4; block scales two e4m3fn bytes per (row, chunk) (low byte:
 *                 elements 0-15 of the chunk, high byte: 16-31), one 16-bit pair per (row, chunk)
 *                 interleaved as for Q4_0, for all slots; then the fp32 matrix scales, one per slot
 * Array sizes per format: ft_moe_bank_bytes.  Divisibility: d a multiple of 128 and I a multiple of 64
 * (so every matrix has whole 64-row blocks and whole chunks; FP8_B128 also needs I % 128 == 0).
 */
typedef struct ft_moe_bank {
  int32_t fmt, n_slots, d, I;
  const void* w13;
  const void* w2;
  const void* s13;
  const void* s2;
} ft_moe_bank;

/* FT_MOE_ABI_VERSION of the built library. */
int ft_moe_abi_version(void);

/* Text of the last non-OK status on this host thread ("" if none).  Owned by the library. */
const char* ft_moe_last_error(void);

/*
 * Router: top-k experts per token and their renormalised softmax weights.
 *   logits fp32 [T][E]  ->  ids int32 [T][k], w fp32 [T][k]
 * ids[t] lists the k largest logits of row t in descending order; equal logits are taken in
 * ascending expert order (IEEE comparison, so -0.0 == +0.0).  w[t][j] = p_j / sum_i p_i with
 * p_j = exp(logit_j - max logit) over the k chosen experts: the softmax over all E experts
 * restricted to the chosen ones and renormalised (the normaliser over all E cancels).
 * Logits must be finite or -inf; a row whose k chosen logits are all -inf gets NaN weights.
 * Sparse activation of a few experts per token: [article] "为什么 MoE 模型适合做 CPU–GPU 协同？".
 */
int ft_moe_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t stream);

/*
 * Router projection and router in one launch (the step before the path, fused into route).
 *   x bf16 [T][d], w_router bf16 [E][d] (row-major)  ->  logits fp32 [T][E], ids int32 [T][k],
 *   w fp32 [T][k]
 * logits[t][e] = sum_c x[t][c] * w_router[e][c]: bf16 products accumulated in fp32 on the matrix
 * cores (the order of the fp32 additions is the kernel's; the result is within the rounding bound
 * of an fp32 sum of d terms).  ids and w are then exactly what ft_moe_route returns for those
 * logits.  Requires d > 0 with d % 32 == 0, 1 <= E <= 512, 1 <= k <= min(E, 32); T = 0 is a no-op.
 * ws: ft_moe_route_proj_workspace(T) bytes of device memory, zero-filled once by the caller; every
 * call leaves it zero again.  Calls that may overlap need their own workspaces.
 * The gate that picks k of E experts: [article] "为什么 MoE 模型适合做 CPU–GPU 协同？"; FreeToken
 * walk-through "深入FreeToken架构…全链路剖析", section 五.
 */
size_t ft_moe_route_proj_workspace(int T);
int ft_moe_route_proj(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int d, int E, int k,
                      float* logits, int32_t* ids, float* w, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of workspace ft_moe_permute needs for (T, E, k); 0 when none is needed.
 */
size_t ft_moe_permute_workspace(int T, int E, int k);

/*
 * Token -> expert permutation (the expert-dispatch stage of [walk-through] section 一).
 *   ids int32 [T][k]  ->  counts int32 [E], offsets int32 [E+1], gather int32 [T*k], inv int32 [T*k]
 * With flat index f = t*k + j: counts[e] = #{f : ids[f] == e}; offsets = exclusive prefix sum of
 * counts (offsets[E] = T*k); gather[p] = f lists flat indices grouped by expert id ascending and,
 * inside a group, by ascending f; inv[gather[p]] = p.  Every id must lie in [0, E).
 * ws: device workspace of at least ft_moe_permute_workspace(T, E, k) bytes (may be NULL if 0).
 */
int ft_moe_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                   int32_t* gather, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of workspace ft_moe_grouped_ffn needs.  `bank` is a host pointer.
 */
size_t ft_moe_grouped_ffn_workspace(const ft_moe_bank* bank, int T, int E, int k, int shared_slot, int flags);

/*
 * Grouped SwiGLU expert FFN over the resident experts ([walk-through] section 五: expert FFNs in
 * per-format banks; hot experts resident on the GPU and found through a lookup table).
 *   bank            host pointer to the bank description (device arrays inside)
 *   slot_of_expert  int32 [E]: bank slot of each expert, -1 when the expert is not resident
 *   shared_slot     bank slot of an always-on shared expert applied to every token, or -1
 *   x               bf16 [T][d] activations
 *   offsets, gather the permutation of ft_moe_permute for the same routing
 *   y_sorted        bf16 [T*k][d]: row p = offsets[e] + i receives FFN_e(x[gather[p] / k]) for every
 *                   resident expert e; rows of non-resident experts are not written
 *   y_shared        bf16 [T][d]: FFN_shared(x[t]); required iff shared_slot >= 0, else NULL
 * FFN_s(x) = (SiLU(x Wg^T) * (x Wu^T)) W2^T with Wg = W13[0:I], Wu = W13[I:2I], SiLU(g) = g/(1+e^-g);
 * products accumulate in fp32; the intermediate h is rounded to bf16 once, y to bf16 once.
 * flags: FT_PATH_*, FT_GEMM_WIDEN (which kernels run; results agree within rounding).
 * ws: device workspace of at least ft_moe_grouped_ffn_workspace(...) bytes.
 */
int ft_moe_grouped_ffn(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot,
                       const uint16_t* x, int T, int E, int k, const int32_t* offsets,
                       const int32_t* gather, uint16_t* y_sorted, uint16_t* y_shared, void* ws,
                       size_t ws_bytes, int flags, hipStream_t stream);

/*
 * Weighted combine back to token order, and the residual mask of non-resident experts
 * ([walk-through] section 五: experts not resident on the GPU are left to another path).
 *   out[t][c] = sum over j ascending with slot_of_expert[ids[t][j]] >= 0 of
 *               w[t][j] * y_sorted[inv[t*k+j]][c]   (+ y_shared[t][c] when y_shared != NULL)
 *   residual_mask[t] bit j = 1 iff expert ids[t][j] is not resident (may be NULL)
 * Weights are not renormalised over the resident subset: the masked share belongs to the other
 * path.  out is fp32 [T][d], or bf16 [T][d] with FT_OUT_BF16.
 */
int ft_moe_combine(const uint16_t* y_sorted, const uint16_t* y_shared, const int32_t* ids,
                   const float* w, const int32_t* inv, const int32_t* slot_of_expert, int T, int E,
                   int k, int d, void* out, uint32_t* residual_mask, int flags, hipStream_t stream);

/*
 * Bytes of workspace ft_moe_layer needs (0 for invalid arguments).  `bank` is a host pointer.
 */
size_t ft_moe_layer_workspace(const ft_moe_bank* bank, int T, int E, int k, int shared_slot, int flags);

/*
 * The whole layer in one call: exactly ft_moe_route, ft_moe_permute, ft_moe_grouped_ffn and
 * ft_moe_combine on the same arguments, with every intermediate result written to the caller's
 * buffers (ids, w, counts, offsets, gather, inv, y_sorted, y_shared) and the same definitions.
 * For decode batches (1 <= T <= 16, path not FT_PATH_GEMM, no FT_LAYER_UNFUSED, and a shape whose
 * per-block working set fits the 160 KiB LDS of a CU) it runs one kernel instead of the calls' five
 * or more: every block routes and permutes the tokens itself, then takes gate/up and down work
 * items from device queues, ordered by device-side dependency counters, and combines (no host
 * synchronisation; graph-capturable).  Its results
 * equal the four calls' within rounding (the partial sums of a row may be added in another
 * grouping); here a slot_of_expert entry outside [0, n_slots) counts as not resident everywhere.
 * Dispatch and combine follow [walk-through] sections 一 and 五.
 * ws: device workspace of ft_moe_layer_workspace(...) bytes, zero-filled by the caller before its
 * first use; every call leaves it ready for the next call of the same shape (bank shape, T, E, k,
 * shared_slot, flags): the fused kernel returns its counters to zero.  A call of another shape may
 * find other data where its counters lie: zero the workspace again before it, or give each shape a
 * workspace of its own.  Its first int32 is a status word that the fused kernel sets non-zero if an internal
 * dependency wait gave up (results are then invalid); the library never clears it, and it stays 0
 * in every correct run.  Calls that may overlap need separate workspaces.
 * The one-kernel path sizes its grid to the blocks the device holds at once and its waits end
 * promptly only when all of them run together: it expects the device's compute units to itself.
 * Beside a long kernel on another stream its waits can last until that kernel ends, or give up
 * after 2^20 polls (about a second) with the status word set; use FT_LAYER_UNFUSED for such
 * overlap.
 * flags: FT_PATH_*, FT_GEMM_WIDEN, FT_OUT_BF16, FT_LAYER_UNFUSED.  T == 0 only writes counts = offsets = 0.
 */
int ft_moe_layer(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot,
                 const float* logits, const uint16_t* x, int T, int E, int k, int32_t* ids, float* w,
                 int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* inv, uint16_t* y_sorted,
                 uint16_t* y_shared, void* out, uint32_t* residual_mask, void* ws, size_t ws_bytes,
                 int flags, hipStream_t stream);

/*
 * The layer from the activations: the router projection of ft_moe_route_proj (logits[t][e] =
 * x[t] . w_router[e], bf16 products summed in fp32, written to `logits` fp32 [T][E]), then
 * ft_moe_layer on those logits, with every output of both.  Where ft_moe_layer runs its one-launch
 * path and the T x E logits fit in a block's LDS, the projection runs inside that launch: a group of
 * 8 blocks computes each token's logits (the experts dealt over their waves, each logit an fp32 sum
 * in a fixed order: within the rounding bound of ft_moe_route_proj's), publishes them, and every
 * block routes once all T rows are published; ids and w are exactly what ft_moe_route returns for the written
 * logits.  Otherwise ft_moe_route_proj runs first.  w_router bf16 [E][d]; requires E <= 512 besides
 * ft_moe_layer's conditions.  ws: ft_moe_layer_workspace(...) bytes (the same
 * workspace serves both calls), zero-filled once by the caller.  The expert routing of a decode
 * layer from its input in one launch: [walk-through] sections 一 and 五; [article]
 * "为什么 MoE 模型适合做 CPU–GPU 协同？".
 */
int ft_moe_layer_proj(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot,
                      const uint16_t* x, const uint16_t* w_router, int T, int E, int k, float* logits,
                      int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* gather,
                      int32_t* inv, uint16_t* y_sorted, uint16_t* y_shared, void* out,
                      uint32_t* residual_mask, void* ws, size_t ws_bytes, int flags, hipStream_t stream);

/*
 * Scratch bytes of ft_moe_layer_noalloc: one static array per device that the library runs on,
 * held until the process ends.
 */
#define FT_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * ft_moe_layer for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid allocation): the same call, arguments, results and
 * kernels, with the workspace taken from a static device array of the library
 * (FT_NOALLOC_SCRATCH_BYTES per device) instead of a ws argument.  Nothing is allocated.
 *   - A layer whose workspace (ft_moe_layer_workspace with the same arguments) exceeds
 *     FT_NOALLOC_SCRATCH_BYTES is refused with FT_E_WORKSPACE and enqueues nothing.
 *   - The counters a call needs at zero sit at the start of the scratch.  Before the layer, a clear
 *     kernel zeroes the part of them that earlier calls (of other shapes) may have used for other
 *     data; every call leaves its own counters at zero.
 *   - status: optional device int32, 4-byte aligned: receives this call's status word (0 in every
 *     correct run; non-zero when a dependency wait of the one-kernel path gave up and the results
 *     are invalid).  A one-thread kernel after the layer moves the word there and clears it, also
 *     when status is NULL.
 *   - Every call on a device shares that device's scratch: calls that may overlap on one device
 *     (different streams, or host threads without ordering) race and give wrong results.  Order
 *     them on one stream.
 */
int ft_moe_layer_noalloc(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot,
                         const float* logits, const uint16_t* x, int T, int E, int k, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* inv,
                         uint16_t* y_sorted, uint16_t* y_shared, void* out, uint32_t* residual_mask,
                         int32_t* status, int flags, hipStream_t stream);

/* ------------------------------------------------------------------------- start-up rates */

/*
 * Rates of the device at hand, measured by ft_moe_measure_rates (the start-up measurement of the
 * [walk-through] section 五: the engine measures the host link and memory bandwidths and sizes its
 * CPU-GPU split from them).  Rates are the best of `reps` timed launches.
 */
typedef struct ft_moe_rates {
  double hbm_read_gbs;        /* device memory read by a streaming kernel on every CU (GB/s) */
  double host_read_gbs;       /* pinned host memory read by the same kernel with the cache fill's 8
                                 blocks: the host link rate P of the load fraction (0: no host_buf) */
  double mfma_bf16_tflops;    /* dense v_mfma_f32_32x32x16_bf16, register operands, every SIMD */
  double mfma_fp8_tflops;     /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3 operands */
  double mfma_fp6_fp4_tflops; /* the same instruction with e2m3 x e2m1 operands (the MXFP4 prefill path) */
  double mfma_clock_ghz;      /* the clock at which the bf16 rate is one MFMA per 32 cycles per SIMD */
  int compute_units;
  int stream_blocks;          /* blocks of the device-memory streaming launch (resident per CU x CUs) */
} ft_moe_rates;

/*
 * Measures the rates above.  dev_buf: device memory of dev_bytes >= 64 MiB, 256-byte aligned, whose
 * contents are overwritten (its first MiB takes the kernels' results; the rest is read).  host_buf:
 * pinned host memory of host_bytes >= 1 MiB, 16-byte aligned, only read; NULL skips the host link.
 * reps in [1, 100].  Unlike every other call this one blocks: it records HIP events on `stream` and
 * waits for them (about 10 ms with reps = 3 on a 1 GiB buffer), so it is a start-up call and cannot be
 * captured into a graph.  It allocates no device memory (two HIP events for the length of the call).
 * On success *out holds the rates; on error it is left unchanged.
 */
int ft_moe_measure_rates(void* dev_buf, size_t dev_bytes, const void* host_buf, size_t host_bytes, int reps,
                         ft_moe_rates* out, hipStream_t stream);

/* ------------------------------------------------------------------------- expert cache */

/*
 * One step of the global LRU expert cache (FreeToken article on zuoshipin.com, mechanism four:
 * frequently used experts stay on the GPU under one global LRU policy; FreeToken walk-through,
 * section 五: hot experts resident on the GPU, cold experts in pinned host memory; FreeToken paper
 * summary, key insights: an LRU that CUDA Graphs can hold).  Everything it reads and writes is in
 * device memory, so a step needs no host round trip.
 *
 * counts [E] int32: tokens per expert in this step (the `counts` of ft_moe_permute); an expert
 * with counts > 0 is demanded.  Cache state, updated in place (caller-owned device memory, kept
 * between steps; start: every entry -1, last_use and tick 0, or any consistent preload):
 *   slot_of_expert [E] int32    slot of each expert in the device bank, -1 = not resident;
 *   expert_of_slot [n_slots]    expert held by each slot, -1 = empty (the inverse of the former);
 *   last_use [n_slots] uint32   step at which the slot was last used;  tick [1] uint32: step clock.
 * One step, at clock now = tick + 1:
 *   - each demanded resident expert marks its slot used now;
 *   - the demanded absent experts, by counts descending then expert index, are paired with the
 *     slots whose expert is not demanded, empty slots first, then by last_use ascending, then slot
 *     index; min(#absent, #such slots, max_loads) pairs are made, and with load_fraction q > 0 at
 *     most ceil(q * #absent) (fp32 product; q in [0, 1], 0 = no such limit): the share of the cold
 *     experts copied to the GPU, the rest being left to the host (the bandwidth-adaptive CPU-GPU
 *     split of the walk-through, section 五, and the zuoshipin.com article, mechanism two).  Each
 *     pair evicts the slot's expert (its slot_of_expert becomes -1), puts the new expert there and
 *     marks the slot used now;
 *   - compute_slot [E] int32 (out): an expert's slot when it was resident before the step and still
 *     is, else -1.  Pass it as the slot table of this step's ft_moe_grouped_ffn: the experts being
 *     loaded are not computed from it;
 *   - load_slot [E] int32 (out, may be NULL): an expert's slot when it was loaded in this step, else
 *     -1.  A caller that computes the loaded experts in the same step runs a second
 *     ft_moe_grouped_ffn with this table after the fill, and combines with slot_of_expert (the
 *     table after the step); one that leaves them to the next step combines with compute_slot;
 *   - loads [max_loads][2] int32 (out): (expert, slot) per load in pairing order; n_loads [1] int32
 *     (out): their number.  Copy them with ft_moe_cache_fill before the next step's update.
 * Limits: 1 <= E <= 1024, 1 <= n_slots <= 1024, 0 <= max_loads <= n_slots.  Pointers 16-byte
 * aligned.  Entries of the tables outside their ranges are read as -1.  last_use wraps after 2^32
 * steps.  One kernel launch (one block); none allocates or syncs.
 */
int ft_moe_cache_update(const int32_t* counts, int E, int n_slots, int max_loads, float load_fraction,
                        int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use, uint32_t* tick,
                        int32_t* compute_slot, int32_t* load_slot, int32_t* loads, int32_t* n_loads,
                        hipStream_t stream);

/*
 * Copy the experts listed by ft_moe_cache_update from the bank that holds every expert (`src`,
 * expert e in slot e, normally in pinned host memory: the walk-through's cold tier) into their slots
 * of the device bank `dst` (same fmt, d and I): every array of the format, byte for byte.  The load
 * list is read on the device (loads [max_loads][2], n_loads [1]: the update's outputs), so the copy
 * is enqueued without knowing it on the host; run it on a second stream beside the step's grouped
 * FFN (the walk-through's copies overlapped with compute): the slots it writes hold no expert that
 * this step's compute_slot names.  The caller orders the streams: the fill after the update, and
 * the next step's update and FFN after the fill.
 * `src` and `dst` are host pointers to bank descriptions; src's arrays are pinned host memory
 * (hipHostMalloc; the kernel reads it over the bus) or device memory; pageable host memory is
 * refused (FT_E_INVAL).  Entries naming an expert >= src->n_slots or a slot >= dst->n_slots are
 * skipped.  max_loads = 0 is a no-op.
 */
int ft_moe_cache_fill(const ft_moe_bank* src, const ft_moe_bank* dst, const int32_t* loads, const int32_t* n_loads,
                      int max_loads, hipStream_t stream);

/* ---------------------------------------------------------------------- cold-expert residual */

/*
 * The pairs the device layer leaves to another path, computed on the host cores (FreeToken
 * walk-through, section 五: cold experts stay in host memory and run on the CPU beside the GPU;
 * zuoshipin.com FreeToken article, mechanism two: CPU-GPU co-execution).  For every token t and
 * slot j whose pair is cold and e = ids[t][j] < min(E, host_bank->n_slots): y = SiLU(x[t] Wg_e^T) * (x[t] Wu_e^T) Wd_e^T with fp32 sums,
 * h and y rounded to bf16 as on the device; then out[t] = sum over those j, in order j, of
 * w[t][j] * y.  out [T][d] fp32 is overwritten (zero for a token with no such pair).  A pair is
 * cold when bit j of residual_mask[t] is set (the mask ft_moe_combine or ft_moe_layer wrote), or,
 * with residual_mask NULL, when slot_of_expert[e] < 0 (a host copy of the slot table the device
 * layer uses, so the host can start as soon as the routing is known, beside the device layer; the
 * host does not know the device bank's slot count, so such a table marks every expert without a
 * valid slot with -1, as the tables of ft_moe_cache_update do).  Exactly one of the two is given.
 * Everything is host memory: host_bank (a host pointer to a bank description whose arrays are in
 * host memory, pinned or not, in the device layout of ft_moe_pack_bank, expert e in slot e: the bank
 * ft_moe_cache_fill reads), x bf16 [T][d], ids [T][k], w [T][k], residual_mask [T], out.  Runs on
 * n_threads host threads (0: the hardware's thread count, at most 256) and returns when done; it
 * does not touch the GPU.  Add the result to the device output with ft_moe_residual_add.
 */
int ft_moe_residual_host(const ft_moe_bank* host_bank, const uint16_t* x, const int32_t* ids, const float* w,
                         const uint32_t* residual_mask, const int32_t* slot_of_expert, int T, int E, int k,
                         float* out, int n_threads);

/*
 * out[t][c] += residual[t][c] on the device, out fp32 or (FT_OUT_BF16) bf16 rounded to nearest even,
 * both [T][d] device memory: the merge of the host residual into the layer output.
 */
int ft_moe_residual_add(void* out, const float* residual, int T, int d, int flags, hipStream_t stream);

/* ------------------------------------------------------------------------------ set-up calls */

/*
 * Bytes of one bank array in device layout: which = 0 w13, 1 w2, 2 s13, 3 s2 (0 if the format has
 * no such array).  Returns 0 for an invalid request.
 */
size_t ft_moe_bank_bytes(int fmt, int n_slots, int d, int I, int which);

/*
 * Build a device-layout bank from canonical stored bytes (all pointers are device pointers).
 * Canonical layouts, per slot, row-major over rows:
 *   FT_W_BF16     w uint16 [rows][K]
 *   FT_W_Q4_0     GGUF blocks [rows][K/32][18]: fp16 scale (little endian), then 16 bytes where byte i
 *                 holds element i (low nibble) and element i+16 (high nibble); canon_s13/s2 NULL
 *   FT_W_MXFP4    codes uint8 [rows][K/2] (element 2i low nibble), scales uint8 E8M0 [rows][K/32]
 *   FT_W_FP8_B128 codes uint8 [rows][K], scales fp32 [rows/128][K/128]
 *   FT_W_NVFP4    codes uint8 [rows][K/2] (element 2i low nibble), scales uint8 [rows*K/16 + 4]:
 *                 e4m3fn scales [rows][K/16], then the matrix's fp32 scale (little endian)
 * `dst` is a host pointer to a bank whose device arrays are already allocated (sizes from
 * ft_moe_bank_bytes); its fmt/n_slots/d/I must match the arguments.  Source and destination
 * must not overlap.
 */
int ft_moe_pack_bank(int fmt, int n_slots, int d, int I, const void* canon_w13, const void* canon_w2,
                     const void* canon_s13, const void* canon_s2, const ft_moe_bank* dst,
                     hipStream_t stream);

/*
 * Decode one bank matrix to fp32 with the same per-format decode routine the GEMV kernels use (for
 * checking the dequantisation bit for bit): which = 0: W13 of `slot` -> out fp32 [2I][d] row-major;
 * which = 1: W2 of `slot` -> out fp32 [d][I] row-major.
 */
int ft_moe_dequant(const ft_moe_bank* bank, int slot, int which, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FT_MOE_H */
