// C ABI of the MoE layer (declared in include/ft_moe.h): host-side validation, workspace sizing,
// path selection and kernel launches on the caller's stream.  No device call allocates device
// memory or synchronises, and nothing throws across the ABI; the host residual call computes on the
// host threads it starts and returns when done.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <exception>
#include <mutex>
#include <new>
#include <thread>

#include "../../include/ft_moe.h"
#include "ft_kernels.h"

namespace {

thread_local char g_err[512] = {0};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return FT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FT_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define CHECK_PTR(p, name) \
  do {                                                               \
    if ((p) == nullptr) return fail(FT_E_INVAL, "%s is null", name); \
    if (!aligned16(p)) return fail(FT_E_INVAL, "%s is not 16-byte aligned", name); \
  } while (0)

int check_tek(int T, int E, int k) {
  REQUIRE(T >= 0, FT_E_INVAL, "T must be >= 0 (got %d)", T);
  REQUIRE(E >= 1 && E <= 1024, FT_E_INVAL, "E must be in [1, 1024] (got %d)", E);
  REQUIRE(k >= 1 && k <= E && k <= 32, FT_E_INVAL, "k must be in [1, min(E, 32)] (got k=%d, E=%d)", k, E);
  REQUIRE((long long)T * k <= (1LL << 30), FT_E_INVAL, "T*k too large (%lld)", (long long)T * k);
  return FT_OK;
}


int check_bank_shape(int fmt, int n_slots, int d, int I) {
  REQUIRE(fmt >= FT_W_BF16 && fmt <= FT_W_NVFP4, FT_E_UNSUPPORTED, "unknown weight format %d", fmt);
  REQUIRE(n_slots >= 1, FT_E_INVAL, "n_slots must be >= 1 (got %d)", n_slots);
  REQUIRE(d > 0 && I > 0, FT_E_INVAL, "d and I must be positive (got d=%d, I=%d)", d, I);
  REQUIRE(d % 128 == 0 && I % 64 == 0, FT_E_INVAL,
          "d must be a multiple of 128 and I a multiple of 64 (got d=%d, I=%d)", d, I);
  REQUIRE(fmt != FT_W_FP8_B128 || I % 128 == 0, FT_E_INVAL,
          "FP8_B128 needs I to be a multiple of 128 (got I=%d)", I);
  REQUIRE((long long)d * I <= (1LL << 31), FT_E_INVAL, "d*I too large");
  return FT_OK;
}

int check_bank(const ft_moe_bank* b) {
  REQUIRE(b != nullptr, FT_E_INVAL, "bank is null");
  int rc = check_bank_shape(b->fmt, b->n_slots, b->d, b->I);
  if (rc) return rc;
  CHECK_PTR(b->w13, "bank->w13");
  CHECK_PTR(b->w2, "bank->w2");
  if (b->fmt != FT_W_BF16) {
    REQUIRE(b->s13 != nullptr && b->s2 != nullptr, FT_E_INVAL, "format %d needs scale arrays s13 and s2", b->fmt);
    REQUIRE(aligned16(b->s13) && aligned16(b->s2), FT_E_INVAL, "bank scale arrays must be 16-byte aligned");
  }
  return FT_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// groups with at most this many routed rows go through the GEMV kernels when the path is automatic
constexpr int kGemvMaxRows = ftk::GEMV_MAX_ROWS;
constexpr int kWideAllRows = 256;  // from this many tokens the wide GEMM kernels take every group

size_t h_bytes(int T, int k, int I, bool shared) {
  return round256((size_t)((long long)T * k + (shared ? T : 0)) * I * 2);
}

// MXFP4 and FP8-B128 banks whose shapes the scaled low-precision MFMA kernels take run their GEMM
// groups there (weights in their stored format, activations as two terms of the operand format).
// (The kernels address each array of activation terms with 32-bit offsets: both stay below 4 GiB.)
bool mx_path(const ft_moe_bank* b, int T, int E, int k, bool shared, int flags) {
  if ((flags & FT_GEMM_WIDEN) != 0) return false;
  if (!((b->fmt == FT_W_MXFP4 || b->fmt == FT_W_FP8_B128) && ftk::gemm_mx_fits(b->fmt, 2 * b->I, b->d, E) &&
        ftk::gemm_mx_fits(b->fmt, b->d, b->I, E)))
    return false;
  const long long rows = (long long)T * k + (shared ? T : 0);
  return ftk::mx_term_bytes(b->fmt, T, b->d) < (1ull << 32) && ftk::mx_term_bytes(b->fmt, rows, b->I) < (1ull << 32);
}
// Workspace after the h rows: the activation terms of x (T rows of d) and of h (every h row, of I)
size_t mx_ws_bytes(const ft_moe_bank* b, int T, int E, int k, bool shared, int flags) {
  if (T <= 0 || !mx_path(b, T, E, k, shared, flags)) return 0;
  const long long rows = (long long)T * k + (shared ? T : 0);
  return ftk::mx_term_bytes(b->fmt, T, b->d) + ftk::mx_term_bytes(b->fmt, rows, b->I);
}

// Bytes of the work-queue counters at the start of a grouped-FFN workspace (cleared by each call).
constexpr size_t kQctrBytes = (ftk::FFN_QCTR_INTS * 4 + 255) & ~(size_t)255;

// FfnArgs for one grouped-FFN call and its launches (arguments already validated).  terms: the
// mx_ws_bytes region (unused by the other formats); qctr: kQctrBytes of queue counters, cleared
// here unless the caller's permutation kernel already cleared them (qctr_zeroed).
int launch_grouped_ffn(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const uint16_t* x,
                       int T, int E, int k, const int32_t* offsets, const int32_t* gather, uint16_t* y_sorted,
                       uint16_t* y_shared, uint16_t* h, uint8_t* terms, int32_t* qctr, int flags,
                       hipStream_t stream, bool qctr_zeroed = false) {
  const int path = flags & FT_PATH_MASK;
  const bool shared = shared_slot >= 0;
  ftk::FfnArgs a{};
  a.fmt = bank->fmt;
  a.d = bank->d;
  a.I = bank->I;
  a.n_slots = bank->n_slots;
  a.w13 = (const uint8_t*)bank->w13;
  a.w2 = (const uint8_t*)bank->w2;
  a.s13 = (const uint8_t*)bank->s13;
  a.s2 = (const uint8_t*)bank->s2;
  a.slot_of = slot_of_expert;
  a.shared_slot = shared_slot;
  a.x = x;
  a.T = T;
  a.E = E;
  a.k = k;
  a.offsets = offsets;
  a.gather = gather;
  a.h = h;
  a.y_sorted = y_sorted;
  a.y_shared = y_shared;

  // Which groups each kernel family takes (by routed-row count).  A group never has more than
  // T rows (top-k ids of a token are distinct); the shared group has exactly T.
  const long long TK = (long long)T * k;
  const long long rows_total = TK + (shared ? T : 0);
  const long long groups_upper = (long long)(E < TK ? E : TK) + (shared ? 1 : 0);
  int gemv_max, gemm_min;
  if (path == FT_PATH_GEMV) {
    gemv_max = 0x7fffffff;
    gemm_min = 0x7fffffff;
  } else if (path == FT_PATH_GEMM) {
    gemv_max = 0;
    gemm_min = 1;
  } else if (T >= kWideAllRows && ftk::gemm_wide_fits(a.fmt, 2 * a.I, a.d, E) && ftk::gemm_wide_fits(a.fmt, a.d, a.I, E)) {
    // Many tokens on the wide GEMM kernels: small groups go there too.  A 128-row tile streams its
    // weights at close to the HBM share of one CU while the MFMAs run, which beats the GEMV
    // kernel's rate for groups of a few rows once the launch has enough tiles to fill the device.
    gemv_max = 0;
    gemm_min = 1;
  } else {
    gemv_max = kGemvMaxRows;
    gemm_min = kGemvMaxRows + 1;
  }
  const int BM = ftk::GEMM_BM;
  const bool run_gemv = gemv_max > 0;
  const bool run_gemm = gemm_min <= T;  // no group has more than T rows
  long long gemm_tiles = 0;
  if (run_gemm) {
    const long long big_upper = rows_total / gemm_min + 1;
    const long long g_up = big_upper < groups_upper ? big_upper : groups_upper;
    gemm_tiles = (rows_total + BM - 1) / BM + g_up;
  }
  const bool mx = run_gemm && mx_path(bank, T, E, k, shared, flags);
  uint8_t* xterms = terms;
  uint8_t* hterms = mx ? terms + ftk::mx_term_bytes(bank->fmt, T, bank->d) : nullptr;
  // every launch below takes its items from its own queue counters, cleared here (or already)
  hipError_t e = hipSuccess;
  if (!qctr_zeroed) {
    e = ftk::launch_zero_ints(qctr, ftk::FFN_QCTR_INTS, stream);
    if (e != hipSuccess) return hip_status(e, "grouped_ffn queue clear launch");
  }
  constexpr int QL = ftk::FFN_QCTR_INTS / 4;  // counters of one launch
  if (run_gemv) {
    a.min_cnt = 1;
    a.max_cnt = gemv_max;
    a.qctr = qctr;
    e = ftk::launch_gemv_gateup(a, (int)groups_upper, rows_total, stream);
    if (e != hipSuccess) return hip_status(e, "grouped_ffn gemv gate/up launch");
  }
  if (run_gemm) {
    a.min_cnt = gemm_min;
    a.max_cnt = 0x7fffffff;
    a.qctr = qctr + QL;
    if (mx) {
      e = ftk::launch_quant_act(bank->fmt, x, T, bank->d, xterms, stream);
      if (e != hipSuccess) return hip_status(e, "grouped_ffn activation terms launch");
      e = ftk::launch_gemm_mx(a, true, xterms, T, (int)gemm_tiles, stream);
    } else {
      e = ftk::launch_gemm_gateup(a, (int)gemm_tiles, stream);
    }
    if (e != hipSuccess) return hip_status(e, "grouped_ffn gemm gate/up launch");
  }
  if (run_gemv) {
    a.min_cnt = 1;
    a.max_cnt = gemv_max;
    a.qctr = qctr + 2 * QL;
    e = ftk::launch_gemv_down(a, (int)groups_upper, rows_total, stream);
    if (e != hipSuccess) return hip_status(e, "grouped_ffn gemv down launch");
  }
  if (run_gemm) {
    a.min_cnt = gemm_min;
    a.max_cnt = 0x7fffffff;
    a.qctr = qctr + 3 * QL;
    if (mx) {
      e = ftk::launch_quant_act(bank->fmt, h, rows_total, bank->I, hterms, stream);
      if (e != hipSuccess) return hip_status(e, "grouped_ffn h terms launch");
      e = ftk::launch_gemm_mx(a, false, hterms, rows_total, (int)gemm_tiles, stream);
    } else {
      e = ftk::launch_gemm_down(a, (int)gemm_tiles, stream);
    }
    if (e != hipSuccess) return hip_status(e, "grouped_ffn gemm down launch");
  }
  return ok();
}

// Workspace of ft_moe_layer: control words and the fused path's counters (every one of them zero
// when a fused call starts and again when it ends; they end at `zeroed`), then the grouped FFN's
// queue counters (cleared by each unfused call), the h rows, the activation terms and the
// permutation workspace of the unfused path.
struct LayerWs {
  size_t ctl, rproj, done13, cdone, zeroed, qctr, h, terms, perm, total;
  int n_rc;
};

bool layer_fused(const ft_moe_bank* b, int T, int E, int k, int flags) {
  return T >= 1 && T <= ftk::LAYER_MAX_T && (flags & FT_LAYER_UNFUSED) == 0 &&
         (flags & FT_PATH_MASK) != FT_PATH_GEMM && ftk::layer_decode_fits(b->fmt, T, E, k, b->d, b->I);
}

LayerWs layer_ws(const ft_moe_bank* b, int T, int E, int k, bool shared, bool fused, int flags) {
  const int d = b->d, I = b->I;
  LayerWs L{};
  size_t o = 0;
  L.ctl = o;
  o += round256((size_t)ftk::CTL_INTS * 4);
  // ft_moe_layer_proj: the router projection's counters (zero between calls), also the per-token
  // flags of the one-launch path's projection
  L.rproj = o;
  o += round256(ftk::route_proj_workspace_bytes(T > 0 ? T : 1));
  L.n_rc = fused ? ftk::layer_decode_rowchunks_upper(T, E, k, shared) : 0;
  L.done13 = o;
  o += round256((size_t)L.n_rc * ftk::CNT_STRIDE * 4);
  L.cdone = o;
  o += fused ? round256((size_t)T * (d / 64) * ftk::CNT_STRIDE * 4) : 0;
  L.zeroed = o;
  L.qctr = o;
  o += fused ? 0 : kQctrBytes;
  L.h = o;
  o += h_bytes(T, k, I, shared);
  L.terms = o;
  o += fused ? 0 : round256(mx_ws_bytes(b, T, E, k, shared, flags));
  L.perm = o;
  o += round256(ftk::permute_workspace_bytes(T, E, k));
  L.total = o;
  return L;
}

int id_bits_of(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

}  // namespace

extern "C" {

int ft_moe_abi_version(void) { return FT_MOE_ABI_VERSION; }

const char* ft_moe_last_error(void) { return g_err; }

int ft_moe_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t stream) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    if (T == 0) return ok();
    CHECK_PTR(logits, "logits");
    CHECK_PTR(ids, "ids");
    CHECK_PTR(w, "w");
    return hip_status(ftk::launch_route(logits, T, E, k, ids, w, stream), "ft_moe_route launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_route: unexpected exception");
  }
}

size_t ft_moe_route_proj_workspace(int T) { return T < 0 ? 0 : ftk::route_proj_workspace_bytes(T); }

int ft_moe_route_proj(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int k, float* logits,
                      int32_t* ids, float* w, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    REQUIRE(E <= 512, FT_E_INVAL, "E must be at most 512 for ft_moe_route_proj (got %d)", E);
    REQUIRE(d > 0 && d % 32 == 0, FT_E_INVAL, "d must be a positive multiple of 32 (got %d)", d);
    if (T == 0) return ok();
    CHECK_PTR(x, "x");
    CHECK_PTR(w_router, "w_router");
    CHECK_PTR(logits, "logits");
    CHECK_PTR(ids, "ids");
    CHECK_PTR(w, "w");
    CHECK_PTR(ws, "ws");
    const size_t need = ftk::route_proj_workspace_bytes(T);
    REQUIRE(ws_bytes >= need, FT_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    return hip_status(ftk::launch_route_proj(x, w_router, T, d, E, k, logits, ids, w, ws, stream),
                      "ft_moe_route_proj launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_route_proj: unexpected exception");
  }
}

size_t ft_moe_permute_workspace(int T, int E, int k) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32) return 0;
  return ftk::permute_workspace_bytes(T, E, k);
}

int ft_moe_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* gather,
                   int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    CHECK_PTR(counts, "counts");
    CHECK_PTR(offsets, "offsets");
    if (T > 0) {
      CHECK_PTR(ids, "ids");
      CHECK_PTR(gather, "gather");
      CHECK_PTR(inv, "inv");
    }
    const size_t need = ftk::permute_workspace_bytes(T, E, k);
    if (need) {
      REQUIRE(ws != nullptr && ws_bytes >= need, FT_E_WORKSPACE, "permute needs %zu bytes of workspace (got %zu%s)",
              need, ws_bytes, ws ? "" : ", null pointer");
      REQUIRE(aligned16(ws), FT_E_INVAL, "ws is not 16-byte aligned");
    }
    // T == 0 still defines counts = 0 and offsets = 0: the small kernel handles n = 0.
    return hip_status(ftk::launch_permute(ids, T, E, k, counts, offsets, gather, inv, ws, stream),
                      "ft_moe_permute launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_permute: unexpected exception");
  }
}

size_t ft_moe_grouped_ffn_workspace(const ft_moe_bank* bank, int T, int E, int k, int shared_slot, int flags) {
  if (!bank || T < 0 || k < 1 || E < 1) return 0;
  return kQctrBytes + h_bytes(T, k, bank->I, shared_slot >= 0) + mx_ws_bytes(bank, T, E, k, shared_slot >= 0, flags);
}

int ft_moe_grouped_ffn(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const uint16_t* x,
                       int T, int E, int k, const int32_t* offsets, const int32_t* gather, uint16_t* y_sorted,
                       uint16_t* y_shared, void* ws, size_t ws_bytes, int flags, hipStream_t stream) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    rc = check_bank(bank);
    if (rc) return rc;
    REQUIRE((flags & ~(FT_PATH_MASK | FT_GEMM_WIDEN)) == 0, FT_E_INVAL, "unknown flags 0x%x", flags);
    const int path = flags & FT_PATH_MASK;
    REQUIRE(path != 3, FT_E_INVAL, "FT_PATH_GEMV and FT_PATH_GEMM are exclusive");
    REQUIRE(shared_slot >= -1 && shared_slot < bank->n_slots, FT_E_INVAL, "shared_slot %d out of range [-1, %d)",
            shared_slot, bank->n_slots);
    REQUIRE((shared_slot >= 0) == (y_shared != nullptr), FT_E_INVAL,
            "y_shared must be given exactly when shared_slot >= 0");
    if (T == 0) return ok();
    CHECK_PTR(slot_of_expert, "slot_of_expert");
    CHECK_PTR(x, "x");
    CHECK_PTR(offsets, "offsets");
    CHECK_PTR(gather, "gather");
    CHECK_PTR(y_sorted, "y_sorted");
    if (y_shared) CHECK_PTR(y_shared, "y_shared");
    const bool shared = shared_slot >= 0;
    const size_t hb = h_bytes(T, k, bank->I, shared);
    const size_t need = kQctrBytes + hb + mx_ws_bytes(bank, T, E, k, shared, flags);
    REQUIRE(ws != nullptr && ws_bytes >= need, FT_E_WORKSPACE, "grouped_ffn needs %zu bytes of workspace (got %zu%s)",
            need, ws_bytes, ws ? "" : ", null pointer");
    REQUIRE(aligned16(ws), FT_E_INVAL, "ws is not 16-byte aligned");

    uint8_t* wsb = (uint8_t*)ws;
    return launch_grouped_ffn(bank, slot_of_expert, shared_slot, x, T, E, k, offsets, gather, y_sorted, y_shared,
                              (uint16_t*)(wsb + kQctrBytes), wsb + kQctrBytes + hb, (int32_t*)wsb, flags, stream);
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_grouped_ffn: unexpected exception");
  }
}

int ft_moe_combine(const uint16_t* y_sorted, const uint16_t* y_shared, const int32_t* ids, const float* w,
                   const int32_t* inv, const int32_t* slot_of_expert, int T, int E, int k, int d, void* out,
                   uint32_t* residual_mask, int flags, hipStream_t stream) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    REQUIRE(d > 0 && d % 8 == 0, FT_E_INVAL, "d must be a positive multiple of 8 (got %d)", d);
    REQUIRE((flags & ~FT_OUT_BF16) == 0, FT_E_INVAL, "unknown flags 0x%x", flags);
    if (T == 0) return ok();
    CHECK_PTR(y_sorted, "y_sorted");
    if (y_shared) CHECK_PTR(y_shared, "y_shared");
    CHECK_PTR(ids, "ids");
    CHECK_PTR(w, "w");
    CHECK_PTR(inv, "inv");
    CHECK_PTR(slot_of_expert, "slot_of_expert");
    CHECK_PTR(out, "out");
    if (residual_mask) CHECK_PTR(residual_mask, "residual_mask");
    return hip_status(ftk::launch_combine(y_sorted, y_shared, ids, w, inv, slot_of_expert, INT_MAX, T, E, k, d, out,
                                          residual_mask,
                                          (flags & FT_OUT_BF16) != 0, stream),
                      "ft_moe_combine launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_combine: unexpected exception");
  }
}

size_t ft_moe_bank_bytes(int fmt, int n_slots, int d, int I, int which) {
  if (check_bank_shape(fmt, n_slots, d, I) != FT_OK || which < 0 || which > 3) {
    g_err[0] = 0;
    return 0;
  }
  const size_t n = (size_t)n_slots, r13 = 2 * (size_t)I, r2 = (size_t)d;
  const size_t K13 = (size_t)d, K2 = (size_t)I;
  switch (fmt) {
    case FT_W_BF16:
      return which == 0 ? n * r13 * K13 * 2 : which == 1 ? n * r2 * K2 * 2 : 0;
    case FT_W_Q4_0:
      return which == 0 ? n * r13 * K13 / 2 : which == 1 ? n * r2 * K2 / 2 : which == 2 ? n * r13 * (K13 / 32) * 2
                                                                                       : n * r2 * (K2 / 32) * 2;
    case FT_W_MXFP4:
      return which == 0 ? n * r13 * K13 / 2 : which == 1 ? n * r2 * K2 / 2 : which == 2 ? n * r13 * (K13 / 32)
                                                                                       : n * r2 * (K2 / 32);
    case FT_W_NVFP4:  // two e4m3 bytes per (row, chunk), then one fp32 matrix scale per slot
      return which == 0 ? n * r13 * K13 / 2 : which == 1 ? n * r2 * K2 / 2 : which == 2 ? n * r13 * (K13 / 32) * 2 + n * 4
                                                                                       : n * r2 * (K2 / 32) * 2 + n * 4;
    default:
      return which == 0 ? n * r13 * K13 : which == 1 ? n * r2 * K2 : which == 2 ? n * (r13 / 128) * (K13 / 128) * 4
                                                                               : n * (r2 / 128) * (K2 / 128) * 4;
  }
}

int ft_moe_pack_bank(int fmt, int n_slots, int d, int I, const void* canon_w13, const void* canon_w2,
                     const void* canon_s13, const void* canon_s2, const ft_moe_bank* dst, hipStream_t stream) {
  try {
    int rc = check_bank_shape(fmt, n_slots, d, I);
    if (rc) return rc;
    rc = check_bank(dst);
    if (rc) return rc;
    REQUIRE(dst->fmt == fmt && dst->n_slots == n_slots && dst->d == d && dst->I == I, FT_E_INVAL,
            "dst bank description does not match (fmt, n_slots, d, I)");
    REQUIRE(canon_w13 != nullptr && canon_w2 != nullptr, FT_E_INVAL, "canonical weight arrays are null");
    if (fmt == FT_W_Q4_0) {
      REQUIRE(((uintptr_t)canon_w13 & 1u) == 0 && ((uintptr_t)canon_w2 & 1u) == 0, FT_E_INVAL,
              "canonical Q4_0 arrays must be 2-byte aligned");
    } else {
      REQUIRE(aligned16(canon_w13) && aligned16(canon_w2), FT_E_INVAL, "canonical code arrays must be 16-byte aligned");
      if (fmt != FT_W_BF16)
        REQUIRE(canon_s13 != nullptr && canon_s2 != nullptr, FT_E_INVAL, "canonical scale arrays are null");
    }
    hipError_t e = ftk::launch_pack_matrix(fmt, (const uint8_t*)canon_w13, (const uint8_t*)canon_s13,
                                           (uint8_t*)dst->w13, (uint8_t*)dst->s13, (long long)n_slots * 2 * I, d, I,
                                           2 * I, stream);
    if (e == hipSuccess)
      e = ftk::launch_pack_matrix(fmt, (const uint8_t*)canon_w2, (const uint8_t*)canon_s2, (uint8_t*)dst->w2,
                                  (uint8_t*)dst->s2, (long long)n_slots * d, I, 0, d, stream);
    if (e != hipSuccess) return hip_status(e, "ft_moe_pack_bank launch");
    return ok();
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_pack_bank: unexpected exception");
  }
}

int ft_moe_dequant(const ft_moe_bank* bank, int slot, int which, float* out, hipStream_t stream) {
  try {
    int rc = check_bank(bank);
    if (rc) return rc;
    REQUIRE(slot >= 0 && slot < bank->n_slots, FT_E_INVAL, "slot %d out of range [0, %d)", slot, bank->n_slots);
    REQUIRE(which == 0 || which == 1, FT_E_INVAL, "which must be 0 (W13) or 1 (W2), got %d", which);
    CHECK_PTR(out, "out");
    const int rows = which == 0 ? 2 * bank->I : bank->d;
    const int K = which == 0 ? bank->d : bank->I;
    const size_t per_slot = ft_moe_bank_bytes(bank->fmt, 1, bank->d, bank->I, which);
    const size_t per_slot_s = ft_moe_bank_bytes(bank->fmt, 1, bank->d, bank->I, which + 2);
    const uint8_t* codes = (const uint8_t*)(which == 0 ? bank->w13 : bank->w2) + per_slot * slot;
    const uint8_t* scales = nullptr;
    const float* tscale = nullptr;
    if (bank->fmt == FT_W_NVFP4) {  // block scales of every slot, then the slots' matrix scales
      const uint8_t* base = (const uint8_t*)(which == 0 ? bank->s13 : bank->s2);
      const size_t blk = (size_t)rows * (K / 32) * 2;
      scales = base + blk * slot;
      tscale = (const float*)(base + blk * bank->n_slots) + slot;
    } else if (bank->fmt != FT_W_BF16) {
      scales = (const uint8_t*)(which == 0 ? bank->s13 : bank->s2) + per_slot_s * slot;
    }
    return hip_status(ftk::launch_dequant(bank->fmt, codes, scales, rows, K, which == 0 ? bank->I : 0, tscale, out,
                                          stream),
                      "ft_moe_dequant launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_dequant: unexpected exception");
  }
}

int ft_moe_cache_update(const int32_t* counts, int E, int n_slots, int max_loads, float load_fraction,
                        int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use, uint32_t* tick,
                        int32_t* compute_slot, int32_t* load_slot, int32_t* loads, int32_t* n_loads,
                        hipStream_t stream) {
  try {
    REQUIRE(E >= 1 && E <= 1024, FT_E_INVAL, "E must be in [1, 1024] (got %d)", E);
    REQUIRE(n_slots >= 1 && n_slots <= 1024, FT_E_INVAL, "n_slots must be in [1, 1024] (got %d)", n_slots);
    REQUIRE(max_loads >= 0 && max_loads <= n_slots, FT_E_INVAL, "max_loads must be in [0, n_slots] (got %d)",
            max_loads);
    REQUIRE(load_fraction >= 0.0f && load_fraction <= 1.0f, FT_E_INVAL, "load_fraction must be in [0, 1] (got %g)",
            (double)load_fraction);
    if (load_slot) CHECK_PTR(load_slot, "load_slot");
    CHECK_PTR(counts, "counts");
    CHECK_PTR(slot_of_expert, "slot_of_expert");
    CHECK_PTR(expert_of_slot, "expert_of_slot");
    CHECK_PTR(last_use, "last_use");
    CHECK_PTR(tick, "tick");
    CHECK_PTR(compute_slot, "compute_slot");
    CHECK_PTR(loads, "loads");
    CHECK_PTR(n_loads, "n_loads");
    return hip_status(ftk::launch_cache_update(counts, E, n_slots, max_loads, load_fraction, slot_of_expert,
                                               expert_of_slot, last_use, tick, compute_slot, load_slot, loads,
                                               n_loads, stream),
                      "ft_moe_cache_update launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_cache_update: unexpected exception");
  }
}

// Device-visible address of a source-bank array: pinned host memory (its mapped address) or device
// memory (as is).  Pageable host memory is refused.
static int source_view(const void* p, const char* name, const uint8_t** out) {
  hipPointerAttribute_t attr{};
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FT_E_INVAL, "%s is neither pinned host memory nor device memory (%s)", name, hipGetErrorString(e));
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = (const uint8_t*)p;
    return FT_OK;
  }
  REQUIRE(attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr, FT_E_INVAL,
          "%s is neither pinned host memory nor device memory", name);
  const uint8_t* dev = (const uint8_t*)attr.devicePointer;
  *out = attr.hostPointer ? dev + ((const uint8_t*)p - (const uint8_t*)attr.hostPointer) : dev;
  return FT_OK;
}

constexpr int kFillBlocks = 8;  // 128 KiB in flight saturate the host link; every other CU is left to the FFN

int ft_moe_cache_fill(const ft_moe_bank* src, const ft_moe_bank* dst, const int32_t* loads, const int32_t* n_loads,
                      int max_loads, hipStream_t stream) {
  try {
    int rc = check_bank(src);
    if (rc) return rc;
    rc = check_bank(dst);
    if (rc) return rc;
    REQUIRE(src->fmt == dst->fmt && src->d == dst->d && src->I == dst->I, FT_E_INVAL,
            "source and destination banks differ in format or shape");
    REQUIRE(max_loads >= 0 && max_loads <= dst->n_slots, FT_E_INVAL, "max_loads must be in [0, dst->n_slots] (got %d)",
            max_loads);
    if (max_loads == 0) return ok();
    CHECK_PTR(loads, "loads");
    CHECK_PTR(n_loads, "n_loads");
    const int fmt = dst->fmt, d = dst->d, I = dst->I;
    ftk::CacheFillArgs a{};
    const uint8_t* sv[4] = {nullptr, nullptr, nullptr, nullptr};
    rc = source_view(src->w13, "src->w13", &sv[0]);
    if (rc == FT_OK) rc = source_view(src->w2, "src->w2", &sv[1]);
    if (rc == FT_OK && fmt != FT_W_BF16) rc = source_view(src->s13, "src->s13", &sv[2]);
    if (rc == FT_OK && fmt != FT_W_BF16) rc = source_view(src->s2, "src->s2", &sv[3]);
    if (rc) return rc;
    a.seg[0] = {sv[0], (uint8_t*)dst->w13, (long long)ft_moe_bank_bytes(fmt, 1, d, I, 0)};
    a.seg[1] = {sv[1], (uint8_t*)dst->w2, (long long)ft_moe_bank_bytes(fmt, 1, d, I, 1)};
    a.nseg = 2;
    if (fmt == FT_W_NVFP4) {  // per-slot block scales, then one matrix scale per slot after every slot's blocks
      const long long b13 = 2LL * I * (d / 32) * 2, b2 = (long long)d * (I / 32) * 2;
      a.seg[2] = {sv[2], (uint8_t*)dst->s13, b13};
      a.seg[3] = {sv[3], (uint8_t*)dst->s2, b2};
      a.seg[4] = {sv[2] + b13 * src->n_slots, (uint8_t*)dst->s13 + b13 * dst->n_slots, 4};
      a.seg[5] = {sv[3] + b2 * src->n_slots, (uint8_t*)dst->s2 + b2 * dst->n_slots, 4};
      a.nseg = 6;
    } else if (fmt != FT_W_BF16) {
      a.seg[2] = {sv[2], (uint8_t*)dst->s13, (long long)ft_moe_bank_bytes(fmt, 1, d, I, 2)};
      a.seg[3] = {sv[3], (uint8_t*)dst->s2, (long long)ft_moe_bank_bytes(fmt, 1, d, I, 3)};
      a.nseg = 4;
    }
    a.n_src = src->n_slots;
    a.n_dst = dst->n_slots;
    a.max_loads = max_loads;
    a.loads = loads;
    a.n_loads = n_loads;
    return hip_status(ftk::launch_cache_fill(a, kFillBlocks, stream), "ft_moe_cache_fill launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_cache_fill: unexpected exception");
  }
}

int ft_moe_residual_host(const ft_moe_bank* host_bank, const uint16_t* x, const int32_t* ids, const float* w,
                         const uint32_t* residual_mask, const int32_t* slot_of_expert, int T, int E, int k,
                         float* out, int n_threads) {
  try {
    int rc = check_tek(T, E, k);
    if (rc) return rc;
    rc = check_bank(host_bank);
    if (rc) return rc;
    REQUIRE(n_threads >= 0, FT_E_INVAL, "n_threads must be >= 0 (got %d)", n_threads);
    if (T == 0) return ok();
    REQUIRE(x != nullptr && ids != nullptr && w != nullptr && out != nullptr, FT_E_INVAL,
            "x, ids, w and out must not be null");
    REQUIRE((residual_mask != nullptr) != (slot_of_expert != nullptr), FT_E_INVAL,
            "exactly one of residual_mask and slot_of_expert must be given");
    int threads = n_threads;
    if (threads == 0) threads = (int)std::thread::hardware_concurrency();
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    const ft_moe_bank* b = host_bank;
    ftk::residual_host(b->fmt, b->n_slots, b->d, b->I, (const uint8_t*)b->w13, (const uint8_t*)b->w2,
                       (const uint8_t*)b->s13, (const uint8_t*)b->s2, x, ids, w, residual_mask, slot_of_expert, T, E, k,
                       out, threads);
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(FT_E_INTERNAL, "ft_moe_residual_host: out of host memory");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_residual_host: unexpected exception");
  }
}

int ft_moe_residual_add(void* out, const float* residual, int T, int d, int flags, hipStream_t stream) {
  try {
    REQUIRE(T >= 0, FT_E_INVAL, "T must be >= 0 (got %d)", T);
    REQUIRE(d > 0 && d % 8 == 0, FT_E_INVAL, "d must be a positive multiple of 8 (got %d)", d);
    REQUIRE((flags & ~FT_OUT_BF16) == 0, FT_E_INVAL, "unknown flags 0x%x", flags);
    if (T == 0) return ok();
    CHECK_PTR(out, "out");
    CHECK_PTR(residual, "residual");
    return hip_status(ftk::launch_residual_add(out, residual, (long long)T * d, (flags & FT_OUT_BF16) != 0, stream),
                      "ft_moe_residual_add launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_residual_add: unexpected exception");
  }
}

// ---- start-up rates

constexpr size_t kRatesSink = 1u << 20;          // sink words at the start of dev_buf
constexpr size_t kRatesMinDev = 64u << 20;       // device bytes: the sink, then at least 63 MiB to stream
constexpr int kRatesMfmaIters = 4096;            // x 4 MFMAs per wave and launch

int ft_moe_measure_rates(void* dev_buf, size_t dev_bytes, const void* host_buf, size_t host_bytes, int reps,
                         ft_moe_rates* out, hipStream_t stream) {
  try {
    CHECK_PTR(out, "out");
    CHECK_PTR(dev_buf, "dev_buf");
    REQUIRE(((uintptr_t)dev_buf & 255u) == 0, FT_E_INVAL, "dev_buf is not 256-byte aligned");
    REQUIRE(dev_bytes >= kRatesMinDev, FT_E_INVAL, "dev_bytes must be at least %zu (got %zu)", kRatesMinDev,
            dev_bytes);
    REQUIRE(reps >= 1 && reps <= 100, FT_E_INVAL, "reps must be in [1, 100] (got %d)", reps);
    const uint8_t* hv = nullptr;
    if (host_buf != nullptr) {
      REQUIRE(((uintptr_t)host_buf & 15u) == 0, FT_E_INVAL, "host_buf is not 16-byte aligned");
      REQUIRE(host_bytes >= (1u << 20), FT_E_INVAL, "host_bytes must be at least 1 MiB (got %zu)", host_bytes);
      int rc = source_view(host_buf, "host_buf", &hv);
      if (rc) return rc;
    }
    int blocks = 0, cus = 0;
    hipError_t e = ftk::rate_launch_facts(&blocks, &cus);
    if (e != hipSuccess) return hip_status(e, "ft_moe_measure_rates: launch facts");
    const int mfma_blocks = 2 * cus;  // two 4-wave blocks per CU: two waves per SIMD
    REQUIRE((size_t)mfma_blocks * 256 * 4 <= kRatesSink && (size_t)blocks * 16 <= kRatesSink, FT_E_UNSUPPORTED,
            "%d compute units need more sink than the %zu bytes at the start of dev_buf", cus, kRatesSink);
    uint8_t* base = (uint8_t*)dev_buf;
    const long long dev_stream = (long long)((dev_bytes - kRatesSink) & ~(size_t)15);
    const long long host_stream = (long long)(host_bytes & ~(size_t)15);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e != hipSuccess) {
      if (e0) (void)hipEventDestroy(e0);
      return hip_status(e, "ft_moe_measure_rates: event create");
    }
    // best (shortest) of reps timed launches after one untimed, in seconds; negative on a HIP error
    auto best = [&](auto launch) -> double {
      double t = 1e30;
      for (int r = 0; r <= reps; ++r) {
        if ((e = hipEventRecord(e0, stream)) != hipSuccess) return -1.0;
        if ((e = launch()) != hipSuccess) return -1.0;
        if ((e = hipEventRecord(e1, stream)) != hipSuccess) return -1.0;
        if ((e = hipEventSynchronize(e1)) != hipSuccess) return -1.0;
        float ms = 0.0f;
        if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) return -1.0;
        if (r > 0 && ms * 1e-3 < t) t = ms * 1e-3;
      }
      return t;
    };
    ft_moe_rates R{};
    R.compute_units = cus;
    R.stream_blocks = blocks;
    double t = best([&] { return ftk::launch_stream_read(base + kRatesSink, dev_stream, blocks, (uint32_t*)base, stream); });
    if (t > 0) R.hbm_read_gbs = (double)dev_stream / t / 1e9;
    if (t > 0 && hv != nullptr) {
      t = best([&] { return ftk::launch_stream_read(hv, host_stream, kFillBlocks, (uint32_t*)base, stream); });
      if (t > 0) R.host_read_gbs = (double)host_stream / t / 1e9;
    }
    const double per_launch = (double)mfma_blocks * 4 * kRatesMfmaIters * 4;  // MFMA instructions
    double* rate[3] = {&R.mfma_bf16_tflops, &R.mfma_fp8_tflops, &R.mfma_fp6_fp4_tflops};
    const double flops[3] = {2.0 * 32 * 32 * 16, 2.0 * 32 * 32 * 64, 2.0 * 32 * 32 * 64};
    for (int kind = 0; kind < 3 && t > 0; ++kind) {
      t = best([&] { return ftk::launch_mfma_rate(kind, mfma_blocks, kRatesMfmaIters, (float*)base, stream); });
      if (t > 0) *rate[kind] = per_launch * flops[kind] / t / 1e12;
    }
    // a bf16 32x32x16 MFMA occupies a SIMD for 32 cycles (1024 flops per SIMD and cycle)
    R.mfma_clock_ghz = R.mfma_bf16_tflops * 1e12 / ((double)cus * 4 * 1024) / 1e9;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (t <= 0) return hip_status(e != hipSuccess ? e : hipErrorUnknown, "ft_moe_measure_rates");
    *out = R;
    return ok();
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_measure_rates: unexpected exception");
  }
}

size_t ft_moe_layer_workspace(const ft_moe_bank* bank, int T, int E, int k, int shared_slot, int flags) {
  if (bank == nullptr || check_tek(T, E, k) != FT_OK || check_bank_shape(bank->fmt, bank->n_slots, bank->d, bank->I)) {
    g_err[0] = 0;
    return 0;
  }
  return layer_ws(bank, T, E, k, shared_slot >= 0, layer_fused(bank, T, E, k, flags), flags).total;
}

}  // extern "C"

namespace {

// ft_moe_layer after its checks of T, E, k, the bank, the flags and shared_slot: the rest of the
// validation and the launches, with the workspace `wsb` (ws_bytes long; null when missing).
// w_router (ft_moe_layer_proj): the logits are first computed from x and the router rows into
// `logits`, inside the one launch where that fits, else by the router projection kernel.
int layer_checked(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const float* logits,
                  const uint16_t* x, int T, int E, int k, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                  int32_t* gather, int32_t* inv, uint16_t* y_sorted, uint16_t* y_shared, void* out,
                  uint32_t* residual_mask, uint8_t* wsb, size_t ws_bytes, int flags, hipStream_t stream,
                  bool check_only = false, const uint16_t* w_router = nullptr) {
  int rc;
  CHECK_PTR(counts, "counts");
  CHECK_PTR(offsets, "offsets");
  const bool shared = shared_slot >= 0;
  const bool fused = layer_fused(bank, T, E, k, flags);
  const LayerWs W = layer_ws(bank, T, E, k, shared, fused, flags);
  REQUIRE(wsb != nullptr && ws_bytes >= W.total, FT_E_WORKSPACE, "layer needs %zu bytes of workspace (got %zu%s)",
          W.total, ws_bytes, wsb ? "" : ", null pointer");
  REQUIRE(aligned16(wsb), FT_E_INVAL, "ws is not 16-byte aligned");
  if (T == 0) {  // counts and offsets are still defined (all zero)
    if (check_only) return FT_OK;
    return hip_status(ftk::launch_permute(ids, 0, E, k, counts, offsets, gather, inv, wsb + W.perm, stream),
                      "ft_moe_layer permute launch");
  }
  CHECK_PTR(slot_of_expert, "slot_of_expert");
  CHECK_PTR(logits, "logits");
  CHECK_PTR(x, "x");
  CHECK_PTR(ids, "ids");
  CHECK_PTR(w, "w");
  CHECK_PTR(gather, "gather");
  CHECK_PTR(inv, "inv");
  CHECK_PTR(y_sorted, "y_sorted");
  if (y_shared) CHECK_PTR(y_shared, "y_shared");
  CHECK_PTR(out, "out");
  if (residual_mask) CHECK_PTR(residual_mask, "residual_mask");
  if (w_router) CHECK_PTR(w_router, "w_router");
  if (check_only) return FT_OK;
  const bool out_bf16 = (flags & FT_OUT_BF16) != 0;
  const bool proj_fused = w_router && fused && ftk::layer_decode_fits(bank->fmt, T, E, k, bank->d, bank->I, true);
  if (w_router && !proj_fused) {
    hipError_t e = ftk::launch_route_proj(x, w_router, T, bank->d, E, k, (float*)logits, ids, w, wsb + W.rproj, stream);
    if (e != hipSuccess) return hip_status(e, "ft_moe_layer_proj router projection launch");
  }
  if (!fused) {
    hipError_t e = ftk::launch_route(logits, T, E, k, ids, w, stream);
    if (e != hipSuccess) return hip_status(e, "ft_moe_layer route launch");
    // the permutation also clears the grouped FFN's queue counters (one launch fewer)
    e = ftk::launch_permute(ids, T, E, k, counts, offsets, gather, inv, wsb + W.perm, stream, (int32_t*)(wsb + W.qctr),
                            ftk::FFN_QCTR_INTS);
    if (e != hipSuccess) return hip_status(e, "ft_moe_layer permute launch");
    rc = launch_grouped_ffn(bank, slot_of_expert, shared_slot, x, T, E, k, offsets, gather, y_sorted, y_shared,
                            (uint16_t*)(wsb + W.h), wsb + W.terms, (int32_t*)(wsb + W.qctr),
                            flags & (FT_PATH_MASK | FT_GEMM_WIDEN), stream, true);
    if (rc) return rc;
    return hip_status(ftk::launch_combine(y_sorted, y_shared, ids, w, inv, slot_of_expert, bank->n_slots, T, E, k,
                                          bank->d, out, residual_mask, out_bf16, stream),
                      "ft_moe_layer combine launch");
  }
  ftk::LayerArgs L{};
  ftk::FfnArgs& a = L.f;
  a.fmt = bank->fmt;
  a.d = bank->d;
  a.I = bank->I;
  a.n_slots = bank->n_slots;
  a.w13 = (const uint8_t*)bank->w13;
  a.w2 = (const uint8_t*)bank->w2;
  a.s13 = (const uint8_t*)bank->s13;
  a.s2 = (const uint8_t*)bank->s2;
  a.slot_of = slot_of_expert;
  a.shared_slot = shared_slot;
  a.x = x;
  a.T = T;
  a.E = E;
  a.k = k;
  a.offsets = offsets;
  a.gather = gather;
  a.h = (uint16_t*)(wsb + W.h);
  a.y_sorted = y_sorted;
  a.y_shared = y_shared;
  a.min_cnt = 1;
  a.max_cnt = 0x7fffffff;
  L.logits = logits;
  L.ids = ids;
  L.w = w;
  L.counts = counts;
  L.offsets = offsets;
  L.gather = gather;
  L.inv = inv;
  L.mask = residual_mask;
  L.out = out;
  L.out_bf16 = out_bf16 ? 1 : 0;
  L.id_bits = id_bits_of(E);
  L.ctl = (int32_t*)(wsb + W.ctl);
  L.done13 = (int32_t*)(wsb + W.done13);
  L.n_rc = W.n_rc;
  L.cdone = (int32_t*)(wsb + W.cdone);
  if (proj_fused) {
    L.w_router = w_router;
    L.proj_logits = (float*)logits;
    L.pflag = (int32_t*)(wsb + W.rproj);
  }
  return hip_status(ftk::launch_layer_decode(L, stream), "ft_moe_layer fused launch");
}

// ft_moe_layer's own checks of the arguments that are not buffers
int layer_args(const ft_moe_bank* bank, int shared_slot, int T, int E, int k, const uint16_t* y_shared, int flags) {
  int rc = check_tek(T, E, k);
  if (rc) return rc;
  rc = check_bank(bank);
  if (rc) return rc;
  REQUIRE((flags & ~(FT_PATH_MASK | FT_GEMM_WIDEN | FT_OUT_BF16 | FT_LAYER_UNFUSED)) == 0, FT_E_INVAL,
          "unknown flags 0x%x", flags);
  REQUIRE((flags & FT_PATH_MASK) != 3, FT_E_INVAL, "FT_PATH_GEMV and FT_PATH_GEMM are exclusive");
  REQUIRE(shared_slot >= -1 && shared_slot < bank->n_slots, FT_E_INVAL, "shared_slot %d out of range [-1, %d)",
          shared_slot, bank->n_slots);
  REQUIRE((shared_slot >= 0) == (y_shared != nullptr), FT_E_INVAL,
          "y_shared must be given exactly when shared_slot >= 0");
  return FT_OK;
}

}  // namespace

extern "C" {

int ft_moe_layer(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const float* logits,
                 const uint16_t* x, int T, int E, int k, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                 int32_t* gather, int32_t* inv, uint16_t* y_sorted, uint16_t* y_shared, void* out,
                 uint32_t* residual_mask, void* ws, size_t ws_bytes, int flags, hipStream_t stream) {
  try {
    const int rc = layer_args(bank, shared_slot, T, E, k, y_shared, flags);
    if (rc) return rc;
    return layer_checked(bank, slot_of_expert, shared_slot, logits, x, T, E, k, ids, w, counts, offsets, gather, inv,
                         y_sorted, y_shared, out, residual_mask, (uint8_t*)ws, ws_bytes, flags, stream);
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_layer: unexpected exception");
  }
}

int ft_moe_layer_proj(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const uint16_t* x,
                      const uint16_t* w_router, int T, int E, int k, float* logits, int32_t* ids, float* w,
                      int32_t* counts, int32_t* offsets, int32_t* gather, int32_t* inv, uint16_t* y_sorted,
                      uint16_t* y_shared, void* out, uint32_t* residual_mask, void* ws, size_t ws_bytes, int flags,
                      hipStream_t stream) {
  try {
    int rc = layer_args(bank, shared_slot, T, E, k, y_shared, flags);
    if (rc) return rc;
    REQUIRE(E <= 512, FT_E_INVAL, "E must be at most 512 for ft_moe_layer_proj (got %d)", E);
    if (T > 0) {
      CHECK_PTR(w_router, "w_router");
      CHECK_PTR(logits, "logits");
    }
    return layer_checked(bank, slot_of_expert, shared_slot, logits, x, T, E, k, ids, w, counts, offsets, gather, inv,
                         y_sorted, y_shared, out, residual_mask, (uint8_t*)ws, ws_bytes, flags, stream, false,
                         T > 0 ? w_router : nullptr);
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_layer_proj: unexpected exception");
  }
}

}  // extern "C"

// ---- ft_moe_layer_noalloc: the layer workspace in a static device array of the library

// The scratch of ft_moe_layer_noalloc: one copy per device, loaded with the code object and held
// until the process ends.  Host code never uses this name as an address (in host code it stands for
// a host-side shadow); it uses the device address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[FT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device
// Bytes at the start of each device's scratch that hold zeros once the work enqueued so far has run
// (the counters a fused call needs zero at its start lie in such a prefix; calls of other shapes
// leave other data past their own counters).  Starts at 0: the array's initial contents are not
// relied on.
size_t g_scratch_zero[kMaxDevices] = {};

__global__ void scratch_clear_kernel(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Moves the status word of the call that ran before it on the stream into *status (when given) and
// clears it, so that every call starts with a clear word.
__global__ void scratch_status_kernel(int32_t* word, int32_t* status) {
  const int v = __hip_atomic_exchange(word, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (status) *status = v;
}

// Device address of the scratch on the current device (looked up once per device, with that device
// current) and the device's index.
int scratch_of_device(uint8_t** ptr, int* device) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "ft_moe_layer_noalloc: hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, FT_E_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "ft_moe_layer_noalloc: hipGetSymbolAddress of the scratch");
    REQUIRE(p != nullptr && ((uintptr_t)p & 255u) == 0, FT_E_INTERNAL, "scratch address %p is not 256-byte aligned",
            p);
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *ptr = g_scratch_ptr[dev];
  *device = dev;
  return FT_OK;
}

}  // namespace

extern "C" {

int ft_moe_layer_noalloc(const ft_moe_bank* bank, const int32_t* slot_of_expert, int shared_slot, const float* logits,
                         const uint16_t* x, int T, int E, int k, int32_t* ids, float* w, int32_t* counts,
                         int32_t* offsets, int32_t* gather, int32_t* inv, uint16_t* y_sorted, uint16_t* y_shared,
                         void* out, uint32_t* residual_mask, int32_t* status, int flags, hipStream_t stream) {
  try {
    int rc = layer_args(bank, shared_slot, T, E, k, y_shared, flags);
    if (rc) return rc;
    const LayerWs W = layer_ws(bank, T, E, k, shared_slot >= 0, layer_fused(bank, T, E, k, flags), flags);
    REQUIRE(W.total <= FT_NOALLOC_SCRATCH_BYTES, FT_E_WORKSPACE,
            "ft_moe_layer_noalloc: this layer needs %zu bytes of scratch, more than the %zu of the static scratch "
            "(call ft_moe_layer with a workspace)",
            W.total, (size_t)FT_NOALLOC_SCRATCH_BYTES);
    REQUIRE(status == nullptr || ((uintptr_t)status & 3u) == 0, FT_E_INVAL, "status is not 4-byte aligned");
    // every check of the call runs before anything is enqueued (the scratch's address stands in)
    uint8_t* sp = nullptr;
    int dev = 0;
    rc = scratch_of_device(&sp, &dev);
    if (rc) return rc;
    rc = layer_checked(bank, slot_of_expert, shared_slot, logits, x, T, E, k, ids, w, counts, offsets, gather, inv,
                       y_sorted, y_shared, out, residual_mask, sp, FT_NOALLOC_SCRATCH_BYTES, flags, stream, true);
    if (rc) return rc;
    // the control words and counters this call needs zero: clear what earlier calls may have left
    // there (the status word, the first of them, is zero after every call)
    std::unique_lock<std::mutex> lock(g_scratch_mu);
    const size_t zero = g_scratch_zero[dev];
    g_scratch_zero[dev] = 0;  // unknown until this call's work is enqueued
    lock.unlock();
    if (W.zeroed > zero) {
      hipLaunchKernelGGL(scratch_clear_kernel, dim3(64), dim3(256), 0, stream, (uint4*)(sp + zero),
                         (W.zeroed - zero) / 16);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_status(e, "ft_moe_layer_noalloc scratch clear launch");
    }
    rc = layer_checked(bank, slot_of_expert, shared_slot, logits, x, T, E, k, ids, w, counts, offsets, gather, inv,
                       y_sorted, y_shared, out, residual_mask, sp, FT_NOALLOC_SCRATCH_BYTES, flags, stream);
    if (rc) return rc;
    // the call leaves its counters at zero and other data after them
    lock.lock();
    g_scratch_zero[dev] = W.zeroed;
    lock.unlock();
    // the status word is the first int32 of the layer workspace's control block
    hipLaunchKernelGGL(scratch_status_kernel, dim3(1), dim3(1), 0, stream, (int32_t*)sp, status);
    return hip_status(hipGetLastError(), "ft_moe_layer_noalloc status launch");
  } catch (...) {
    return fail(FT_E_INTERNAL, "ft_moe_layer_noalloc: unexpected exception");
  }
}

}  // extern "C"
