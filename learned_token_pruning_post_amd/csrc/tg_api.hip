// C ABI of libtokengate: host-side validation, workspace carving and kernel
// launches. Arguments are checked before any HIP call, so argument errors
// come back synchronously with nothing enqueued.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstring>

#include "../../include/tokengate.h"
#include "tg_internal.hpp"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline size_t elt_size(tg_dtype d) { return d == TG_BF16 ? 2 : 4; }
inline bool dtype_ok(tg_dtype d) { return d == TG_F32 || d == TG_BF16; }

// gfx950 check, cached per device (the cache is idempotent; races only repeat the query)
std::atomic<int> g_arch[64];

tg_status check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_LAUNCH;
  if (dev >= 0 && dev < 64) {
    const int c = g_arch[dev].load(std::memory_order_relaxed);
    if (c == 1) return TG_OK;
    if (c == -1) return TG_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TG_ERR_LAUNCH;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? TG_OK : TG_ERR_UNSUPPORTED;
}

inline tg_status launched(hipError_t e) { return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH; }

// The bf16 kernels address each operand through a buffer resource whose range
// is a 32-bit byte count: every such operand must stay below 4 GiB.
inline bool fits32(int64_t rows, int64_t row_elems, int64_t elt = 2) {
  return rows >= 0 && row_elems >= 0 && rows * row_elems * elt < ((int64_t)1 << 32);
}

#define TG_CHECK(cond, code) \
  do {                       \
    if (!(cond)) return (code); \
  } while (0)
#define TG_LAUNCH(expr)                  \
  do {                                   \
    hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return TG_ERR_LAUNCH; \
  } while (0)

bool layer_dims_ok(const tg_layer_dims* dm) {
  constexpr int known = TG_LAYER_ROPE_READY | TG_LAYER_NORMS_FOLDED | TG_LAYER_INPUT_SSQ |
                        TG_LAYER_ATTN_ONLY | TG_LAYER_FFN_ONLY;
  const bool halves = (dm->flags & TG_LAYER_ATTN_ONLY) && (dm->flags & TG_LAYER_FFN_ONLY);
  return dm->D > 0 && dm->Hq > 0 && dm->Hkv > 0 && dm->d > 0 && dm->I > 0 &&
         dm->Hq % dm->Hkv == 0 && dm->rms_eps >= 0.f && dm->rope_base > 0.f &&
         (dm->flags & ~known) == 0 && !halves &&
         (!(dm->flags & TG_LAYER_INPUT_SSQ) || (dm->flags & TG_LAYER_NORMS_FOLDED));
}

tg_status layer_dims_supported(const tg_layer_dims* dm) {
  if (!dtype_ok(dm->dtype)) return TG_ERR_UNSUPPORTED;
  if (dm->d != 64 && dm->d != 128) return TG_ERR_UNSUPPORTED;
  if ((dm->flags & TG_LAYER_NORMS_FOLDED) && dm->dtype != TG_BF16) return TG_ERR_UNSUPPORTED;
  if (dm->dtype == TG_BF16) {
    const int G = dm->Hq / dm->Hkv;
    if (G != 1 && G != 2 && G != 4) return TG_ERR_UNSUPPORTED;
    if (dm->D % 64 || dm->I % 64 || (dm->Hq * dm->d) % 64) return TG_ERR_UNSUPPORTED;
  }
  return TG_OK;
}

}  // namespace

// Scratch of tg_topk_select_noalloc. Every GPU the library runs on holds its
// own copy at its own address until the process ends; host code reaches it
// only through the address hipGetSymbolAddress gives for the current device
// (the array's name on the host is a stand-in, not a device address). Calls
// that overlap on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[TG_SELECT_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_ptr[64];  // device address of `scratch`, per device (idempotent cache)

tg_status noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_LAUNCH;
  if (dev < 0 || dev >= 64) return TG_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TG_ERR_LAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return TG_OK;
}
}  // namespace

extern "C" {

const char* tg_status_string(tg_status s) {
  switch (s) {
    case TG_OK: return "ok";
    case TG_ERR_INVALID_ARG: return "invalid argument";
    case TG_ERR_UNSUPPORTED: return "unsupported dtype, shape or device";
    case TG_ERR_WORKSPACE: return "workspace too small";
    case TG_ERR_LAUNCH: return "HIP launch error";
    default: return "unknown status";
  }
}

int tg_abi_version(void) { return (3 << 16) | 1; }

// ---------------------------------------------------------------------------
size_t tg_gate_score_workspace_size(int64_t T_in, int D, int H1, tg_dtype dtype) {
  (void)D;
  if (T_in <= 0 || H1 <= 0) return 0;
  if (dtype == TG_BF16) return tg::gemm_bf16_score_ws(T_in, H1);
  return align_up((size_t)T_in * (size_t)H1 * sizeof(float));
}

tg_status tg_gate_score(const void* h, int64_t T_in, int D, int H1, const void* W1, const void* b1,
                        const void* w2, const void* b2, tg_dtype dtype, float* s_out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  TG_CHECK(T_in >= 0 && T_in <= INT_MAX && D > 0 && H1 > 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  if (T_in == 0) return TG_OK;
  TG_CHECK(h && W1 && b1 && w2 && b2 && s_out, TG_ERR_INVALID_ARG);
  if (dtype == TG_BF16) TG_CHECK(D % 64 == 0 && H1 % 4 == 0, TG_ERR_UNSUPPORTED);
  if (dtype == TG_BF16) TG_CHECK(fits32(T_in, D) && fits32(H1, D), TG_ERR_UNSUPPORTED);
  const size_t need = tg_gate_score_workspace_size(T_in, D, H1, dtype);
  TG_CHECK(ws_bytes >= need && (need == 0 || ws), TG_ERR_WORKSPACE);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  if (dtype == TG_BF16) {
    return launched(tg::gemm_bf16_score((const bf16*)h, (const bf16*)W1, (const bf16*)b1,
                                        (const bf16*)w2, (const bf16*)b2, s_out, (float*)ws,
                                        (int)T_in, H1, D, stream));
  }
  float* z = (float*)ws;
  TG_LAUNCH(tg::gemm_f32((const float*)h, (const float*)W1, nullptr, z, (int)T_in, H1, D, H1, stream));
  return launched(tg::score_epilogue_f32(z, (const float*)b1, (const float*)w2, (const float*)b2,
                                         s_out, T_in, H1, stream));
}

// ---------------------------------------------------------------------------
size_t tg_topk_select_workspace_size(int B, int64_t T_in, int max_n) {
  if (B <= 0 || T_in < 0 || max_n < 0 || !tg::select_supported(max_n)) return 0;
  return tg::select_workspace_bytes(B, T_in, max_n);
}

// Arguments shared by the selection entry points (checked before any HIP call).
static tg_status select_args(const float* s, const int32_t* d_cu_in, const int32_t* d_cu_kept, int B,
                             int64_t T_in, int64_t T, int max_n, const int32_t* kept_idx, void* ws,
                             size_t ws_bytes) {
  TG_CHECK(B >= 0 && T_in >= 0 && T >= 0 && max_n >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(T_in <= INT_MAX && T <= INT_MAX, TG_ERR_INVALID_ARG);
  TG_CHECK(T <= T_in, TG_ERR_INVALID_ARG);  // K_b <= N_b summed over the batch
  if (B == 0) return TG_OK;
  TG_CHECK(d_cu_in && d_cu_kept, TG_ERR_INVALID_ARG);
  TG_CHECK(T_in == 0 || s, TG_ERR_INVALID_ARG);
  TG_CHECK(T == 0 || kept_idx, TG_ERR_INVALID_ARG);
  TG_CHECK(tg::select_supported(max_n), TG_ERR_UNSUPPORTED);
  // one workgroup per (sequence, chunk of at least 256 tokens)
  TG_CHECK(((int64_t)max_n + 255) / 256 * B <= INT_MAX, TG_ERR_INVALID_ARG);
  const size_t need = tg::select_workspace_bytes(B, T_in, max_n);
  TG_CHECK(ws && ws_bytes >= need, TG_ERR_WORKSPACE);
  TG_CHECK(((uintptr_t)ws & 255u) == 0, TG_ERR_INVALID_ARG);
  return TG_OK;
}

tg_status tg_topk_select(const float* s, const uint8_t* keep_mask, const int32_t* d_cu_in,
                         const int32_t* d_cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                         int32_t* kept_idx, int32_t* d_status, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  const tg_status st = select_args(s, d_cu_in, d_cu_kept, B, T_in, T, max_n, kept_idx, ws, ws_bytes);
  if (st != TG_OK || B == 0) return st;
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_select_compact(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n,
                                            kept_idx, d_status, ws, nullptr, nullptr, 0, nullptr,
                                            nullptr, nullptr, stream));
}

tg_status tg_select_compact(const float* s, const uint8_t* keep_mask, const int32_t* d_cu_in,
                            const int32_t* d_cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                            const void* h, const int32_t* pos, int D, tg_dtype dtype,
                            int32_t* kept_idx, int32_t* d_status, void* h_out, int32_t* pos_out,
                            float* s_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  TG_CHECK(D > 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  const tg_status st = select_args(s, d_cu_in, d_cu_kept, B, T_in, T, max_n, kept_idx, ws, ws_bytes);
  if (st != TG_OK || B == 0) return st;
  TG_CHECK(T == 0 || (h && h_out && pos_out), TG_ERR_INVALID_ARG);
  TG_CHECK((int64_t)D * (int64_t)elt_size(dtype) < ((int64_t)1 << 31), TG_ERR_UNSUPPORTED);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_select_compact(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n,
                                            kept_idx, d_status, ws, h, pos,
                                            (size_t)D * elt_size(dtype), T > 0 ? h_out : nullptr,
                                            pos_out, s_out, stream));
}

tg_status tg_topk_select_noalloc(const float* s, const uint8_t* keep_mask, const int32_t* d_cu_in,
                                 const int32_t* d_cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                                 int32_t* kept_idx, int32_t* d_status, hipStream_t stream) {
  // every argument check before the first HIP call, with the scratch standing
  // in for the workspace (its size; any 256-aligned address)
  const tg_status chk = select_args(s, d_cu_in, d_cu_kept, B, T_in, T, max_n, kept_idx,
                                    reinterpret_cast<void*>(256), TG_SELECT_NOALLOC_SCRATCH_BYTES);
  if (chk != TG_OK || B == 0) return chk;
  const size_t need = tg::select_workspace_bytes(B, T_in, max_n);
  void* ws = nullptr;
  const tg_status st = noalloc_scratch(&ws);
  if (st != TG_OK) return st;
  return tg_topk_select(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n, kept_idx, d_status,
                        ws, need, stream);
}

// ---------------------------------------------------------------------------
tg_status tg_compact(const void* h, const int32_t* pos, const float* s, const int32_t* kept_idx,
                     const int32_t* d_cu_in, const int32_t* d_cu_kept, int B, int64_t T, int D,
                     tg_dtype dtype, void* h_out, int32_t* pos_out, float* s_out,
                     hipStream_t stream) {
  TG_CHECK(T >= 0 && D > 0 && B >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  if (T == 0) return TG_OK;
  TG_CHECK(B >= 1, TG_ERR_INVALID_ARG);
  TG_CHECK(h && kept_idx && h_out && pos_out && d_cu_kept, TG_ERR_INVALID_ARG);
  TG_CHECK(pos || d_cu_in, TG_ERR_INVALID_ARG);
  TG_CHECK(!s_out || s, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_compact(h, pos, s, kept_idx, d_cu_in, d_cu_kept, B, T,
                                     (size_t)D * elt_size(dtype), h_out, pos_out, s_out, stream));
}

// ---------------------------------------------------------------------------
size_t tg_gated_attn_workspace_size(int B, int max_k, int Hq, int Hkv, int d, tg_dtype dtype) {
  (void)B;
  (void)max_k;
  (void)Hq;
  (void)Hkv;
  (void)d;
  (void)dtype;
  return 0;
}

static tg_status attn_args(int B, int max_k, int Hq, int Hkv, int d, tg_dtype dtype) {
  TG_CHECK(B >= 0 && max_k >= 0 && Hq > 0 && Hkv > 0 && d > 0, TG_ERR_INVALID_ARG);
  TG_CHECK(Hq % Hkv == 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  TG_CHECK(d == 64 || d == 128, TG_ERR_UNSUPPORTED);
  if (dtype == TG_BF16) {
    const int G = Hq / Hkv;
    TG_CHECK(G == 1 || G == 2 || G == 4, TG_ERR_UNSUPPORTED);
    TG_CHECK(fits32(max_k, (int64_t)Hkv * d), TG_ERR_UNSUPPORTED);  // one sequence's K or V
  }
  return TG_OK;
}

tg_status tg_gated_attn_fwd(const void* q, const void* k, const void* v, const float* s_c,
                            const float* t, const float* g, const int32_t* d_cu_kept, int B,
                            int max_k, int Hq, int Hkv, int d, tg_dtype dtype, void* o,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  tg_status st = attn_args(B, max_k, Hq, Hkv, d, dtype);
  if (st != TG_OK) return st;
  if (B == 0 || max_k == 0) return TG_OK;
  TG_CHECK(q && k && v && s_c && t && g && d_cu_kept && o, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::attn_fwd(q, k, v, s_c, t, g, d_cu_kept, B, max_k, Hq, Hkv, d,
                               dtype == TG_BF16, o, lse, stream));
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// backward of the gated attention
// ---------------------------------------------------------------------------

size_t tg_gated_attn_bwd_workspace_size(int B, int64_t T, int max_k, int Hq, int Hkv, int d,
                                        tg_dtype dtype) {
  if (dtype != TG_BF16 || B <= 0 || T < 0 || max_k < 0 || !tg::attn_bwd_supported(Hq, Hkv, d)) return 0;
  return tg::attn_bwd_workspace_bytes(B, T, max_k, Hq, Hkv, d);
}

tg_status tg_gated_attn_bwd(const void* q, const void* k, const void* v, const float* s_c,
                            const float* t, const float* g, const int32_t* d_cu_kept, int B, int64_t T,
                            int max_k, int Hq, int Hkv, int d, tg_dtype dtype, const void* o,
                            const float* lse, const void* dO, float* dq, float* dk, float* dv, float* ds,
                            float* dt, float* dg, void* ws, size_t ws_bytes, hipStream_t stream) {
  TG_CHECK(B >= 0 && T >= 0 && T <= INT_MAX && max_k >= 0 && Hq > 0 && Hkv > 0 && d > 0,
           TG_ERR_INVALID_ARG);
  TG_CHECK(Hq % Hkv == 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype == TG_BF16, TG_ERR_UNSUPPORTED);
  TG_CHECK(tg::attn_bwd_supported(Hq, Hkv, d), TG_ERR_UNSUPPORTED);
  TG_CHECK((int64_t)T * Hq * (d / 8) / 256 < INT_MAX, TG_ERR_UNSUPPORTED);  // prep grid
  // one sequence's q / dO rows (Hq heads; k / v have Hkv <= Hq) through 32-bit buffer ranges
  TG_CHECK(fits32(max_k, (int64_t)Hq * d), TG_ERR_UNSUPPORTED);
  if (B == 0 || T == 0 || max_k == 0) return TG_OK;
  TG_CHECK(q && k && v && s_c && t && g && d_cu_kept && o && lse && dO, TG_ERR_INVALID_ARG);
  TG_CHECK(dq && dk && dv && ds && dt && dg, TG_ERR_INVALID_ARG);
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  TG_CHECK(a16(q) && a16(k) && a16(v) && a16(o) && a16(dO) && a16(dq) && a16(dk) && a16(dv),
           TG_ERR_INVALID_ARG);
  const size_t need = tg::attn_bwd_workspace_bytes(B, T, max_k, Hq, Hkv, d);
  TG_CHECK(ws && ws_bytes >= need, TG_ERR_WORKSPACE);
  TG_CHECK(((uintptr_t)ws & 255u) == 0, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_attn_bwd(q, k, v, s_c, t, g, d_cu_kept, B, T, max_k, Hq, Hkv, d, o, lse, dO,
                                      dq, dk, dv, ds, dt, dg, ws, stream));
}

// ---------------------------------------------------------------------------
// backward of the scorer and of the compaction
// ---------------------------------------------------------------------------

size_t tg_gate_score_bwd_workspace_size(int64_t T_in, int D, int H1, tg_dtype dtype) {
  if (dtype != TG_BF16 || T_in <= 0 || D <= 0 || H1 <= 0) return 0;
  return tg::score_bwd_workspace_bytes(T_in, D, H1);
}

tg_status tg_gate_score_bwd(const void* h, int64_t T_in, int D, int H1, const void* W1, const void* b1,
                            const void* w2, tg_dtype dtype, const float* s, const float* ds, void* dh,
                            float* dW1, float* db1, float* dw2, float* db2, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  TG_CHECK(T_in >= 0 && T_in <= INT_MAX && D > 0 && H1 > 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype == TG_BF16, TG_ERR_UNSUPPORTED);
  TG_CHECK(D % 64 == 0 && H1 % 64 == 0, TG_ERR_UNSUPPORTED);
  // 32-bit buffer ranges of the products' operands
  TG_CHECK(fits32(T_in, D) && fits32(T_in, H1) && fits32(H1, D), TG_ERR_UNSUPPORTED);
  TG_CHECK(W1 && b1 && w2 && dW1 && db1 && dw2 && db2, TG_ERR_INVALID_ARG);
  TG_CHECK(T_in == 0 || (h && s && ds && dh), TG_ERR_INVALID_ARG);
  auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  TG_CHECK(a16(h) && a16(W1) && a16(dh) && a16(dW1), TG_ERR_INVALID_ARG);
  const size_t need = tg::score_bwd_workspace_bytes(T_in, D, H1);
  TG_CHECK(T_in == 0 || (ws && ws_bytes >= need && ((uintptr_t)ws & 255u) == 0), TG_ERR_WORKSPACE);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  if (T_in == 0) {  // no tokens: every gradient is zero
    TG_LAUNCH(tg::launch_fill_f32(dW1, (int64_t)H1 * D, 0.f, stream));
    TG_LAUNCH(tg::launch_fill_f32(db1, H1, 0.f, stream));
    TG_LAUNCH(tg::launch_fill_f32(dw2, H1, 0.f, stream));
    return launched(tg::launch_fill_f32(db2, 1, 0.f, stream));
  }
  return launched(tg::launch_score_bwd(h, T_in, D, H1, W1, b1, w2, s, ds, dh, dW1, db1, dw2, db2, ws, stream));
}

tg_status tg_compact_scores_bwd(const float* ds_c, const int32_t* kept_idx, int64_t T, int64_t T_in,
                                float* ds, hipStream_t stream) {
  TG_CHECK(T >= 0 && T_in >= 0 && T <= T_in && T_in <= INT_MAX, TG_ERR_INVALID_ARG);
  if (T_in == 0) return TG_OK;
  TG_CHECK(ds && (T == 0 || (ds_c && kept_idx)), TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_scatter_scores(ds_c, kept_idx, T, T_in, ds, stream));
}

// ---------------------------------------------------------------------------
// Gated DeltaNet mixer of the hybrid variant
// ---------------------------------------------------------------------------

size_t tg_gdn_workspace_size(int64_t T, int B, int H, int dk, int dv, tg_dtype dtype) {
  if (dtype != TG_BF16 || T <= 0 || B <= 0 || H <= 0 || !tg::gdn_supported(dk, dv)) return 0;
  return tg::gdn_chunk_workspace_bytes(T, B, H, dk, dv);
}

tg_status tg_gdn_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                     const int32_t* d_cu, int64_t T, int B, int H, int dk, int dv, tg_dtype dtype,
                     const float* state_in, void* o, float* state_out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  TG_CHECK(B >= 0 && H > 0 && dk > 0 && dv > 0 && T >= 0 && T <= INT_MAX, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  TG_CHECK(tg::gdn_supported(dk, dv), TG_ERR_UNSUPPORTED);
  TG_CHECK((int64_t)B * H * (dv / 16) <= INT_MAX, TG_ERR_UNSUPPORTED);
  TG_CHECK(((T + 63) / 64 + B) * (int64_t)H <= INT_MAX, TG_ERR_UNSUPPORTED);
  if (B == 0) return TG_OK;
  TG_CHECK(d_cu && (T == 0 || (q && k && v && o && alpha && beta)), TG_ERR_INVALID_ARG);
  auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  TG_CHECK(a16(q) && a16(k) && a16(v) && a16(o) && a16(state_in) && a16(state_out), TG_ERR_INVALID_ARG);
  const bool bf = dtype == TG_BF16;
  if (bf && T > 0) {
    const size_t need = tg::gdn_chunk_workspace_bytes(T, B, H, dk, dv);
    TG_CHECK(ws && ws_bytes >= need && ((uintptr_t)ws & 255u) == 0, TG_ERR_WORKSPACE);
  }
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  if (bf)
    return launched(tg::launch_gdn_chunked(q, k, v, alpha, beta, d_cu, T, B, H, dk, dv, state_in, o, state_out,
                                           ws, stream));
  return launched(tg::launch_gdn(q, k, v, alpha, beta, d_cu, B, H, dk, dv, false, state_in, o, state_out, stream));
}

// ---------------------------------------------------------------------------
// decode attention over the pruned cache
// ---------------------------------------------------------------------------

size_t tg_decode_attn_workspace_size(int B, int max_len, int Hq, int Hkv, int d, tg_dtype dtype) {
  if (!dtype_ok(dtype) || B <= 0 || max_len < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
  return tg::decode_workspace_bytes(B, max_len, Hq, Hkv, d);
}

tg_status tg_decode_attn_fwd(const void* q, const void* kA, const void* vA, const float* sA,
                             const int32_t* d_cuA, const void* kB, const void* vB, const float* sB,
                             const int32_t* d_lenB, int capB, const float* t, const float* g, int B,
                             int max_len, int Hq, int Hkv, int d, tg_dtype dtype, void* o, float* lse,
                             int32_t* d_status, void* ws, size_t ws_bytes, hipStream_t stream) {
  TG_CHECK(B >= 0 && max_len >= 0 && capB >= 0 && Hq > 0 && Hkv > 0 && d > 0, TG_ERR_INVALID_ARG);
  TG_CHECK(Hq % Hkv == 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  TG_CHECK(tg::decode_supported(Hq, Hkv, d), TG_ERR_UNSUPPORTED);
  // one workgroup per (sequence, kv head, chunk of at least 128 keys)
  TG_CHECK((int64_t)B * Hkv * (((int64_t)max_len + 127) / 128) <= INT_MAX, TG_ERR_UNSUPPORTED);
  if (B == 0) return TG_OK;
  TG_CHECK(q && kA && vA && sA && d_cuA && d_lenB && t && g && o, TG_ERR_INVALID_ARG);
  TG_CHECK(capB == 0 || (kB && vB && sB), TG_ERR_INVALID_ARG);
  auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  TG_CHECK(a16(q) && a16(kA) && a16(vA) && a16(kB) && a16(vB) && a16(o), TG_ERR_INVALID_ARG);
  const size_t need = tg::decode_workspace_bytes(B, max_len, Hq, Hkv, d);
  TG_CHECK(need == 0 || (ws && ws_bytes >= need), TG_ERR_WORKSPACE);
  TG_CHECK(need == 0 || ((uintptr_t)ws & 255u) == 0, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_decode_attn(q, kA, vA, sA, d_cuA, kB, vB, sB, d_lenB, capB, t, g, B,
                                         max_len, Hq, Hkv, d, dtype == TG_BF16, o, lse, d_status,
                                         ws, stream));
}

tg_status tg_fold_norm_weights(const void* norm_w, void* W, int64_t rows, int cols,
                               tg_dtype dtype, hipStream_t stream) {
  TG_CHECK(rows >= 0 && cols >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dtype), TG_ERR_UNSUPPORTED);
  if (rows == 0 || cols == 0) return TG_OK;
  TG_CHECK(norm_w && W, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_fold_norm(norm_w, W, rows, cols, dtype == TG_BF16, stream));
}

// ---------------------------------------------------------------------------
tg_status tg_upper_layer_ws_layout(const tg_layer_dims* dm, int64_t T, tg_layer_ws_layout* out) {
  TG_CHECK(dm && out && T >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(layer_dims_ok(dm), TG_ERR_INVALID_ARG);
  TG_CHECK(dtype_ok(dm->dtype), TG_ERR_UNSUPPORTED);
  const size_t e = elt_size(dm->dtype);
  const size_t t = (size_t)T;
  size_t off = 0;
  out->norm = off;
  off += align_up(t * dm->D * e);
  out->q = off;
  off += align_up(t * dm->Hq * dm->d * e);
  out->attn = off;
  off += align_up(t * dm->Hq * dm->d * e);
  out->x1 = off;
  off += align_up(t * dm->D * e);
  out->act = off;
  off += align_up(t * dm->I * e);
  out->rope = off;
  off += align_up(t * dm->d * sizeof(float));
  out->ssq = off;  // [2][T][D/64] fp32, fused RMSNorm
  off += align_up(2 * t * (size_t)((dm->D + 63) / 64) * sizeof(float));
  if (dm->dtype == TG_F32) {  // raw q|k|v and the up projection
    off += align_up(t * (dm->Hq + 2 * dm->Hkv) * dm->d * sizeof(float));
    off += align_up(t * dm->I * sizeof(float));
  }
  out->total = off;
  return TG_OK;
}

size_t tg_upper_layer_workspace_size(const tg_layer_dims* dm, int64_t T, int B, int max_k) {
  (void)B;
  (void)max_k;
  tg_layer_ws_layout l;
  if (tg_upper_layer_ws_layout(dm, T, &l) != TG_OK) return 0;
  return l.total;
}

static tg_status upper_layer_impl(const tg_layer_weights* w, const tg_layer_dims* dm,
                                  const void* x_in, void* x_out, const int32_t* pos_c,
                                  const float* s_c, const int32_t* d_cu_kept, int B, int64_t T,
                                  int max_k, void* kcache, void* vcache, void* ws, size_t ws_bytes,
                                  hipStream_t stream, hipEvent_t* ev) {
  TG_CHECK(w && dm, TG_ERR_INVALID_ARG);
  TG_CHECK(layer_dims_ok(dm), TG_ERR_INVALID_ARG);
  TG_CHECK(B >= 0 && T >= 0 && T <= INT_MAX && max_k >= 0, TG_ERR_INVALID_ARG);
  tg_status st = layer_dims_supported(dm);
  if (st != TG_OK) return st;
  if (T == 0 || B == 0) return TG_OK;
  const bool fused = (dm->flags & TG_LAYER_NORMS_FOLDED) != 0;
  const bool attn_half = !(dm->flags & TG_LAYER_FFN_ONLY);  // stages 0-4
  const bool ffn_half = !(dm->flags & TG_LAYER_ATTN_ONLY);  // stages 5-7
  TG_CHECK(!attn_half || max_k > 0, TG_ERR_INVALID_ARG);
  if (dm->dtype == TG_BF16) {  // activations and weights of every GEMM, one sequence's K/V
    const int64_t qd = (int64_t)dm->Hq * dm->d, kvd = (int64_t)dm->Hkv * dm->d;
    TG_CHECK(fits32(T, dm->D) && fits32(T, qd) && fits32(T, dm->I) && fits32(qd, dm->D) &&
                 fits32(dm->I, dm->D) && fits32(max_k, kvd),
             TG_ERR_UNSUPPORTED);
  }
  TG_CHECK(!attn_half || (w->wq && w->wk && w->wv && w->wo && w->t && w->g), TG_ERR_INVALID_ARG);
  TG_CHECK(!ffn_half || (w->wg && w->wu && w->wd), TG_ERR_INVALID_ARG);
  TG_CHECK(fused || ((!attn_half || w->attn_norm) && (!ffn_half || w->ffn_norm)), TG_ERR_INVALID_ARG);
  TG_CHECK(x_in && x_out, TG_ERR_INVALID_ARG);
  TG_CHECK(!attn_half || (pos_c && s_c && d_cu_kept && kcache && vcache), TG_ERR_INVALID_ARG);
  tg_layer_ws_layout L;
  st = tg_upper_layer_ws_layout(dm, T, &L);
  if (st != TG_OK) return st;
  TG_CHECK(ws && ws_bytes >= L.total, TG_ERR_WORKSPACE);
  tg_status a = check_arch();
  if (a != TG_OK) return a;

  char* base = (char*)ws;
  void* norm = base + L.norm;
  void* qb = base + L.q;
  void* attn = base + L.attn;
  void* act = base + L.act;
  float* rope = (float*)(base + L.rope);
  float* ssq_x = (float*)(base + L.ssq);                   // x_in, then x_out
  float* ssq_x1 = ssq_x + (size_t)T * (size_t)(dm->D / 64);  // x1
  // the post-attention residual: the workspace's x1 for a whole layer, the
  // output of an attention half, the input of an FFN half
  void* x1 = attn_half ? (ffn_half ? (void*)(base + L.x1) : x_out) : const_cast<void*>(x_in);
  const int M = (int)T;
  const int D = dm->D, Hq = dm->Hq, Hkv = dm->Hkv, d = dm->d, I = dm->I;
  const bool bf = dm->dtype == TG_BF16;

  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if (attn_half) {
    TG_LAUNCH(mark(0));
    if (!(dm->flags & TG_LAYER_ROPE_READY))
      TG_LAUNCH(tg::launch_rope_table(pos_c, T, d, dm->rope_base, rope, stream));
    TG_LAUNCH(mark(1));
    if (!fused)
      TG_LAUNCH(tg::launch_rmsnorm(x_in, w->attn_norm, norm, T, D, dm->rms_eps, bf, stream));
    else if (!(dm->flags & TG_LAYER_INPUT_SSQ))
      TG_LAUNCH(tg::launch_row_ssq(x_in, ssq_x, T, D, stream));
    TG_LAUNCH(mark(2));
    if (bf) {
      tg::QkvOut qo{(bf16*)qb, (bf16*)kcache, (bf16*)vcache, rope, Hq, Hkv, d};
      TG_LAUNCH(tg::gemm_bf16_qkv((const bf16*)(fused ? x_in : norm), (const bf16*)w->wq,
                                  (const bf16*)w->wk, (const bf16*)w->wv, qo, M, D, stream,
                                  fused ? ssq_x : nullptr, dm->rms_eps));
    } else {
      float* raw = (float*)(base + L.rope + align_up((size_t)T * d * sizeof(float)));
      const int ldr = (Hq + 2 * Hkv) * d;
      TG_LAUNCH(tg::gemm_f32((const float*)norm, (const float*)w->wq, nullptr, raw, M, Hq * d, D, ldr, stream));
      TG_LAUNCH(tg::gemm_f32((const float*)norm, (const float*)w->wk, nullptr, raw + Hq * d, M,
                             Hkv * d, D, ldr, stream));
      TG_LAUNCH(tg::gemm_f32((const float*)norm, (const float*)w->wv, nullptr,
                             raw + (Hq + Hkv) * d, M, Hkv * d, D, ldr, stream));
      TG_LAUNCH(tg::qkv_split_rope_f32(raw, rope, (float*)qb, (float*)kcache, (float*)vcache, T, Hq,
                                       Hkv, d, stream));
    }
    TG_LAUNCH(mark(3));
    TG_LAUNCH(tg::attn_fwd(qb, kcache, vcache, s_c, w->t, w->g, d_cu_kept, B, max_k, Hq, Hkv, d, bf,
                           attn, nullptr, stream));
    TG_LAUNCH(mark(4));
    // the residual is read and the output written element by element by the
    // same thread, so x1 may be x_in (an attention half in place)
    if (bf) {
      TG_LAUNCH(tg::gemm_bf16_plain((const bf16*)attn, (const bf16*)w->wo, (const bf16*)x_in,
                                    (bf16*)x1, M, D, Hq * d, stream,
                                    fused && ffn_half ? ssq_x1 : nullptr));
    } else {
      TG_LAUNCH(tg::gemm_f32((const float*)attn, (const float*)w->wo, (const float*)x_in, (float*)x1,
                             M, D, Hq * d, D, stream));
    }
  } else {
    for (int i = 0; i <= 4; ++i) TG_LAUNCH(mark(i));
  }
  TG_LAUNCH(mark(5));
  if (!ffn_half) {
    for (int i = 6; i <= 8; ++i) TG_LAUNCH(mark(i));
    return TG_OK;
  }
  if (!fused)
    TG_LAUNCH(tg::launch_rmsnorm(x1, w->ffn_norm, norm, T, D, dm->rms_eps, bf, stream));
  else if (!attn_half)  // an FFN half: its input's sums of squares
    TG_LAUNCH(tg::launch_row_ssq(x1, ssq_x1, T, D, stream));
  TG_LAUNCH(mark(6));
  if (bf) {
    TG_LAUNCH(tg::gemm_bf16_swiglu((const bf16*)(fused ? x1 : norm), (const bf16*)w->wg,
                                   (const bf16*)w->wu, (bf16*)act, M, I, D, stream,
                                   fused ? ssq_x1 : nullptr, dm->rms_eps));
    TG_LAUNCH(mark(7));
    TG_LAUNCH(tg::gemm_bf16_plain((const bf16*)act, (const bf16*)w->wd, (const bf16*)x1,
                                  (bf16*)x_out, M, D, I, stream, fused ? ssq_x : nullptr));
    return launched(mark(8));
  }
  float* raw = (float*)(base + L.rope + align_up((size_t)T * d * sizeof(float)));
  float* up = (float*)((char*)raw + align_up((size_t)T * (Hq + 2 * Hkv) * d * sizeof(float)));
  TG_LAUNCH(tg::gemm_f32((const float*)norm, (const float*)w->wg, nullptr, (float*)act, M, I, D, I, stream));
  TG_LAUNCH(tg::gemm_f32((const float*)norm, (const float*)w->wu, nullptr, up, M, I, D, I, stream));
  TG_LAUNCH(tg::swiglu_f32((const float*)act, up, (float*)act, (int64_t)T * I, stream));
  TG_LAUNCH(mark(7));
  TG_LAUNCH(tg::gemm_f32((const float*)act, (const float*)w->wd, (const float*)x1, (float*)x_out,
                         M, D, I, D, stream));
  return launched(mark(8));
}

tg_status tg_upper_layer_fwd(const tg_layer_weights* w, const tg_layer_dims* dm, const void* x_in,
                             void* x_out, const int32_t* pos_c, const float* s_c,
                             const int32_t* d_cu_kept, int B, int64_t T, int max_k, void* kcache,
                             void* vcache, void* ws, size_t ws_bytes, hipStream_t stream) {
  return upper_layer_impl(w, dm, x_in, x_out, pos_c, s_c, d_cu_kept, B, T, max_k, kcache, vcache,
                          ws, ws_bytes, stream, nullptr);
}

tg_status tg_upper_layer_stack_fwd(const tg_layer_weights* w, int n_layers, const tg_layer_dims* dm,
                                   void* x, const int32_t* pos_c, const float* s_c,
                                   const int32_t* d_cu_kept, int B, int64_t T, int max_k,
                                   void* kcache, void* vcache, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  TG_CHECK(n_layers >= 0 && dm, TG_ERR_INVALID_ARG);
  if (n_layers == 0) return TG_OK;
  TG_CHECK(w, TG_ERR_INVALID_ARG);
  TG_CHECK((dm->flags & ~TG_LAYER_NORMS_FOLDED) == 0, TG_ERR_INVALID_ARG);
  const bool fused = (dm->flags & TG_LAYER_NORMS_FOLDED) != 0;
  // every layer's weights before the first launch (the other arguments are
  // shared, and layer 0 checks them before it launches anything)
  for (int l = 0; l < n_layers; ++l) {
    const tg_layer_weights& wl = w[l];
    TG_CHECK(wl.wq && wl.wk && wl.wv && wl.wo && wl.wg && wl.wu && wl.wd && wl.t && wl.g,
             TG_ERR_INVALID_ARG);
    TG_CHECK(fused || (wl.attn_norm && wl.ffn_norm), TG_ERR_INVALID_ARG);
  }
  TG_CHECK(dm->Hkv > 0 && dm->d > 0, TG_ERR_INVALID_ARG);
  const size_t cache_layer = (size_t)(T > 0 ? T : 0) * (size_t)dm->Hkv * (size_t)dm->d * elt_size(dm->dtype);
  for (int l = 0; l < n_layers; ++l) {
    tg_layer_dims dl = *dm;
    if (l > 0) dl.flags |= TG_LAYER_ROPE_READY | (fused ? TG_LAYER_INPUT_SSQ : 0);
    const tg_status st = upper_layer_impl(&w[l], &dl, x, x, pos_c, s_c, d_cu_kept, B, T, max_k,
                                          kcache ? (char*)kcache + l * cache_layer : nullptr,
                                          vcache ? (char*)vcache + l * cache_layer : nullptr, ws,
                                          ws_bytes, stream, nullptr);
    if (st != TG_OK) return st;
  }
  return TG_OK;
}

size_t tg_gated_prefill_workspace_size(const tg_layer_dims* dm, int H1, int64_t T_in, int64_t T,
                                       int B, int max_k) {
  if (!dm) return 0;
  const size_t a = tg_gate_score_workspace_size(T_in, dm->D, H1, dm->dtype);
  tg_layer_dims base = *dm;
  base.flags &= TG_LAYER_NORMS_FOLDED;
  const size_t b = tg_upper_layer_workspace_size(&base, T, B, max_k);
  const size_t c = B > 0 && T_in >= 0 ? tg::select_workspace_bound(B, T_in) : 0;
  const size_t ab = a > b ? a : b;
  return ab > c ? ab : c;
}

tg_status tg_gated_prefill(const void* h, const int32_t* pos, const uint8_t* keep_mask,
                           const int32_t* d_cu_in, const int32_t* d_cu_kept, int B, int64_t T_in,
                           int64_t T, int max_n, int max_k, const tg_gate_weights* gate,
                           const tg_layer_weights* layers, int n_layers, const tg_layer_dims* dm,
                           float* s, int32_t* kept_idx, int32_t* d_status, void* x, int32_t* pos_c,
                           float* s_c, void* kcache, void* vcache, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  TG_CHECK(gate && dm, TG_ERR_INVALID_ARG);
  tg_status st = tg_gate_score(h, T_in, dm->D, gate->H1, gate->W1, gate->b1, gate->w2, gate->b2,
                               dm->dtype, s, ws, ws_bytes, stream);
  if (st != TG_OK) return st;
  st = tg_select_compact(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n, h, pos, dm->D,
                         dm->dtype, kept_idx, d_status, x, pos_c, s_c, ws, ws_bytes, stream);
  if (st != TG_OK) return st;
  return tg_upper_layer_stack_fwd(layers, n_layers, dm, x, pos_c, s_c, d_cu_kept, B, T, max_k,
                                  kcache, vcache, ws, ws_bytes, stream);
}

size_t tg_full_prefill_workspace_size(const tg_layer_dims* dm, int H1, int64_t T_in, int64_t T,
                                      int B, int max_n, int max_k) {
  if (!dm || T_in < 0 || T < 0 || B < 0) return 0;
  tg_layer_dims base = *dm;
  base.flags &= TG_LAYER_NORMS_FOLDED;
  size_t m = tg_gate_score_workspace_size(T_in, dm->D, H1, dm->dtype);
  m = std::max(m, tg_upper_layer_workspace_size(&base, T_in, B, max_n));
  m = std::max(m, tg_upper_layer_workspace_size(&base, T, B, max_k));
  m = std::max(m, tg_topk_select_workspace_size(B, T_in, max_n));
  // plus the plain-attention constants: t = 1 and g = 0 per head, zero scores per token
  return align_up(m) + align_up(((size_t)2 * (size_t)std::max(dm->Hq, 0) + (size_t)T_in) * sizeof(float));
}

tg_status tg_full_prefill(const void* h, const int32_t* pos, const uint8_t* keep_mask,
                          const int32_t* d_cu_in, const int32_t* d_cu_kept, int B, int64_t T_in,
                          int64_t T, int max_n, int max_k, const tg_gate_weights* gate,
                          const tg_layer_weights* below, int n_below,
                          const tg_layer_weights* gate_layer, const tg_layer_weights* above,
                          int n_above, const tg_layer_dims* dm, void* x_full, void* kcache_full,
                          void* vcache_full, float* s, int32_t* kept_idx, int32_t* d_status, void* x,
                          int32_t* pos_c, float* s_c, void* kcache, void* vcache, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  TG_CHECK(gate && dm && gate_layer && n_below >= 0 && n_above >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(n_below == 0 || below, TG_ERR_INVALID_ARG);
  TG_CHECK(n_above == 0 || above, TG_ERR_INVALID_ARG);
  TG_CHECK((dm->flags & ~TG_LAYER_NORMS_FOLDED) == 0, TG_ERR_INVALID_ARG);
  TG_CHECK(B >= 0 && T_in >= 0 && T_in <= INT_MAX && T >= 0 && T <= T_in && max_n >= 0 && max_k >= 0,
           TG_ERR_INVALID_ARG);
  if (B == 0 || T_in == 0) return TG_OK;
  TG_CHECK(h && pos && x_full && kcache_full && vcache_full && s, TG_ERR_INVALID_ARG);
  TG_CHECK(T == 0 || (kept_idx && x && pos_c && s_c), TG_ERR_INVALID_ARG);
  TG_CHECK(n_above == 0 || T == 0 || (kcache && vcache), TG_ERR_INVALID_ARG);
  const size_t need = tg_full_prefill_workspace_size(dm, gate->H1, T_in, T, B, max_n, max_k);
  TG_CHECK(ws && ws_bytes >= need, TG_ERR_WORKSPACE);
  TG_CHECK(dtype_ok(dm->dtype), TG_ERR_UNSUPPORTED);
  // every layer's weights before the first launch
  auto weights_ok = [&](const tg_layer_weights& wl) {
    return wl.wq && wl.wk && wl.wv && wl.wo && wl.wg && wl.wu && wl.wd &&
           ((dm->flags & TG_LAYER_NORMS_FOLDED) || (wl.attn_norm && wl.ffn_norm));
  };
  for (int l = 0; l < n_below; ++l) TG_CHECK(weights_ok(below[l]), TG_ERR_INVALID_ARG);
  TG_CHECK(weights_ok(*gate_layer), TG_ERR_INVALID_ARG);
  for (int l = 0; l < n_above; ++l) TG_CHECK(weights_ok(above[l]) && above[l].t && above[l].g, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;

  // plain attention below the gate and in layer L: t = 1, g = 0 (the layers'
  // own t and g are not used), zero scores; kept at the end of the workspace,
  // past what every stage uses
  const size_t stage_ws = need - align_up(((size_t)2 * dm->Hq + (size_t)T_in) * sizeof(float));
  float* plain = (float*)((char*)ws + stage_ws);
  TG_LAUNCH(tg::launch_fill_f32(plain, dm->Hq, 1.f, stream));
  TG_LAUNCH(tg::launch_fill_f32(plain + dm->Hq, (int64_t)dm->Hq + T_in, 0.f, stream));
  auto plain_weights = [&](const tg_layer_weights& wl) {
    tg_layer_weights p = wl;
    p.t = plain;
    p.g = plain + dm->Hq;
    return p;
  };
  const float* zero_s = plain + 2 * dm->Hq;
  const bool fused = (dm->flags & TG_LAYER_NORMS_FOLDED) != 0;
  const size_t elt = elt_size(dm->dtype);
  const size_t cache_full = (size_t)T_in * (size_t)dm->Hkv * (size_t)dm->d * elt;
  // ---- layers below the gate on every token ----
  for (int l = 0; l < n_below; ++l) {
    tg_layer_dims dl = *dm;
    if (l > 0) dl.flags |= TG_LAYER_ROPE_READY | (fused ? TG_LAYER_INPUT_SSQ : 0);
    const tg_layer_weights wl = plain_weights(below[l]);
    tg_status st = upper_layer_impl(&wl, &dl, l == 0 ? h : x_full, x_full, pos, zero_s, d_cu_in, B,
                                    T_in, max_n, (char*)kcache_full + l * cache_full,
                                    (char*)vcache_full + l * cache_full, ws, stage_ws, stream, nullptr);
    if (st != TG_OK) return st;
  }
  // ---- layer L's attention on every token: x_full = its post-attention residual ----
  {
    tg_layer_dims dl = *dm;
    dl.flags |= TG_LAYER_ATTN_ONLY;
    if (n_below > 0) dl.flags |= TG_LAYER_ROPE_READY | (fused ? TG_LAYER_INPUT_SSQ : 0);
    const tg_layer_weights wl = plain_weights(*gate_layer);
    tg_status st = upper_layer_impl(&wl, &dl, n_below > 0 ? x_full : h, x_full, pos, zero_s, d_cu_in,
                                    B, T_in, max_n, (char*)kcache_full + n_below * cache_full,
                                    (char*)vcache_full + n_below * cache_full, ws, stage_ws, stream,
                                    nullptr);
    if (st != TG_OK) return st;
  }
  // ---- the gate: scores, selection, compaction of the residual rows ----
  tg_status st = tg_gate_score(x_full, T_in, dm->D, gate->H1, gate->W1, gate->b1, gate->w2, gate->b2,
                               dm->dtype, s, ws, stage_ws, stream);
  if (st != TG_OK) return st;
  st = tg_select_compact(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n, x_full, pos, dm->D,
                         dm->dtype, kept_idx, d_status, x, pos_c, s_c, ws, stage_ws, stream);
  if (st != TG_OK) return st;
  if (T == 0) return TG_OK;
  // ---- layer L's FFN on the kept rows, then the layers above ----
  {
    tg_layer_dims dl = *dm;
    dl.flags |= TG_LAYER_FFN_ONLY;
    st = upper_layer_impl(gate_layer, &dl, x, x, pos_c, s_c, d_cu_kept, B, T, max_k, nullptr, nullptr,
                          ws, stage_ws, stream, nullptr);
    if (st != TG_OK) return st;
  }
  return tg_upper_layer_stack_fwd(above, n_above, dm, x, pos_c, s_c, d_cu_kept, B, T, max_k, kcache,
                                  vcache, ws, stage_ws, stream);
}

tg_status tg_upper_layer_fwd_timed(const tg_layer_weights* w, const tg_layer_dims* dm,
                                   const void* x_in, void* x_out, const int32_t* pos_c,
                                   const float* s_c, const int32_t* d_cu_kept, int B, int64_t T,
                                   int max_k, void* kcache, void* vcache, void* ws,
                                   size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  TG_CHECK(events, TG_ERR_INVALID_ARG);
  for (int i = 0; i <= TG_LAYER_STAGES; ++i) TG_CHECK(events[i], TG_ERR_INVALID_ARG);
  return upper_layer_impl(w, dm, x_in, x_out, pos_c, s_c, d_cu_kept, B, T, max_k, kcache, vcache,
                          ws, ws_bytes, stream, events);
}

}  // extern "C"
