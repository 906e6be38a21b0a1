// C ABI of libtokengate: host-side validation, workspace carving and kernel
// launches. Arguments are checked before any HIP call, so argument errors
// come back synchronously with nothing enqueued.
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
  return dm->D > 0 && dm->Hq > 0 && dm->Hkv > 0 && dm->d > 0 && dm->I > 0 &&
         dm->Hq % dm->Hkv == 0 && dm->rms_eps >= 0.f && dm->rope_base > 0.f &&
         (dm->flags & ~(TG_LAYER_ROPE_READY | TG_LAYER_NORMS_FOLDED | TG_LAYER_INPUT_SSQ)) == 0 &&
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
  if (B < 0 || T_in < 0) return 0;
  return tg::topk_select_workspace_bytes(B, T_in, max_n);
}

tg_status tg_topk_select(const float* s, const uint8_t* keep_mask, const int32_t* d_cu_in,
                         const int32_t* d_cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                         int32_t* kept_idx, int32_t* d_status, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  TG_CHECK(B >= 0 && T_in >= 0 && T >= 0 && max_n >= 0, TG_ERR_INVALID_ARG);
  TG_CHECK(T_in <= INT_MAX && T <= INT_MAX, TG_ERR_INVALID_ARG);
  TG_CHECK(T <= T_in, TG_ERR_INVALID_ARG);  // K_b <= N_b summed over the batch
  if (B == 0) return TG_OK;
  TG_CHECK(d_cu_in && d_cu_kept, TG_ERR_INVALID_ARG);
  TG_CHECK(T_in == 0 || s, TG_ERR_INVALID_ARG);
  TG_CHECK(T == 0 || kept_idx, TG_ERR_INVALID_ARG);
  // one workgroup per (sequence, 4096-token chunk) on the long-sequence path
  TG_CHECK(((int64_t)max_n + 4095) / 4096 * B <= INT_MAX, TG_ERR_INVALID_ARG);
  const size_t need = tg::topk_select_workspace_bytes(B, T_in, max_n);
  TG_CHECK(need == 0 || (ws && ws_bytes >= need), TG_ERR_WORKSPACE);
  TG_CHECK(need == 0 || ((uintptr_t)ws & 255u) == 0, TG_ERR_INVALID_ARG);
  tg_status a = check_arch();
  if (a != TG_OK) return a;
  return launched(tg::launch_topk_select(s, keep_mask, d_cu_in, d_cu_kept, B, max_n, kept_idx,
                                         d_status, ws, stream));
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
  TG_CHECK(max_k > 0, TG_ERR_INVALID_ARG);
  const bool fused = (dm->flags & TG_LAYER_NORMS_FOLDED) != 0;
  TG_CHECK(w->wq && w->wk && w->wv && w->wo && w->wg && w->wu && w->wd && w->t && w->g,
           TG_ERR_INVALID_ARG);
  TG_CHECK(fused || (w->attn_norm && w->ffn_norm), TG_ERR_INVALID_ARG);
  TG_CHECK(x_in && x_out && pos_c && s_c && d_cu_kept && kcache && vcache, TG_ERR_INVALID_ARG);
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
  void* x1 = base + L.x1;
  void* act = base + L.act;
  float* rope = (float*)(base + L.rope);
  float* ssq_x = (float*)(base + L.ssq);                   // x_in, then x_out
  float* ssq_x1 = ssq_x + (size_t)T * (size_t)(dm->D / 64);  // x1
  const int M = (int)T;
  const int D = dm->D, Hq = dm->Hq, Hkv = dm->Hkv, d = dm->d, I = dm->I;
  const bool bf = dm->dtype == TG_BF16;

  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
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
  if (bf) {
    TG_LAUNCH(tg::gemm_bf16_plain((const bf16*)attn, (const bf16*)w->wo, (const bf16*)x_in,
                                  (bf16*)x1, M, D, Hq * d, stream, fused ? ssq_x1 : nullptr));
  } else {
    TG_LAUNCH(tg::gemm_f32((const float*)attn, (const float*)w->wo, (const float*)x_in, (float*)x1,
                           M, D, Hq * d, D, stream));
  }
  TG_LAUNCH(mark(5));
  if (!fused) TG_LAUNCH(tg::launch_rmsnorm(x1, w->ffn_norm, norm, T, D, dm->rms_eps, bf, stream));
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
  const size_t c = tg_topk_select_workspace_size(B, T_in, INT_MAX);
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
  st = tg_topk_select(s, keep_mask, d_cu_in, d_cu_kept, B, T_in, T, max_n, kept_idx, d_status,
                      ws, ws_bytes, stream);
  if (st != TG_OK) return st;
  st = tg_compact(h, pos, s, kept_idx, d_cu_in, d_cu_kept, B, T, dm->D, dm->dtype, x, pos_c, s_c,
                  stream);
  if (st != TG_OK) return st;
  return tg_upper_layer_stack_fwd(layers, n_layers, dm, x, pos_c, s_c, d_cu_kept, B, T, max_k,
                                  kcache, vcache, ws, ws_bytes, stream);
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
