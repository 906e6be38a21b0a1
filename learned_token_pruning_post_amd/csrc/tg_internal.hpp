// Internal launchers of libtokengate (host side). Every launcher enqueues on
// `stream`, assumes validated arguments, and returns hipGetLastError().
#pragma once
#include <atomic>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "tg_common.hpp"

namespace tg {

// Raise a kernel's dynamic-LDS limit to `bytes`, once per device (the limit
// is a per-device function attribute; later calls on that device skip it).
template <auto Kernel>
hipError_t ensure_dynamic_lds(int bytes) {
  static std::atomic<bool> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const bool slot = dev >= 0 && dev < 64;
  if (slot && done[dev].load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && slot) done[dev].store(true, std::memory_order_relaxed);
  return e;
}

// Compute units of the current device, cached per device (idempotent: a race
// only repeats the query); 256 if the query fails.
inline int device_cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (slot) cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Top-K selection with forced keep (and, with h_out, the compaction of the
// kept rows in the same pass). Supported for max_n up to 1M tokens per sequence.
bool select_supported(int max_n);
size_t select_workspace_bytes(int B, int64_t T_in, int max_n);
size_t select_workspace_bound(int B, int64_t T_in);  // over every max_n <= T_in
hipError_t launch_select_compact(const float* s, const uint8_t* mask, const int32_t* cu_in,
                                 const int32_t* cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                                 int32_t* kept, int32_t* status, void* ws, const void* h,
                                 const int32_t* pos, size_t row_bytes, void* h_out,
                                 int32_t* pos_out, float* s_out, hipStream_t stream);

hipError_t launch_compact(const void* h, const int32_t* pos, const float* s, const int32_t* kept,
                          const int32_t* cu_in, const int32_t* cu_kept, int B, int64_t T,
                          size_t row_bytes, void* h_out, int32_t* pos_out, float* s_out,
                          hipStream_t stream);

// RMSNorm rows: y = x * rsqrt(mean(x^2) + eps) * w  (is_bf16 selects the storage type)
hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int D, float eps,
                          bool is_bf16, hipStream_t stream);

// fused RMSNorm: ssq[r, s] = sum of x[r, 64s .. 64s+63]^2 (bf16 x, fp32 ssq, D % 64 == 0)
hipError_t launch_row_ssq(const void* x, float* ssq, int64_t rows, int D, hipStream_t stream);

// W[r, c] *= w[c] (fp32 product, rounded to the storage type)
hipError_t launch_fold_norm(const void* w, void* W, int64_t rows, int cols, bool is_bf16,
                            hipStream_t stream);

// p[i] = v for i < n
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);

// cos/sin table [T, d] fp32: [.., i] = cos(pos*base^(-2i/d)), [.., d/2 + i] = sin(..)
hipError_t launch_rope_table(const int32_t* pos, int64_t T, int d, float base, float* table,
                             hipStream_t stream);

// ---- bf16 MFMA GEMMs: out = f(W x) with W rows as output features ----
struct QkvOut {
  bf16* q;        // [M, Hq*d]
  bf16* kc;       // [M, Hkv*d]
  bf16* vc;       // [M, Hkv*d]
  const float* rope;  // [M, d]
  int Hq, Hkv, d;
};

// Fused RMSNorm (all optional, NULL = off): ssq_out [M][N/64] receives the row
// sums of squares of the stored output (PLAIN); with ssq_in [M][K/64] the QKV and
// SwiGLU products of row m are scaled by rsqrt(sum(ssq_in[m]) / K + eps).
hipError_t gemm_bf16_plain(const bf16* X, const bf16* W, const bf16* resid, bf16* out, int M,
                           int N, int K, hipStream_t stream, float* ssq_out = nullptr);
hipError_t gemm_bf16_qkv(const bf16* X, const bf16* wq, const bf16* wk, const bf16* wv,
                         const QkvOut& o, int M, int K, hipStream_t stream,
                         const float* ssq_in = nullptr, float eps = 0.f);
hipError_t gemm_bf16_swiglu(const bf16* X, const bf16* wg, const bf16* wu, bf16* act, int M,
                            int I, int K, hipStream_t stream, const float* ssq_in = nullptr,
                            float eps = 0.f);
// scorer; partial [nblk, M] fp32 scratch needed when H1 > 256 (nblk = ceil(H1/256))
hipError_t gemm_bf16_score(const bf16* X, const bf16* W1, const bf16* b1, const bf16* w2,
                           const bf16* b2, float* s_out, float* partial, int M, int H1, int K,
                           hipStream_t stream);
size_t gemm_bf16_score_ws(int64_t M, int H1);

// ---- fp32 SIMT path ----
hipError_t gemm_f32(const float* X, const float* W, const float* resid, float* out, int M, int N,
                    int K, int ldo, hipStream_t stream);
hipError_t score_epilogue_f32(const float* z, const float* b1, const float* w2, const float* b2,
                              float* s_out, int64_t M, int H1, hipStream_t stream);
hipError_t qkv_split_rope_f32(const float* qkv, const float* rope, float* q, float* kc, float* vc,
                              int64_t M, int Hq, int Hkv, int d, hipStream_t stream);
hipError_t swiglu_f32(const float* gate, const float* up, float* act, int64_t n,
                      hipStream_t stream);

// ---- attention ----
hipError_t attn_fwd(const void* q, const void* k, const void* v, const float* s_c, const float* t,
                    const float* g, const int32_t* cu_kept, int B, int max_k, int Hq, int Hkv,
                    int d, bool is_bf16, void* o, float* lse, hipStream_t stream);

// ---- decode attention over the pruned cache (two segments per sequence) ----
bool decode_supported(int Hq, int Hkv, int d);
size_t decode_workspace_bytes(int B, int max_len, int Hq, int Hkv, int d);
hipError_t launch_decode_attn(const void* q, const void* kA, const void* vA, const float* sA,
                              const int32_t* cuA, const void* kB, const void* vB, const float* sB,
                              const int32_t* lenB, int capB, const float* t, const float* g, int B,
                              int max_len, int Hq, int Hkv, int d, bool is_bf16, void* o, float* lse,
                              int32_t* status, void* ws, hipStream_t stream);

// ---- backward of the gated attention (bf16; d in {64, 128}, Hq / Hkv in {1, 2, 4}) ----
bool attn_bwd_supported(int Hq, int Hkv, int d);
size_t attn_bwd_workspace_bytes(int B, int64_t T, int max_k, int Hq, int Hkv, int d);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* s_c, const float* t,
                           const float* g, const int32_t* cu, int B, int64_t T, int max_k, int Hq, int Hkv,
                           int d, const void* o, const float* lse, const void* dO, float* dq, float* dk,
                           float* dv, float* ds, float* dt, float* dg, void* ws, hipStream_t stream);

// ---- backward of the scorer (bf16; D % 64 == 0, H1 % 64 == 0) and of the compaction ----
size_t score_bwd_workspace_bytes(int64_t T, int D, int H1);
hipError_t launch_score_bwd(const void* h, int64_t T, int D, int H1, const void* W1, const void* b1,
                            const void* w2, const float* s, const float* ds, void* dh, float* dW1,
                            float* db1, float* dw2, float* db2, void* ws, hipStream_t stream);
// ds[kept[r]] = ds_c[r] for r < T, every other ds[i] (i < T_in) = 0
hipError_t launch_scatter_scores(const float* ds_c, const int32_t* kept, int64_t T, int64_t T_in, float* ds,
                                 hipStream_t stream);

// ---- Gated DeltaNet mixer (dk in {64, 128}, dv % 32 == 0) ----
bool gdn_supported(int dk, int dv);
hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                      const int32_t* cu, int B, int H, int dk, int dv, bool is_bf16, const float* state_in,
                      void* o, float* state_out, hipStream_t stream);
// chunked form for bf16 (matrix cores): workspace of chunk records
size_t gdn_chunk_workspace_bytes(int64_t T, int B, int H, int dk, int dv);
hipError_t launch_gdn_chunked(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                              const int32_t* cu, int64_t T, int B, int H, int dk, int dv, const float* state_in,
                              void* o, float* state_out, void* ws, hipStream_t stream);

}  // namespace tg
