// Row-parallel HBM-bound kernels: compaction gather, RMSNorm, RoPE table.
#include <algorithm>

#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

// ---------------------------------------------------------------------------
// Compaction: h_out[k] = h[kept[k]], pos_out[k] = pos[kept[k]] (or the local
// index), s_out[k] = s[kept[k]]. Only kept tokens continue above the gate
// (Tencent Cloud TokenGate article, early token filtering). One wave moves
// one row per step with 16-byte loads, all loads of a row in flight before
// its stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int seq_of_slot(const int32_t* cu, int B, int64_t row) {
  int lo = 0, hi = B;  // find b with cu[b] <= row < cu[b+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <bool VEC>
__global__ __launch_bounds__(256) void compact_kernel(
    const uint8_t* __restrict__ h, const int32_t* __restrict__ pos, const float* __restrict__ s,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ cu_in,
    const int32_t* __restrict__ cu_kept, int B, int64_t T, size_t row_bytes,
    uint8_t* __restrict__ h_out, int32_t* __restrict__ pos_out, float* __restrict__ s_out) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < T; row += stride) {
    const int src = kept[row];
    uint8_t* dp = h_out + (size_t)row * row_bytes;
    if (src < 0 || (cu_in && src >= cu_in[B])) {  // slot of a sequence the selection rejected
      for (size_t c = lane; c < row_bytes / 2; c += 64) reinterpret_cast<uint16_t*>(dp)[c] = 0;
      if (lane == 0) {
        pos_out[row] = -1;
        if (s_out) s_out[row] = 0.f;
      }
      continue;
    }
    const uint8_t* sp = h + (size_t)src * row_bytes;
    if (VEC) {
      const u32x4* sv = reinterpret_cast<const u32x4*>(sp);
      u32x4* dv = reinterpret_cast<u32x4*>(dp);
      const int nvec = (int)(row_bytes >> 4);
      int c = lane;
      for (; c + 192 < nvec; c += 256) {
        u32x4 a0 = __builtin_nontemporal_load(sv + c);
        u32x4 a1 = __builtin_nontemporal_load(sv + c + 64);
        u32x4 a2 = __builtin_nontemporal_load(sv + c + 128);
        u32x4 a3 = __builtin_nontemporal_load(sv + c + 192);
        __builtin_nontemporal_store(a0, dv + c);
        __builtin_nontemporal_store(a1, dv + c + 64);
        __builtin_nontemporal_store(a2, dv + c + 128);
        __builtin_nontemporal_store(a3, dv + c + 192);
      }
      for (; c < nvec; c += 64) dv[c] = sv[c];
    } else {
      const uint16_t* sv = reinterpret_cast<const uint16_t*>(sp);
      uint16_t* dv = reinterpret_cast<uint16_t*>(dp);
      const int ne = (int)(row_bytes >> 1);
      for (int c = lane; c < ne; c += 64) dv[c] = sv[c];
    }
    if (lane == 0) {
      int p;
      if (pos) {
        p = pos[src];
      } else {
        const int b = seq_of_slot(cu_kept, B, row);
        p = src - cu_in[b];
      }
      pos_out[row] = p;
      if (s_out) s_out[row] = s[src];
    }
  }
}

hipError_t launch_compact(const void* h, const int32_t* pos, const float* s, const int32_t* kept,
                          const int32_t* cu_in, const int32_t* cu_kept, int B, int64_t T,
                          size_t row_bytes, void* h_out, int32_t* pos_out, float* s_out,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  int64_t blocks = (T + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  const bool vec = (row_bytes % 16 == 0) && ((uintptr_t)h % 16 == 0) && ((uintptr_t)h_out % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(compact_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)h, pos, s, kept, cu_in, cu_kept, B, T, row_bytes,
                       (uint8_t*)h_out, pos_out, s_out);
  else
    hipLaunchKernelGGL(compact_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)h, pos, s, kept, cu_in, cu_kept, B, T, row_bytes,
                       (uint8_t*)h_out, pos_out, s_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm (pre-norm of the Qwen3-shaped layer): y = x * rsqrt(mean x^2 + eps) * w,
// one wave per row, fp32 statistics.
// ---------------------------------------------------------------------------
// Wave-wide float sum on DPP lane moves (VALU; no LDS round trip): row_shr
// 1, 2, 4, 8 sum each 16-lane row, row_bcast 15 / 31 carry the row totals,
// lane 63 ends with the total.
__device__ __forceinline__ float wave_sum_dpp(float x) {
#define TG_DPP_ADD(ctrl, rmask)                                                                 \
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xf, false))
  TG_DPP_ADD(0x111, 0xf);
  TG_DPP_ADD(0x112, 0xf);
  TG_DPP_ADD(0x114, 0xf);
  TG_DPP_ADD(0x118, 0xf);
  TG_DPP_ADD(0x142, 0xa);
  TG_DPP_ADD(0x143, 0xc);
#undef TG_DPP_ADD
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// One wave per row; the row (NVL 16-byte vectors per lane) stays in
// registers between the sum of squares and the scaling, so x is read once.
template <int NVL>
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const bf16* __restrict__ x,
                                                           const bf16* __restrict__ w,
                                                           bf16* __restrict__ y, int64_t rows,
                                                           int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bf16x8* xr = reinterpret_cast<const bf16x8*>(x + row * D);
  const bf16x8* wr = reinterpret_cast<const bf16x8*>(w);
  bf16x8* yr = reinterpret_cast<bf16x8*>(y + row * D);
  const int nv = D >> 3;
  bf16x8 v[NVL];
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) v[i] = xr[c];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NVL; ++i)
    if (lane + 64 * i < nv)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = bf2f(v[i][e]);
        ss += f * f;
      }
  ss = wave_sum_dpp(ss);
  const float r = rsqrtf(ss / (float)D + eps);
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      const bf16x8 ww = wr[c];
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f2bf(bf2f(v[i][e]) * r * bf2f(ww[e]));
      yr[c] = o;
    }
  }
}

// rows wider than the register budget: two passes over the row
__global__ __launch_bounds__(256) void rmsnorm_bf16_wide_kernel(const bf16* __restrict__ x,
                                                                const bf16* __restrict__ w,
                                                                bf16* __restrict__ y, int64_t rows,
                                                                int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bf16x8* xr = reinterpret_cast<const bf16x8*>(x + row * D);
  const bf16x8* wr = reinterpret_cast<const bf16x8*>(w);
  bf16x8* yr = reinterpret_cast<bf16x8*>(y + row * D);
  const int nv = D >> 3;
  float ss = 0.f;
  for (int c = lane; c < nv; c += 64) {
    bf16x8 v = xr[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f = bf2f(v[e]);
      ss += f * f;
    }
  }
  ss = wave_sum_dpp(ss);
  const float r = rsqrtf(ss / (float)D + eps);
  for (int c = lane; c < nv; c += 64) {
    bf16x8 v = xr[c], ww = wr[c], o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f2bf(bf2f(v[e]) * r * bf2f(ww[e]));
    yr[c] = o;
  }
}

__global__ __launch_bounds__(256) void rmsnorm_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ y, int64_t rows,
                                                          int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * D;
  float* yr = y + row * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss += xr[c] * xr[c];
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  for (int c = lane; c < D; c += 64) yr[c] = xr[c] * r * w[c];
}

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int D, float eps,
                          bool is_bf16, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
  const int nvl = ((D >> 3) + 63) / 64;  // 16-byte vectors per lane
  if (is_bf16 && nvl <= 4)
    hipLaunchKernelGGL(rmsnorm_bf16_kernel<4>, grid, dim3(256), 0, stream, (const bf16*)x,
                       (const bf16*)w, (bf16*)y, rows, D, eps);
  else if (is_bf16 && nvl <= 8)
    hipLaunchKernelGGL(rmsnorm_bf16_kernel<8>, grid, dim3(256), 0, stream, (const bf16*)x,
                       (const bf16*)w, (bf16*)y, rows, D, eps);
  else if (is_bf16)
    hipLaunchKernelGGL(rmsnorm_bf16_wide_kernel, grid, dim3(256), 0, stream, (const bf16*)x,
                       (const bf16*)w, (bf16*)y, rows, D, eps);
  else
    hipLaunchKernelGGL(rmsnorm_f32_kernel, grid, dim3(256), 0, stream, (const float*)x,
                       (const float*)w, (float*)y, rows, D, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RoPE angle table at the kept tokens' original positions. The angle
// pos * base^(-2i/d) reaches 1.3e5 rad at 128K positions, where an fp32
// product would already be off by ~1e-2 rad, so angles and sincos run in
// fp64 and only the results are rounded to fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ pos,
                                                         int64_t T, int d, double base,
                                                         float* __restrict__ table) {
  const int half = d >> 1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * half) return;
  const int64_t t = idx / half;
  const int i = (int)(idx - t * half);
  const double inv = pow(base, -2.0 * (double)i / (double)d);
  const double th = (double)pos[t] * inv;
  double sn, cs;
  sincos(th, &sn, &cs);
  table[t * d + i] = (float)cs;
  table[t * d + half + i] = (float)sn;
}

hipError_t launch_rope_table(const int32_t* pos, int64_t T, int d, float base, float* table,
                             hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t n = T * (d / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     pos, T, d, (double)base, table);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row sums of squares for the fused RMSNorm: ssq[r, s] = sum of x[r, c]^2
// over the 64 features c = 64s..64s+63 (fp32), one thread per (row, slot):
// consecutive threads read consecutive 128-byte segments of a row. The sum
// is taken in the order of the GEMM epilogue that writes the same values for
// the layer's later rows (8-feature fma chains, then pairwise), so a layer
// reading sums from either source computes bit-identical results.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void row_ssq_bf16_kernel(const bf16* __restrict__ x,
                                                           float* __restrict__ ssq, int64_t rows,
                                                           int nslot) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * nslot) return;
  const bf16x8* src = reinterpret_cast<const bf16x8*>(x) + idx * 8;
  bf16x8 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = src[i];
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf2f(v[i][e]);
      c[i] = fmaf(f, f, c[i]);
    }
  }
  ssq[idx] = ((c[7] + c[6]) + (c[5] + c[4])) + ((c[3] + c[2]) + (c[1] + c[0]));
}

hipError_t launch_row_ssq(const void* x, float* ssq, int64_t rows, int D, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int nslot = D / 64;
  const int64_t n = rows * nslot;
  hipLaunchKernelGGL(row_ssq_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const bf16*)x, ssq, rows, nslot);
  return hipGetLastError();
}

// Norm-weight folding: W[r, c] *= w[c] in fp32, rounded to the storage type.
template <class T>
__global__ __launch_bounds__(256) void fold_norm_kernel(const T* __restrict__ w, T* __restrict__ W,
                                                        int64_t n, int cols) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % cols);
  if constexpr (sizeof(T) == 2)
    W[i] = f2bf(bf2f(W[i]) * bf2f(w[c]));
  else
    W[i] = W[i] * w[c];
}

hipError_t launch_fold_norm(const void* w, void* W, int64_t rows, int cols, bool is_bf16,
                            hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (is_bf16)
    hipLaunchKernelGGL(fold_norm_kernel<bf16>, grid, dim3(256), 0, stream, (const bf16*)w, (bf16*)W,
                       n, cols);
  else
    hipLaunchKernelGGL(fold_norm_kernel<float>, grid, dim3(256), 0, stream, (const float*)w,
                       (float*)W, n, cols);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// p[i] = v for i < n (workspace constants; a kernel, so it captures into a graph)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// gradient of the prompt scores through the compaction: zero, then scatter
__global__ void scatter_scores_kernel(const float* __restrict__ ds_c, const int32_t* __restrict__ kept, int64_t T,
                                      int64_t T_in, float* __restrict__ ds) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= T) return;
  const int32_t i = kept[r];
  if (i >= 0 && i < T_in) ds[i] = ds_c[r];  // -1 slots of a rejected sequence carry nothing
}

hipError_t launch_scatter_scores(const float* ds_c, const int32_t* kept, int64_t T, int64_t T_in, float* ds,
                                 hipStream_t stream) {
  hipError_t e = launch_fill_f32(ds, T_in, 0.f, stream);
  if (e != hipSuccess || T == 0) return e;
  scatter_scores_kernel<<<dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream>>>(ds_c, kept, T, T_in, ds);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace tg
