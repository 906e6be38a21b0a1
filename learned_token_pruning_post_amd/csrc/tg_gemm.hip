// Dense projections of the gated path on CDNA4 matrix cores.
//
// out[m, n] = f( sum_k W[n, k] * X[m, k] ): weights in nn.Linear layout
// [out_features, in_features], activations row-major [tokens, features]; both
// operands are K-contiguous. The weight tile is the MFMA A operand and the
// token tile the B operand, so every lane ends with 4 consecutive output
// features of one token and stores 8 bytes at a time.
//
// Tiling: BK = 64; each wave owns a 64 (features) x 128 (tokens) tile made of
// 2 x 4 MFMA 32x32x16 bf16 blocks (128 fp32 accumulators per lane). A
// workgroup is WN x WM waves. Tiles are staged global -> registers -> LDS
// (double buffer, one barrier per k-step; the next tile's global loads are in
// flight while the current one feeds the MFMAs). LDS rows are 128 B with the
// 16-byte chunk index XOR-swizzled by (row & 7) so the 16-byte fragment reads
// of 8 consecutive rows hit distinct banks.
//
// Epilogues, fused on the accumulators:
//   PLAIN  : out = acc (+ residual)                         (O and down proj)
//   QKV    : rotate-half RoPE of q and k, scatter to q / k-cache / v-cache.
//            Weight rows are loaded permuted so each lane holds both halves
//            (i, i + d/2) of its rotary pairs.
//   SWIGLU : gate and up rows interleaved per 32 -> silu(g) * u
//   SCORE  : scorer logit: sum_n GELU(acc + b1[n]) * w2[n], then sigmoid
//            (the [tokens, H1] activations never reach memory)
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

enum { MODE_PLAIN = 0, MODE_QKV = 1, MODE_SWIGLU = 2, MODE_SCORE = 3 };

struct GemmParams {
  const bf16* X;
  int M, N, K;
  const bf16* W0;
  const bf16* W1;
  const bf16* W2;
  // PLAIN
  const bf16* resid;
  bf16* out;
  // QKV
  bf16* q;
  bf16* kc;
  bf16* vc;
  const float* rope;
  int Hq, Hkv, hd;
  // SWIGLU
  bf16* act;
  int I;
  // SCORE
  const bf16* b1;
  const bf16* w2;
  const bf16* b2;
  float* s_out;
  float* partial;
};

template <int MODE>
__device__ __forceinline__ const bf16* weight_row(const GemmParams& p, int n0, int ln) {
  if (MODE == MODE_PLAIN || MODE == MODE_SCORE) {
    const int gn = n0 + ln;
    return gn < p.N ? p.W0 + (size_t)gn * p.K : nullptr;
  } else if (MODE == MODE_QKV) {
    int gn;
    if (p.hd == 128) {
      const int c = ln & 127;
      const int perm = (((c >> 5) & 1) << 6) | (((c >> 6) & 1) << 5) | (c & 31);
      gn = n0 + (ln & ~127) + perm;
    } else {
      gn = n0 + ln;
    }
    const int nq = p.Hq * p.hd, nk = p.Hkv * p.hd;
    if (gn < nq) return p.W0 + (size_t)gn * p.K;
    if (gn < nq + nk) return p.W1 + (size_t)(gn - nq) * p.K;
    if (gn < nq + 2 * nk) return p.W2 + (size_t)(gn - nq - nk) * p.K;
    return nullptr;
  } else {  // SWIGLU
    const int idx = (n0 >> 1) + (ln >> 6) * 32 + (ln & 31);
    if (idx >= p.I) return nullptr;
    return (((ln >> 5) & 1) ? p.W1 : p.W0) + (size_t)idx * p.K;
  }
}

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ void store_bf16x4(bf16* dst, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = f2bf(a);
  v[1] = f2bf(b);
  v[2] = f2bf(c);
  v[3] = f2bf(d);
  *reinterpret_cast<bf16x4*>(dst) = v;
}

template <int MODE, int WN, int WM>
__global__ __launch_bounds__(WN* WM * 64) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WN * WM * 64;
  constexpr int BN = WN * 64;
  constexpr int BM = WM * 128;
  constexpr int WCH = BN * 8 / NT;  // 16-byte chunks of the W tile per thread
  constexpr int XCH = BM * 8 / NT;
  constexpr int STAGE = (BN + BM) * 64;  // bf16 elements per stage

  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;
  const int wm = wave / WN;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int K = p.K;

  // per-thread global source rows (fixed across k-steps)
  const bf16* wsrc[WCH];
  const bf16* xsrc[XCH];
  int wdst[WCH], xdst[XCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + i * NT;
    const int row = c >> 3, kc = c & 7;
    const bf16* r = weight_row<MODE>(p, n0, row);
    wsrc[i] = r ? r + kc * 8 : nullptr;
    wdst[i] = row * 64 + ((kc ^ (row & 7)) << 3);
  }
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + i * NT;
    const int row = c >> 3, kc = c & 7;
    const int gm = m0 + row;
    xsrc[i] = gm < p.M ? p.X + (size_t)gm * K + kc * 8 : nullptr;
    xdst[i] = BN * 64 + row * 64 + ((kc ^ (row & 7)) << 3);
  }

  uint4 wreg[WCH], xreg[XCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < WCH; ++i)
      wreg[i] = wsrc[i] ? *reinterpret_cast<const uint4*>(wsrc[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      xreg[i] = xsrc[i] ? *reinterpret_cast<const uint4*>(xsrc[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int stage) {
    bf16* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < WCH; ++i) *reinterpret_cast<uint4*>(base + wdst[i]) = wreg[i];
#pragma unroll
    for (int i = 0; i < XCH; ++i) *reinterpret_cast<uint4*>(base + xdst[i]) = xreg[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = zero_f32x16();

  // fragment read offsets (elements) inside a stage
  const int half = lane >> 5;
  int woff[2], xoff[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wn * 64 + j * 32 + (lane & 31);
    woff[j] = row * 64;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32 + (lane & 31);
    xoff[i] = BN * 64 + row * 64;
  }
  const int rsw = lane & 7;  // (row & 7) is lane & 7 for every fragment row

  const int KT = K / 64;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload((kt + 1) * 64);
    const bf16* base = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = ((ks * 2 + half) ^ rsw) << 3;
      bf16x8 wf[2], xf[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) wf[j] = *reinterpret_cast<const bf16x8*>(base + woff[j] + ch);
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[i] = *reinterpret_cast<const bf16x8*>(base + xoff[i] + ch);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mfma32(wf[j], xf[i], acc[j][i]);
    }
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---------------- epilogues ----------------
  const int ml = lane & 31;
  if (MODE == MODE_PLAIN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + i * 32 + ml;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + wn * 64 + j * 32 + rq * 8 + half * 4;
          if (n >= p.N) continue;
          float v0 = acc[j][i][rq * 4 + 0], v1 = acc[j][i][rq * 4 + 1];
          float v2 = acc[j][i][rq * 4 + 2], v3 = acc[j][i][rq * 4 + 3];
          const size_t o = (size_t)m * p.N + n;
          if (p.resid) {
            const bf16x4 r = *reinterpret_cast<const bf16x4*>(p.resid + o);
            v0 += bf2f(r[0]);
            v1 += bf2f(r[1]);
            v2 += bf2f(r[2]);
            v3 += bf2f(r[3]);
          }
          store_bf16x4(p.out + o, v0, v1, v2, v3);
        }
    }
  } else if (MODE == MODE_QKV) {
    const int hd = p.hd, hh = hd >> 1;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      // global column of the j = 0 element (the j = 1 partner is + d/2)
      const int e = rq * 8 + half * 4;
      int gn0;
      if (hd == 128) {
        const int c = (wn * 64 + e) & 127;  // j = 0 -> bit 5 clear
        const int perm = (((c >> 6) & 1) << 5) | (c & 31);
        gn0 = n0 + ((wn * 64) & ~127) + perm;
      } else {
        gn0 = n0 + wn * 64 + e;
      }
      const int gh = gn0 / hd;
      const int dim = gn0 - gh * hd;  // < d/2
      if (gh >= p.Hq + 2 * p.Hkv) continue;
      const bool rot = gh < p.Hq + p.Hkv;
      bf16* dst;
      int ld;
      if (gh < p.Hq) {
        dst = p.q + gh * hd + dim;
        ld = p.Hq * hd;
      } else if (gh < p.Hq + p.Hkv) {
        dst = p.kc + (gh - p.Hq) * hd + dim;
        ld = p.Hkv * hd;
      } else {
        dst = p.vc + (gh - p.Hq - p.Hkv) * hd + dim;
        ld = p.Hkv * hd;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + ml;
        if (m >= p.M) continue;
        float y0[4], y1[4];
        if (rot) {
          const f32x4 cs = *reinterpret_cast<const f32x4*>(p.rope + (size_t)m * hd + dim);
          const f32x4 sn = *reinterpret_cast<const f32x4*>(p.rope + (size_t)m * hd + hh + dim);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float x0 = acc[0][i][rq * 4 + t], x1 = acc[1][i][rq * 4 + t];
            y0[t] = x0 * cs[t] - x1 * sn[t];
            y1[t] = x1 * cs[t] + x0 * sn[t];
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            y0[t] = acc[0][i][rq * 4 + t];
            y1[t] = acc[1][i][rq * 4 + t];
          }
        }
        bf16* row = dst + (size_t)m * ld;
        store_bf16x4(row, y0[0], y0[1], y0[2], y0[3]);
        store_bf16x4(row + hh, y1[0], y1[1], y1[2], y1[3]);
      }
    }
  } else if (MODE == MODE_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + i * 32 + ml;
      if (m >= p.M) continue;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int idx = (n0 >> 1) + wn * 32 + rq * 8 + half * 4;
        if (idx >= p.I) continue;
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float gt = acc[0][i][rq * 4 + t], up = acc[1][i][rq * 4 + t];
          y[t] = gt / (1.0f + __expf(-gt)) * up;
        }
        store_bf16x4(p.act + (size_t)m * p.I + idx, y[0], y[1], y[2], y[3]);
      }
    }
  } else {  // SCORE
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int n = n0 + wn * 64 + j * 32 + rq * 8 + half * 4 + t;
          if (n < p.N) {
            const float bb = bf2f(p.b1[n]), ww = bf2f(p.w2[n]);
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i] += gelu_erf(acc[j][i][rq * 4 + t] + bb) * ww;
          }
        }
    float* red = reinterpret_cast<float*>(smem);  // pipeline buffers are free now
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[i] += __shfl_xor(part[i], 32, 64);
      if (half == 0) red[wn * BM + wm * 128 + i * 32 + ml] = part[i];
    }
    __syncthreads();
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      if (m >= p.M) continue;
      float u = 0.f;
#pragma unroll
      for (int w = 0; w < WN; ++w) u += red[w * BM + r];
      if (gridDim.x == 1) {
        u += bf2f(p.b2[0]);
        p.s_out[m] = 1.0f / (1.0f + expf(-u));
      } else {
        p.partial[(size_t)blockIdx.x * p.M + m] = u;
      }
    }
  }
}

__global__ void score_finish_kernel(const float* __restrict__ partial, int nblk, int64_t M,
                                    const bf16* __restrict__ b2, float* __restrict__ s_out) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  float u = 0.f;
  for (int b = 0; b < nblk; ++b) u += partial[(size_t)b * M + m];
  u += bf2f(b2[0]);
  s_out[m] = 1.0f / (1.0f + expf(-u));
}

template <int MODE, int WN, int WM>
static hipError_t launch_gemm(const GemmParams& p, int Ncols, hipStream_t stream) {
  constexpr int BN = WN * 64, BM = WM * 128;
  constexpr size_t lds = (size_t)2 * (BN + BM) * 64 * sizeof(bf16);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<MODE, WN, WM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((Ncols + BN - 1) / BN, (p.M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, WN, WM>), grid, dim3(WN * WM * 64), lds, stream, p);
  return hipGetLastError();
}

// config choice: the biggest tile that still gives >= 256 workgroups (one per CU)
template <int MODE>
static hipError_t launch_auto(const GemmParams& p, int Ncols, hipStream_t stream) {
  const long tA = (long)((Ncols + 255) / 256) * ((p.M + 255) / 256);
  const long tC = (long)((Ncols + 255) / 256) * ((p.M + 127) / 128);
  if (tA >= 256) return launch_gemm<MODE, 4, 2>(p, Ncols, stream);
  if (tC >= 256) return launch_gemm<MODE, 4, 1>(p, Ncols, stream);
  return launch_gemm<MODE, 2, 1>(p, Ncols, stream);
}

hipError_t gemm_bf16_plain(const bf16* X, const bf16* W, const bf16* resid, bf16* out, int M,
                           int N, int K, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  GemmParams p{};
  p.X = X;
  p.M = M;
  p.N = N;
  p.K = K;
  p.W0 = W;
  p.resid = resid;
  p.out = out;
  return launch_auto<MODE_PLAIN>(p, N, stream);
}

hipError_t gemm_bf16_qkv(const bf16* X, const bf16* wq, const bf16* wk, const bf16* wv,
                         const QkvOut& o, int M, int K, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  GemmParams p{};
  p.X = X;
  p.M = M;
  p.N = (o.Hq + 2 * o.Hkv) * o.d;
  p.K = K;
  p.W0 = wq;
  p.W1 = wk;
  p.W2 = wv;
  p.q = o.q;
  p.kc = o.kc;
  p.vc = o.vc;
  p.rope = o.rope;
  p.Hq = o.Hq;
  p.Hkv = o.Hkv;
  p.hd = o.d;
  return launch_auto<MODE_QKV>(p, p.N, stream);
}

hipError_t gemm_bf16_swiglu(const bf16* X, const bf16* wg, const bf16* wu, bf16* act, int M,
                            int I, int K, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  GemmParams p{};
  p.X = X;
  p.M = M;
  p.N = 2 * I;
  p.K = K;
  p.W0 = wg;
  p.W1 = wu;
  p.act = act;
  p.I = I;
  return launch_auto<MODE_SWIGLU>(p, 2 * I, stream);
}

size_t gemm_bf16_score_ws(int64_t M, int H1) {
  const int nblk = (H1 + 255) / 256;
  return nblk > 1 ? (size_t)nblk * (size_t)M * sizeof(float) : 0;
}

hipError_t gemm_bf16_score(const bf16* X, const bf16* W1, const bf16* b1, const bf16* w2,
                           const bf16* b2, float* s_out, float* partial, int M, int H1, int K,
                           hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  GemmParams p{};
  p.X = X;
  p.M = M;
  p.N = H1;
  p.K = K;
  p.W0 = W1;
  p.b1 = b1;
  p.w2 = w2;
  p.b2 = b2;
  p.s_out = s_out;
  p.partial = partial;
  const int nblk = (H1 + 255) / 256;
  hipError_t e;
  if ((long)((M + 255) / 256) * nblk >= 256)
    e = launch_gemm<MODE_SCORE, 4, 2>(p, H1, stream);
  else
    e = launch_gemm<MODE_SCORE, 4, 1>(p, H1, stream);
  if (e != hipSuccess || nblk == 1) return e;
  hipLaunchKernelGGL(score_finish_kernel, dim3((M + 255) / 256), dim3(256), 0, stream,
                     (const float*)partial, nblk, (int64_t)M, b2, s_out);
  return hipGetLastError();
}

// ===========================================================================
// fp32 SIMT path (the fp32 configurations): 64x64 tiles, 16x16 threads,
// 4x4 outputs each, BK = 16 staged in LDS.
// ===========================================================================
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W,
                                                       const float* __restrict__ R,
                                                       float* __restrict__ out, int M, int N,
                                                       int K, int ldo) {
  __shared__ float xs[16][64 + 4];
  __shared__ float ws[16][64 + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int r = e >> 4, c = e & 15;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      xs[c][r] = (gm < M && gk < K) ? X[(size_t)gm * K + gk] : 0.f;
      ws[c][r] = (gn < N && gk < K) ? W[(size_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j];
      if (R) v += R[(size_t)m * ldo + n];
      out[(size_t)m * ldo + n] = v;
    }
  }
}

hipError_t gemm_f32(const float* X, const float* W, const float* resid, float* out, int M, int N,
                    int K, int ldo, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, stream, X, W, resid, out, M, N, K, ldo);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void score_epi_f32_kernel(const float* __restrict__ z,
                                                            const float* __restrict__ b1,
                                                            const float* __restrict__ w2,
                                                            const float* __restrict__ b2,
                                                            float* __restrict__ s, int64_t M,
                                                            int H1) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  float u = 0.f;
  for (int n = lane; n < H1; n += 64) u += gelu_erf(z[m * H1 + n] + b1[n]) * w2[n];
  u = wave_sum(u);
  if (lane == 0) s[m] = 1.0f / (1.0f + expf(-(u + b2[0])));
}

hipError_t score_epilogue_f32(const float* z, const float* b1, const float* w2, const float* b2,
                              float* s_out, int64_t M, int H1, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(score_epi_f32_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream,
                     z, b1, w2, b2, s_out, M, H1);
  return hipGetLastError();
}

__global__ void qkv_split_rope_f32_kernel(const float* __restrict__ qkv,
                                          const float* __restrict__ rope, float* __restrict__ q,
                                          float* __restrict__ kc, float* __restrict__ vc,
                                          int64_t M, int Hq, int Hkv, int d) {
  const int hh = d >> 1;
  const int H = Hq + 2 * Hkv;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * H * hh) return;
  const int i = (int)(idx % hh);
  const int h = (int)((idx / hh) % H);
  const int64_t m = idx / ((int64_t)hh * H);
  const float* src = qkv + (m * H + h) * d;
  float a = src[i], b = src[i + hh];
  float* dst;
  if (h < Hq) {
    dst = q + (m * Hq + h) * d;
  } else if (h < Hq + Hkv) {
    dst = kc + (m * Hkv + (h - Hq)) * d;
  } else {
    dst = vc + (m * Hkv + (h - Hq - Hkv)) * d;
  }
  if (h < Hq + Hkv) {
    const float c = rope[m * d + i], s = rope[m * d + hh + i];
    const float a2 = a * c - b * s, b2 = b * c + a * s;
    a = a2;
    b = b2;
  }
  dst[i] = a;
  dst[i + hh] = b;
}

hipError_t qkv_split_rope_f32(const float* qkv, const float* rope, float* q, float* kc, float* vc,
                              int64_t M, int Hq, int Hkv, int d, hipStream_t stream) {
  const int64_t n = M * (Hq + 2 * Hkv) * (d / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_split_rope_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, qkv, rope, q, kc, vc, M, Hq, Hkv, d);
  return hipGetLastError();
}

__global__ void swiglu_f32_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                  float* __restrict__ a, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float x = g[i];
  a[i] = x / (1.0f + expf(-x)) * u[i];
}

hipError_t swiglu_f32(const float* gate, const float* up, float* act, int64_t n,
                      hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     gate, up, act, n);
  return hipGetLastError();
}

}  // namespace tg
