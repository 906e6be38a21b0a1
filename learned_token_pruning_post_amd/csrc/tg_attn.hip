// Token-gated causal GQA flash attention.
//
// Logit of query i, key j <= i, q-head h, kv-head h' = h / (Hq/Hkv):
//   L_ij = t_h * (q_i . k_j) / sqrt(d) + g_h * s_c[j]
// (the kept tokens' gate scores enter the upper layers' attention as a bias
// on each key's logit, with a learnable gain and temperature per head:
// Tencent Cloud TokenGate article, gradient-path and engineering sections;
// ai.866data article, mechanism-design section).
//
// bf16 kernel (gfx950 MFMA 32x32x16, fp32 accumulate):
//  * one workgroup = one kv-head, all G q-heads of its group, and a tile of
//    BQ = 128/G queries; 4 waves, each owning 32 queries of one q-head, so
//    each K/V tile staged in LDS serves every head of the group;
//  * S^T = K Q^T and O^T = V^T P^T: the 32x32 accumulator layout puts one
//    query per lane (column), so the row max / row sum are per lane plus one
//    exchange with lane ^ 32, and P goes from the S accumulator straight into
//    the B operand of the PV product without touching LDS (the k-slot order
//    of P is matched by a fixed permutation of keys in the transposed V tile);
//  * log2-domain online softmax: t_h*log2(e)/sqrt(d) is one multiply, the bias
//    g_h*log2(e)*s_c[j] is precomputed per key and head when the tile is
//    staged;
//  * K/V tiles of 64 keys double-buffered through registers -> LDS; K rows
//    XOR-swizzled, V stored transposed ([d][key]) with a swizzle that keeps
//    both the transposing writes and the fragment reads spread over banks;
//  * the heaviest (last) query tiles are dispatched first.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

__device__ __forceinline__ int vperm16(int p) {  // swap bits 2 and 3
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}
__device__ __forceinline__ int vswz(int dd) { return (dd ^ (dd >> 3)) & 7; }

template <int G, int HD>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ s_c, const float* __restrict__ t, const float* __restrict__ g,
    const int32_t* __restrict__ cu_kept, int B, int Hq, int Hkv, int n_qt, bf16* __restrict__ o,
    float* __restrict__ lse) {
  constexpr int WPH = 4 / G;     // waves per q-head
  constexpr int BQ = 32 * WPH;   // queries per workgroup
  constexpr int KCH = HD / 8;    // 16-byte chunks per K row
  constexpr int KSTAGE = 64 * HD;
  constexpr int VSTAGE = HD * 64;
  constexpr int NKL = HD / 32;   // K chunks loaded per thread
  constexpr int ND = HD / 32;    // 32-wide d blocks of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char attn_smem[];
  bf16* Ks = reinterpret_cast<bf16*>(attn_smem);
  bf16* Vs = Ks + 2 * KSTAGE;
  float* bias = reinterpret_cast<float*>(Vs + 2 * VSTAGE);  // [2][G][64]

  const int tid = threadIdx.x;
  const int L = blockIdx.x;
  const int per = Hkv * B;
  const int qt = n_qt - 1 - L / per;
  const int rem = L - (L / per) * per;
  const int hk = rem % Hkv, b = rem / Hkv;
  const int seq0 = cu_kept[b];
  const int Kb = cu_kept[b + 1] - seq0;
  const int q0 = qt * BQ;
  if (q0 >= Kb) return;
  const int Ttot = cu_kept[B];

  const int wave = tid >> 6, lane = tid & 63, l31 = lane & 31, half = lane >> 5;
  const int gi = wave / WPH, qs = wave % WPH;
  const int h = hk * G + gi;
  const int qw0 = q0 + qs * 32;
  const int qi = qw0 + l31;
  const bool qvalid = qi < Kb;
  const bool wave_any = qw0 < Kb;
  const int qend = min(Kb, q0 + BQ);
  const int n_kt = (qend + 63) >> 6;

  bf16x8 qf[HD / 16];
  {
    const bf16* qrow = q + ((size_t)(seq0 + qi) * Hq + h) * HD + half * 8;
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks)
      qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16) : zero_bf16x8();
  }
  const float cscale = t[h] * TG_LOG2E / sqrtf((float)HD);

  // ---- tile loader state ----
  uint4 kreg[NKL];
  bf16x8 vreg[4];
  float sreg = 0.f;
  const int vdc = tid % KCH, vkg = tid / KCH;
  const bool vloader = tid < KCH * 16;

  auto gload = [&](int kt) {
    const int kb0 = kt * 64;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int c = tid + i * 256;
      const int key = c / KCH, kc = c % KCH;
      const int gk = kb0 + key;
      kreg[i] = gk < Kb ? *reinterpret_cast<const uint4*>(
                              k + ((size_t)(seq0 + gk) * Hkv + hk) * HD + kc * 8)
                        : make_uint4(0, 0, 0, 0);
    }
    if (vloader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gk = kb0 + vkg * 4 + i;
        vreg[i] = gk < Kb ? *reinterpret_cast<const bf16x8*>(
                                v + ((size_t)(seq0 + gk) * Hkv + hk) * HD + vdc * 8)
                          : zero_bf16x8();
      }
    }
    if (tid < 64) {
      const int gk = kb0 + tid;
      sreg = gk < Kb ? s_c[seq0 + gk] : 0.f;
    }
  };
  auto sstore = [&](int st) {
    bf16* kd = Ks + st * KSTAGE;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int c = tid + i * 256;
      const int key = c / KCH, kc = c % KCH;
      *reinterpret_cast<uint4*>(kd + key * HD + ((kc ^ (key & (KCH - 1))) << 3)) = kreg[i];
    }
    if (vloader) {
      bf16* vd = Vs + st * VSTAGE;
      const int p = vperm16((vkg * 4) & 15) | ((vkg * 4) & ~15);
      const int chunk = p >> 3, off = p & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = vdc * 8 + e;
        bf16x4 pk;
        pk[0] = vreg[0][e];
        pk[1] = vreg[1][e];
        pk[2] = vreg[2][e];
        pk[3] = vreg[3][e];
        *reinterpret_cast<bf16x4*>(vd + dd * 64 + ((chunk ^ vswz(dd)) << 3) + off) = pk;
      }
    }
    if (tid < 64) {
#pragma unroll
      for (int j = 0; j < G; ++j) bias[(st * G + j) * 64 + tid] = sreg * g[hk * G + j] * TG_LOG2E;
    }
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = zero_f32x16();
  float m_run = -INFINITY, l_run = 0.f;

  const int ksw = l31 & (KCH - 1);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) gload(kt + 1);
    const int st = kt & 1;
    const int kbase = kt * 64;
    if (wave_any && kbase <= qw0 + 31) {
      const bf16* kd = Ks + st * KSTAGE;
      f32x16 sacc[2];
      sacc[0] = zero_f32x16();
      sacc[1] = zero_f32x16();
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const int ch = ((ks * 2 + half) ^ ksw) << 3;
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kd + l31 * HD + ch);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kd + (32 + l31) * HD + ch);
        sacc[0] = mfma32(k0, qf[ks], sacc[0]);
        sacc[1] = mfma32(k1, qf[ks], sacc[1]);
      }
      const float* bs = bias + (st * G + gi) * 64;
      const bool diag = kbase + 63 > qw0;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int kl = kb * 32 + rq * 8 + half * 4;
          const f32x4 bv = *reinterpret_cast<const f32x4*>(bs + kl);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = fmaf(sacc[kb][rq * 4 + e], cscale, bv[e]);
            if (diag && kbase + kl + e > qi) x = -INFINITY;
            sacc[kb][rq * 4 + e] = x;
            mx = fmaxf(mx, x);
          }
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float rs = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_new);
          rs += pv;
          pf[kb * 2 + (r >> 3)][r & 7] = f2bf(pv);
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      const bf16* vd = Vs + st * VSTAGE;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int dd = db * 32 + l31;
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vd + dd * 64 + (((kk * 2 + half) ^ vswz(dd)) << 3));
          oacc[db] = mfma32(vf, pf[kk], oacc[db]);
        }
    }
    if (kt + 1 < n_kt) sstore((kt + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    bf16* orow = o + ((size_t)(seq0 + qi) * Hq + h) * HD + half * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = f2bf(oacc[db][rq * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + rq * 8) = w;
      }
    if (lse && half == 0) lse[(size_t)h * Ttot + seq0 + qi] = (m_run + __log2f(l_tot)) * TG_LN2;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per query, keys streamed through LDS in tiles of 32,
// exact-exp online softmax.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ s_c, const float* __restrict__ t, const float* __restrict__ g,
    const int32_t* __restrict__ cu_kept, int B, int Hq, int Hkv, float* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ float ks[32][HD + 1];
  __shared__ float vs[32][HD + 1];
  __shared__ float sb[32];
  const int b = blockIdx.z, h = blockIdx.y;
  const int seq0 = cu_kept[b], Kb = cu_kept[b + 1] - seq0;
  const int q0 = blockIdx.x * 64;
  if (q0 >= Kb) return;
  const int Ttot = cu_kept[B];
  const int hk = h / (Hq / Hkv);
  const int qi = q0 + threadIdx.x;
  const bool valid = qi < Kb;
  float qr[HD], acc[HD];
  for (int e = 0; e < HD; ++e) {
    qr[e] = valid ? q[((size_t)(seq0 + qi) * Hq + h) * HD + e] : 0.f;
    acc[e] = 0.f;
  }
  const float sc = t[h] / sqrtf((float)HD), gh = g[h];
  float m = -INFINITY, l = 0.f;
  const int kend = min(Kb, q0 + 64);
  for (int k0 = 0; k0 < kend; k0 += 32) {
    for (int e = threadIdx.x; e < 32 * HD; e += 64) {
      const int r = e / HD, c = e % HD;
      const int gk = k0 + r;
      ks[r][c] = gk < Kb ? k[((size_t)(seq0 + gk) * Hkv + hk) * HD + c] : 0.f;
      vs[r][c] = gk < Kb ? v[((size_t)(seq0 + gk) * Hkv + hk) * HD + c] : 0.f;
    }
    if (threadIdx.x < 32) sb[threadIdx.x] = (k0 + threadIdx.x < Kb) ? s_c[seq0 + k0 + threadIdx.x] : 0.f;
    __syncthreads();
    for (int j = 0; j < 32; ++j) {
      const int key = k0 + j;
      if (key > qi || key >= Kb) break;
      float dot = 0.f;
      for (int e = 0; e < HD; ++e) dot = fmaf(qr[e], ks[j][e], dot);
      const float x = dot * sc + gh * sb[j];
      if (x > m) {
        const float r = expf(m - x);
        for (int e = 0; e < HD; ++e) acc[e] *= r;
        l *= r;
        m = x;
      }
      const float p = expf(x - m);
      l += p;
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(p, vs[j][e], acc[e]);
    }
    __syncthreads();
  }
  if (valid) {
    const float inv = 1.0f / l;
    for (int e = 0; e < HD; ++e) o[((size_t)(seq0 + qi) * Hq + h) * HD + e] = acc[e] * inv;
    if (lse) lse[(size_t)h * Ttot + seq0 + qi] = m + logf(l);
  }
}

template <int G, int HD>
static hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const float* s_c,
                                   const float* t, const float* g, const int32_t* cu_kept, int B,
                                   int max_k, int Hq, int Hkv, void* o, float* lse,
                                   hipStream_t stream) {
  constexpr int BQ = 32 * (4 / G);
  constexpr size_t lds = (size_t)2 * 2 * 64 * HD * sizeof(bf16) + (size_t)2 * G * 64 * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<G, HD>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_qt = (max_k + BQ - 1) / BQ;
  const long blocks = (long)n_qt * Hkv * B;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<G, HD>), dim3((unsigned)blocks), dim3(256), lds, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, s_c, t, g, cu_kept, B, Hq,
                     Hkv, n_qt, (bf16*)o, lse);
  return hipGetLastError();
}

hipError_t attn_fwd(const void* q, const void* k, const void* v, const float* s_c, const float* t,
                    const float* g, const int32_t* cu_kept, int B, int max_k, int Hq, int Hkv,
                    int d, bool is_bf16, void* o, float* lse, hipStream_t stream) {
  if (B <= 0 || max_k <= 0) return hipSuccess;
  if (!is_bf16) {
    dim3 grid((max_k + 63) / 64, Hq, B);
    if (d == 64)
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, (const float*)q,
                         (const float*)k, (const float*)v, s_c, t, g, cu_kept, B, Hq, Hkv,
                         (float*)o, lse);
    else
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, (const float*)q,
                         (const float*)k, (const float*)v, s_c, t, g, cu_kept, B, Hq, Hkv,
                         (float*)o, lse);
    return hipGetLastError();
  }
  const int G = Hq / Hkv;
#define TG_ATTN_CASE(GG, DD)                                                                    \
  if (G == GG && d == DD)                                                                       \
    return launch_attn_bf16<GG, DD>(q, k, v, s_c, t, g, cu_kept, B, max_k, Hq, Hkv, o, lse, \
                                    stream);
  TG_ATTN_CASE(1, 64)
  TG_ATTN_CASE(2, 64)
  TG_ATTN_CASE(4, 64)
  TG_ATTN_CASE(1, 128)
  TG_ATTN_CASE(2, 128)
  TG_ATTN_CASE(4, 128)
#undef TG_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace tg
