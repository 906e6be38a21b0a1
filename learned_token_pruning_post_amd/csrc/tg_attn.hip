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
//    the B operand of the PV product without touching LDS;
//  * K, V and the tile's gate scores move global -> LDS with direct-to-LDS
//    buffer loads into a 2-stage ring (one barrier per 64-key tile). V stays
//    row-major: its V^T fragments come from ds_read_b64_tr_b16, which hands
//    each lane of a 16-lane group 4 keys of one feature column; the key order
//    of those fragments matches the k-slot order of P in the accumulator.
//    LDS rows are XOR-swizzled so that both the K fragment reads and the
//    transposing V reads of a phase hit distinct banks;
//  * log2-domain online softmax, t_h*log2(e)/sqrt(d) folded into one
//    multiply, g_h*log2(e)*s_c[j] added per key; the output accumulator is
//    rescaled only when a row maximum grows by more than 8 (log2 units);
//  * heavy (late) and light (early) query tiles are dispatched in pairs.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

template <int HD>
struct AttnLayout {
  static constexpr int RB = HD * 2;          // bytes per K or V row
  static constexpr int KCH = HD / 8;         // 16-byte chunks per row
  static constexpr int RPB = 1024 / RB;      // rows per 1 KB load block
  static constexpr int TILE = 64 * RB;       // bytes of a 64-key K (or V) tile
  static constexpr int STAGE = 2 * TILE + 256;  // K, V, 64 fp32 scores
  // K fragment reads: 16 lanes read 16 consecutive keys, same logical chunk
  __device__ static int kswz(int key) { return HD == 128 ? (key & 15) : ((key >> 1) & 7); }
  // V transposing reads: 32 lanes read 4 consecutive (4-aligned) keys x 4 chunks
  __device__ static int vswz(int key) { return HD == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); }
};

template <int G, int HD>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ s_c, const float* __restrict__ t, const float* __restrict__ g,
    const int32_t* __restrict__ cu_kept, int B, int Hq, int Hkv, int n_qt, bf16* __restrict__ o,
    float* __restrict__ lse) {
  using LY = AttnLayout<HD>;
  constexpr int WPH = 4 / G;     // waves per q-head
  constexpr int BQ = 32 * WPH;   // queries per workgroup
  constexpr int ND = HD / 32;    // 32-wide d blocks of O^T
  constexpr int NKB = 64 / LY::RPB;  // load blocks per K (or V) tile
  constexpr int LPW = NKB / 4;       // of them per wave
  extern __shared__ __attribute__((aligned(1024))) unsigned char attn_smem[];
  const uint32_t lds0 = lds_addr(attn_smem);

  const int tid = threadIdx.x;
  // Work order: the first half of the grid takes query tiles from the last
  // (heaviest: most keys under the causal mask) down, the second half from
  // the first up. Workgroups L and L + grid/2 land on the same XCD and, with
  // breadth-first dispatch, on the same CU, so every CU gets about n_qt + 1
  // key tiles of work.
  const int L = blockIdx.x;
  const int per = Hkv * B;
  const int rank = L / per;
  const int hn = (n_qt + 1) >> 1;
  const int qt = rank < hn ? n_qt - 1 - rank : rank - hn;
  const int rem = L - rank * per;
  const int hk = rem % Hkv, b = rem / Hkv;
  const int seq0 = cu_kept[b];
  const int Kb = cu_kept[b + 1] - seq0;
  const int q0 = qt * BQ;
  if (q0 >= Kb) return;
  const int Ttot = cu_kept[B];

  const int lane = tid & 63, l31 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const bf16* qrow = q + ((size_t)(seq0 + min(qi, Kb - 1)) * Hq + h) * HD + half * 8;
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }
  const float cscale = t[h] * TG_LOG2E / sqrtf((float)HD);
  const float gl = g[h] * TG_LOG2E;

  // ---- direct-to-LDS tile loads (buffer loads, range = this sequence, so
  // keys past its end read as zeros and are masked). Lane l of a 1 KB block
  // lands in row l / KCH, slot l % KCH, and fetches the logical chunk that the
  // swizzle puts there. A wave's blocks are blk = wave + 4i: for K the
  // swizzle depends on blk only through blk & 3 (= wave & 3), for V not at
  // all, so each lane has one fixed byte offset per operand. ----
  const int rib = lane / LY::KCH, slot = lane % LY::KCH;
  const uint32_t row_bytes = (uint32_t)Hkv * HD * 2u;  // bytes between consecutive tokens
  const i32x4 rk = make_rsrc(k + (size_t)seq0 * Hkv * HD + (size_t)hk * HD, (uint32_t)Kb * row_bytes);
  const i32x4 rv = make_rsrc(v + (size_t)seq0 * Hkv * HD + (size_t)hk * HD, (uint32_t)Kb * row_bytes);
  const i32x4 rsc = make_rsrc(s_c + seq0, (uint32_t)Kb * 4u);
  const int krow0 = (wave & 3) * LY::RPB + rib;  // row of this lane in the wave's first block
  const uint32_t koff = rib * row_bytes + ((slot ^ LY::kswz(krow0)) << 4);
  const uint32_t voff_l = rib * row_bytes + ((slot ^ LY::vswz(krow0)) << 4);
  auto issue = [&](int kt, int st) {
    const uint32_t sb = lds0 + st * LY::STAGE;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const uint32_t rowoff = (uint32_t)(kt * 64 + blk * LY::RPB) * row_bytes;
      buf_dma16(rk, koff + rowoff, __builtin_amdgcn_readfirstlane(sb + blk * 1024));
      buf_dma16(rv, voff_l + rowoff, __builtin_amdgcn_readfirstlane(sb + LY::TILE + blk * 1024));
    }
    if (wave == 0)  // one gate score per lane
      buf_dma4(rsc, (uint32_t)(kt * 64 + lane) * 4u, __builtin_amdgcn_readfirstlane(sb + 2 * LY::TILE));
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = zero_f32x16();
  float m_run = -INFINITY, l_run = 0.f;

  // V^T fragment source (bytes inside a stage) for key-step kk, d block db:
  // group G = lane / 16 of the wave: k-slot group G / 2, d half G % 2
  const int vg = (lane >> 4) & 3, vs = lane & 15;
  const int vkey_lo = 4 * (vg >> 1) + (vs >> 2);         // + 16*kk (+8 for the high half)
  const int vd = 16 * (vg & 1) + 4 * (vs & 3);            // + 32*db
  // byte offsets of the low-half reads; +16 keys (next kk) and +8 keys (high
  // half) keep key & 3 and (key >> 1) & 1, hence the swizzle: constant offsets
  int voff[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int d = 32 * db + vd;
    voff[db] = vkey_lo * LY::RB + (((d >> 3) ^ LY::vswz(vkey_lo)) << 4) + (d & 7) * 2;
  }

  issue(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < n_kt) issue(kt + 1, (kt + 1) & 1);
    const int st = kt & 1;
    const int kbase_key = kt * 64;
    if (wave_any && kbase_key <= qw0 + 31) {
      const unsigned char* ks_ = attn_smem + st * LY::STAGE;
      const unsigned char* vs_ = ks_ + LY::TILE;
      const float* ss_ = reinterpret_cast<const float*>(ks_ + 2 * LY::TILE);
      f32x16 sacc[2];
      sacc[0] = zero_f32x16();
      sacc[1] = zero_f32x16();
      const int ksw = LY::kswz(l31);  // same for key l31 and 32 + l31
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const int ch = ((ks * 2 + half) ^ ksw) << 4;
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks_ + l31 * LY::RB + ch);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(ks_ + (32 + l31) * LY::RB + ch);
        sacc[0] = mfma32(k0, qf[ks], sacc[0]);
        sacc[1] = mfma32(k1, qf[ks], sacc[1]);
      }
      // logits in the log2 domain; keys past a query (diagonal tiles only) -> -inf
      float mx = -INFINITY;
      if (kbase_key + 63 > qw0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int kl = kb * 32 + rq * 8 + half * 4;
            const f32x4 sv = *reinterpret_cast<const f32x4*>(ss_ + kl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = fmaf(sacc[kb][rq * 4 + e], cscale, sv[e] * gl);
              x = (kbase_key + kl + e > qi) ? -INFINITY : x;
              sacc[kb][rq * 4 + e] = x;
              mx = fmaxf(mx, x);
            }
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const f32x4 sv = *reinterpret_cast<const f32x4*>(ss_ + kb * 32 + rq * 8 + half * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = fmaf(sacc[kb][rq * 4 + e], cscale, sv[e] * gl);
              sacc[kb][rq * 4 + e] = x;
              mx = fmaxf(mx, x);
            }
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescale: keep the running max while no row exceeds it by more
      // than 8 (p <= 2^8, far from fp32/bf16 overflow; exact after the final
      // division by the row sum, which uses the same reference).
      if (__any(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }
      float rs = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_run);
          rs += pv;
          pf[kb * 2 + (r >> 3)][r & 7] = f2bf(pv);
        }
      l_run += rs;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const unsigned char* a_lo = vs_ + voff[db] + kk * 16 * LY::RB;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(a_lo));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(a_lo + 8 * LY::RB));
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = mfma32(vf, pf[kk], oacc[db]);
        }
      }
    }
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
  constexpr size_t lds = (size_t)2 * AttnLayout<HD>::STAGE;
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
