// Backward of the token-gated causal GQA attention.
//
// Tencent Cloud TokenGate article, gradient-path section: the kept tokens'
// scores enter the upper layers' attention logits, so the loss reaches the
// scorer through them, and the per-head gain and temperature are learned with
// it. Forward (as in the forward kernel): L_ij = t_h q_i.k_j / sqrt(d) +
// g_h s_c[j] for j <= i, P = softmax_j L, o_i = sum_j P_ij v_j. Given dO:
//   dv_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;  dL_ij = P_ij (dP_ij - D_i)
//   with D_i = dO_i . o_i (= sum_j P_ij dP_ij);  dq_i = t_h/sqrt(d) sum_j dL_ij k_j;
//   dk_j = t_h/sqrt(d) sum_i dL_ij q_i;  ds_j = sum_h g_h sum_i dL_ij;
//   dg_h = sum_ij dL_ij s_j;  dt_h = sum_ij dL_ij q_i.k_j / sqrt(d).
// P is recomputed from the forward's log-sum-exp (no [T, T] matrix is stored).
//
// Kernels (bf16 operands, fp32 accumulation on 32x32x16 MFMA):
//  * prep: D_i and the log-sum-exp in log2 units, per (query, head);
//  * dK/dV: one workgroup per (sequence, kv head, pair of key tiles p and
//    n-1-p, so every workgroup sees about the same number of query tiles);
//    its 4 waves cover (q head of the group, 32-key sub-tile). Per 32-query
//    step the Q and dO rows of the group's heads are staged in LDS; a wave
//    computes S = Q K^T and dP = dO V^T with K and V of its keys held as
//    register B operands, so the accumulators put one key per lane and P and
//    dL feed dV^T += dO^T P and dK^T += Q^T dL straight from registers (the
//    A operands dO^T and Q^T come from transposing LDS reads). The per-key
//    sums for ds, dg and dt are then per lane. The heads of a group meet in
//    LDS at the end;
//  * dQ: mirrors the forward's layout (S^T = K Q^T, one query per lane), one
//    workgroup per (sequence, kv head, pair of query tiles), K, V and scores
//    of each 32-key tile staged in LDS; dQ^T += K^T dL^T (K^T by transposing
//    LDS reads); like the forward, two groups of four waves take the two
//    halves of the key range and their partial dQ meet in LDS;
//  * staging: direct-to-LDS buffer loads over the sequence's rows (reads past
//    its end give zeros), double-buffered: the next step's tiles are in flight
//    while the current one is computed, one barrier per step;
//  * reductions: ds over kv heads, dt and dg over workgroups, in a fixed
//    order (deterministic).
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace abwd {

constexpr int NT = 256;

// row-major bf16 tile in LDS, HD columns, 16-byte chunks XOR-swizzled by row
template <int HD>
struct Tile {
  static constexpr int RB = HD * 2;
  static constexpr int NCH = HD / 8;
  __device__ static int swz(int r) { return HD == 128 ? (r & 15) : (r & 7); }
  __device__ static const bf16x8& chunk(const bf16* base, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + r * RB + ((c ^ swz(r)) << 4));
  }
};

// A operand of a transposed tile (rows of A = feature columns, k-slots = tile
// rows): lane l holds feature 32*db + l%32 and the 8 tile rows 16*ks + {0..3,
// 8..11} + 4*(l/32), the row order of registers 8*ks .. 8*ks+7 of an
// accumulator (acc_row). Two ds_read_tr16_b64: within 16 lanes, lane 4e+m
// addresses row e, features 4m .. 4m+3, and lane i receives feature i of
// rows 0..3.
template <int HD>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* base, int ks, int db, int lane) {
  const int vg = (lane >> 4) & 3, vs = lane & 15;
  const int r = 16 * ks + 4 * (vg >> 1) + (vs >> 2);
  const int d = 32 * db + 16 * (vg & 1) + 4 * (vs & 3);
  const char* b = reinterpret_cast<const char*>(base);
  const char* lo = b + r * Tile<HD>::RB + (((d >> 3) ^ Tile<HD>::swz(r)) << 4) + (d & 7) * 2;
  const char* hi = b + (r + 8) * Tile<HD>::RB + (((d >> 3) ^ Tile<HD>::swz(r + 8)) << 4) + (d & 7) * 2;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(lo));
  const bf16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(hi));
  return __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct-to-LDS load of 32 rows of a row-strided bf16 tensor into a swizzled
// Tile: 1 KB blocks of RPB rows; lane l of a block lands in row l / NCH, slot
// l % NCH and fetches the logical chunk the swizzle puts there. `rs` covers the
// sequence's rows (reads past its end give zeros); `row0` is the tile's first
// row in the sequence, `rstride` the bytes between rows, `col` the byte offset
// of the tile's columns inside a row (the head).
template <int HD>
__device__ __forceinline__ void dma_tile(const i32x4& rs, uint32_t row0, uint32_t rstride, uint32_t col,
                                         uint32_t lds_tile, int blk, int lane) {
  constexpr int NCH = Tile<HD>::NCH, RPB = 1024 / Tile<HD>::RB;
  const int r = blk * RPB + lane / NCH, slot = lane % NCH;
  const uint32_t off = (row0 + (uint32_t)r) * rstride + col + (uint32_t)((slot ^ Tile<HD>::swz(r)) << 4);
  buf_dma16(rs, off, __builtin_amdgcn_readfirstlane(lds_tile + blk * 1024));
}

// query / key index of accumulator register r of lane group g (rows of a 32x32 tile)
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// bf16x8 of v[8*ks .. 8*ks+7] (B operand taken from an accumulator)
__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = f2bf(v[j]);
  return b;
}

__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dO;
  const float* lse;  // [Hq, T] natural log (forward)
  const float* s_c;
  const float* t;
  const float* g;
  const int32_t* cu;
  float* dq;  // [T, Hq, d]
  float* dk;  // [T, Hkv, d]
  float* dv;
  float* ds;  // [T]
  float* dt;  // [Hq]
  float* dg;
  float* lse2;     // ws [Hq, T]
  float* delta;    // ws [Hq, T]
  float* ds_part;  // ws [Hkv, T]
  float* tg_part;  // ws [nwg_kv, G, 2]
  int B, T, Hq, Hkv, n_kt, n_qt;
};

// D_i = dO_i . o_i and lse in log2 units, one group of HD/8 lanes per (query, head)
template <int HD>
__global__ __launch_bounds__(NT) void prep_kernel(Args a) {
  constexpr int LPR = HD / 8;
  const int64_t row = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPR;  // (query, head)
  const int c = threadIdx.x % LPR;
  const bool live = row < (int64_t)a.T * a.Hq;
  const int64_t rr = live ? row : 0;
  const int i = (int)(rr / a.Hq), h = (int)(rr % a.Hq);
  const u32x4 x = *reinterpret_cast<const u32x4*>(a.o + (size_t)rr * HD + c * 8);
  const u32x4 y = *reinterpret_cast<const u32x4*>(a.dO + (size_t)rr * HD + c * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(__uint_as_float(x[e] << 16), __uint_as_float(y[e] << 16), acc);
    acc = fmaf(__uint_as_float(x[e] & 0xffff0000u), __uint_as_float(y[e] & 0xffff0000u), acc);
  }
#pragma unroll
  for (int sh = 1; sh < LPR; sh <<= 1) acc += __shfl_xor(acc, sh, 64);
  if (live && c == 0) {
    a.delta[(size_t)h * a.T + i] = acc;
    a.lse2[(size_t)h * a.T + i] = a.lse[(size_t)h * a.T + i] * TG_LOG2E;
  }
}

template <int G, int HD>
struct KvSmem {
  static constexpr int WPK = 4 / G;
  struct Stage {
    bf16 q[G][32 * HD];
    bf16 o[G][32 * HD];  // dO
  };
  union {
    Stage st[2];  // double-buffered Q and dO rows of the query step
    // after the query loop, the heads of a group meet here: dK^T and dV^T of a
    // 32-key sub-tile ([d][key])
    float red[G > 1 ? WPK : 1][2][HD * 32];
  };
  __attribute__((aligned(16))) float l2[2][G][32];
  __attribute__((aligned(16))) float dl[2][G][32];
  float dsr[4][32];
  float tgr[4][2];
};

template <int G, int HD>
__global__ __launch_bounds__(NT, 1) void dkdv_kernel(Args a) {
  constexpr int WPK = 4 / G;  // 32-key sub-tiles per key tile
  constexpr int BK = 32 * WPK;
  constexpr int NS = HD / 16, ND = HD / 32;
  constexpr int NBLK = 32 * Tile<HD>::RB / 1024;  // 1 KB blocks per 32-row tile
  constexpr int BPW = 2 * G * NBLK / 4;            // of them per wave and step
  using TL = Tile<HD>;
  using SM = KvSmem<G, HD>;
  static_assert(sizeof(SM) <= 160 * 1024, "dK/dV LDS fits a CU");
  extern __shared__ __attribute__((aligned(1024))) unsigned char dkdv_smem[];
  auto& S = *reinterpret_cast<SM*>(dkdv_smem);

  const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, grp = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gi = w / WPK, ksub = w % WPK;
  const int npair = (a.n_kt + 1) >> 1;
  const int wg = blockIdx.x;
  const int hk = wg % a.Hkv, p = (wg / a.Hkv) % npair, b = wg / (a.Hkv * npair);
  const int seq0 = a.cu[b], Kb = a.cu[b + 1] - seq0;
  const int nk = (Kb + BK - 1) / BK, nq = (Kb + 31) / 32;
  const int h = hk * G + gi;
  const float c2 = a.t[h] * TG_LOG2E * rsqrtf((float)HD);
  const float cnat = a.t[h] * rsqrtf((float)HD);
  const float g2 = a.g[h] * TG_LOG2E;
  float dg_acc = 0.f, dt_acc = 0.f;

  // Q and dO rows of the group's heads: resources over the sequence's rows
  const uint32_t rstride = (uint32_t)a.Hq * HD * 2u;
  const i32x4 rq = make_rsrc(a.q + (size_t)seq0 * a.Hq * HD + (size_t)hk * G * HD, (uint32_t)Kb * rstride);
  const i32x4 ro = make_rsrc(a.dO + (size_t)seq0 * a.Hq * HD + (size_t)hk * G * HD, (uint32_t)Kb * rstride);
  const uint32_t lds0 = lds_addr(dkdv_smem);
  // one step's loads into stage buffer sb: 2 * G * NBLK blocks, BPW per wave
  auto issue = [&](int qt, int sb) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int bi = w * BPW + i;
      const int tens = bi / (G * NBLK), gg = (bi / NBLK) % G, blk = bi % NBLK;
      const uint32_t dst = lds0 + (uint32_t)((char*)(tens ? &S.st[sb].o[gg][0] : &S.st[sb].q[gg][0]) -
                                             (char*)dkdv_smem);
      // rows of head gg sit gg * HD elements further into each token's row
      dma_tile<HD>(tens ? ro : rq, (uint32_t)(qt * 32), rstride, (uint32_t)(gg * HD * 2), dst, blk, lane);
    }
  };
  float pl2 = INFINITY, pdl = 0.f;  // this thread's (head, row) of the next step's lse and D
  auto fetch_ld = [&](int qt) {
    if (tid < G * 32) {
      const int gg = tid / 32, r = tid % 32;
      const bool qv = qt * 32 + r < Kb;
      const size_t at = (size_t)(hk * G + gg) * a.T + seq0 + qt * 32 + r;
      pl2 = qv ? a.lse2[at] : INFINITY;  // P = 0 for rows past the sequence
      pdl = qv ? a.delta[at] : 0.f;
    }
  };
  auto put_ld = [&](int sb) {
    if (tid < G * 32) {
      S.l2[sb][tid / 32][tid % 32] = pl2;
      S.dl[sb][tid / 32][tid % 32] = pdl;
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    const int kt = pass == 0 ? p : nk - 1 - p;
    if (p >= (nk + 1) / 2 || (pass == 1 && kt == p)) break;  // uniform over the workgroup
    const int kb = kt * BK + 32 * ksub;                        // first key of this wave
    const int kj = kb + l31;
    const bool kval = kj < Kb;
    bf16x8 kfr[NS], vfr[NS];
    {
      const size_t off = ((size_t)(seq0 + (kval ? kj : 0)) * a.Hkv + hk) * HD + 8 * grp;
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) {
        kfr[s_] = kval ? *reinterpret_cast<const bf16x8*>(a.k + off + 16 * s_) : zero_bf16x8();
        vfr[s_] = kval ? *reinterpret_cast<const bf16x8*>(a.v + off + 16 * s_) : zero_bf16x8();
      }
    }
    const float sj = kval ? a.s_c[seq0 + kj] : 0.f;
    const float bias2 = g2 * sj;
    f32x16 dkT[ND], dvT[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      dkT[db] = zero_f32x16();
      dvT[db] = zero_f32x16();
    }
    float dl_acc = 0.f;

    const int qt0 = (kt * BK) / 32;
    __syncthreads();  // the stage buffers (and the reduction area aliasing them) are free
    issue(qt0, 0);
    fetch_ld(qt0);
    put_ld(0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int qt = qt0; qt < nq; ++qt) {
      const int sb = (qt - qt0) & 1;
      // the accumulators stay in AGPRs across steps (no copies at the loop back edge)
#pragma unroll
      for (int db = 0; db < ND; ++db) asm volatile("" : "+a"(dkT[db]), "+a"(dvT[db]));
      if (qt + 1 < nq) {
        issue(qt + 1, sb ^ 1);
        fetch_ld(qt + 1);
      }
      const int q0 = qt * 32;
      {  // a step no query of which sees this wave's keys gives P = 0 through the mask
        const bf16* sq = S.st[sb].q[gi];
        const bf16* so = S.st[sb].o[gi];
        f32x16 sacc = zero_f32x16(), pacc = zero_f32x16();
#pragma unroll
        for (int s_ = 0; s_ < NS; ++s_) {
          sacc = mfma32(TL::chunk(sq, l31, 2 * s_ + grp), kfr[s_], sacc);
          pacc = mfma32(TL::chunk(so, l31, 2 * s_ + grp), vfr[s_], pacc);
        }
        // the fragment reads run two k-steps ahead of their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s_ = 0; s_ < NS - 2; ++s_) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
        // dV / dK products: MFMA i takes (ks, db) = (i / (2 ND), (i / 2) % ND), even i dV
        // (dO^T, P), odd i dK (Q^T, dL); the transposed fragments are read PF MFMAs ahead,
        // the first PF of them under the softmax
        constexpr int NM = 4 * ND, PF = 4;
        auto trf = [&](int i) { return tr_frag<HD>(i & 1 ? sq : so, i / (2 * ND), (i >> 1) % ND, lane); };
        bf16x8 fq[NM];
#pragma unroll
        for (int i = 0; i < PF; ++i) fq[i] = trf(i);
        __builtin_amdgcn_sched_barrier(0);
        // P and dL eight rows at a time (one k-step of the dV / dK products),
        // packed to bf16 right away; the rows' lse and D four rows per read
        bf16x8 pbk[2], lbk[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float P[8], dL[8];
#pragma unroll
          for (int r4 = 0; r4 < 2; ++r4) {
            const int rb = 8 * ks + 4 * r4;
            const f32x4 l2v = *reinterpret_cast<const f32x4*>(&S.l2[sb][gi][acc_row(rb, grp)]);
            const f32x4 dlv = *reinterpret_cast<const f32x4*>(&S.dl[sb][gi][acc_row(rb, grp)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = rb + e;
              const int qi = acc_row(r, grp);
              const bool vis = kval && kj <= q0 + qi;
              // the exponent is <= 0 up to rounding (P <= 1); hardware exp2, then the mask
              const float ex = __builtin_amdgcn_exp2f(fmaf(c2, sacc[r], bias2) - l2v[e]);
              const float pr = vis ? ex : 0.f;
              P[4 * r4 + e] = pr;
              dL[4 * r4 + e] = pr * (pacc[r] - dlv[e]);
              dl_acc += dL[4 * r4 + e];
              dt_acc = fmaf(dL[4 * r4 + e], sacc[r], dt_acc);
            }
          }
          pbk[ks] = pack8(P);
          lbk[ks] = pack8(dL);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i + PF < NM) fq[i + PF] = trf(i + PF);
          const int ks = i / (2 * ND), db = (i >> 1) % ND;
          if (i & 1)
            dkT[db] = mfma32(fq[i], lbk[ks], dkT[db]);
          else
            dvT[db] = mfma32(fq[i], pbk[ks], dvT[db]);
        }
#pragma unroll
        for (int i = 0; i < NM - PF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }
      if (qt + 1 < nq) put_ld(sb ^ 1);
      wait_vmcnt<0>();
      __syncthreads();
    }
    // per-key sums of this head: dL summed over the queries (both lane groups)
    const float dl_key = xsum32(dl_acc);
    dg_acc = fmaf(sj, dl_acc, dg_acc);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dkT[db][r] *= cnat;
    if constexpr (G > 1) {
      for (int src = 1; src < G; ++src) {
        if (gi == src) {
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int d = 32 * db + acc_row(r, grp);
              S.red[ksub][0][d * 32 + l31] = dkT[db][r];
              S.red[ksub][1][d * 32 + l31] = dvT[db][r];
            }
        }
        __syncthreads();
        if (gi == 0) {
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int d = 32 * db + acc_row(r, grp);
              dkT[db][r] += S.red[ksub][0][d * 32 + l31];
              dvT[db][r] += S.red[ksub][1][d * 32 + l31];
            }
        }
        __syncthreads();
      }
    }
    if (lane < 32) S.dsr[w][l31] = a.g[h] * dl_key;
    __syncthreads();
    if (gi == 0 && kval) {
      float* dkr = a.dk + ((size_t)(seq0 + kj) * a.Hkv + hk) * HD;
      float* dvr = a.dv + ((size_t)(seq0 + kj) * a.Hkv + hk) * HD;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * grp;
          *reinterpret_cast<f32x4*>(dkr + d) =
              f32x4{dkT[db][4 * r4], dkT[db][4 * r4 + 1], dkT[db][4 * r4 + 2], dkT[db][4 * r4 + 3]};
          *reinterpret_cast<f32x4*>(dvr + d) =
              f32x4{dvT[db][4 * r4], dvT[db][4 * r4 + 1], dvT[db][4 * r4 + 2], dvT[db][4 * r4 + 3]};
        }
      if (lane < 32) {
        float sum = 0.f;
        for (int gg = 0; gg < G; ++gg) sum += S.dsr[gg * WPK + ksub][l31];
        a.ds_part[(size_t)hk * a.T + seq0 + kj] = sum;
      }
    }
  }
  // this workgroup's dg and dt of each head of the group (zeros when it had no keys)
  dg_acc = wave_sum(dg_acc);
  dt_acc = wave_sum(dt_acc) * rsqrtf((float)HD);
  if (lane == 0) {
    S.tgr[w][0] = dg_acc;
    S.tgr[w][1] = dt_acc;
  }
  __syncthreads();
  if (tid < G) {
    float sg = 0.f, st = 0.f;
    for (int ww = 0; ww < WPK; ++ww) {
      sg += S.tgr[tid * WPK + ww][0];
      st += S.tgr[tid * WPK + ww][1];
    }
    a.tg_part[((size_t)wg * G + tid) * 2] = sg;
    a.tg_part[((size_t)wg * G + tid) * 2 + 1] = st;
  }
}

template <int HD>
struct QSmem {
  struct Ring {  // double-buffered K and V rows and scores of one key-half group
    bf16 k[2][32 * HD];
    bf16 v[2][32 * HD];
    __attribute__((aligned(16))) float s[2][64];
  };
  union {
    Ring r[2];
    // after the key loop: the second group's dQ^T partials, [wave][d block][register][lane]
    float red[4][HD / 32][16][64];
  };
};

template <int G, int HD>
__global__ __launch_bounds__(2 * NT, 1) void dq_kernel(Args a) {
  constexpr int WPH = 4 / G;  // 32-query sub-tiles per query tile
  constexpr int BQ = 32 * WPH;
  constexpr int NS = HD / 16, ND = HD / 32;
  constexpr int NBLK = 32 * Tile<HD>::RB / 1024;  // 1 KB blocks per 32-row tile
  constexpr int BPW = 2 * NBLK / 4;               // of them per wave and step (K and V)
  using TL = Tile<HD>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char dq_smem[];
  QSmem<HD>& SQ = *reinterpret_cast<QSmem<HD>*>(dq_smem);

  // two groups of four waves split each query tile's key range in halves (two
  // waves per SIMD); the second group's dQ partials join the first's through
  // LDS at the end, in a fixed order
  const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, grp = lane >> 5;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w8 >> 2, w = w8 & 3;  // key-half group, wave inside the group
  auto& S = SQ.r[kg];
  const int gi = w / WPH, qs = w % WPH;
  const int npair = (a.n_qt + 1) >> 1;
  const int wg = blockIdx.x;
  const int hk = wg % a.Hkv, p = (wg / a.Hkv) % npair, b = wg / (a.Hkv * npair);
  const int seq0 = a.cu[b], Kb = a.cu[b + 1] - seq0;
  const int nq = (Kb + BQ - 1) / BQ;
  const int h = hk * G + gi;
  const float c2 = a.t[h] * TG_LOG2E * rsqrtf((float)HD);
  const float cnat = a.t[h] * rsqrtf((float)HD);
  const float g2 = a.g[h] * TG_LOG2E;

  const uint32_t rstride = (uint32_t)a.Hkv * HD * 2u;
  const i32x4 rk = make_rsrc(a.k + (size_t)seq0 * a.Hkv * HD + (size_t)hk * HD, (uint32_t)Kb * rstride);
  const i32x4 rv = make_rsrc(a.v + (size_t)seq0 * a.Hkv * HD + (size_t)hk * HD, (uint32_t)Kb * rstride);
  const i32x4 rsc = make_rsrc(a.s_c + seq0, (uint32_t)Kb * 4u);
  const uint32_t lk = lds_addr(&S.k[0][0]), lv = lds_addr(&S.v[0][0]), ls = lds_addr(&S.s[0][0]);
  auto issue = [&](int kt, int sb) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int bi = w * BPW + i;
      const int tens = bi / NBLK, blk = bi % NBLK;
      dma_tile<HD>(tens ? rv : rk, (uint32_t)(kt * 32), rstride, 0u,
                   (tens ? lv : lk) + (uint32_t)(sb * 32 * HD * 2), blk, lane);
    }
    if (w == 0)  // one score per lane (lanes past the 32 keys read zeros or another tile's keys; unused)
      buf_dma4(rsc, (uint32_t)(kt * 32 + lane) * 4u, __builtin_amdgcn_readfirstlane(ls + (uint32_t)(sb * 256)));
  };

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? p : nq - 1 - p;
    if (p >= (nq + 1) / 2 || (pass == 1 && qt == p)) break;  // uniform over the workgroup
    const int q0 = qt * BQ + 32 * qs;
    const int qi = q0 + l31;
    const bool qval = qi < Kb;
    bf16x8 qfr[NS], ofr[NS];
    {
      const size_t off = ((size_t)(seq0 + (qval ? qi : 0)) * a.Hq + h) * HD + 8 * grp;
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) {
        qfr[s_] = qval ? *reinterpret_cast<const bf16x8*>(a.q + off + 16 * s_) : zero_bf16x8();
        ofr[s_] = qval ? *reinterpret_cast<const bf16x8*>(a.dO + off + 16 * s_) : zero_bf16x8();
      }
    }
    const size_t at = (size_t)h * a.T + seq0 + (qval ? qi : 0);
    const float l2 = qval ? a.lse2[at] : INFINITY;
    const float dl = qval ? a.delta[at] : 0.f;
    f32x16 dqT[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) dqT[db] = zero_f32x16();
    const int last_key = min(qt * BQ + BQ, Kb) - 1;
    const int nkt = last_key / 32 + 1;
    const int nh = (nkt + 1) >> 1;        // key tiles of group 0 (also the loop count)
    const int t0 = kg ? nh : 0;           // first key tile of this group
    const int nt = kg ? nkt - nh : nh;    // key tiles of this group
    __syncthreads();  // the previous pass's readers (and the merge) are done with the buffers
    if (nt > 0) issue(t0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int j = 0; j < nh; ++j) {
      const int sb = j & 1;
      if (j + 1 < nt) issue(t0 + j + 1, sb ^ 1);
      const int k0 = (t0 + j) * 32;
      if (j < nt) {  // uniform per group; a tile no key of which precedes a query of this wave gives P = 0 through the mask
        const bf16* sk = S.k[sb];
        f32x16 sacc = zero_f32x16(), pacc = zero_f32x16();
#pragma unroll
        for (int s_ = 0; s_ < NS; ++s_) {
          sacc = mfma32(TL::chunk(sk, l31, 2 * s_ + grp), qfr[s_], sacc);
          pacc = mfma32(TL::chunk(S.v[sb], l31, 2 * s_ + grp), ofr[s_], pacc);
        }
        // the fragment reads run two k-steps ahead of their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s_ = 0; s_ < NS - 2; ++s_) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
        // dQ products: MFMA i takes (ks, db) = (i / ND, i % ND); the transposed K
        // fragments are read PF MFMAs ahead, the first PF of them under the softmax
        constexpr int NM = 2 * ND, PF = 4;
        bf16x8 fq[NM];
#pragma unroll
        for (int i = 0; i < PF; ++i) fq[i] = tr_frag<HD>(sk, i / ND, i % ND, lane);
        __builtin_amdgcn_sched_barrier(0);
        // the keys' scores, four consecutive keys per read (acc_row order)
        f32x4 sv[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) sv[r4] = *reinterpret_cast<const f32x4*>(&S.s[sb][acc_row(4 * r4, grp)]);
        float dL[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = acc_row(r, grp);
          const int kj = k0 + kr;
          const bool vis = qval && kj <= qi && kj < Kb;
          // the exponent is <= 0 up to rounding (P <= 1); hardware exp2, then the mask
          const float e = __builtin_amdgcn_exp2f(fmaf(c2, sacc[r], g2 * sv[r >> 2][r & 3]) - l2);
          const float pr = vis ? e : 0.f;
          dL[r] = pr * (pacc[r] - dl);
        }
        const bf16x8 lb[2] = {pack8(dL), pack8(dL + 8)};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i + PF < NM) fq[i + PF] = tr_frag<HD>(sk, (i + PF) / ND, (i + PF) % ND, lane);
          dqT[i % ND] = mfma32(fq[i], lb[i / ND], dqT[i % ND]);
        }
#pragma unroll
        for (int i = 0; i < NM - PF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }
      wait_vmcnt<0>();
      __syncthreads();
    }
    // the key halves meet: group 1 leaves its partials in the idle rings, group 0 adds them
    if (kg == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) SQ.red[w][db][r][lane] = dqT[db][r];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqT[db][r] += SQ.red[w][db][r][lane];
    }
    if (kg == 0 && qval) {
      float* dqr = a.dq + ((size_t)(seq0 + qi) * a.Hq + h) * HD;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * grp;
          *reinterpret_cast<f32x4*>(dqr + d) =
              f32x4{cnat * dqT[db][4 * r4], cnat * dqT[db][4 * r4 + 1], cnat * dqT[db][4 * r4 + 2],
                    cnat * dqT[db][4 * r4 + 3]};
        }
    }
  }
}

// ds_j = sum over kv heads of the partials; dt_h, dg_h = sum over the dK/dV workgroups
__global__ __launch_bounds__(NT) void reduce_ds_kernel(Args a) {
  const int64_t j = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (j >= a.T) return;
  float s = 0.f;
  for (int hk = 0; hk < a.Hkv; ++hk) s += a.ds_part[(size_t)hk * a.T + j];
  a.ds[j] = s;
}

template <int G>
__global__ __launch_bounds__(NT) void reduce_tg_kernel(Args a, int nwg) {
  __shared__ float red[2][NT];
  const int h = blockIdx.x, hk = h / G, gi = h % G;
  float sg = 0.f, st = 0.f;
  for (int wg = hk + threadIdx.x * a.Hkv; wg < nwg; wg += NT * a.Hkv) {
    sg += a.tg_part[((size_t)wg * G + gi) * 2];
    st += a.tg_part[((size_t)wg * G + gi) * 2 + 1];
  }
  red[0][threadIdx.x] = sg;
  red[1][threadIdx.x] = st;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      red[0][threadIdx.x] += red[0][threadIdx.x + o];
      red[1][threadIdx.x] += red[1][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.dg[h] = red[0][0];
    a.dt[h] = red[1][0];
  }
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int n_kv_wg(int B, int max_k, int Hkv, int G) {
  const int BK = 32 * (4 / G);
  const int n_kt = (max_k + BK - 1) / BK;
  return B * ((n_kt + 1) / 2) * Hkv;
}

template <int G, int HD>
hipError_t launch_gh(Args a, int max_k, void* ws, hipStream_t stream) {
  const int BK = 32 * (4 / G), BQ = 32 * (4 / G);
  a.n_kt = (max_k + BK - 1) / BK;
  a.n_qt = (max_k + BQ - 1) / BQ;
  const int nwg_kv = a.B * ((a.n_kt + 1) / 2) * a.Hkv;
  const int nwg_q = a.B * ((a.n_qt + 1) / 2) * a.Hkv;
  char* p = static_cast<char*>(ws);
  a.lse2 = reinterpret_cast<float*>(p);
  p += al256((size_t)a.Hq * a.T * 4);
  a.delta = reinterpret_cast<float*>(p);
  p += al256((size_t)a.Hq * a.T * 4);
  a.ds_part = reinterpret_cast<float*>(p);
  p += al256((size_t)a.Hkv * a.T * 4);
  a.tg_part = reinterpret_cast<float*>(p);

  const int64_t rows = (int64_t)a.T * a.Hq;
  const int64_t prep_blocks = (rows * (HD / 8) + NT - 1) / NT;
  prep_kernel<HD><<<dim3((unsigned)prep_blocks), dim3(NT), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int smem = (int)sizeof(KvSmem<G, HD>);
  e = ensure_dynamic_lds<dkdv_kernel<G, HD>>(smem);
  if (e != hipSuccess) return e;
  dkdv_kernel<G, HD><<<dim3((unsigned)nwg_kv), dim3(NT), smem, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int smem_q = (int)sizeof(QSmem<HD>);
  e = ensure_dynamic_lds<dq_kernel<G, HD>>(smem_q);
  if (e != hipSuccess) return e;
  dq_kernel<G, HD><<<dim3((unsigned)nwg_q), dim3(2 * NT), smem_q, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  reduce_ds_kernel<<<dim3((unsigned)((a.T + NT - 1) / NT)), dim3(NT), 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  reduce_tg_kernel<G><<<dim3((unsigned)a.Hq), dim3(NT), 0, stream>>>(a, nwg_kv);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_h(const Args& a, int max_k, int G, void* ws, hipStream_t stream) {
  switch (G) {
    case 1: return launch_gh<1, HD>(a, max_k, ws, stream);
    case 2: return launch_gh<2, HD>(a, max_k, ws, stream);
    case 4: return launch_gh<4, HD>(a, max_k, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace abwd

bool attn_bwd_supported(int Hq, int Hkv, int d) {
  if (Hkv <= 0 || Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4);
}

size_t attn_bwd_workspace_bytes(int B, int64_t T, int max_k, int Hq, int Hkv, int d) {
  (void)d;
  if (B <= 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return 0;
  return 2 * abwd::al256((size_t)Hq * T * 4) + abwd::al256((size_t)Hkv * T * 4) +
         abwd::al256((size_t)abwd::n_kv_wg(B, max_k, Hkv, G) * G * 2 * 4);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* s_c, const float* t,
                           const float* g, const int32_t* cu, int B, int64_t T, int max_k, int Hq, int Hkv,
                           int d, const void* o, const float* lse, const void* dO, float* dq, float* dk,
                           float* dv, float* ds, float* dt, float* dg, void* ws, hipStream_t stream) {
  abwd::Args a{};
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = static_cast<const bf16*>(o);
  a.dO = static_cast<const bf16*>(dO);
  a.lse = lse;
  a.s_c = s_c;
  a.t = t;
  a.g = g;
  a.cu = cu;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ds = ds;
  a.dt = dt;
  a.dg = dg;
  a.B = B;
  a.T = (int)T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  const int G = Hq / Hkv;
  return d == 64 ? abwd::launch_h<64>(a, max_k, G, ws, stream) : abwd::launch_h<128>(a, max_k, G, ws, stream);
}

}  // namespace tg
