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
//    exchange with lane ^ 32 (v_permlane32_swap), and P goes from the S
//    accumulator straight into the B operand of the PV product;
//  * the gate-score bias rides in the logit product: one extra 16-wide
//    k-slice per 32 keys holds (s_hi, s_lo, s_hi) of each key's score split
//    into two bf16 and, on the query side, (f_hi, f_hi, f_lo) of
//    f = g_h log2(e) / c with c = |t_h| log2(e) / sqrt(d), so the
//    accumulator is q.k + f s_c[j] to ~2^-16 relative and the log2-domain
//    logit is one multiply by c away (the sign of t_h moves into q, which is
//    exact in bf16). Per logit the softmax is then: max, one FMA (scale and
//    running-max shift), exp2, and half a bf16 pack and half a bf16 dot2
//    (the row sum adds the same rounded P that the PV product uses);
//  * software pipeline: while the VALU works on the softmax of key tile j,
//    the matrix cores compute the logits of tile j+1; K (with the tile's
//    gate scores) and V have separate 2-slot rings filled by direct-to-LDS
//    buffer loads, K two tiles ahead and V one, one barrier per 64-key tile.
//    V stays row-major: its V^T fragments come from ds_read_b64_tr_b16,
//    which hands each lane of a 16-lane group 4 keys of one feature column;
//    the key order of those fragments matches the k-slot order of P in the
//    accumulator. LDS rows are XOR-swizzled so that both the K fragment
//    reads and the transposing V reads of a phase hit distinct banks;
//  * online softmax in the log2 domain with a lazy running maximum: the
//    output rows are rescaled only when some row's tile maximum exceeds the
//    running one by more than 8 (P <= 2^8, far from overflow; exact after
//    the final division by the row sum, which uses the same reference);
//  * heavy (late) and light (early) query tiles are dispatched in pairs, so
//    every workgroup sees about the same number of key tiles; when all query
//    tiles fit one workgroup per CU, each workgroup takes a single tile,
//    heaviest first.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

template <int HD>
struct AttnLayout {
  static constexpr int RB = HD * 2;          // bytes per K or V row
  static constexpr int KCH = HD / 8;         // 16-byte chunks per row
  static constexpr int RPB = 1024 / RB;      // rows per 1 KB load block
  static constexpr int TILE = 64 * RB;       // bytes of a 64-key K (or V) tile
  // LDS: K slots 0/1, V slots 0/1, gate-score slots 0/1 (64 fp32 each)
  static constexpr int KOFF = 0, VOFF = 2 * TILE, SOFF = 4 * TILE;
  static constexpr int BYTES = 4 * TILE + 2 * 256;
  // K fragment reads: 16 lanes read 16 consecutive keys, same logical chunk
  __device__ static int kswz(int key) { return HD == 128 ? (key & 15) : ((key >> 1) & 7); }
  // V transposing reads: 32 lanes read 4 consecutive (4-aligned) keys x 4 chunks
  __device__ static int vswz(int key) { return HD == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); }
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float xmax32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int G, int HD>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ s_c, const float* __restrict__ t, const float* __restrict__ g,
    const int32_t* __restrict__ cu_kept, int B, int Hq, int Hkv, int n_qt, int single, bf16* __restrict__ o,
    float* __restrict__ lse) {
  using LY = AttnLayout<HD>;
  constexpr int WPH = 4 / G;     // waves per q-head in a group
  constexpr int BQ = 32 * WPH;   // queries per query tile
  constexpr int ND = HD / 32;    // 32-wide d blocks of O^T
  constexpr int NKB = 64 / LY::RPB;  // load blocks per K (or V) tile
  constexpr int LPW = NKB / 4;       // of them per wave
  static_assert(4 * ND * 16 * 64 * 4 + 4 * 2 * 64 * 4 <= 2 * LY::BYTES, "merge buffer fits");
  extern __shared__ __attribute__((aligned(1024))) unsigned char attn_smem[];

  const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, half = lane >> 5;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave8 >> 2;   // key-range group: 0 = first half of the keys, 1 = second
  const int wave = wave8 & 3;   // wave inside the group
  unsigned char* gsm = attn_smem + grp * LY::BYTES;  // this group's K/V/score rings
  const uint32_t glds = lds_addr(gsm);

  // Work: workgroup L takes the query-tile pair (n_qt-1-p, p) of one
  // (sequence, kv-head), one tile after the other, so every workgroup sees
  // about n_qt + 1 key tiles. Consecutive L differ in kv-head first: with 8
  // kv-heads, each XCD (L % 8) serves one head, whose K and V stay in its L2.
  // Then pairs, then sequences: the workgroups of one sequence are dispatched
  // together, so those of a head sweep its keys at about the same time and
  // share K/V tiles in L2 (with the sequences interleaved, a 16K-key sequence
  // next to short ones ran 3x slower).
  // With `single` (few query tiles: pairing would leave CUs idle) workgroup
  // L takes only the tile n_qt-1-p, p < n_qt, heavy tiles first.
  const int L = blockIdx.x;
  const int npair = single ? n_qt : (n_qt + 1) >> 1;
  const int hk = L % Hkv;
  const int p = (L / Hkv) % npair, b = L / (Hkv * npair);
  const int seq0 = cu_kept[b];
  const int Kb = cu_kept[b + 1] - seq0;
  const int Ttot = cu_kept[B];
  const int gi = wave / WPH, qs = wave % WPH;
  const int h = hk * G + gi;

  // logit scale c > 0 in log2 units; a negative t_h flips the sign of q
  // (exact in bf16); c is floored so that f = g log2(e) / c stays finite
  // (with t_h = 0 the q.k term then weighs 1e-20, i.e. nothing).
  const float cq = t[h] * TG_LOG2E / sqrtf((float)HD);
  const uint32_t qsign = cq < 0.f ? 0x80008000u : 0u;
  const float cs = fmaxf(fabsf(cq), 1e-20f);
  const float fb = g[h] * TG_LOG2E / cs;
  bf16x8 qaug;
  {
    const bf16 fh = f2bf(fb);
    const bf16 fl = f2bf(fb - bf2f(fh));
    const bf16 z = f2bf(0.f);
    qaug = bf16x8{fh, fh, fl, z, z, z, z, z};
    if (half) qaug = bf16x8{z, z, z, z, z, z, z, z};
  }

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
  const int krow0 = wave * LY::RPB + rib;  // row of this lane in the wave's first block
  const uint32_t koff = rib * row_bytes + ((slot ^ LY::kswz(krow0)) << 4);
  const uint32_t voff_l = rib * row_bytes + ((slot ^ LY::vswz(krow0)) << 4);
  // K tile kt and its gate scores -> K slot sl
  auto issue_k = [&](int kt, int sl) {
    const uint32_t sb = glds + LY::KOFF + sl * LY::TILE;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const uint32_t rowoff = (uint32_t)(kt * 64 + blk * LY::RPB) * row_bytes;
      buf_dma16(rk, koff + rowoff, __builtin_amdgcn_readfirstlane(sb + blk * 1024));
    }
    if (wave == 0)  // one gate score per lane
      buf_dma4(rsc, (uint32_t)(kt * 64 + lane) * 4u,
               __builtin_amdgcn_readfirstlane(glds + LY::SOFF + sl * 256));
  };
  auto issue_v = [&](int kt, int sl) {
    const uint32_t sb = glds + LY::VOFF + sl * LY::TILE;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const uint32_t rowoff = (uint32_t)(kt * 64 + blk * LY::RPB) * row_bytes;
      buf_dma16(rv, voff_l + rowoff, __builtin_amdgcn_readfirstlane(sb + blk * 1024));
    }
  };

  // V^T fragment source (bytes inside a V slot) for key-step kk, d block db:
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
  const int ksw = LY::kswz(l31);  // same for key l31 and 32 + l31
  const bf16x2 ones = {f2bf(1.f), f2bf(1.f)};

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? n_qt - 1 - p : p;
    if (pass == 1 && (single || qt == n_qt - 1 - p)) break;  // (or the middle tile of an odd count)
    const int q0 = qt * BQ;
    if (q0 >= Kb) continue;  // uniform over the workgroup
    const int qw0 = q0 + qs * 32;
    const int qi = qw0 + l31;
    const bool qvalid = qi < Kb;
    const int qend = min(Kb, q0 + BQ);
    const int n_kt = (qend + 63) >> 6;
    const int nh = (n_kt + 1) >> 1;      // key tiles of group 0 (also the loop count)
    const int t0 = grp ? nh : 0;         // first key tile of this group
    const int nt = grp ? n_kt - nh : nh; // key tiles of this group
    // last group-relative tile with a key <= one of this wave's queries
    const int jw = (qw0 < Kb ? min(n_kt - 1, (qw0 + 31) >> 6) : -1) - t0;

    bf16x8 qf[HD / 16];
    {
      const bf16* qrow = q + ((size_t)(seq0 + min(qi, Kb - 1)) * Hq + h) * HD + half * 8;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        u32x4 w = *reinterpret_cast<const u32x4*>(qrow + ks * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] ^= qsign;
        qf[ks] = __builtin_bit_cast(bf16x8, w);
      }
    }
    // S^T of the key tile in K slot sl: rows = keys (two blocks of 32), one
    // query per lane column; includes f * s_c[key] through the augmented slice
    auto logits = [&](int sl, f32x16(&sa)[2]) {
      const unsigned char* kb_ = gsm + LY::KOFF + sl * LY::TILE;
      const float* ss_ = reinterpret_cast<const float*>(gsm + LY::SOFF + sl * 256);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float s = ss_[kb * 32 + l31];
        const bf16 sh = f2bf(s);
        const bf16 sl_ = f2bf(s - bf2f(sh));
        const bf16 z = f2bf(0.f);
        sa[kb] = mfma32(bf16x8{sh, sl_, sh, z, z, z, z, z}, qaug, zero_f32x16());
      }
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks) {
        const int ch = ((ks * 2 + half) ^ ksw) << 4;
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kb_ + l31 * LY::RB + ch);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kb_ + (32 + l31) * LY::RB + ch);
        sa[0] = mfma32(k0, qf[ks], sa[0]);
        sa[1] = mfma32(k1, qf[ks], sa[1]);
      }
    };

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = zero_f32x16();
    float m_run = -INFINITY, l_run = 0.f;

    __syncthreads();  // the previous tile's merge has read its LDS
    if (nt > 0) {
      issue_k(t0, 0);
      issue_v(t0, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (1 < nt) issue_k(t0 + 1, 1);
    f32x16 sa[2];
    if (0 <= jw && 0 < nt) logits(0, sa);
    for (int j = 0; j < nh; ++j) {
      wait_vmcnt<0>();
      __syncthreads();  // K/scores of tile j+1 and V of tile j landed; slots of j-1 free
      if (j + 2 < nt) issue_k(t0 + j + 2, j & 1);
      if (j + 1 < nt) issue_v(t0 + j + 1, (j + 1) & 1);
      if (j >= nt || j > jw) continue;  // uniform per wave; it stays for the barriers
      const int kbase = (t0 + j) * 64;
      // keys past a query (diagonal tiles only) -> -inf
      float mr = -INFINITY;
      if (kbase + 63 > qw0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            sa[kb][r] = key > qi ? -INFINITY : sa[kb][r];
            mr = fmaxf(mr, sa[kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mr = fmaxf(mr, sa[kb][r]);
      }
      const float mx = xmax32(mr) * cs;
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
      // logits of the next tile (its K slot is ready; past the wave's last
      // tile the result is unused) overlap the exponentials of this one
      f32x16 sn[2];
      logits((j + 1) & 1, sn);
      // P in the B-operand layout of the PV product; the row sum adds the
      // same bf16 values
      bf16x8 pf[4];
      const float nm = -m_run;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[kb * 2 + (r >> 3)][r & 7] = f2bf(__builtin_amdgcn_exp2f(fmaf(sa[kb][r], cs, nm)));
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[i], pf[i], 0, 1), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[i], pf[i], 2, 3), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[i], pf[i], 4, 5), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[i], pf[i], 6, 7), ones, rs, false);
      }
      l_run += rs;
      const unsigned char* vs_ = gsm + LY::VOFF + (j & 1) * LY::TILE;
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
      sa[0] = sn[0];
      sa[1] = sn[1];
    }

    // merge the second key half into the first through LDS: wave w of group 1
    // holds the same queries and head as wave w of group 0; per lane, its 16*ND
    // unnormalised outputs (16-byte chunks, lane-fastest), running max and sum
    __syncthreads();  // both rings are idle (no load is in flight after the loop)
    f32x4* mo = reinterpret_cast<f32x4*>(attn_smem) + wave * (ND * 4 * 64) + lane;
    float* mml = reinterpret_cast<float*>(attn_smem + 4 * ND * 16 * 64 * 4) + wave * 128 + lane;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          mo[(db * 4 + rq) * 64] = f32x4{oacc[db][rq * 4], oacc[db][rq * 4 + 1], oacc[db][rq * 4 + 2],
                                         oacc[db][rq * 4 + 3]};
      mml[0] = m_run;
      mml[64] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = mml[0], l1 = mml[64];
      const float m = fmaxf(m_run, m1);
      const float a0 = __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = __builtin_amdgcn_exp2f(m1 - m);
      const float l_tot = xsum32(l_run * a0 + l1 * a1);
      if (qvalid) {
        const float inv = 1.0f / l_tot;
        const float s0 = a0 * inv, s1 = a1 * inv;
        bf16* orow = o + ((size_t)(seq0 + qi) * Hq + h) * HD + half * 4;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const f32x4 o1 = mo[(db * 4 + rq) * 64];
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = f2bf(oacc[db][rq * 4 + e] * s0 + o1[e] * s1);
            *reinterpret_cast<bf16x4*>(orow + db * 32 + rq * 8) = w;
          }
        if (lse && half == 0) lse[(size_t)h * Ttot + seq0 + qi] = (m + __log2f(l_tot)) * TG_LN2;
      }
    }
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
  constexpr size_t lds = (size_t)2 * AttnLayout<HD>::BYTES;
  {
    const hipError_t e = ensure_dynamic_lds<attn_bf16_kernel<G, HD>>((int)lds);
    if (e != hipSuccess) return e;
  }
  const int n_qt = (max_k + BQ - 1) / BQ;
  // one query-tile pair per workgroup; single tiles while they fit one
  // workgroup per CU
  const int single = (long)n_qt * Hkv * B <= device_cu_count();
  const long blocks = (long)(single ? n_qt : (n_qt + 1) / 2) * Hkv * B;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<G, HD>), dim3((unsigned)blocks), dim3(512), lds, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, s_c, t, g, cu_kept, B, Hq,
                     Hkv, n_qt, single, (bf16*)o, lse);
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
