// Dense projections of the gated path on CDNA4 matrix cores.
//
// out[m, n] = f( sum_k W[n, k] * X[m, k] ): weights in nn.Linear layout
// [out_features, in_features], activations row-major [tokens, features]; both
// operands are K-contiguous. The weight tile is the MFMA A operand and the
// token tile the B operand, so every lane ends with 4 consecutive output
// features of one token and stores 8 bytes at a time.
//
// Tiling: BK = 64 (128-byte LDS rows). A workgroup of WN x WM waves owns a
// BN (features) x BM (tokens) tile; each wave owns (BN/WN) x (BM/WM) made of
// 32x32x16 bf16 MFMA blocks with fp32 accumulators. Tiles move global -> LDS
// with gfx950 direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): no
// register staging, no per-lane predication (the buffer range check zeroes
// rows past the end), NSTAGE k-tiles in flight in an LDS ring,
// one barrier per k-tile. Each 1 KB load instruction fills 8 rows; the lane
// that lands in 16-byte slot (row, c) fetches logical chunk c ^ ((row>>1)&7),
// so the MFMA fragment reads (16 consecutive rows per 16-lane phase, same
// logical chunk) hit distinct banks of the 64-bank LDS. Rows past M or N
// read as zeros (their results are never stored).
//
// Workgroups are ordered for the 8 XCDs (private L2 each): hardware id L
// runs on XCD L % 8, in order of L / 8. The token-block x weight-block tile
// grid is cut into 8 rectangles, one per XCD, and each XCD walks its
// rectangle in groups of 4 token blocks, so the ~32 tiles an XCD runs at
// once cover about 4 token blocks x 8 weight blocks: 12 row blocks of operand
// data per round through its L2 instead of 2 + 16 (token-block-fastest
// order).
//
// Epilogues, fused on the accumulators:
//   PLAIN  : out = acc (+ residual)                         (O and down proj)
//   QKV    : rotate-half RoPE of q and k, scatter to q / k-cache / v-cache
//            (staged through LDS so rotary pairs and stores are row-wise).
//   SWIGLU : gate and up rows interleaved per 32 -> silu(g) * u (staged).
//   SCORE  : scorer logit: sum_n GELU(acc + b1[n]) * w2[n], then sigmoid
//            (the [tokens, H1] activations never reach memory)
#include <type_traits>

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
  // fused RMSNorm: row sums of squares [M][N/64] of the stored output (PLAIN),
  // and of the input rows [M][K/64] that scale QKV / SwiGLU products by
  // rsqrt(sum / K + rs_eps)
  float* ssq_out;
  const float* ssq_in;
  float rs_eps;
};

// Buffer resources of the operands: W0..W2 (weights; QKV uses all three,
// SwiGLU two) and X. Each range covers exactly its matrix, so rows past the
// end read as zeros (their results are never stored).
struct GemmRsrc {
  i32x4 w[3];
  i32x4 x;
};

// Source of load block `blk` (8 consecutive LDS rows; W rows first, then X
// rows): which resource and its first row. Every block lies inside one
// matrix (head and chunk sizes are multiples of 8), so both are uniform.
template <int MODE, int BN, int TN>
__device__ __forceinline__ void block_src(const GemmParams& p, int n0, int m0, int blk, int& which,
                                          int& r0) {
  if (blk >= BN / 8) {
    which = 3;
    r0 = m0 + (blk - BN / 8) * 8;
  } else if (MODE == MODE_SWIGLU) {
    // per wave: subtiles alternate gate (even) / up (odd) over the same 32 features
    const int ln = blk * 8;
    const int wv = ln / TN, j = (ln % TN) >> 5;
    which = j & 1;
    r0 = (n0 >> 1) + wv * (TN >> 1) + (j >> 1) * 32 + (ln & 31);
  } else if (MODE == MODE_QKV) {
    const int gn = n0 + blk * 8;
    const int nq = p.Hq * p.hd, nk = p.Hkv * p.hd;
    if (gn < nq) {
      which = 0;
      r0 = gn;
    } else if (gn < nq + nk) {
      which = 1;
      r0 = gn - nq;
    } else {
      which = 2;
      r0 = gn - nq - nk;  // past the last head: out of range, zeros
    }
  } else {
    which = 0;
    r0 = n0 + blk * 8;
  }
}

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erf_fast(z * 0.70710678118654752f));
}

template <int MODE, int BN, int BM, int WN, int WM, int NSTAGE>
__global__ __launch_bounds__(WN* WM * 64) void gemm_bf16_kernel(GemmParams p, int NB, int MB) {
  constexpr int NW = WN * WM;
  constexpr int TN = BN / WN, TM = BM / WM;   // wave tile
  constexpr int SN = TN / 32, SM = TM / 32;   // MFMA blocks per wave
  constexpr int STAGE = (BN + BM) * 128;      // bytes per LDS stage
  constexpr int NBLK = (BN + BM) / 8;         // 1 KB load blocks per stage
  // the tile loads are issued by one wave per SIMD (waves 0 .. NW/2 - 1); the
  // other wave of each SIMD only reads fragments and multiplies
  constexpr int NI = NW / 2;
  constexpr int LPW = NBLK / NI;              // load instructions per issuing wave per stage
  static_assert(NBLK % NI == 0, "load blocks must split evenly over the issuing waves");
  static_assert(MODE != MODE_SWIGLU || SN % 2 == 0, "SwiGLU pairs gate/up subtiles");

  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  // SCORE: b1 and w2 of the tile's features (zero past N), staged once; the
  // first k-tile's barrier makes them visible to the epilogue
  __shared__ float sbw[MODE == MODE_SCORE ? 2 * BN : 1];

  // XCD-aware tile order (see the file header)
  int mb, nb;
  {
    const int L = blockIdx.x;
    int RX = 0;  // XCD rectangles along the token blocks (8 / RX along weight blocks)
    if (((NB * MB) & 7) == 0) {
      if (MB % 4 == 0 && NB % 2 == 0) RX = 4;
      else if (MB % 2 == 0 && NB % 4 == 0) RX = 2;
      else if (MB % 8 == 0) RX = 8;
      else if (NB % 8 == 0) RX = 1;
    }
    if (RX) {
      const int xcd = L & 7, j = L >> 3;
      const int mbr = MB / RX, nbr = NB / (8 / RX);
      const int G = (mbr & 3) == 0 ? 4 : ((mbr & 1) == 0 ? 2 : 1);
      const int gi = j / (G * nbr), jj = j - gi * (G * nbr);
      mb = (xcd % RX) * mbr + gi * G + jj % G;
      nb = (xcd / RX) * nbr + jj / G;
    } else {
      mb = L % MB;
      nb = L / MB;
    }
  }
  const int n0 = nb * BN, m0 = mb * BM;
  if constexpr (MODE == MODE_SCORE) {
    for (int i = threadIdx.x; i < BN; i += WN * WM * 64) {
      const bool ok = n0 + i < p.N;
      sbw[i] = ok ? bf2f(p.b1[n0 + i]) : 0.f;
      sbw[BN + i] = ok ? bf2f(p.w2[n0 + i]) : 0.f;
    }
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int K = p.K;

  // lane l of a load block lands in row l/8, 16-byte slot l%8, and fetches
  // logical chunk (l%8) ^ swz(row) with swz(row) = (row >> 1) & 7: a 16-lane
  // ds_read_b128 phase covers 16 consecutive rows, whose 128-byte rows fall
  // on two halves of the 256-byte bank space, and swz takes 8 distinct values
  // over the even and over the odd rows of any aligned 16, so the phase hits
  // 16 distinct 16-byte bank groups. The swizzle of row 8*blk + l/8 depends
  // on the block's parity only, giving two per-lane byte offsets.
  const int rl = lane >> 3;
  const uint32_t lane_off0 = (uint32_t)(rl * K + ((lane & 7) ^ (rl >> 1)) * 8) * 2u;
  const uint32_t lane_off1 = (uint32_t)(rl * K + ((lane & 7) ^ (4 + (rl >> 1))) * 8) * 2u;
  GemmRsrc rs;
  {
    const uint32_t kb = (uint32_t)K * 2u;
    if (MODE == MODE_SWIGLU) {
      rs.w[0] = make_rsrc(p.W0, (uint32_t)p.I * kb);
      rs.w[1] = make_rsrc(p.W1, (uint32_t)p.I * kb);
      rs.w[2] = rs.w[1];
    } else if (MODE == MODE_QKV) {
      rs.w[0] = make_rsrc(p.W0, (uint32_t)(p.Hq * p.hd) * kb);
      rs.w[1] = make_rsrc(p.W1, (uint32_t)(p.Hkv * p.hd) * kb);
      rs.w[2] = make_rsrc(p.W2, (uint32_t)(p.Hkv * p.hd) * kb);
    } else {
      rs.w[0] = make_rsrc(p.W0, (uint32_t)p.N * kb);
      rs.w[1] = rs.w[0];
      rs.w[2] = rs.w[0];
    }
    rs.x = make_rsrc(p.X, (uint32_t)p.M * kb);
  }
  // An issuing wave's load blocks are blk = wave + NI*i. Their source (resource
  // and first row) does not depend on the k-tile, so it is resolved once; the
  // k-tile's byte offset goes in the instruction's scalar offset.
  const bool issuer = wave < NI;
  i32x4 brs[LPW];
  uint32_t bvoff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = (issuer ? wave : 0) + NI * i;
    int which, r0;
    block_src<MODE, BN, TN>(p, n0, m0, blk, which, r0);
    brs[i] = which == 3 ? rs.x : (which == 2 ? rs.w[2] : (which == 1 ? rs.w[1] : rs.w[0]));
    bvoff[i] = ((blk & 1) ? lane_off1 : lane_off0) + (uint32_t)r0 * (uint32_t)K * 2u;
  }
  auto issue = [&](int kt, int st) {
    const uint32_t base_lds = lds0 + st * STAGE + wave * 1024;
    if (issuer) {
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        buf_dma16_soff(brs[i], bvoff[i], (uint32_t)kt * 128u,
                       __builtin_amdgcn_readfirstlane(base_lds + NI * i * 1024));
    }
  };

  // fused RMSNorm (QKV, SwiGLU): threads 2t and 2t+1 request one half each of
  // the 64-feature sums of squares of token m0 + t now (held through the main
  // loop: 16 registers, not 32); the epilogue reduces them. Loading them in
  // the epilogue instead exposes their latency once per tile.
  constexpr bool ROWSCALE = MODE == MODE_QKV || MODE == MODE_SWIGLU;
  constexpr int SQV = 4;  // f32x4 per thread: up to 32 slots per token
  const int nslot = K >> 6;
  const bool sq_vec = ROWSCALE && p.ssq_in && (nslot & 7) == 0 && nslot <= 8 * SQV;
  f32x4 sqv[ROWSCALE ? SQV : 1];
  if (ROWSCALE && sq_vec && (tid >> 1) < BM && m0 + (tid >> 1) < p.M) {
    const f32x4* src =
        reinterpret_cast<const f32x4*>(p.ssq_in + (size_t)(m0 + (tid >> 1)) * nslot) + (tid & 1) * (nslot >> 3);
#pragma unroll
    for (int i = 0; i < SQV; ++i)
      if (8 * i < nslot) sqv[i] = src[i];
  }

  f32x16 acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = zero_f32x16();

  const int half = lane >> 5, rsw = (lane >> 1) & 7;  // swz of fragment row (32-aligned base + lane%32)
  const int KT = K / 64;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) issue(s, s);
  // One k-tile. Its wave's share of the loads for k-tile kt+NSTAGE-1 (ISSUE)
  // goes out after the MFMAs of k-steps 0 and 1: issuing them back to back
  // right after the barrier stalls the wave for ~500-1000 cycles (64 KB per
  // CU per k-tile through the vector-memory path) before its first MFMA, and
  // issuing them as late as k-step 3 leaves them in flight at the next wait.
  // The last NSTAGE-1 k-tiles (no loads) use a separate copy of the loop so
  // the body has no branch.
  constexpr int NR = SN + SM, NMF = SN * SM;
  static_assert(NR <= NMF, "one read per MFMA slot");
  constexpr int LPK = (LPW + 1) / 2;  // loads after each of k-steps 0 and 1
  auto ktile = [&](int kt, auto issue_c) {
    constexpr bool ISSUE = decltype(issue_c)::value;
    if (kt + NSTAGE - 2 < KT)
      wait_vmcnt<LPW * (NSTAGE - 2)>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    const int kn = kt + NSTAGE - 1, sn = kn % NSTAGE;
    const uint32_t base_lds = lds0 + sn * STAGE + wave * 1024;
    const unsigned char* st = smem + (kt % NSTAGE) * STAGE;
    const unsigned char* wb = st + (wn * TN + (lane & 31)) * 128;
    const unsigned char* xb = st + (BN + wm * TM + (lane & 31)) * 128;
    // fragments of k-step ks+1 are read while the MFMAs of ks run
    bf16x8 wf[2][SN], xf[2][SM];
    auto frag = [&](int ks, int b) {
      const int ch = ((ks * 2 + half) ^ rsw) << 4;
#pragma unroll
      for (int j = 0; j < SN; ++j) wf[b][j] = *reinterpret_cast<const bf16x8*>(wb + j * 32 * 128 + ch);
#pragma unroll
      for (int i = 0; i < SM; ++i) xf[b][i] = *reinterpret_cast<const bf16x8*>(xb + i * 32 * 128 + ch);
    };
    frag(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) frag(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int i = 0; i < SM; ++i) acc[j][i] = mfma32(wf[ks & 1][j], xf[ks & 1][i], acc[j][i]);
      if (ISSUE && issuer) {
#pragma unroll
        for (int i = ks * LPK; i < (ks + 1) * LPK; ++i)
          if (i < LPW)
            buf_dma16_soff(brs[i], bvoff[i], (uint32_t)kn * 128u,
                           __builtin_amdgcn_readfirstlane(base_lds + NI * i * 1024));
      }
    }
    // Issue order of reads and MFMAs (the scheduler would otherwise put each
    // step's reads after the previous step's MFMAs): k-step 0 reads, then
    // each later read between the MFMAs of the step before, so LDS latency
    // hides under them.
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF - NR, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
  };
  int kt = 0;
  for (; kt + NSTAGE - 1 < KT; ++kt) ktile(kt, std::true_type());
  for (; kt < KT; ++kt) ktile(kt, std::false_type());

  // ---------------- epilogues ----------------
  const int ml = lane & 31;
  if (MODE == MODE_PLAIN) {
    static_assert(MODE != MODE_PLAIN || TN == 64,
                  "the fused sum of squares for the next RMSNorm covers 64-feature slots, one per wave");
    // Stage the wave's fp32 tile in LDS ([token][feature], rows padded by 16
    // bytes so the 16 rows of a write phase hit distinct banks), then each
    // lane adds the residual and stores 8 consecutive features (16 bytes):
    // full 128-byte row segments instead of 32 scattered 16-byte pieces.
    constexpr int PADW = TN + 4;                    // floats per staged row
    constexpr int CH = NW * 64 * PADW * 4 <= STAGE * NSTAGE ? 64 : 32;  // tokens per round
    static_assert(NW * CH * PADW * 4 <= STAGE * NSTAGE, "staging fits in the LDS ring");
    float* stg = reinterpret_cast<float*>(smem) + wave * CH * PADW;
    __syncthreads();  // every wave is done with the LDS ring
#pragma unroll
    for (int c0 = 0; c0 < SM; c0 += CH / 32) {
#pragma unroll
      for (int ii = 0; ii < CH / 32; ++ii)
#pragma unroll
        for (int j = 0; j < SN; ++j)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            f32x4 v;
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = acc[j][c0 + ii][rq * 4 + t];
            *reinterpret_cast<f32x4*>(stg + (ii * 32 + ml) * PADW + j * 32 + rq * 8 + half * 4) = v;
          }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      constexpr int LPR = TN / 8;          // lanes per staged row
      constexpr int RPI = 64 / LPR;        // rows per pass
#pragma unroll
      for (int r0 = 0; r0 < CH; r0 += RPI) {
        const int r = r0 + lane / LPR, c = (lane % LPR) * 8;
        const int m = m0 + wm * TM + c0 * 32 + r;
        const int n = n0 + wn * TN + c;
        float ss = 0.f;
        if (m < p.M && n < p.N) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(stg + r * PADW + c);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(stg + r * PADW + c + 4);
          float y[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const size_t o = (size_t)m * p.N + n;
          if (p.resid) {
            const bf16x8 rr = *reinterpret_cast<const bf16x8*>(p.resid + o);
#pragma unroll
            for (int t = 0; t < 8; ++t) y[t] += bf2f(rr[t]);
          }
          bf16x8 w;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            w[t] = f2bf(y[t]);
            const float f = bf2f(w[t]);
            ss = fmaf(f, f, ss);
          }
          *reinterpret_cast<bf16x8*>(p.out + o) = w;
        }
        {
          // fused RMSNorm of the next projection: the 8 lanes of a row hold
          // its 64 features of this wave; row shifts 1, 2, 4 gather their
          // sum in lane 8c+7 (all lanes take part in the moves)
          if (p.ssq_out) {
            ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x111, 0xf, 0xf, false));
            ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x112, 0xf, 0xf, false));
            ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x114, 0xf, 0xf, false));
            if ((lane & 7) == 7 && m < p.M && n < p.N)
              p.ssq_out[(size_t)m * (p.N >> 6) + ((n0 + wn * TN) >> 6)] = ss;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next round overwrites
    }
  } else if (MODE == MODE_QKV || MODE == MODE_SWIGLU) {
    // Stage 64 tokens at a time in LDS as fp32 [token][feature] over the
    // whole workgroup tile, then let every thread finish 8-feature chunks of
    // token rows with 16-byte stores of contiguous row segments. Inside a
    // staged row the 4-feature halves of each 8-feature chunk are split into
    // two runs, so the f32x4 writes (one token per lane) and the f32x4 reads
    // (16 lanes on 16 consecutive rows, or on 16 consecutive chunks of a row)
    // are conflict-free. QKV: RoPE pairs (i, i + d/2) are both in the tile
    // (heads never straddle a 256-feature tile, and a tile holds an even
    // number of heads); a thread takes one token and one 8-dim slice j of a
    // head pair, i.e. the chunks at dims 8j and d/2 + 8j of both heads, so
    // each cos/sin value read from the RoPE table serves four outputs and
    // the two chunks of a pair are each other's partner.
    constexpr int W = MODE == MODE_QKV ? BN : BN / 2;  // staged features per token
    constexpr int RW = W + 4;                           // floats per staged row
    constexpr int CHT = 64;                             // tokens per round
    static_assert(CHT * RW * 4 <= STAGE * NSTAGE, "staging fits in the LDS ring");
    static_assert(BM % CHT == 0 && TM % 32 == 0, "token rounds cover whole MFMA blocks");
    float* stg = reinterpret_cast<float*>(smem);
    auto fpos = [](int f) { return ((f >> 2) & 1) * (W / 2) + (f >> 3) * 4 + (f & 3); };
    constexpr int CPR = W / 8;  // chunks per staged row
    // fused RMSNorm: 1 / rms of each token of the tile, after the staging rows
    float* rstd_s = stg + CHT * RW;
    static_assert(CHT * RW * 4 + BM * 4 <= STAGE * NSTAGE, "row scales fit in the LDS ring");
    if (p.ssq_in) {
      float rs = 1.f;
      if (sq_vec) {
        float a = 0.f;
        if ((tid >> 1) < BM && m0 + (tid >> 1) < p.M) {
#pragma unroll
          for (int i = 0; i < SQV; ++i)
            if (8 * i < nslot) a += (sqv[i][0] + sqv[i][1]) + (sqv[i][2] + sqv[i][3]);
        }
        // add the other half from lane ^ 1 (quad_perm 1,0,3,2; every lane takes part)
        a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xb1, 0xf, 0xf, false));
        rs = rsqrtf(a / (float)K + p.rs_eps);
      } else if (tid < BM) {
        const int m = m0 + tid;
        float a = 0.f;
        if (m < p.M)
          for (int sl = 0; sl < nslot; ++sl) a += p.ssq_in[(size_t)m * nslot + sl];
        rs = rsqrtf(a / (float)K + p.rs_eps);
      }
      __syncthreads();  // the LDS ring is no longer read
      if (sq_vec ? ((tid >> 1) < BM && (tid & 1) == 0) : tid < BM) rstd_s[sq_vec ? (tid >> 1) : tid] = rs;
    }
    static_assert(MODE != MODE_QKV || (BN == 256 && NW * 64 == CHT * 8),
                  "QKV: one (token, head pair, 8-dim slice) task per thread and round");
    // QKV task of this thread: token row qr of the round, head pair qhp, slice qj
    const int qlane = tid & 63, qwv = tid >> 6;
    const int qr = (qlane & 15) + 16 * (qwv >> 1), qu = (qlane >> 4) + 4 * (qwv & 1);
    const int qnpc = MODE == MODE_QKV ? (p.hd >> 4) : 1;  // slices per head
    const int qhp = qu / qnpc, qj = qu - qhp * qnpc;
#pragma unroll
    for (int c0 = 0; c0 < BM; c0 += CHT) {
      // QKV: cos and sin of the task's 8 dims, requested before the staging
      // barriers so that their latency overlaps the staging
      f32x4 tab[4];
      if (MODE == MODE_QKV) {
        const int m = m0 + c0 + qr, gh0 = n0 / p.hd + 2 * qhp;
        if (m < p.M && gh0 < p.Hq + p.Hkv) {
          const float* cs = p.rope + (size_t)m * p.hd + 8 * qj;
          tab[0] = *reinterpret_cast<const f32x4*>(cs);
          tab[1] = *reinterpret_cast<const f32x4*>(cs + 4);
          tab[2] = *reinterpret_cast<const f32x4*>(cs + (p.hd >> 1));
          tab[3] = *reinterpret_cast<const f32x4*>(cs + (p.hd >> 1) + 4);
        }
      }
      __syncthreads();  // the LDS ring (or the previous round) is no longer read
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        const int tl = wm * TM + i * 32;  // first tile-local token of block i
        if (tl < c0 || tl >= c0 + CHT) continue;
        float* row = stg + (tl - c0 + ml) * RW;
        if (MODE == MODE_QKV) {
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int f = wn * TN + j * 32 + rq * 8 + half * 4;
              *reinterpret_cast<f32x4*>(row + fpos(f)) =
                  f32x4{acc[j][i][rq * 4], acc[j][i][rq * 4 + 1], acc[j][i][rq * 4 + 2], acc[j][i][rq * 4 + 3]};
            }
        } else {
          const float rs = p.ssq_in ? rstd_s[tl + ml] : 1.f;  // this lane's token
#pragma unroll
          for (int jj = 0; jj < SN / 2; ++jj)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              f32x4 y;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const float gt = acc[2 * jj][i][rq * 4 + t] * rs, up = acc[2 * jj + 1][i][rq * 4 + t] * rs;
                y[t] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;  // v_rcp_f32: 1 ulp
              }
              *reinterpret_cast<f32x4*>(row + fpos(wn * (TN / 2) + jj * 32 + rq * 8 + half * 4)) = y;
            }
        }
      }
      __syncthreads();
      if (MODE == MODE_QKV) {
        const int m = m0 + c0 + qr;
        const int hd = p.hd, hh = hd >> 1;
        const float* row = stg + qr * RW;
        const float rs = p.ssq_in ? rstd_s[c0 + qr] : 1.f;
        const float c[8] = {tab[0][0], tab[0][1], tab[0][2], tab[0][3], tab[1][0], tab[1][1], tab[1][2], tab[1][3]};
        const float sn[8] = {tab[2][0], tab[2][1], tab[2][2], tab[2][3], tab[3][0], tab[3][1], tab[3][2], tab[3][3]};
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int h = 2 * qhp + e2;  // head inside the tile
          const int gh = n0 / hd + h;
          if (m >= p.M || gh >= p.Hq + 2 * p.Hkv) continue;
          const int flo = h * hd + 8 * qj, fhi = flo + hh;
          const f32x4 la = *reinterpret_cast<const f32x4*>(row + fpos(flo));
          const f32x4 lb = *reinterpret_cast<const f32x4*>(row + fpos(flo + 4));
          const f32x4 ha = *reinterpret_cast<const f32x4*>(row + fpos(fhi));
          const f32x4 hb = *reinterpret_cast<const f32x4*>(row + fpos(fhi + 4));
          float ylo[8] = {la[0] * rs, la[1] * rs, la[2] * rs, la[3] * rs,
                          lb[0] * rs, lb[1] * rs, lb[2] * rs, lb[3] * rs};
          float yhi[8] = {ha[0] * rs, ha[1] * rs, ha[2] * rs, ha[3] * rs,
                          hb[0] * rs, hb[1] * rs, hb[2] * rs, hb[3] * rs};
          if (gh < p.Hq + p.Hkv) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float xl = ylo[t], xh = yhi[t];
              ylo[t] = xl * c[t] - xh * sn[t];
              yhi[t] = xh * c[t] + xl * sn[t];
            }
          }
          bf16* dst;
          if (gh < p.Hq)
            dst = p.q + (size_t)m * p.Hq * hd + gh * hd;
          else if (gh < p.Hq + p.Hkv)
            dst = p.kc + (size_t)m * p.Hkv * hd + (gh - p.Hq) * hd;
          else
            dst = p.vc + (size_t)m * p.Hkv * hd + (gh - p.Hq - p.Hkv) * hd;
          bf16x8 wl, wh;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            wl[t] = f2bf(ylo[t]);
            wh[t] = f2bf(yhi[t]);
          }
          *reinterpret_cast<bf16x8*>(dst + 8 * qj) = wl;
          *reinterpret_cast<bf16x8*>(dst + hh + 8 * qj) = wh;
        }
      } else {
        for (int task = tid; task < CHT * CPR; task += NW * 64) {
          const int r = task / CPR, f = (task % CPR) * 8;
          const int m = m0 + c0 + r;
          if (m >= p.M) continue;
          const float* row = stg + r * RW;
          const f32x4 xa = *reinterpret_cast<const f32x4*>(row + fpos(f));
          const f32x4 xb = *reinterpret_cast<const f32x4*>(row + fpos(f + 4));
          const int idx = (n0 >> 1) + f;
          if (idx >= p.I) continue;
          bf16x8 w;
          w[0] = f2bf(xa[0]);
          w[1] = f2bf(xa[1]);
          w[2] = f2bf(xa[2]);
          w[3] = f2bf(xa[3]);
          w[4] = f2bf(xb[0]);
          w[5] = f2bf(xb[1]);
          w[6] = f2bf(xb[2]);
          w[7] = f2bf(xb[3]);
          *reinterpret_cast<bf16x8*>(p.act + (size_t)m * p.I + idx) = w;
        }
      }
    }
  } else {  // SCORE
    float part[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) part[i] = 0.f;
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int nl = wn * TN + j * 32 + rq * 8 + half * 4 + t;  // features past N: b1 = w2 = 0
          const float bb = sbw[nl], ww = sbw[BN + nl];
#pragma unroll
          for (int i = 0; i < SM; ++i) part[i] += gelu_erf(acc[j][i][rq * 4 + t] + bb) * ww;
        }
    __syncthreads();  // every wave is done with the LDS ring
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      part[i] += __shfl_xor(part[i], 32, 64);
      if (half == 0) red[wn * BM + wm * TM + i * 32 + ml] = part[i];
    }
    __syncthreads();
    for (int r = tid; r < BM; r += NW * 64) {
      const int m = m0 + r;
      if (m >= p.M) continue;
      float u = 0.f;
#pragma unroll
      for (int w = 0; w < WN; ++w) u += red[w * BM + r];
      if (NB == 1) {
        u += bf2f(p.b2[0]);
        p.s_out[m] = 1.0f / (1.0f + expf(-u));
      } else {
        p.partial[(size_t)nb * p.M + m] = u;
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

template <int MODE, int BN, int BM, int WN, int WM, int NSTAGE>
static hipError_t launch_gemm(const GemmParams& p, int Ncols, hipStream_t stream) {
  constexpr size_t lds = (size_t)NSTAGE * (BN + BM) * 128;
  static_assert(lds <= 160 * 1024, "LDS budget");
  {
    const hipError_t e = ensure_dynamic_lds<gemm_bf16_kernel<MODE, BN, BM, WN, WM, NSTAGE>>((int)lds);
    if (e != hipSuccess) return e;
  }
  const int NB = (Ncols + BN - 1) / BN, MB = (p.M + BM - 1) / BM;
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, BN, BM, WN, WM, NSTAGE>), dim3(NB * MB),
                     dim3(WN * WM * 64), lds, stream, p, NB, MB);
  return hipGetLastError();
}

// Tile choice (measured on MI355X at M = 4096 tokens): 8 waves per workgroup
// (two per SIMD, so one wave's MFMAs cover the other's LDS and barrier
// waits). 256 x 256 tiles (64 x 128 per wave, 2-stage ring) whenever they
// give every CU at least one tile (gate/up, QKV); 256 x 128 tiles (64 x 64
// per wave, 3-stage ring) when 256 x 256 would leave CUs idle (O, down).
// A 32-wide k-tile with a deeper ring measured slower for every shape.
template <int MODE>
static hipError_t launch_auto(const GemmParams& p, int Ncols, hipStream_t stream) {
  const long tA = (long)((Ncols + 255) / 256) * ((p.M + 255) / 256);
  if (tA >= 256) return launch_gemm<MODE, 256, 256, 4, 2, 2>(p, Ncols, stream);
  return launch_gemm<MODE, 256, 128, 4, 2, 3>(p, Ncols, stream);
}

hipError_t gemm_bf16_plain(const bf16* X, const bf16* W, const bf16* resid, bf16* out, int M,
                           int N, int K, hipStream_t stream, float* ssq_out) {
  if (M <= 0) return hipSuccess;
  GemmParams p{};
  p.X = X;
  p.M = M;
  p.N = N;
  p.K = K;
  p.W0 = W;
  p.resid = resid;
  p.out = out;
  p.ssq_out = ssq_out;  // both PLAIN tilings have 64-feature wave tiles
  return launch_auto<MODE_PLAIN>(p, N, stream);
}

hipError_t gemm_bf16_qkv(const bf16* X, const bf16* wq, const bf16* wk, const bf16* wv,
                         const QkvOut& o, int M, int K, hipStream_t stream, const float* ssq_in,
                         float eps) {
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
  p.ssq_in = ssq_in;
  p.rs_eps = eps;
  return launch_auto<MODE_QKV>(p, p.N, stream);
}

hipError_t gemm_bf16_swiglu(const bf16* X, const bf16* wg, const bf16* wu, bf16* act, int M,
                            int I, int K, hipStream_t stream, const float* ssq_in, float eps) {
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
  p.ssq_in = ssq_in;
  p.rs_eps = eps;
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
  hipError_t e = launch_gemm<MODE_SCORE, 256, 128, 4, 2, 3>(p, H1, stream);
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
