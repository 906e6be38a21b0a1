// Gated DeltaNet mixer, chunked form (bf16 inputs): the token recurrence of
// the gated delta rule rewritten over chunks of C = 64 tokens so that the
// work is matrix products on the matrix cores instead of a per-token chain.
//
// The recurrence (Tencent Cloud TokenGate article, section on the gate
// position: the hybrid model's Gated DeltaNet layers run on the kept tokens),
// per head with state S [dv, dk]:
//   k^ = k / |k|,  q^ = q / (|q| sqrt(dk))
//   S_t = a_t S_{t-1} + b_t (v_t - a_t S_{t-1} k^_t) k^_t^T,  o_t = S_t q^_t
// Inside a chunk with start state S0 and cumulative decay g_i = a_1 ... a_i,
// S_i = g_i S0 + sum_{j<=i} (g_i / g_j) u_j k^_j^T holds with
//   u_i = b_i (v_i - g_i S0 k^_i - sum_{j<i} (g_i / g_j) (k^_j . k^_i) u_j),
// i.e. (I + diag(b) A) U = diag(b) (V - diag(g) K^ S0^T) with A the strictly
// lower (g_i / g_j) k^_i . k^_j. With T = (I + diag(b) A)^-1:
//   U   = T diag(b) V - T diag(b g) K^ S0^T            (= Ut + WN S0^T)
//   O   = diag(g) Q^ S0^T + (Q^ K^T o (g_i / g_j) [j <= i]) U
//   S_C = g_C S0 + U^T diag(g_C / g) K^
// (the chunked gated delta rule of the Gated DeltaNet paper, Yang, Kautz and
// Hatamizadeh, 2024, derived here in this notation).
//
//  prep kernel (one workgroup per chunk and head, all chunks in parallel):
//    norms, log-decay prefix, K K^T and Q K^T on MFMA, the unit lower system
//    solved for T by forward substitution in fp32, then WN = -T diag(b g) K^
//    and Ut = T diag(b) V on MFMA (T split into two bf16 halves); writes WN,
//    QG = diag(g) Q^, PG = the masked decayed Q^ K^T, KT = (diag(g_C/g) K^)^T,
//    Ut and g_C per chunk and head to the workspace.
//  scan kernel (one workgroup per sequence, head and 32 rows of S, chunks in
//    order): per chunk U = Ut + WN S0^T and O = QG S0^T (phase A), then
//    S^T <- g_C S^T + KT U and O += PG U (phase B); the state stays in the
//    accumulator registers (fp32), with a bf16 copy in LDS as the MFMA
//    operand; the next chunk's operands are loaded during the current one.
// Rows past a sequence's end are padded with a = 1, b = 0, k = q = v = 0,
// which leaves the state unchanged; their outputs are not stored.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace gdnc {

constexpr int C = 64, NT = 256;
constexpr float EPS = 1e-6f;
constexpr float LOGA_MIN = -80.f;  // log-decay floor: a = 0 acts as e^-80 inside a chunk

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One (chunk, head) record of the workspace. Every matrix is stored with the
// 16-byte pieces of each row permuted (piece c of row r at c ^ swz(r)), so
// that the scan kernel's linear copies into LDS give a layout in which a
// 16-lane read of 16 consecutive rows, same logical piece, hits 16 distinct
// 16-byte bank groups: swz(r) = r & 15 for 256-byte rows, (r >> 1) & 7 for
// 128-byte rows (two rows share the 256-byte bank space).
template <int DK>
struct Rec {
  static constexpr size_t WN = 0;                          // [C][DK] bf16
  static constexpr size_t QG = WN + (size_t)C * DK * 2;    // [C][DK] bf16
  static constexpr size_t PG = QG + (size_t)C * DK * 2;    // [C][C] bf16
  static constexpr size_t KT = PG + (size_t)C * C * 2;     // [DK][C] bf16
  static constexpr size_t GC = KT + (size_t)DK * C * 2;    // fp32 (its own 1 KB)
  static constexpr size_t UT = GC + 1024;                  // dv / 32 blocks of [32 features][C] fp32
  static constexpr size_t HEAD = UT;                       // bytes every scan workgroup copies
  __host__ __device__ static size_t bytes(int dv) { return UT + (size_t)C * dv * 4; }
};

// byte offset of element e (of `esz` bytes) of row r in a row of `rb` bytes
__device__ __forceinline__ uint32_t swz_off(int r, int e, int esz, int rb) {
  const int c = e * esz / 16, in = e * esz % 16;
  const int sw = rb == 256 ? (r & 15) : ((r >> 1) & 7);
  return (uint32_t)(r * rb + ((c ^ sw) << 4) + in);
}
// byte offset of 16-byte piece c of row r
__device__ __forceinline__ uint32_t swz_piece(int r, int c, int rb) {
  const int sw = rb == 256 ? (r & 15) : ((r >> 1) & 7);
  return (uint32_t)(r * rb + ((c ^ sw) << 4));
}

// first chunk slot of sequence b: cu[b] / C + b (slot ranges of consecutive
// sequences never overlap; ceil(T / C) + B slots cover a batch)
__device__ __forceinline__ int slot_base(const int32_t* cu, int b) { return cu[b] / C + b; }

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of 16 lanes
__device__ __forceinline__ float sum16(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  return v;
}

__device__ __forceinline__ float sq8(const u32x4& r) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(r[i] << 16), hi = __uint_as_float(r[i] & 0xffff0000u);
    acc = fmaf(lo, lo, fmaf(hi, hi, acc));
  }
  return acc;
}

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* alpha;
  const float* beta;
  const int32_t* cu;
  const float* state_in;
  bf16* o;
  float* state_out;
  unsigned char* ws;
  int64_t T;      // rows of q, k, v and o: tokens at or past T are never read or written
  int64_t nslot;  // chunk records in the workspace
  int B, H, dv;
};

// ---------------------------------------------------------------------------
// prep kernel
// ---------------------------------------------------------------------------
template <int DK>
struct PrepSmem {
  bf16 k[C][DK + 8];  // raw k rows of the chunk (zeros past the end)
  union {
    bf16 q[C][DK + 8];   // raw q rows (first phase)
    float m[C][C + 4];   // strictly lower part of the system matrix (substitution)
    struct {
      bf16 hi[C][C + 8];
      bf16 lo[C][C + 8];
    } t;                 // T = hi + lo (products)
  } u;
  bf16 xt[DK][C + 8];  // right operand of T X, transposed: (b g k^)^T, then (b v)^T blocks
  float tf[C][C + 4];  // T in fp32 (blocked solve)
  float xb[3][16][17]; // block products of one block diagonal of the solve
  float nk[C], nq[C], lg[C], be[C];
  float eg[C], egc[C];  // g_j and g_C / g_j
};

// Y = T X for 2 * DK / 32 output tiles of 32 x 32 (rows of T, columns of X),
// X^T in xt; tile index ti = (row block, column block); fn(ti, acc) consumes each
template <int DK, class Fn>
__device__ __forceinline__ void t_times_x(PrepSmem<DK>& S, int w, int lane, Fn&& fn) {
  constexpr int NTILE = 2 * (DK / 32);
  const int l31 = lane & 31, hf = lane >> 5;
  for (int ti = w; ti < NTILE; ti += 4) {
    const int rb = ti & 1, cb = ti >> 1;
    f32x16 acc = zero_f32x16();
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int kc = 16 * ks + 8 * hf;
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&S.u.t.hi[32 * rb + l31][kc]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&S.u.t.lo[32 * rb + l31][kc]);
      const bf16x8 bx = *reinterpret_cast<const bf16x8*>(&S.xt[32 * cb + l31][kc]);
      acc = mfma32(ah, bx, acc);
      acc = mfma32(al, bx, acc);
    }
    fn(rb, cb, acc);
  }
}

// Both kernels are bounded to two waves per SIMD (256 registers per wave): with
// that bound the compiler accumulates the MFMAs in ordinary vector registers;
// allowed the whole register file it used the accumulation registers and
// copied every accumulator in and out around the MFMAs (their results are
// read by vector instructions right after).
template <int DK>
__global__ __launch_bounds__(NT, 2) void prep_kernel(Args A) {
  using R = Rec<DK>;
  __shared__ __attribute__((aligned(16))) PrepSmem<DK> S;
  const int H = A.H, dv = A.dv;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  // sequence of this slot: the last b with slot_base(b) <= slot
  int b;
  {
    int lo = 0, hi = A.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (slot_base(A.cu, mid) <= slot)
        lo = mid;
      else
        hi = mid - 1;
    }
    b = lo;
  }
  const int t0 = A.cu[b], L = A.cu[b + 1] - t0;
  const int c = slot - slot_base(A.cu, b);
  const int tb = t0 + c * C;  // first token of the chunk
  // rows of the chunk: past the sequence's end (or past T) they are padding
  const int n = (int)min((int64_t)min(C, L - c * C), A.T - tb);
  if (n <= 0 || c < 0 || tb < 0) return;  // a gap slot (uniform over the workgroup)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l31 = lane & 31, hf = lane >> 5;
  unsigned char* rec = A.ws + ((size_t)slot * H + h) * R::bytes(dv);

  // ---- rows of k and q into LDS, their norms; decay prefix and b ----
  constexpr int KCH = DK / 8;                // 16-byte pieces per row
  constexpr int PPT = C * KCH / NT;          // pieces per thread and matrix
  static_assert(C * KCH % NT == 0 && NT % KCH == 0, "piece split");
  {
    // every load in flight before the first use
    u32x4 x[2][PPT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int p = tid + i * NT, r = p / KCH, c16 = p % KCH;
        x[m][i] = u32x4{0u, 0u, 0u, 0u};
        if (r < n)
          x[m][i] = *reinterpret_cast<const u32x4*>((m ? A.q : A.k) + ((size_t)(tb + r) * H + h) * DK + 8 * c16);
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int p = tid + i * NT, r = p / KCH, c16 = p % KCH;
        *reinterpret_cast<u32x4*>(m ? &S.u.q[r][8 * c16] : &S.k[r][8 * c16]) = x[m][i];
        // the KCH pieces of a row sit in KCH consecutive lanes
        float s2 = sq8(x[m][i]);
        if constexpr (KCH == 16) {
          s2 = sum16(s2);
        } else {
          s2 += dppf<0xB1>(s2);
          s2 += dppf<0x4E>(s2);
          s2 += dppf<0x141>(s2);
        }
        if (c16 == 0) {
          const float inv = rsqrtf(s2 + EPS);
          if (m)
            S.nq[r] = inv * rsqrtf((float)DK);
          else
            S.nk[r] = inv;
        }
      }
  }
  if (w == 0) {
    const bool live = lane < n;
    const float a = live ? A.alpha[(size_t)(tb + lane) * H + h] : 1.f;
    float la = fmaxf(__logf(a), LOGA_MIN);
    // inclusive prefix sum over the 64 lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(la, o, 64);
      if (lane >= o) la += y;
    }
    S.lg[lane] = la;
    S.eg[lane] = __expf(la);
    S.egc[lane] = __expf(__shfl(la, 63, 64) - la);
    S.be[lane] = live ? A.beta[(size_t)(tb + lane) * H + h] : 0.f;
  }
  __syncthreads();

  // ---- K K^T and K Q^T (raw bf16 products, fp32 accumulators), QG ----
  // wave w: tile (rows 32 ti.., columns 32 tj..) of K K^T and tile (rows j in
  // 32 tj.., columns i in 32 ti..) of K Q^T, so that a lane ends with four
  // consecutive j of one row i of the stored product
  const int ti = w >> 1, tj = w & 1;
  f32x16 g = zero_f32x16(), pq = zero_f32x16();
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks) {
    const int kc = 16 * ks + 8 * hf;
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&S.k[32 * ti + l31][kc]);
    const bf16x8 qb = *reinterpret_cast<const bf16x8*>(&S.u.q[32 * ti + l31][kc]);
    const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&S.k[32 * tj + l31][kc]);
    g = mfma32(ka, kb, g);
    pq = mfma32(kb, qb, pq);
  }
  // QG[i][d] = g_i nq_i q_i[d]
  for (int p = tid; p < C * DK / 8; p += NT) {
    const int r = p / KCH, c16 = p % KCH;
    const float sc = S.eg[r] * S.nq[r];
    const u32x4 x = *reinterpret_cast<const u32x4*>(&S.u.q[r][8 * c16]);
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = f2bf(__uint_as_float(x[e] << 16) * sc);
      y[2 * e + 1] = f2bf(__uint_as_float(x[e] & 0xffff0000u) * sc);
    }
    *reinterpret_cast<bf16x8*>(rec + R::QG + swz_piece(r, c16, DK * 2)) = y;
  }
  __syncthreads();  // q is no longer read: its space becomes the system matrix
  {
    // K K^T: lane holds column j = 32 tj + l31, rows i = 32 ti + 8 (r/4) + 4 hf + r%4
    const int j = 32 * tj + l31;
    const float nkj = S.nk[j], lgj = S.lg[j];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hf + (r & 3);
      const float dec = j < i ? __expf(S.lg[i] - lgj) : 0.f;  // g_i / g_j <= 1 below the diagonal
      S.u.m[i][j] = S.be[i] * dec * S.nk[i] * nkj * g[r];
    }
    // K Q^T: lane holds column i = 32 ti + l31, rows j = 32 tj + 8 (r/4) + 4 hf + r%4;
    // PG[i][j] = nq_i nk_j (g_i / g_j) q_i . k_j for j <= i, four j per 8-byte store
    const int i = 32 * ti + l31;
    const float nqi = S.nq[i], lgi = S.lg[i];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int j0 = 32 * tj + 8 * g4 + 4 * hf;
      bf16x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = j0 + e;
        const float dec = jj <= i ? __expf(lgi - S.lg[jj]) : 0.f;
        y[e] = f2bf(nqi * S.nk[jj] * dec * pq[4 * g4 + e]);
      }
      *reinterpret_cast<bf16x4*>(rec + R::PG + swz_off(i, j0, 2, C * 2)) = y;
    }
  }
  __syncthreads();

  // ---- T = (I + M)^-1, blocked in 16 x 16: wave 0 solves the four diagonal
  // blocks by forward substitution (lane = block and column); then every
  // thread takes part in the off-diagonal blocks, one block diagonal at a
  // time: X_IJ = sum_{J<=K<I} M_IK T_KJ, T_IJ = -T_II X_IJ ----
  if (w == 0) {
    const int bb = lane >> 4, c = lane & 15;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a0 = i == c ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < i; j4 += 4) {
        const f32x4_t mr = *reinterpret_cast<const f32x4_t*>(&S.u.m[16 * bb + i][16 * bb + j4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j4 + e < i) {
            if (e & 1)
              a1 = fmaf(-mr[e], tc[j4 + e], a1);
            else
              a0 = fmaf(-mr[e], tc[j4 + e], a0);
          }
      }
      tc[i] = a0 + a1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) S.tf[16 * bb + i][16 * bb + c] = tc[i];  // zeros above the diagonal
  }
  {
    // KT[d][j] = (g_C / g_j) k^_j[d] to the workspace, (b g k^)^T into xt (16 bytes at a time)
    for (int p = tid; p < DK * (C / 8); p += NT) {
      const int d = p / (C / 8), jc = p % (C / 8);
      bf16x8 ykt, yx;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 8 * jc + e;
        const float kv = bf2f(S.k[j][d]) * S.nk[j];
        ykt[e] = f2bf(S.egc[j] * kv);
        yx[e] = f2bf(S.be[j] * S.eg[j] * kv);
      }
      *reinterpret_cast<bf16x8*>(rec + R::KT + swz_piece(d, jc, C * 2)) = ykt;
      *reinterpret_cast<bf16x8*>(&S.xt[d][8 * jc]) = yx;
    }
    if (tid == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(S.lg[C - 1]);
  }
  __syncthreads();
  {
    const int oi = tid >> 4, oc = tid & 15;
#pragma unroll
    for (int dd = 1; dd < 4; ++dd) {
#pragma unroll
      for (int I = dd; I < 4; ++I) {
        const int J = I - dd;
        float x0 = 0.f, x1 = 0.f;
#pragma unroll
        for (int K = J; K < I; ++K)
#pragma unroll
          for (int k4 = 0; k4 < 16; k4 += 4) {
            const f32x4_t mr = *reinterpret_cast<const f32x4_t*>(&S.u.m[16 * I + oi][16 * K + k4]);
            x0 = fmaf(mr[0], S.tf[16 * K + k4][16 * J + oc], x0);
            x1 = fmaf(mr[1], S.tf[16 * K + k4 + 1][16 * J + oc], x1);
            x0 = fmaf(mr[2], S.tf[16 * K + k4 + 2][16 * J + oc], x0);
            x1 = fmaf(mr[3], S.tf[16 * K + k4 + 3][16 * J + oc], x1);
          }
        S.xb[I - dd][oi][oc] = x0 + x1;
      }
      __syncthreads();
#pragma unroll
      for (int I = dd; I < 4; ++I) {
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < 16; k4 += 4) {
          const f32x4_t tr = *reinterpret_cast<const f32x4_t*>(&S.tf[16 * I + oi][16 * I + k4]);
          y0 = fmaf(tr[0], S.xb[I - dd][k4][oc], y0);
          y1 = fmaf(tr[1], S.xb[I - dd][k4 + 1][oc], y1);
          y0 = fmaf(tr[2], S.xb[I - dd][k4 + 2][oc], y0);
          y1 = fmaf(tr[3], S.xb[I - dd][k4 + 3][oc], y1);
        }
        S.tf[16 * I + oi][16 * (I - dd) + oc] = -(y0 + y1);
      }
      __syncthreads();
    }
  }
  // every read of M is done: T overwrites it, split in two bf16 (zero above the diagonal)
  for (int p = tid; p < C * C; p += NT) {
    const int i = p / C, j = p % C;
    const float t = j > i ? 0.f : S.tf[i][j];
    const bf16 th = f2bf(t);
    S.u.t.hi[i][j] = th;
    S.u.t.lo[i][j] = f2bf(t - bf2f(th));
  }
  __syncthreads();

  // ---- WN = -T diag(b g) K^, as W^T = X^T T^T (rows d, columns i): a lane
  // ends with four consecutive d of one row i ----
  {
    constexpr int NTILE = 2 * (DK / 32);
    for (int tt = w; tt < NTILE; tt += 4) {
      const int ib = tt & 1, db = tt >> 1;
      f32x16 acc = zero_f32x16();
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const int kc = 16 * ks + 8 * hf;
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&S.xt[32 * db + l31][kc]);
        const bf16x8 th = *reinterpret_cast<const bf16x8*>(&S.u.t.hi[32 * ib + l31][kc]);
        const bf16x8 tl = *reinterpret_cast<const bf16x8*>(&S.u.t.lo[32 * ib + l31][kc]);
        acc = mfma32(xa, th, acc);
        acc = mfma32(xa, tl, acc);
      }
      const int i = 32 * ib + l31;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = f2bf(-acc[4 * g4 + e]);
        *reinterpret_cast<bf16x4*>(rec + R::WN + swz_off(i, d0, 2, DK * 2)) = y;
      }
    }
  }
  // ---- Ut = T diag(b) V, DK columns of V at a time ----
  unsigned char* ut = rec + R::UT;  // block col / 32: [32 features][C rows] fp32
  for (int c0 = 0; c0 < dv; c0 += DK) {
    __syncthreads();  // the previous product has read xt
    constexpr int VPT = C * (DK / 8) / NT;  // 16-byte pieces of V per thread
    u32x4 xv[VPT];
#pragma unroll
    for (int ii = 0; ii < VPT; ++ii) {
      const int p = tid + ii * NT, j = p / (DK / 8), cp = p % (DK / 8);
      xv[ii] = u32x4{0u, 0u, 0u, 0u};
      if (j < n && c0 + 8 * cp < dv)
        xv[ii] = *reinterpret_cast<const u32x4*>(A.v + ((size_t)(tb + j) * H + h) * dv + c0 + 8 * cp);
    }
#pragma unroll
    for (int ii = 0; ii < VPT; ++ii) {
      const int p = tid + ii * NT, j = p / (DK / 8), cp = p % (DK / 8);
      const float bj = S.be[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S.xt[8 * cp + 2 * e][j] = f2bf(bj * __uint_as_float(xv[ii][e] << 16));
        S.xt[8 * cp + 2 * e + 1][j] = f2bf(bj * __uint_as_float(xv[ii][e] & 0xffff0000u));
      }
    }
    __syncthreads();
    t_times_x<DK>(S, w, lane, [&](int rb, int cb, const f32x16& acc) {
      const int col = c0 + 32 * cb + l31;
      if (col < dv) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int i0 = 32 * rb + 8 * g4 + 4 * hf;
          f32x4_t y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[4 * g4 + e];
          *reinterpret_cast<f32x4_t*>(ut + (size_t)(col >> 5) * (32 * C * 4) + swz_off(col & 31, i0, 4, C * 4)) = y;
        }
      }
    });
  }
}

// ---------------------------------------------------------------------------
// scan kernel
// ---------------------------------------------------------------------------
template <int DK>
struct ScanSmem {
  static constexpr int STAGE = (int)Rec<DK>::HEAD + 32 * C * 4;  // a record's shared part + one U block
  unsigned char st[2][STAGE];  // the current and the next chunk's operands
  bf16 s[32][DK + 8];          // chunk-start state, rows r of this block: S[r][d] in bf16
  bf16 u[32][C + 8];           // U^T[r][j] of the chunk
  bf16 o[C][32];               // the chunk's output tile, rows i, features r0 .. r0 + 31
};

template <int DK>
__global__ __launch_bounds__(NT, 2) void scan_kernel(Args A) {
  using R = Rec<DK>;
  using SM = ScanSmem<DK>;
  constexpr int DKT = DK / 32;  // tiles of S^T (one per wave w < DKT)
  constexpr int NP = SM::STAGE / 1024;  // 1 KB copies per stage
  static_assert(SM::STAGE % 1024 == 0, "stage in whole 1 KB copies");
  extern __shared__ __attribute__((aligned(1024))) unsigned char gdn_smem[];
  SM& S = *reinterpret_cast<SM*>(gdn_smem);
  const int H = A.H, dv = A.dv, nrb = dv / 32;
  const int rb = blockIdx.x % nrb, h = (blockIdx.x / nrb) % H, b = blockIdx.x / (nrb * H);
  const int r0 = rb * 32;
  const int t0 = A.cu[b], L = A.cu[b + 1] - t0;
  const int sb = slot_base(A.cu, b);
  // chunks of the sequence (none past the workspace's records)
  const int nch = t0 < 0 ? 0 : (int)min((int64_t)((L + C - 1) / C), A.nslot - sb);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l31 = lane & 31, hf = lane >> 5;
  const size_t rbytes = R::bytes(dv);

  // copy chunk c's operands into stage sl: the record's shared part, then
  // this workgroup's U block (1 KB per wave instruction, direct to LDS);
  // wave w copies pieces w, w + 4, ...; part k of PARTS issues its share k
  constexpr int PPW = (NP + 3) / 4, PARTS = 4, PPP = (PPW + PARTS - 1) / PARTS;
  auto issue = [&](int c, int sl, int part) {
    const unsigned char* rec = A.ws + ((size_t)(sb + c) * H + h) * rbytes;
    const uint32_t dst = lds_addr(&S.st[sl][0]);
#pragma unroll
    for (int ii = 0; ii < PPP; ++ii) {
      const int p = w + 4 * (part * PPP + ii);
      if (part * PPP + ii < PPW && p < NP) {
        const unsigned char* src = p < (int)(R::HEAD / 1024) ? rec + (size_t)p * 1024
                                                              : rec + R::UT + (size_t)rb * (32 * C * 4) +
                                                                    (size_t)(p - R::HEAD / 1024) * 1024;
        lds_dma16(src + lane * 16, __builtin_amdgcn_readfirstlane(dst + p * 1024));
      }
    }
  };

  // S^T tile of wave w: lane holds column r = l31, rows d = 32 w + 8 (q/4) + 4 hf + q%4
  f32x16 st = zero_f32x16();
  const size_t so = (((size_t)b * H + h) * dv + r0 + l31) * DK;
  if (w < DKT && A.state_in) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(A.state_in + so + 32 * w + 8 * g4 + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) st[4 * g4 + e] = x[e];
    }
  }
  auto put_state = [&]() {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = f2bf(st[4 * g4 + e]);
      *reinterpret_cast<bf16x4*>(&S.s[l31][32 * w + 8 * g4 + 4 * hf]) = y;
    }
  };
  if (w < DKT) put_state();
  // chunk c's output tile leaves from LDS at the start of the next iteration,
  // 16 bytes per thread (its stores then have a whole chunk to complete
  // before the wave's next wait)
  auto store_o = [&](int c) {
    const int i = tid >> 2, pc = tid & 3;
    const int64_t t = (int64_t)t0 + c * C + i;
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(&S.o[i][8 * pc]);
    if (c * C + i < L && t < A.T) *reinterpret_cast<bf16x8*>(A.o + ((size_t)t * H + h) * dv + r0 + 8 * pc) = y;
  };
  if (nch > 0) {
#pragma unroll
    for (int part = 0; part < PARTS; ++part) issue(0, 0, part);
  }
  wait_vmcnt<0>();
  __syncthreads();  // chunk 0's operands and the bf16 state are in LDS
  const int ta = w & 1;  // row block of U (waves 0, 1) or O (waves 2, 3)
  for (int c = 0; c < nch; ++c) {
    const int sl = c & 1;
    const unsigned char* stg = S.st[sl];
    const bool more = c + 1 < nch;
    if (c > 0) store_o(c - 1);
    // phase A: U = Ut + WN S0^T (waves 0, 1), O = QG S0^T (waves 2, 3);
    // every operand read is issued before the MFMAs, the copies of the next
    // chunk (into the stage read before the previous barrier) between them
    f32x16 acc;
    {
      bf16x8 af[DK / 16], sf[DK / 16];
      const unsigned char* am = stg + (w < 2 ? R::WN : R::QG);
      const int ar = 32 * ta + l31;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) {
        af[ks] = *reinterpret_cast<const bf16x8*>(am + swz_piece(ar, 2 * ks + hf, DK * 2));
        sf[ks] = *reinterpret_cast<const bf16x8*>(&S.s[l31][16 * ks + 8 * hf]);
      }
      if (w < 2) {
        // Ut block: [32 features r][C rows i] fp32; lane reads 4 rows of column l31 at once
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int pc = (32 * ta + 8 * g4 + 4 * hf) >> 2;
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(stg + R::HEAD + swz_piece(l31, pc, C * 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * g4 + e] = x[e];
        }
      } else {
        acc = zero_f32x16();
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc2 = zero_f32x16();
#pragma unroll
      for (int ks = 0; ks < DK / 16; ks += 2) {
        acc = mfma32(af[ks], sf[ks], acc);
        acc2 = mfma32(af[ks + 1], sf[ks + 1], acc2);
        if (more && (ks >> 1) < PARTS) issue(c + 1, sl ^ 1, ks >> 1);
      }
      if (more) {
#pragma unroll
        for (int part = DK / 32; part < PARTS; ++part) issue(c + 1, sl ^ 1, part);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += acc2[r];
    }
    if (w < 2) {
      // U tile (rows j = 32 ta + ..., column r = l31) -> U^T[r][j] in bf16
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = f2bf(acc[4 * g4 + e]);
        *reinterpret_cast<bf16x4*>(&S.u[l31][32 * ta + 8 * g4 + 4 * hf]) = y;
      }
    }
    __syncthreads();  // U^T complete; the chunk-start state and the output buffer were read
    // phase B: S^T <- g_C S^T + KT U (waves w < DKT), O += PG U (waves 2, 3)
    {
      bf16x8 uf[C / 16], kf[C / 16], pf[C / 16];
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) uf[ks] = *reinterpret_cast<const bf16x8*>(&S.u[l31][16 * ks + 8 * hf]);
      if (w < DKT) {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
          kf[ks] = *reinterpret_cast<const bf16x8*>(stg + R::KT + swz_piece(32 * w + l31, 2 * ks + hf, C * 2));
      }
      if (w >= 2) {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
          pf[ks] = *reinterpret_cast<const bf16x8*>(stg + R::PG + swz_piece(32 * ta + l31, 2 * ks + hf, C * 2));
      }
      const float gc = *reinterpret_cast<const float*>(stg + R::GC);
      __builtin_amdgcn_sched_barrier(0);
      if (w < DKT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] *= gc;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) st = mfma32(kf[ks], uf[ks], st);
      }
      if (w >= 2) {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) acc = mfma32(pf[ks], uf[ks], acc);
        // output tile: column r = l31, rows i = 32 ta + 8 (q/4) + 4 hf + q%4
#pragma unroll
        for (int r = 0; r < 16; ++r) S.o[32 * ta + 8 * (r >> 2) + 4 * hf + (r & 3)][l31] = f2bf(acc[r]);
      }
      if (w < DKT) put_state();
    }
    wait_vmcnt<0>();  // the next chunk's operands have landed (and this wave's stores are done)
    __syncthreads();  // the next chunk's state and this chunk's outputs are in LDS; the stage may be refilled
  }
  if (nch > 0) store_o(nch - 1);
  if (A.state_out && w < DKT) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4_t x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = st[4 * g4 + e];
      *reinterpret_cast<f32x4_t*>(A.state_out + so + 32 * w + 8 * g4 + 4 * hf) = x;
    }
  }
}

template <int DK>
hipError_t launch(const Args& a, hipStream_t stream) {
  if (a.T > 0) {
    prep_kernel<DK><<<dim3((unsigned)(a.nslot * a.H)), dim3(NT), 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr size_t lds = sizeof(ScanSmem<DK>);
  const hipError_t e = ensure_dynamic_lds<scan_kernel<DK>>((int)lds);
  if (e != hipSuccess) return e;
  scan_kernel<DK><<<dim3((unsigned)((int64_t)a.B * a.H * (a.dv / 32))), dim3(NT), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gdnc

size_t gdn_chunk_workspace_bytes(int64_t T, int B, int H, int dk, int dv) {
  const int64_t nslot = (T + gdnc::C - 1) / gdnc::C + B;
  const size_t rec = dk == 64 ? gdnc::Rec<64>::bytes(dv) : gdnc::Rec<128>::bytes(dv);
  return (size_t)nslot * H * rec;
}

hipError_t launch_gdn_chunked(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                              const int32_t* cu, int64_t T, int B, int H, int dk, int dv, const float* state_in,
                              void* o, float* state_out, void* ws, hipStream_t stream) {
  gdnc::Args a{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), alpha, beta,
               cu, state_in, static_cast<bf16*>(o), state_out, static_cast<unsigned char*>(ws), T,
               (T + gdnc::C - 1) / gdnc::C + B, B, H, dv};
  return dk == 64 ? gdnc::launch<64>(a, stream) : gdnc::launch<128>(a, stream);
}

}  // namespace tg
