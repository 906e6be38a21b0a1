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

template <int DK>
struct Rec {  // byte offsets inside one (chunk, head) record of the workspace
  static constexpr size_t WN = 0;                          // [C][DK] bf16
  static constexpr size_t QG = WN + (size_t)C * DK * 2;    // [C][DK] bf16
  static constexpr size_t PG = QG + (size_t)C * DK * 2;    // [C][C] bf16
  static constexpr size_t KT = PG + (size_t)C * C * 2;     // [DK][C] bf16
  static constexpr size_t GC = KT + (size_t)DK * C * 2;    // fp32 (padded to 256 bytes)
  static constexpr size_t UT = GC + 256;                   // [C][dv] fp32
  __host__ __device__ static size_t bytes(int dv) { return (UT + (size_t)C * dv * 4 + 255) & ~(size_t)255; }
};

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
  float nk[C], nq[C], lg[C], be[C];
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

template <int DK>
__global__ __launch_bounds__(NT) void prep_kernel(Args A) {
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
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const bf16* src = m ? A.q : A.k;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT, r = p / KCH, c16 = p % KCH;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (r < n) x = *reinterpret_cast<const u32x4*>(src + ((size_t)(tb + r) * H + h) * DK + 8 * c16);
      *reinterpret_cast<u32x4*>(m ? &S.u.q[r][8 * c16] : &S.k[r][8 * c16]) = x;
      // the KCH pieces of a row sit in KCH consecutive lanes
      float s2 = sq8(x);
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
    S.be[lane] = live ? A.beta[(size_t)(tb + lane) * H + h] : 0.f;
  }
  __syncthreads();

  // ---- K K^T and Q K^T (raw bf16 products, fp32 accumulators), QG ----
  const int ti = w >> 1, tj = w & 1;  // this wave's 32 x 32 tile of both
  f32x16 g = zero_f32x16(), pq = zero_f32x16();
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks) {
    const int kc = 16 * ks + 8 * hf;
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&S.k[32 * ti + l31][kc]);
    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&S.u.q[32 * ti + l31][kc]);
    const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&S.k[32 * tj + l31][kc]);
    g = mfma32(ka, kb, g);
    pq = mfma32(qa, kb, pq);
  }
  // QG[i][d] = g_i nq_i q_i[d]
  for (int p = tid; p < C * DK / 8; p += NT) {
    const int r = p / KCH, c16 = p % KCH;
    const float sc = __expf(S.lg[r]) * S.nq[r];
    const u32x4 x = *reinterpret_cast<const u32x4*>(&S.u.q[r][8 * c16]);
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = f2bf(__uint_as_float(x[e] << 16) * sc);
      y[2 * e + 1] = f2bf(__uint_as_float(x[e] & 0xffff0000u) * sc);
    }
    *reinterpret_cast<bf16x8*>(rec + R::QG + ((size_t)r * DK + 8 * c16) * 2) = y;
  }
  __syncthreads();  // q is no longer read: its space becomes the system matrix
  {
    // accumulator: lane holds column j = 32 tj + l31, rows i = 32 ti + 8 (r/4) + 4 hf + r%4
    const int j = 32 * tj + l31;
    const float nkj = S.nk[j], lgj = S.lg[j];
    bf16* pg = reinterpret_cast<bf16*>(rec + R::PG);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hf + (r & 3);
      const float dec = j <= i ? __expf(S.lg[i] - lgj) : 0.f;  // g_i / g_j <= 1 below the diagonal
      S.u.m[i][j] = j < i ? S.be[i] * dec * S.nk[i] * nkj * g[r] : 0.f;
      pg[i * C + j] = f2bf(S.nq[i] * nkj * dec * pq[r]);
    }
  }
  __syncthreads();

  // ---- T = (I + M)^-1 by forward substitution (wave 0: lane = column);
  // waves 1-3 meanwhile write KT and stage (b g k^)^T ----
  if (w == 0) {
    float tc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float a0 = i == lane ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < i; j4 += 4) {
        const f32x4_t mr = *reinterpret_cast<const f32x4_t*>(&S.u.m[i][j4]);
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
    // every read of M is done (program order): T overwrites it, split in two bf16
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const bf16 th = f2bf(tc[i]);
      S.u.t.hi[i][lane] = th;
      S.u.t.lo[i][lane] = f2bf(tc[i] - bf2f(th));
    }
  } else {
    const float lgC = S.lg[C - 1];
    bf16* kt = reinterpret_cast<bf16*>(rec + R::KT);
    for (int p = tid - 64; p < C * DK; p += NT - 64) {
      const int d = p / C, j = p % C;
      const float kv = bf2f(S.k[j][d]) * S.nk[j];
      kt[(size_t)d * C + j] = f2bf(__expf(lgC - S.lg[j]) * kv);
      S.xt[d][j] = f2bf(S.be[j] * __expf(S.lg[j]) * kv);
    }
    if (tid == 64) *reinterpret_cast<float*>(rec + R::GC) = __expf(lgC);
  }
  __syncthreads();

  // ---- WN = -T diag(b g) K^ ----
  {
    bf16* wn = reinterpret_cast<bf16*>(rec + R::WN);
    t_times_x<DK>(S, w, lane, [&](int rb, int cb, const f32x16& acc) {
      const int col = 32 * cb + l31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * rb + 8 * (r >> 2) + 4 * hf + (r & 3);
        wn[(size_t)i * DK + col] = f2bf(-acc[r]);
      }
    });
  }
  // ---- Ut = T diag(b) V, DK columns of V at a time ----
  float* ut = reinterpret_cast<float*>(rec + R::UT);
  for (int c0 = 0; c0 < dv; c0 += DK) {
    __syncthreads();  // the previous product has read xt
    for (int p = tid; p < C * DK; p += NT) {
      const int j = p / DK, col = p % DK;
      float x = 0.f;
      if (j < n && c0 + col < dv) x = S.be[j] * bf2f(A.v[((size_t)(tb + j) * H + h) * dv + c0 + col]);
      S.xt[col][j] = f2bf(x);
    }
    __syncthreads();
    t_times_x<DK>(S, w, lane, [&](int rb, int cb, const f32x16& acc) {
      const int col = c0 + 32 * cb + l31;
      if (col < dv) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = 32 * rb + 8 * (r >> 2) + 4 * hf + (r & 3);
          ut[(size_t)i * dv + col] = acc[r];
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
  bf16 s[32][DK + 8];  // chunk-start state, rows r of this block: S[r][d] in bf16
  bf16 u[32][C + 8];   // U^T[r][j] of the chunk
};

template <int DK>
struct Frags {  // one chunk's operands of this wave (A-operand rows, fp32 U start)
  bf16x8 a[DK / 16];  // WN rows (waves 0, 1) or QG rows (waves 2, 3)
  bf16x8 p[C / 16];   // PG rows (waves 2, 3)
  bf16x8 kt[C / 16];  // KT rows (waves holding a tile of S^T)
  float ut[16];       // Ut entries of the wave's U tile (waves 0, 1)
  float gc;
};

template <int DK>
__global__ __launch_bounds__(NT) void scan_kernel(Args A) {
  using R = Rec<DK>;
  constexpr int DKT = DK / 32;  // tiles of S^T (one per wave w < DKT)
  __shared__ __attribute__((aligned(16))) ScanSmem<DK> S;
  const int H = A.H, dv = A.dv, nrb = dv / 32;
  const int rb = blockIdx.x % nrb, h = (blockIdx.x / nrb) % H, b = blockIdx.x / (nrb * H);
  const int r0 = rb * 32;
  const int t0 = A.cu[b], L = A.cu[b + 1] - t0;
  const int sb = slot_base(A.cu, b);
  // chunks of the sequence (none past the workspace's records)
  const int nch = t0 < 0 ? 0 : (int)min((int64_t)((L + C - 1) / C), A.nslot - sb);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l31 = lane & 31, hf = lane >> 5;
  const size_t rbytes = R::bytes(dv);

  // S^T tile of wave w: lane holds column r = l31, rows d = 32 w + 8 (q/4) + 4 hf + q%4
  f32x16 st = zero_f32x16();
  const size_t so = (((size_t)b * H + h) * dv + r0 + l31) * DK;
  if (w < DKT) {
    if (A.state_in) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(A.state_in + so + 32 * w + 8 * g4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) st[4 * g4 + e] = x[e];
      }
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

  auto fetch = [&](int c, Frags<DK>& F) {
    const unsigned char* rec = A.ws + ((size_t)(sb + c) * H + h) * rbytes;
    const int kc = 8 * hf;
    if (w < 2) {
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks)
        F.a[ks] = *reinterpret_cast<const bf16x8*>(rec + R::WN + ((size_t)(32 * w + l31) * DK + 16 * ks + kc) * 2);
      const float* ut = reinterpret_cast<const float*>(rec + R::UT);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * w + 8 * (r >> 2) + 4 * hf + (r & 3);
        F.ut[r] = ut[(size_t)i * dv + r0 + l31];
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks)
        F.a[ks] =
            *reinterpret_cast<const bf16x8*>(rec + R::QG + ((size_t)(32 * (w - 2) + l31) * DK + 16 * ks + kc) * 2);
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks)
        F.p[ks] = *reinterpret_cast<const bf16x8*>(rec + R::PG + ((size_t)(32 * (w - 2) + l31) * C + 16 * ks + kc) * 2);
    }
    if (w < DKT) {
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks)
        F.kt[ks] = *reinterpret_cast<const bf16x8*>(rec + R::KT + ((size_t)(32 * w + l31) * C + 16 * ks + kc) * 2);
    }
    F.gc = *reinterpret_cast<const float*>(rec + R::GC);
  };

  Frags<DK> cur;
  if (nch > 0) fetch(0, cur);
  __syncthreads();  // the bf16 state is in LDS
  for (int c = 0; c < nch; ++c) {
    Frags<DK> nxt;
    if (c + 1 < nch) fetch(c + 1, nxt);
    // phase A: U = Ut + WN S0^T (waves 0, 1), O = QG S0^T (waves 2, 3)
    f32x16 acc;
    if (w < 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = cur.ut[r];
    } else {
      acc = zero_f32x16();
    }
    {
      f32x16 acc2 = zero_f32x16();
#pragma unroll
      for (int ks = 0; ks < DK / 16; ks += 2) {
        const bf16x8 s0 = *reinterpret_cast<const bf16x8*>(&S.s[l31][16 * ks + 8 * hf]);
        const bf16x8 s1 = *reinterpret_cast<const bf16x8*>(&S.s[l31][16 * ks + 16 + 8 * hf]);
        acc = mfma32(cur.a[ks], s0, acc);
        acc2 = mfma32(cur.a[ks + 1], s1, acc2);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += acc2[r];
    }
    if (w < 2) {
      // U tile (rows j = 32 w + ..., column r = l31) -> U^T[r][j] in bf16
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = f2bf(acc[4 * g4 + e]);
        *reinterpret_cast<bf16x4*>(&S.u[l31][32 * w + 8 * g4 + 4 * hf]) = y;
      }
    }
    __syncthreads();  // U^T complete; every read of the chunk-start state is done
    // phase B: S^T <- g_C S^T + KT U (waves w < DKT), O += PG U (waves 2, 3)
    if (w < DKT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] *= cur.gc;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 ub = *reinterpret_cast<const bf16x8*>(&S.u[l31][16 * ks + 8 * hf]);
        st = mfma32(cur.kt[ks], ub, st);
      }
      put_state();
    }
    if (w >= 2) {
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 ub = *reinterpret_cast<const bf16x8*>(&S.u[l31][16 * ks + 8 * hf]);
        acc = mfma32(cur.p[ks], ub, acc);
      }
      // O tile: column r = l31 (feature r0 + r), rows i = 32 (w-2) + ...
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * (w - 2) + 8 * (r >> 2) + 4 * hf + (r & 3);
        const int64_t t = (int64_t)t0 + c * C + i;
        if (c * C + i < L && t < A.T) A.o[((size_t)t * H + h) * dv + r0 + l31] = f2bf(acc[r]);
      }
    }
    __syncthreads();  // the next chunk's state copy is in LDS; U^T may be overwritten
    if (c + 1 < nch) cur = nxt;
  }
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
  scan_kernel<DK><<<dim3((unsigned)((int64_t)a.B * a.H * (a.dv / 32))), dim3(NT), 0, stream>>>(a);
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
