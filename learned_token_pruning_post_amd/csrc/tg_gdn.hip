// Gated DeltaNet mixer of the hybrid variant, run on the kept tokens.
//
// Tencent Cloud TokenGate article, section on the gate position: in a hybrid
// model (Qwen3.5-2B) only some layers use full attention and the rest are
// Gated DeltaNet; the scorer reads hidden states, so the gate can sit on a
// GDN layer, and a GDN layer above it has no attention logits to bias, so it
// simply runs on the kept tokens. Per head, state S [dv, dk] (zero, or given,
// at a sequence's start), for each token in order:
//   k^ = k / |k|,  q^ = q / (|q| sqrt(dk))
//   S <- alpha S;  S <- S + beta (v - S k^) k^T;  o = S q^
//
// The rows of S evolve independently (row i only needs v_i and the shared
// k, q, alpha, beta), so the recurrence runs in parallel over rows and stays
// sequential over tokens. A workgroup takes RPWG rows of one (sequence, head);
// a row's state lives in the registers of dk / 8 lanes (8 fp32 each). Per
// token, S k finishes with DPP butterflies inside those lanes; 1/|k| and
// 1/(|q| sqrt(dk)) are computed for the whole chunk while it is staged, so
// only S k -> write sits on the serial chain (the read S q^ overlaps the next
// token, whose operands are read from LDS during this one). k, q, v, alpha and
// beta of 32-token chunks are staged in LDS, double-buffered: the next chunk's
// global loads are issued before the current chunk is processed and land in
// the other buffer after it; outputs collect in LDS and leave coalesced.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace gdn {

constexpr int NT = 256, NW = 4;
// tokens per staged chunk (fp32 rows are twice as wide: half as many fit the static LDS)
template <typename T>
constexpr int CT = sizeof(T) == 2 ? 32 : 16;
constexpr float EPS = 1e-6f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of N lanes (8 or 16); every lane of a group gets it
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  v += dpp<0xB1>(v);                          // quad permute [1,0,3,2]
  v += dpp<0x4E>(v);                          // quad permute [2,3,0,1]
  v += dpp<0x141>(v);                         // row half mirror
  if constexpr (N >= 16) v += dpp<0x140>(v);  // row mirror
  if constexpr (N == 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// sum of squares of the 8 elements in 16 bytes of T
__device__ __forceinline__ float sq8(const u32x4& r, bf16) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(r[i] << 16), hi = __uint_as_float(r[i] & 0xffff0000u);
    acc = fmaf(lo, lo, fmaf(hi, hi, acc));
  }
  return acc;
}
__device__ __forceinline__ float sq8(const u32x4& r, float) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(r[i]), __uint_as_float(r[i]), acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ void to_f32x8(const T* p, float (&x)[8]);
template <>
__device__ __forceinline__ void to_f32x8<bf16>(const bf16* p, float (&x)[8]) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(r[i] << 16);
    x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void to_f32x8<float>(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ float to_f32(bf16 x) { return bf2f(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ void store(bf16* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void store(float* p, float v) { *p = v; }

template <typename T, int DK>
struct Smem {
  static constexpr int LPR = DK / 8;
  static constexpr int RPWG = NW * (64 / LPR);  // rows per workgroup
  static constexpr int C = CT<T>;
  T k[2][C][DK];
  T q[2][C][DK];
  float v[2][C][RPWG];
  float a[2][C], b[2][C];
  float nk[2][C], nq[2][C];  // 1/|k| and 1/(|q| sqrt(dk)) of each token
  float o[C][RPWG];
};

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const int32_t* cu;
  const float* state_in;
  void* o;
  float* state_out;
  int H, dv;
};

template <typename T, int DK>
__global__ __launch_bounds__(NT) void gdn_kernel(Args A) {
  constexpr int LPR = DK / 8;          // lanes per state row
  constexpr int RPW = 64 / LPR;        // rows per wave
  constexpr int RPWG = NW * RPW;       // rows per workgroup
  constexpr int KCH = DK * (int)sizeof(T) / 16;  // 16-byte pieces per k (or q) row
  constexpr int CT = gdn::CT<T>;
  __shared__ __attribute__((aligned(16))) Smem<T, DK> S;

  const int nrb = A.dv / RPWG;
  const int wg = blockIdx.x;
  const int rb = wg % nrb, h = (wg / nrb) % A.H, b = wg / (nrb * A.H);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ds = lane % LPR;                       // this lane's 8 columns: ds*8 .. ds*8+7
  const int rloc = w * RPW + lane / LPR;           // row within the workgroup
  const int row = rb * RPWG + rloc;                // row of S (and feature of v, o)
  const int t0 = A.cu[b], L = A.cu[b + 1] - t0;
  const int H = A.H, dv = A.dv;
  const T* qg = static_cast<const T*>(A.q);
  const T* kg = static_cast<const T*>(A.k);
  const T* vg = static_cast<const T*>(A.v);
  T* og = static_cast<T*>(A.o);

  float st[8];
  {
    const size_t so = (((size_t)b * H + h) * dv + row) * DK + ds * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) st[e] = A.state_in ? A.state_in[so + e] : 0.f;
  }
  const float qscale = rsqrtf((float)DK);

  // chunk loads: this thread's pieces of k and q rows, v entries, alpha/beta
  constexpr int NKQ = 2 * CT * KCH;  // 16-byte pieces of k and q per chunk
  constexpr int PPT = (NKQ + NT - 1) / NT;
  u32x4 pk[PPT];
  float pv[(CT * RPWG + NT - 1) / NT];
  float pab = 0.f;
  auto load_chunk = [&](int c) {
    const int tc = c * CT;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      pk[i] = u32x4{0u, 0u, 0u, 0u};
      if (p < NKQ) {
        const int which = p / (CT * KCH), r = (p / KCH) % CT, c16 = p % KCH;
        if (tc + r < L) {
          const T* src = (which ? qg : kg) + ((size_t)(t0 + tc + r) * H + h) * DK;
          pk[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) + 16 * c16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (CT * RPWG + NT - 1) / NT; ++i) {
      const int p = tid + i * NT;
      const int r = p / RPWG, f = p % RPWG;
      const bool live = p < CT * RPWG && tc + r < L;
      pv[i] = live ? to_f32(vg[((size_t)(t0 + tc + r) * H + h) * dv + rb * RPWG + f]) : 0.f;
    }
    if (tid < 2 * CT) {
      const int r = tid % CT;
      const float* src = tid < CT ? A.alpha : A.beta;
      pab = tc + r < L ? src[(size_t)(t0 + tc + r) * H + h] : 0.f;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      // the KCH pieces of a row sit in KCH consecutive lanes (KCH divides 64 and NT):
      // their sums of squares reduce inside those lanes (all lanes take part)
      const float n2 = group_sum<KCH>(p < NKQ ? sq8(pk[i], T{}) : 0.f);
      if (p < NKQ) {
        const int which = p / (CT * KCH), r = (p / KCH) % CT, c16 = p % KCH;
        char* dst = reinterpret_cast<char*>(which ? &S.q[buf][r][0] : &S.k[buf][r][0]) + 16 * c16;
        *reinterpret_cast<u32x4*>(dst) = pk[i];
        if (c16 == 0) {
          const float inv = rsqrtf(n2 + EPS);
          if (which)
            S.nq[buf][r] = inv * rsqrtf((float)DK);
          else
            S.nk[buf][r] = inv;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (CT * RPWG + NT - 1) / NT; ++i) {
      const int p = tid + i * NT;
      if (p < CT * RPWG) S.v[buf][p / RPWG][p % RPWG] = pv[i];
    }
    if (tid < CT)
      S.a[buf][tid] = pab;
    else if (tid < 2 * CT)
      S.b[buf][tid - CT] = pab;
  };

  const int nchunk = (L + CT - 1) / CT;
  if (nchunk > 0) {
    load_chunk(0);
    store_chunk(0);
  }
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunk) load_chunk(c + 1);  // in flight while this chunk is processed
    const int nt = min(CT, L - c * CT);
    // operands of token t + 1 are read while token t is computed
    float kx[8], qx[8], al, be, vi, ik, iq;
    auto fetch = [&](int t) {
      to_f32x8<T>(&S.k[buf][t][ds * 8], kx);
      to_f32x8<T>(&S.q[buf][t][ds * 8], qx);
      al = S.a[buf][t];
      be = S.b[buf][t];
      vi = S.v[buf][t][rloc];
      ik = S.nk[buf][t];
      iq = S.nq[buf][t];
    };
    fetch(0);
    for (int t = 0; t < nt; ++t) {
      float ck[8], cq[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ck[e] = kx[e];
        cq[e] = qx[e];
      }
      const float cal = al, cbe = be, cvi = vi, cik = ik, ciq = iq;
      if (t + 1 < nt) fetch(t + 1);
      float dk0 = 0.f, dk1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        dk0 = fmaf(st[e], ck[e], dk0);
        dk1 = fmaf(st[e + 1], ck[e + 1], dk1);
      }
      const float u = cal * group_sum<LPR>(dk0 + dk1) * cik;  // (alpha S) k^
      const float cc = cbe * (cvi - u) * cik;                 // write strength along the raw k
#pragma unroll
      for (int e = 0; e < 8; ++e) st[e] = fmaf(cc, ck[e], cal * st[e]);
      float od0 = 0.f, od1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        od0 = fmaf(st[e], cq[e], od0);
        od1 = fmaf(st[e + 1], cq[e + 1], od1);
      }
      const float od = group_sum<LPR>(od0 + od1) * ciq;
      if (ds == 0) S.o[t][rloc] = od;
    }
    __syncthreads();  // outputs complete; the other buffer is no longer read
    for (int p = tid; p < nt * RPWG; p += NT) {
      const int r = p / RPWG, f = p % RPWG;
      store(og + ((size_t)(t0 + c * CT + r) * H + h) * dv + rb * RPWG + f, S.o[r][f]);
    }
    if (c + 1 < nchunk) store_chunk(buf ^ 1);
    __syncthreads();
  }
  if (A.state_out) {
    const size_t so = (((size_t)b * H + h) * dv + row) * DK + ds * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) A.state_out[so + e] = st[e];
  }
}

template <typename T, int DK>
hipError_t launch_t(const Args& a, int B, hipStream_t stream) {
  constexpr int RPWG = NW * (64 / (DK / 8));
  const int64_t nwg = (int64_t)B * a.H * (a.dv / RPWG);
  gdn_kernel<T, DK><<<dim3((unsigned)nwg), dim3(NT), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gdn

bool gdn_supported(int dk, int dv) { return (dk == 64 || dk == 128) && dv > 0 && dv % 32 == 0; }

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                      const int32_t* cu, int B, int H, int dk, int dv, bool is_bf16, const float* state_in,
                      void* o, float* state_out, hipStream_t stream) {
  gdn::Args a{q, k, v, alpha, beta, cu, state_in, o, state_out, H, dv};
  if (is_bf16)
    return dk == 64 ? gdn::launch_t<bf16, 64>(a, B, stream) : gdn::launch_t<bf16, 128>(a, B, stream);
  return dk == 64 ? gdn::launch_t<float, 64>(a, B, stream) : gdn::launch_t<float, 128>(a, B, stream);
}

}  // namespace tg
