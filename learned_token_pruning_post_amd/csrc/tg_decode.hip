// Decode attention over the pruned K/V cache: one new token per sequence
// attends to its kept prompt tokens and to the tokens generated so far.
//
// Tencent Cloud TokenGate article, engineering section: once prefill has fixed
// the gate bias, decoding folds it into the attention mask and runs ordinary
// attention over the cache; early-token-filtering section: generated tokens are
// never gated out, so each one joins the cache. The logit is the prefill's:
//   L_j = t_h * (q_h . k_j,h') / sqrt(d) + g_h * s_j,   h' = h / (Hq / Hkv),
// over every cached key (all of them precede the query: no causal mask).
//
// Cache: two segments per sequence, so the prefill's kept-token cache is read
// where the prefill wrote it. Segment A (packed, rows cuA[b] .. cuA[b+1]-1 of
// [rows, Hkv, d], scores sA) holds the kept prompt tokens; segment B ([B, capB,
// Hkv, d], scores [B, capB]) the first lenB[b] generated tokens of each sequence.
//
// Decode is bound by reading the cache (two rows of d elements per key and kv
// head, used once), so the kernels run on the vector ALUs, not the matrix
// cores: the q . k dot products of one kv head's G query heads share every K
// row. Work split ("split-K"): one 256-thread workgroup per (sequence, kv head,
// chunk of CK keys). A lane holds a 16-byte slice of a row (8 bf16 or 4 fp32),
// so D / slice lanes hold one key and a wave loads 64 / (D / slice) keys per
// instruction; the dot products finish with DPP butterflies inside those
// lanes, and each lane group keeps its own running maximum, sum and output
// slice (base-2 exponentials, the scale t_h log2(e) / sqrt(d) folded into q).
// The lane groups and the four waves merge at the end of the chunk; a second
// kernel merges the chunks of a (sequence, head). A call whose keys fit in one
// chunk per sequence finishes in the first kernel.
#include "tg_internal.hpp"

namespace tg {
namespace dec {

constexpr int NT = 256;     // threads per workgroup
constexpr int NW = NT / 64; // waves
constexpr int U = 4;        // keys per lane group per step (their loads in flight together)
constexpr int TARGET_WG = 2048;
constexpr int CK_MIN = 128, CK_MAX = 1024;

// keys per workgroup: a power of two giving about TARGET_WG workgroups
inline int chunk_keys(int B, int Hkv, int max_len) {
  const int64_t rows = (int64_t)B * Hkv * (int64_t)(max_len > 0 ? max_len : 1);
  int ck = CK_MIN;
  while (ck < CK_MAX && rows / ck > TARGET_WG) ck <<= 1;
  return ck;
}
inline int n_chunks(int max_len, int ck) { return max_len <= 0 ? 1 : (max_len + ck - 1) / ck; }

// sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a group
// gets the group's sum
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  v += dpp<0xB1>(v);                          // quad permute [1,0,3,2]
  v += dpp<0x4E>(v);                          // quad permute [2,3,0,1]
  v += dpp<0x141>(v);                         // row half mirror: lane i <-> 7 - i within 8
  if constexpr (N >= 16) v += dpp<0x140>(v);  // row mirror: lane i <-> 15 - i within 16
  if constexpr (N == 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// 16 bytes of a row as floats
template <typename T>
struct Slice;
template <>
struct Slice<bf16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(const u32x4& r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ bf16 store(float v) { return f2bf(v); }
};
template <>
struct Slice<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void unpack(const u32x4& r, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
  }
  static __device__ __forceinline__ float store(float v) { return v; }
};

struct Args {
  const void* q;
  const void* kA;
  const void* vA;
  const float* sA;
  const int32_t* cuA;
  const void* kB;
  const void* vB;
  const float* sB;
  const int32_t* lenB;
  const float* t;
  const float* g;
  void* out;
  float* lse;
  int32_t* status;
  float* po;   // [B, Hq, nchunk, D] unnormalised partial outputs
  float* pml;  // [B, Hq, nchunk, 2] (running max in log2 units, sum)
  int capB, Hq, Hkv, CK, nchunk, max_len;
};

constexpr float NEG_FLOOR = -1.0e30f;  // running-max start: finite, so exp2 differences stay defined
constexpr int32_t BAD_LENGTH = 8;      // TG_DEV_LEN_GT_MAX_N

// the sequence's key counts, and whether they fit what the host announced
__device__ __forceinline__ bool lengths(const Args& a, int b, int& lenA, int& nB) {
  lenA = a.cuA[b + 1] - a.cuA[b];
  nB = a.lenB[b];
  return lenA >= 0 && nB >= 0 && nB <= a.capB && (int64_t)lenA + nB <= (int64_t)a.max_len;
}

template <typename T, int D, int G, bool FINAL>
__global__ __launch_bounds__(NT) void decode_partial_kernel(Args a) {
  constexpr int E = Slice<T>::E;
  constexpr int LPR = D / E;          // lanes per key row
  constexpr int KPW = 64 / LPR;       // keys per wave load instruction
  constexpr int STEP = NW * KPW * U;  // keys per workgroup step
  __shared__ float sm_o[NW][G][D];
  __shared__ float sm_m[NW][G], sm_l[NW][G];

  const int wg = blockIdx.x;
  const int c = wg % a.nchunk;
  const int hk = (wg / a.nchunk) % a.Hkv;
  const int b = wg / (a.nchunk * a.Hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ds = lane % LPR, ks = lane / LPR;

  int lenA, nB;
  const bool ok = lengths(a, b, lenA, nB);
  const int L = ok ? lenA + nB : 0;
  const int k0 = c * a.CK, k1 = min(k0 + a.CK, L);
  if (!FINAL && (!ok || k0 >= L)) return;  // the merge kernel covers these

  // q of the G heads, scaled by t_h log2(e) / sqrt(d); bias gains in log2 units
  float qf[G][E], gb[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const int h = hk * G + gg;
    const float cs = a.t[h] * TG_LOG2E * rsqrtf((float)D);
    const T* qp = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + h) * D + ds * E;
    float x[E];
    Slice<T>::unpack(*reinterpret_cast<const u32x4*>(qp), x);
#pragma unroll
    for (int e = 0; e < E; ++e) qf[gg][e] = x[e] * cs;
    gb[gg] = a.g[h] * TG_LOG2E;
  }
  float m[G], l[G], o[G][E];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m[gg] = NEG_FLOOR;
    l[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[gg][e] = 0.f;
  }

  // keys j in [j0, j1) of one segment; key j is row row0 + j of its [rows, Hkv, D] arrays
  auto run = [&](const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ S,
                 int64_t row0, int j0, int j1) {
    for (int base = j0; base < j1; base += STEP) {
      u32x4 kr[U], vr[U];
      float sv[U];
      bool live[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + (w * U + u) * KPW + ks;
        live[u] = j < j1;
        const int64_t row = row0 + (live[u] ? j : j1 - 1);  // past the end: a valid row, masked below
        const size_t off = ((size_t)row * a.Hkv + hk) * D + ds * E;
        kr[u] = *reinterpret_cast<const u32x4*>(K + off);
        vr[u] = *reinterpret_cast<const u32x4*>(V + off);
        sv[u] = S[row];
      }
      float lg[G][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kx[E];
        Slice<T>::unpack(kr[u], kx);
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(qf[gg][e], kx[e], acc);
          acc = group_sum<LPR>(acc);
          lg[gg][u] = live[u] ? fmaf(gb[gg], sv[u], acc) : -INFINITY;
        }
      }
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        float mx = lg[gg][0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, lg[gg][u]);
        const float mn = fmaxf(m[gg], mx);
        const float al = __builtin_amdgcn_exp2f(m[gg] - mn);
        m[gg] = mn;
        l[gg] *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) o[gg][e] *= al;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = __builtin_amdgcn_exp2f(lg[gg][u] - mn);
          l[gg] += p;
          float vx[E];
          Slice<T>::unpack(vr[u], vx);
#pragma unroll
          for (int e = 0; e < E; ++e) o[gg][e] = fmaf(p, vx[e], o[gg][e]);
        }
      }
    }
  };
  if (ok && k0 < L) {
    const int64_t a0 = a.cuA[b];
    if (k0 < lenA)
      run(static_cast<const T*>(a.kA), static_cast<const T*>(a.vA), a.sA, a0, k0, min(k1, lenA));
    if (k1 > lenA)
      run(static_cast<const T*>(a.kB), static_cast<const T*>(a.vB), a.sB, (int64_t)b * a.capB - lenA,
          max(k0, lenA), k1);
  }

  // merge the lane groups of the wave (lanes ds, ds + LPR, ...), then the waves
#pragma unroll
  for (int sh = LPR; sh < 64; sh <<= 1) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float mo = __shfl_xor(m[gg], sh, 64);
      const float mn = fmaxf(m[gg], mo);
      const float as = __builtin_amdgcn_exp2f(m[gg] - mn), ao = __builtin_amdgcn_exp2f(mo - mn);
      l[gg] = l[gg] * as + __shfl_xor(l[gg], sh, 64) * ao;
#pragma unroll
      for (int e = 0; e < E; ++e) o[gg][e] = o[gg][e] * as + __shfl_xor(o[gg][e], sh, 64) * ao;
      m[gg] = mn;
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_o[w][gg][ds * E + e] = o[gg][e];
      if (ds == 0) {
        sm_m[w][gg] = m[gg];
        sm_l[w][gg] = l[gg];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += NT) {
    const int gg = i / D, e = i % D;
    const int h = hk * G + gg;
    float mx = sm_m[0][gg];
#pragma unroll
    for (int v = 1; v < NW; ++v) mx = fmaxf(mx, sm_m[v][gg]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float sc = __builtin_amdgcn_exp2f(sm_m[v][gg] - mx);
      ls = fmaf(sm_l[v][gg], sc, ls);
      os = fmaf(sm_o[v][gg][e], sc, os);
    }
    if constexpr (FINAL) {
      T* out = static_cast<T*>(a.out) + ((size_t)b * a.Hq + h) * D;
      float r, lr;
      if (!ok) {
        r = __builtin_nanf("");
        lr = r;
      } else if (ls > 0.f) {
        r = os / ls;
        lr = (mx + log2f(ls)) * TG_LN2;
      } else {  // no keys
        r = 0.f;
        lr = -INFINITY;
      }
      out[e] = Slice<T>::store(r);
      if (e == 0 && a.lse) a.lse[(size_t)b * a.Hq + h] = lr;
      if (e == 0 && gg == 0 && hk == 0 && a.status) a.status[b] = ok ? 0 : BAD_LENGTH;
    } else {
      const size_t pc = ((size_t)b * a.Hq + h) * a.nchunk + c;
      a.po[pc * D + e] = os;
      if (e == 0) {
        a.pml[2 * pc] = mx;
        a.pml[2 * pc + 1] = ls;
      }
    }
  }
}

// one workgroup of D threads per (sequence, head): merge its chunks
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(Args a) {
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq, e = threadIdx.x;
  int lenA, nB;
  const bool ok = lengths(a, b, lenA, nB);
  T* out = static_cast<T*>(a.out) + ((size_t)b * a.Hq + h) * D;
  float* lse = a.lse ? a.lse + (size_t)b * a.Hq + h : nullptr;
  if (e == 0 && h == 0 && a.status) a.status[b] = ok ? 0 : BAD_LENGTH;
  const int L = ok ? lenA + nB : 0;
  if (!ok || L == 0) {
    const float r = ok ? 0.f : __builtin_nanf("");
    out[e] = Slice<T>::store(r);
    if (e == 0 && lse) *lse = ok ? -INFINITY : r;
    return;
  }
  const int nc = (L + a.CK - 1) / a.CK;
  const size_t p0 = ((size_t)b * a.Hq + h) * a.nchunk;
  float mx = NEG_FLOOR;
  for (int c = 0; c < nc; ++c) mx = fmaxf(mx, a.pml[2 * (p0 + c)]);
  float ls = 0.f, os = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float sc = __builtin_amdgcn_exp2f(a.pml[2 * (p0 + c)] - mx);
    ls = fmaf(a.pml[2 * (p0 + c) + 1], sc, ls);
    os = fmaf(a.po[(p0 + c) * D + e], sc, os);
  }
  out[e] = Slice<T>::store(os / ls);
  if (e == 0 && lse) *lse = (mx + log2f(ls)) * TG_LN2;
}

template <typename T, int D, int G>
hipError_t launch_tdg(const Args& a, int B, hipStream_t stream) {
  const int64_t nwg = (int64_t)B * a.Hkv * a.nchunk;
  if (a.nchunk == 1) {
    decode_partial_kernel<T, D, G, true><<<dim3((unsigned)nwg), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
  }
  decode_partial_kernel<T, D, G, false><<<dim3((unsigned)nwg), dim3(NT), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<T, D><<<dim3((unsigned)((int64_t)B * a.Hq)), dim3(D), 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_td(const Args& a, int B, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_tdg<T, D, 1>(a, B, stream);
    case 2: return launch_tdg<T, D, 2>(a, B, stream);
    case 4: return launch_tdg<T, D, 4>(a, B, stream);
    case 8: return launch_tdg<T, D, 8>(a, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec

bool decode_supported(int Hq, int Hkv, int d) {
  if (Hkv <= 0 || Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

size_t decode_workspace_bytes(int B, int max_len, int Hq, int Hkv, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
  const int ck = dec::chunk_keys(B, Hkv, max_len);
  const int nc = dec::n_chunks(max_len, ck);
  if (nc <= 1) return 0;
  const size_t n = (size_t)B * Hq * nc;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(n * d * sizeof(float)) + al(n * 2 * sizeof(float));
}

hipError_t launch_decode_attn(const void* q, const void* kA, const void* vA, const float* sA,
                              const int32_t* cuA, const void* kB, const void* vB, const float* sB,
                              const int32_t* lenB, int capB, const float* t, const float* g, int B,
                              int max_len, int Hq, int Hkv, int d, bool is_bf16, void* o, float* lse,
                              int32_t* status, void* ws, hipStream_t stream) {
  dec::Args a{};
  a.q = q;
  a.kA = kA;
  a.vA = vA;
  a.sA = sA;
  a.cuA = cuA;
  a.kB = kB;
  a.vB = vB;
  a.sB = sB;
  a.lenB = lenB;
  a.t = t;
  a.g = g;
  a.out = o;
  a.lse = lse;
  a.status = status;
  a.capB = capB;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_len = max_len;
  a.CK = dec::chunk_keys(B, Hkv, max_len);
  a.nchunk = dec::n_chunks(max_len, a.CK);
  if (a.nchunk > 1) {
    const size_t n = (size_t)B * Hq * a.nchunk;
    a.po = static_cast<float*>(ws);
    a.pml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((n * d * sizeof(float) + 255) & ~(size_t)255));
  }
  const int G = Hq / Hkv;
  if (is_bf16)
    return d == 64 ? dec::launch_td<bf16, 64>(a, B, G, stream) : dec::launch_td<bf16, 128>(a, B, G, stream);
  return d == 64 ? dec::launch_td<float, 64>(a, B, G, stream) : dec::launch_td<float, 128>(a, B, G, stream);
}

}  // namespace tg
