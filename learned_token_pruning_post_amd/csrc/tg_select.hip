// Top-K selection with forced keep (one workgroup per sequence).
//
// Rule (Tencent Cloud TokenGate article, section on early token filtering; the
// ai.866data article, mechanism-design section): forced tokens are always
// kept; the other K - F slots go to the highest scores, equal scores to the
// lower index, NaN below every number, -0.0 equal to +0.0. Output ascending.
//
// Algorithm: scores map to order-preserving uint32 keys. A range search
// narrows [kmin, kmax] to the threshold key T with histogram passes whose bin
// width is a power of two sized so the bins span the live range (the range,
// not the fixed top byte: sigmoid scores share their top bits, a fixed-digit
// radix would pile every key into one or two bins). A final pass keeps forced
// tokens, keys > T, and the first `need` keys == T in index order.
//
// Sequences of up to SEL_LDS_MAX tokens keep their keys in LDS (select_lds).
// Longer sequences stream their scores from global memory on every pass
// (select_global) with 16 independent loads in flight per thread.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_BINS = 2048;
constexpr int SEL_LDS_MAX = 32768;                       // keys held in LDS
constexpr int SEL_BATCH = 16;                            // loads in flight (global path)

__device__ __forceinline__ uint32_t score_key(float x, bool& is_nan) {
  uint32_t u = __float_as_uint(x);
  is_nan = (u & 0x7fffffffu) > 0x7f800000u;
  if (is_nan) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide inclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_incl_scan(int v, int* sh /*[SEL_WAVES]*/) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  if (w == 0) {
    int x = lane < SEL_WAVES ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < SEL_WAVES; o <<= 1) {
      int t = __shfl_up(x, o, 64);
      if (lane >= o) x += t;
    }
    if (lane < SEL_WAVES) sh[lane] = x;
  }
  __syncthreads();
  int add = w > 0 ? sh[w - 1] : 0;
  __syncthreads();
  return v + add;
}

__device__ __forceinline__ int block_sum_int(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) tot += sh[i];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  if (lane == 0) sh[w] = v;
  __syncthreads();
  uint32_t r = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) r = min(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  if (lane == 0) sh[w] = v;
  __syncthreads();
  uint32_t r = 0u;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) r = max(r, sh[i]);
  __syncthreads();
  return r;
}

// Scores of one sequence streamed from global memory (sequences longer than
// SEL_LDS_MAX tokens), SEL_BATCH independent loads in flight per thread.
struct GlobalKeys {
  const float* sp;
  const uint8_t* mp;

  // visit (index, key, forced) of the contiguous span [i0, i1) in order
  template <class F>
  __device__ __forceinline__ void blocked(int i0, int i1, F&& f) const {
    for (int b0 = i0; b0 < i1; b0 += SEL_BATCH) {
      float x[SEL_BATCH];
      uint8_t fm[SEL_BATCH];
#pragma unroll
      for (int u = 0; u < SEL_BATCH; ++u) {
        const int i = b0 + u;
        x[u] = i < i1 ? sp[i] : 0.f;
        fm[u] = (i < i1 && mp) ? mp[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < SEL_BATCH; ++u) {
        const int i = b0 + u;
        if (i < i1) {
          bool isn;
          f(i, score_key(x[u], isn), fm[u] != 0);
        }
      }
    }
  }
  // visit (index, key, forced) of the strided set tid, tid+1024, ... (< n)
  template <class F>
  __device__ __forceinline__ void strided(int n, F&& f) const {
    const int tid = threadIdx.x;
    for (int i0 = tid; i0 < n; i0 += SEL_THREADS * SEL_BATCH) {
      float x[SEL_BATCH];
      uint8_t fm[SEL_BATCH];
#pragma unroll
      for (int u = 0; u < SEL_BATCH; ++u) {
        const int i = i0 + u * SEL_THREADS;
        x[u] = i < n ? sp[i] : 0.f;
        fm[u] = (i < n && mp) ? mp[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < SEL_BATCH; ++u) {
        const int i = i0 + u * SEL_THREADS;
        if (i < n) {
          bool isn;
          f(i, score_key(x[u], isn), fm[u] != 0);
        }
      }
    }
  }
};

__device__ __forceinline__ void select_global(const float* __restrict__ sp,
                                              const uint8_t* __restrict__ mp, int n, int K, int in0,
                                              int32_t* __restrict__ kp, int32_t* __restrict__ status_b,
                                              uint32_t* hist, int* shi, uint32_t* shu, int* found) {
  const int tid = threadIdx.x;
  GlobalKeys src{sp, mp};

  // pass 0: forced count, NaN flag, live key range of the candidates
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  for (int i0 = tid; i0 < n; i0 += SEL_THREADS * SEL_BATCH) {
    float x[SEL_BATCH];
    uint8_t fm[SEL_BATCH];
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) {
      const int i = i0 + u * SEL_THREADS;
      x[u] = i < n ? sp[i] : 0.f;
      fm[u] = (i < n && mp) ? mp[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) {
      const int i = i0 + u * SEL_THREADS;
      if (i < n) {
        bool isn;
        const uint32_t k = score_key(x[u], isn);
        nan_seen |= isn;
        if (fm[u]) {
          ++nf;
        } else {
          kmin = min(kmin, k);
          kmax = max(kmax, k);
        }
      }
    }
  }
  nf = block_sum_int(nf, shi);
  nan_seen = block_sum_int(nan_seen, shi);
  kmin = block_min_u32(kmin, shu);
  kmax = block_max_u32(kmax, shu);

  const int flags = (nan_seen ? 4 : 0) | (K > n ? 2 : 0) | (nf > K ? 1 : 0);
  if (tid == 0 && status_b) *status_b = flags;
  if (flags & 3) {
    for (int i = tid; i < K; i += SEL_THREADS) kp[i] = -1;
    return;
  }
  const int C = n - nf;  // candidates
  const int r = K - nf;  // slots for candidates
  uint32_t T;
  int needT;
  if (r == 0) {
    T = 0xffffffffu;  // no key reaches it (largest real key is +inf's)
    needT = 0;
  } else if (r == C) {
    T = 0u;
    needT = C;
  } else {
    uint32_t lo = kmin, hi = kmax;
    int need = r;
    T = lo;
    needT = need;
    for (int iter = 0; iter < 4; ++iter) {
      if (lo == hi) {
        T = lo;
        needT = need;
        break;
      }
      const uint32_t span = hi - lo;
      const int bits = 32 - __clz(span);
      const int shift = bits > 11 ? bits - 11 : 0;
      const int nb = (int)(span >> shift) + 1;
      for (int i = tid; i < nb; i += SEL_THREADS) hist[i] = 0u;
      __syncthreads();
      src.strided(n, [&](int, uint32_t k, bool f) {
        if (!f && k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> shift], 1u);
      });
      __syncthreads();
      // suffix sums over bins: thread t owns bins 2t', 2t'+1 with t' = 1023 - t
      const int t2 = SEL_THREADS - 1 - tid;
      const int b0 = 2 * t2, b1 = 2 * t2 + 1;
      const int h0 = b0 < nb ? (int)hist[b0] : 0;
      const int h1 = b1 < nb ? (int)hist[b1] : 0;
      const int incl = block_incl_scan(h0 + h1, shi);
      const int above_pair = incl - (h0 + h1);  // bins above b1
      if (above_pair < need && incl >= need) {
        if (above_pair + h1 >= need) {
          found[0] = b1;
          found[1] = above_pair;
        } else {
          found[0] = b0;
          found[1] = above_pair + h1;
        }
      }
      __syncthreads();
      const int bstar = found[0];
      need -= found[1];
      const uint64_t nlo = (uint64_t)lo + ((uint64_t)bstar << shift);
      const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
      lo = (uint32_t)nlo;
      hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
      __syncthreads();
      if (shift == 0) {
        T = lo;
        needT = need;
        break;
      }
    }
  }

  // emit: thread t owns the contiguous span [t*chunk, (t+1)*chunk) so that
  // block scans give index-ordered tie ranks and output offsets.
  const int chunk = (n + SEL_THREADS - 1) / SEL_THREADS;
  const int i0 = min(n, tid * chunk), i1 = min(n, i0 + chunk);
  int sure = 0, ties = 0;
  src.blocked(i0, i1, [&](int, uint32_t k, bool f) {
    sure += f || (k > T);
    ties += !f && (k == T);
  });
  const int tie_before = block_incl_scan(ties, shi) - ties;
  int take = needT - tie_before;
  take = take < 0 ? 0 : (take > ties ? ties : take);
  const int cnt = sure + take;
  int off = block_incl_scan(cnt, shi) - cnt;
  int taken = 0;
  src.blocked(i0, i1, [&](int i, uint32_t k, bool f) {
    bool keep = f || k > T;
    if (!keep && k == T && taken < take) {
      keep = true;
      ++taken;
    }
    if (keep && off < K) kp[off++] = in0 + i;  // off < K always holds; the guard keeps a logic slip in bounds
  });
}

// ---------------------------------------------------------------------------
// LDS path (n <= SEL_LDS_MAX): keys stay in LDS after one vectorised load.
//  * load: every thread issues all of its 16-byte score loads and 4-byte
//    mask loads before using any; forced tokens are stored as key 0 and NaN
//    candidates as key 1, below every number's key, so no separate forced
//    bitmap is kept;
//  * one fused reduction of (forced count, NaN flag, candidate min, max);
//  * range passes with SEL_LDS_BINS = 4096 power-of-two bins (the span
//    shrinks by 2^12 per pass). Once the live range holds at most SEL_LIST
//    candidates, the pass that scans all keys also gathers those into a
//    list, and the remaining passes read only the list;
//  * emit: thread t owns tokens 32t..32t+31; one block scan of
//    packed (sure, tie) counts gives every thread its output slot and the
//    tie rank of its first tie, so kept indices are written in ascending
//    order.
// ---------------------------------------------------------------------------
constexpr int SEL_LDS_BINS = 4096;

// LDS position of 4-token chunk g: chunks are XOR-swizzled inside each
// aligned block of 16 (256 bytes, the 64-bank width), so both the strided
// chunk walks (16 consecutive chunks per 16 lanes) and the emit's
// thread-contiguous walk (chunks 8t + q for 16 consecutive t) hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int kchunk(int g) { return g ^ ((g >> 3) & 15); }
constexpr int SEL_LIST = 2048;

// Wave-wide inclusive scans on DPP lane moves (plain VALU: no LDS round trip
// as with ds_bpermute): row_shr 1, 2, 4, 8 scan each 16-lane row, then
// row_bcast 15 and 31 carry the row totals upward. `id` is the identity: it
// fills lanes whose source is outside the row or whose row is masked off.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  return (int)wave_scan_u32((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

__device__ __forceinline__ void select_lds(const float* __restrict__ sp, const uint8_t* __restrict__ mp, int n,
                           int K, int in0, int32_t* __restrict__ kp, int32_t* __restrict__ status_b,
                           uint32_t* keys, uint32_t* hist, int* red, uint32_t* list) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NG = SEL_LDS_MAX / 4 / SEL_THREADS;  // 4-token groups per thread

  // ---- load ----
  // LDS key of a token: 0 if forced, 1 if a NaN candidate, else its order
  // key (>= 0x007fffff, the key of -inf), so range tests skip forced tokens
  // by value and the tail of a partial 4-token chunk (0) is never in range.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  auto take_key = [&](float x, bool f) -> uint32_t {
    bool isn;
    uint32_t k = score_key(x, isn);
    nan_seen |= isn;
    if (f) {
      ++nf;
      return 0u;
    }
    k = isn ? 1u : k;
    kmin = min(kmin, k);
    kmax = max(kmax, k);
    return k;
  };
  const bool vec = (reinterpret_cast<uintptr_t>(sp) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(mp) & 3u) == 0;
  if (vec) {
    // chunk g = u*1024 + tid holds tokens 4g..4g+3: all loads first
    f32x4 xv[NG];
    uint32_t mv[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int i = 4 * (u * SEL_THREADS + tid);
      mv[u] = 0u;
      if (i + 3 < n) {
        xv[u] = *reinterpret_cast<const f32x4*>(sp + i);
        if (mp) mv[u] = *reinterpret_cast<const uint32_t*>(mp + i);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[u][e] = i + e < n ? sp[i + e] : 0.f;
          if (mp && i + e < n && mp[i + e]) mv[u] |= 1u << (8 * e);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int g = u * SEL_THREADS + tid, i = 4 * g;
      u32x4 kv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        kv[e] = i + e < n ? take_key(xv[u][e], ((mv[u] >> (8 * e)) & 0xffu) != 0) : 0u;
      if (i < n) *reinterpret_cast<u32x4*>(keys + 4 * kchunk(g)) = kv;
    }
  } else {
    for (int i = tid; i < ((n + 3) & ~3); i += SEL_THREADS)
      keys[4 * kchunk(i >> 2) + (i & 3)] = i < n ? take_key(sp[i], mp && mp[i]) : 0u;
  }
  // ---- fused reduction ----
  nf = lane63(wave_incl_scan(nf));
  nan_seen = lane63(wave_incl_scan(nan_seen));
  kmin = (uint32_t)lane63((int)wave_scan_u32(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }));
  kmax = (uint32_t)lane63((int)wave_scan_u32(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }));
  if (lane == 0) {
    red[4 * w + 0] = nf;
    red[4 * w + 1] = nan_seen;
    red[4 * w + 2] = (int)kmin;
    red[4 * w + 3] = (int)kmax;
  }
  __syncthreads();
  nf = 0;
  nan_seen = 0;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int v = 0; v < SEL_WAVES; ++v) {
    nf += red[4 * v];
    nan_seen |= red[4 * v + 1];
    kmin = min(kmin, (uint32_t)red[4 * v + 2]);
    kmax = max(kmax, (uint32_t)red[4 * v + 3]);
  }
  const int flags = (nan_seen ? 4 : 0) | (K > n ? 2 : 0) | (nf > K ? 1 : 0);
  if (tid == 0 && status_b) *status_b = flags;
  if (flags & 3) {
    for (int i = tid; i < K; i += SEL_THREADS) kp[i] = -1;
    return;
  }
  const int C = n - nf;  // candidates
  const int r = K - nf;  // slots for candidates
  uint32_t T;
  int needT;
  if (r == 0) {
    T = 0xffffffffu;  // no key reaches it (largest real key is +inf's)
    needT = 0;
  } else if (r == C) {
    T = 0u;
    needT = C;
  } else {
    uint32_t lo = kmin, hi = kmax;
    int need = r;
    int in_range = C;       // candidates with lo <= key <= hi
    bool use_list = false;  // candidates in range are all in list[0, nlist)
    int nlist = 0;
    T = lo;
    needT = need;
    for (int iter = 0; iter < 4; ++iter) {
      if (lo == hi) {
        T = lo;
        needT = need;
        break;
      }
      const uint32_t span = hi - lo;
      const int bits = 32 - __clz(span);
      const int shift = bits > 12 ? bits - 12 : 0;
      const int nb = (int)(span >> shift) + 1;
      const bool build = !use_list && in_range <= SEL_LIST;
      __syncthreads();  // the previous pass's readers of hist / red are done
#pragma unroll
      for (int e = 0; e < 4; ++e) hist[4 * tid + e] = 0u;
      if (tid == 0) red[130] = 0;
      __syncthreads();
      if (use_list) {
        for (int j = tid; j < nlist; j += SEL_THREADS) {
          const uint32_t k = list[j];
          if (k - lo <= span) atomicAdd(&hist[(k - lo) >> shift], 1u);
        }
      } else {
        // candidates of chunk g (tokens 4g..4g+3) inside [lo, hi]; forced
        // tokens and the tail of a partial chunk hold key 0 < lo
        auto in_range4 = [&](int g, u32x4& kv) -> uint32_t {
          kv = *reinterpret_cast<const u32x4*>(keys + 4 * kchunk(g));
          uint32_t m = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) m |= (uint32_t)(kv[e] - lo <= span) << e;
          return m;
        };
        int cnt = 0;
        for (int g = tid; g < (n + 3) / 4; g += SEL_THREADS) {
          u32x4 kv;
          const uint32_t m = in_range4(g, kv);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((m >> e) & 1u) atomicAdd(&hist[(kv[e] - lo) >> shift], 1u);
          cnt += __popc(m);
        }
        if (build) {
          // one list reservation per wave, then a second read writes the keys
          const int incl = wave_incl_scan(cnt);
          int base = 0;
          if (lane == 63) base = atomicAdd(&red[130], incl);
          int pos = __builtin_amdgcn_readlane(base, 63) + incl - cnt;
          for (int g = tid; g < (n + 3) / 4; g += SEL_THREADS) {
            u32x4 kv;
            const uint32_t m = in_range4(g, kv);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if ((m >> e) & 1u) list[pos++] = kv[e];
          }
        }
      }
      __syncthreads();
      if (build) {
        nlist = red[130];
        use_list = true;
      }
      // thread t owns bins 4t'..4t'+3, t' = 1023 - t: an inclusive scan in
      // thread order counts the keys in every bin >= 4t'
      const int tb = 4 * (SEL_THREADS - 1 - tid);
      int h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = tb + e < nb ? (int)hist[tb + e] : 0;
      const int mine = h[0] + h[1] + h[2] + h[3];
      int incl = wave_incl_scan(mine);
      if (lane == 63) red[64 + w] = incl;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < SEL_WAVES; ++v) incl += v < w ? red[64 + v] : 0;
      int above = incl - mine;  // keys in bins above tb + 3
      if (above < need && incl >= need) {
        int bstar = tb, cnt = h[0];
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          if (above + h[e] >= need) {
            bstar = tb + e;
            cnt = h[e];
            break;
          }
          above += h[e];
        }
        red[128] = bstar;
        red[129] = above;
        red[131] = cnt;
      }
      __syncthreads();
      const int bstar = red[128];
      need -= red[129];
      in_range = red[131];
      const uint64_t nlo = (uint64_t)lo + ((uint64_t)bstar << shift);
      const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
      lo = (uint32_t)nlo;
      hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
      if (shift == 0) {
        T = lo;
        needT = need;
        break;
      }
    }
  }

  // ---- emit ----
  // thread t owns tokens [32t, 32t + 32): 32-bit masks of sure keeps (forced,
  // key 0, or key > T) and of ties (candidate key == T), one block scan of
  // the packed (sure, tie) counts, the first needT ties in index order are
  // kept, and each thread writes its kept indices in order. T = 0 keeps
  // every token; T = 0xffffffff (no candidate slot) keeps the forced ones.
  uint32_t sure = 0u, tie = 0u;
  const int i0 = 32 * tid;
  if (i0 < n) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(keys + 4 * kchunk(8 * tid + q));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = 4 * q + e;
        const bool in = i0 + bit < n;
        const uint32_t k = kv[e];
        sure |= (uint32_t)(in && (k == 0u || k > T)) << bit;
        tie |= (uint32_t)(in && k != 0u && k == T) << bit;
      }
    }
  }
  // sure and tie totals are <= 32768, so the packed halves never carry
  const uint32_t packed = (uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16);
  const uint32_t incl = (uint32_t)wave_incl_scan((int)packed);
  __syncthreads();  // red is free
  if (lane == 63) red[w] = (int)incl;
  __syncthreads();
  uint32_t excl = incl - packed;
#pragma unroll
  for (int v = 0; v < SEL_WAVES; ++v) excl += v < w ? (uint32_t)red[v] : 0u;
  const int sure_before = (int)(excl & 0xffffu), tie_before = (int)(excl >> 16);
  const int take = min(max(needT - tie_before, 0), __popc(tie));
  uint32_t rest = tie;  // drop the lowest `take` tie bits from rest: they are kept
  for (int c = 0; c < take; ++c) rest &= rest - 1u;
  uint32_t keep = sure | (tie ^ rest);
  int pos = sure_before + min(tie_before, needT);
  while (keep) {
    const int bit = __builtin_ctz(keep);
    if (pos < K) kp[pos] = in0 + i0 + bit;  // pos < K always holds; the guard keeps a logic slip in bounds
    ++pos;
    keep &= keep - 1u;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(
    const float* __restrict__ s, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
    int32_t* __restrict__ kept, int32_t* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sel_smem[];
  __shared__ uint32_t hist[SEL_LDS_BINS];
  __shared__ int shi[SEL_WAVES];
  __shared__ uint32_t shu[SEL_WAVES];
  __shared__ int found[2];
  __shared__ int red[132];
  __shared__ uint32_t list[SEL_LIST];

  const int b = blockIdx.x;
  const int in0 = cu_in[b];
  const int n = cu_in[b + 1] - in0;
  const int out0 = cu_kept[b];
  const int K = cu_kept[b + 1] - out0;
  const float* sp = s + in0;
  const uint8_t* mp = mask ? mask + in0 : nullptr;
  int32_t* st = status ? status + b : nullptr;
  if (n <= SEL_LDS_MAX)
    select_lds(sp, mp, n, K, in0, kept + out0, st, sel_smem, hist, red, list);
  else
    select_global(sp, mp, n, K, in0, kept + out0, st, hist, shi, shu, found);
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int32_t* kept, int32_t* status,
                              hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  constexpr size_t lds = (size_t)SEL_LDS_MAX * sizeof(uint32_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(SEL_THREADS), lds, stream, s, mask, cu_in,
                     cu_kept, kept, status);
  return hipGetLastError();
}

}  // namespace tg
