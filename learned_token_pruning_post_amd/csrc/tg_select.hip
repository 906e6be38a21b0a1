// Top-K selection with forced keep (one workgroup per sequence).
//
// Rule (Tencent Cloud TokenGate article, section on early token filtering; the
// ai.866data article, mechanism-design section): forced tokens are always
// kept; the other K - F slots go to the highest scores, equal scores to the
// lower index, NaN below every number, -0.0 equal to +0.0. Output ascending.
//
// Algorithm: scores map to order-preserving uint32 keys. A range search
// narrows [kmin, kmax] to the threshold key T with histogram passes whose bin
// width is a power of two sized so at most 2048 bins span the live range
// (the range, not the fixed top byte: sigmoid scores share their top bits, a
// fixed-digit radix would pile every key into one or two bins). Each pass
// shrinks the range by >= 2^10, so three passes resolve any 32-bit key. A
// final pass keeps forced tokens, keys > T, and the first `need` keys == T in
// index order (block-wide exclusive scans give each thread its share and its
// output offset).
//
// Sequences of up to SEL_LDS_MAX tokens keep their keys in LDS after one load
// pass (forced tokens carry a flag bit in a separate bitmap), so the
// histogram and emit passes never touch global memory. The key array is
// padded by one word per 32 so that the blocked per-thread reads of the emit
// pass (thread t reads 32t..32t+31) fall on distinct banks. Longer sequences
// stream their scores from global memory with 16 independent loads in flight
// per thread.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_BINS = 2048;
constexpr int SEL_LDS_MAX = 32768;                       // keys held in LDS
constexpr int SEL_KEY_WORDS = SEL_LDS_MAX + SEL_LDS_MAX / 32;  // padded
constexpr int SEL_BATCH = 16;                            // loads in flight (global path)

__device__ __forceinline__ uint32_t score_key(float x, bool& is_nan) {
  uint32_t u = __float_as_uint(x);
  is_nan = (u & 0x7fffffffu) > 0x7f800000u;
  if (is_nan) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int pidx(int i) { return i + (i >> 5); }

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

// Key source of one sequence: LDS-resident (IN_LDS) or streamed from global.
template <bool IN_LDS>
struct KeySrc {
  const float* sp;
  const uint8_t* mp;
  const uint32_t* keys;   // LDS, padded
  const uint32_t* fbits;  // LDS bitmap of forced tokens

  __device__ __forceinline__ bool forced(int i) const {
    if (IN_LDS) return (fbits[i >> 5] >> (i & 31)) & 1u;
    return mp && mp[i];
  }
  __device__ __forceinline__ uint32_t key(int i) const {
    if (IN_LDS) return keys[pidx(i)];
    bool isn;
    return score_key(sp[i], isn);
  }
  // visit (index, key, forced) of the contiguous span [i0, i1) in order
  template <class F>
  __device__ __forceinline__ void blocked(int i0, int i1, F&& f) const {
    if (IN_LDS) {
      for (int i = i0; i < i1; ++i) f(i, keys[pidx(i)], forced(i));
    } else {
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
  }
  // visit (index, key, forced) of the strided set tid, tid+1024, ... (< n);
  // the global variant keeps SEL_BATCH independent loads in flight
  template <class F>
  __device__ __forceinline__ void strided(int n, F&& f) const {
    const int tid = threadIdx.x;
    if (IN_LDS) {
      for (int i = tid; i < n; i += SEL_THREADS) f(i, keys[pidx(i)], forced(i));
    } else {
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
  }
};

template <bool IN_LDS>
__device__ void select_sequence(const float* __restrict__ sp, const uint8_t* __restrict__ mp,
                                int n, int K, int in0, int32_t* __restrict__ kp,
                                int32_t* __restrict__ status_b, uint32_t* keys, uint32_t* fbits,
                                uint32_t* hist, int* shi, uint32_t* shu, int* found) {
  const int tid = threadIdx.x;
  KeySrc<IN_LDS> src{sp, mp, keys, fbits};

  // pass 0: (LDS variant) load keys and forced bits; forced count, NaN flag,
  // live key range of the candidates
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  if (IN_LDS) {
    for (int w = tid; w < (n + 31) / 32; w += SEL_THREADS) fbits[w] = 0u;
    __syncthreads();
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
          keys[pidx(i)] = k;
          if (fm[u]) {
            ++nf;
            atomicOr(&fbits[i >> 5], 1u << (i & 31));
          } else {
            kmin = min(kmin, k);
            kmax = max(kmax, k);
          }
        }
      }
    }
  } else {
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

__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(
    const float* __restrict__ s, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
    int32_t* __restrict__ kept, int32_t* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sel_smem[];
  __shared__ uint32_t hist[SEL_BINS];
  __shared__ int shi[SEL_WAVES];
  __shared__ uint32_t shu[SEL_WAVES];
  __shared__ int found[2];
  __shared__ uint32_t fbits[SEL_LDS_MAX / 32];

  const int b = blockIdx.x;
  const int in0 = cu_in[b];
  const int n = cu_in[b + 1] - in0;
  const int out0 = cu_kept[b];
  const int K = cu_kept[b + 1] - out0;
  const float* sp = s + in0;
  const uint8_t* mp = mask ? mask + in0 : nullptr;
  int32_t* st = status ? status + b : nullptr;
  if (n <= SEL_LDS_MAX)
    select_sequence<true>(sp, mp, n, K, in0, kept + out0, st, sel_smem, fbits, hist, shi, shu,
                          found);
  else
    select_sequence<false>(sp, mp, n, K, in0, kept + out0, st, sel_smem, fbits, hist, shi, shu,
                           found);
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int32_t* kept, int32_t* status,
                              hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  constexpr size_t lds = (size_t)SEL_KEY_WORDS * sizeof(uint32_t);
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
