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
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_BINS = 2048;

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

__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(
    const float* __restrict__ s, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
    int32_t* __restrict__ kept, int32_t* __restrict__ status) {
  __shared__ uint32_t hist[SEL_BINS];
  __shared__ int shi[SEL_WAVES];
  __shared__ uint32_t shu[SEL_WAVES];
  __shared__ int found_bin, found_above;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int in0 = cu_in[b];
  const int n = cu_in[b + 1] - in0;
  const int out0 = cu_kept[b];
  const int K = cu_kept[b + 1] - out0;
  const float* sp = s + in0;
  const uint8_t* mp = mask ? mask + in0 : nullptr;

  // pass 0: forced count, NaN flag, live key range of the candidates
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  for (int i = tid; i < n; i += SEL_THREADS) {
    bool isn;
    uint32_t k = score_key(sp[i], isn);
    nan_seen |= isn;
    if (mp && mp[i]) {
      ++nf;
    } else {
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  }
  nf = block_sum_int(nf, shi);
  nan_seen = block_sum_int(nan_seen, shi);
  kmin = block_min_u32(kmin, shu);
  kmax = block_max_u32(kmax, shu);

  int flags = (nan_seen ? 4 : 0) | (K > n ? 2 : 0) | (nf > K ? 1 : 0);
  if (tid == 0 && status) status[b] = flags;
  if (flags & 3) {
    for (int i = tid; i < K; i += SEL_THREADS) kept[out0 + i] = -1;
    return;
  }
  const int C = n - nf;   // candidates
  const int r = K - nf;   // slots for candidates
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
      for (int i = tid; i < n; i += SEL_THREADS) {
        if (mp && mp[i]) continue;
        bool isn;
        uint32_t k = score_key(sp[i], isn);
        if (k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> shift], 1u);
      }
      __syncthreads();
      // suffix sums over bins: thread t owns bins 2t, 2t+1; scan in reverse thread order
      const int t2 = SEL_THREADS - 1 - tid;  // thread t2 holds the reversed rank
      const int b0 = 2 * t2, b1 = 2 * t2 + 1;
      const int h0 = b0 < nb ? (int)hist[b0] : 0;
      const int h1 = b1 < nb ? (int)hist[b1] : 0;
      // inclusive scan over tid of (h0 + h1) of bins ordered from the top
      const int incl = block_incl_scan(h0 + h1, shi);
      const int above_pair = incl - (h0 + h1);  // bins above b1
      if (above_pair < need && incl >= need) {
        if (above_pair + h1 >= need) {
          found_bin = b1;
          found_above = above_pair;
        } else {
          found_bin = b0;
          found_above = above_pair + h1;
        }
      }
      __syncthreads();
      const int bstar = found_bin;
      need -= found_above;
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
  for (int i = i0; i < i1; ++i) {
    if (mp && mp[i]) {
      ++sure;
      continue;
    }
    bool isn;
    uint32_t k = score_key(sp[i], isn);
    sure += (k > T);
    ties += (k == T);
  }
  const int tie_before = block_incl_scan(ties, shi) - ties;
  int take = needT - tie_before;
  take = take < 0 ? 0 : (take > ties ? ties : take);
  const int cnt = sure + take;
  int off = block_incl_scan(cnt, shi) - cnt;
  int taken = 0;
  int32_t* kp = kept + out0;
  for (int i = i0; i < i1; ++i) {
    bool keep;
    if (mp && mp[i]) {
      keep = true;
    } else {
      bool isn;
      uint32_t k = score_key(sp[i], isn);
      keep = k > T;
      if (!keep && k == T && taken < take) {
        keep = true;
        ++taken;
      }
    }
    if (keep && off < K) kp[off++] = in0 + i;  // off < K always holds; the guard keeps a logic slip in bounds
  }
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int32_t* kept, int32_t* status,
                              hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(SEL_THREADS), 0, stream, s, mask, cu_in,
                     cu_kept, kept, status);
  return hipGetLastError();
}

}  // namespace tg
