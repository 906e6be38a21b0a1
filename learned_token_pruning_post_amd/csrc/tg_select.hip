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
// Keys live in LDS (select_keys): a sequence of up to SEL_LDS_MAX tokens is
// loaded once; a longer one is walked in rounds of SEL_LDS_MAX tokens, each
// reloaded with coalesced 16-byte loads before every walk over it.
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_LDS_MAX = 32768;                       // keys held in LDS (one round)

__device__ __forceinline__ uint32_t score_key(float x, bool& is_nan) {
  uint32_t u = __float_as_uint(x);
  is_nan = (u & 0x7fffffffu) > 0x7f800000u;
  if (is_nan) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Keys in LDS, in rounds of SEL_LDS_MAX tokens (one round: loaded once).
//  * load: every thread issues all of its 16-byte score loads and 4-byte
//    mask loads before using any; forced tokens are stored as key 0 and NaN
//    candidates as key 1, below every number's key, so no separate forced
//    bitmap is kept;
//  * one fused reduction of (forced count, NaN flag, candidate min, max);
//  * range passes with SEL_LDS_BINS = 4096 power-of-two bins (the span
//    shrinks by 2^12 per pass). Once the live range holds at most SEL_LIST
//    candidates, the pass that scans all keys also gathers those into a
//    list, and the remaining passes read only the list;
//  * emit: thread t owns tokens 32t..32t+31 of a round; one block scan of
//    packed (sure, tie) counts gives every thread its output slot and the
//    tie rank of its first tie (after those of earlier rounds), so kept
//    indices are written in ascending order.
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

template <bool MULTI>
__device__ __forceinline__ void select_keys(const float* __restrict__ sp, const uint8_t* __restrict__ mp, int n,
                           int K, int in0, int32_t* __restrict__ kp, int32_t* __restrict__ status_b,
                           uint32_t* keys, uint32_t* hist, int* red, uint32_t* list) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NG = SEL_LDS_MAX / 4 / SEL_THREADS;  // 4-token groups per thread
  // tokens in rounds of SEL_LDS_MAX: a sequence that fits (!MULTI) stays in
  // LDS after the first load; longer ones reload round r before each walk
  // over it (a separate instantiation, so the one-round code carries none of it)
  const int nrounds = MULTI ? (n + SEL_LDS_MAX - 1) / SEL_LDS_MAX : (n > 0);
  auto round_len = [&](int r) { return min(n - r * SEL_LDS_MAX, SEL_LDS_MAX); };

  // ---- load ----
  // LDS key of a token: 0 if forced, 1 if a NaN candidate, else its order
  // key (>= 0x007fffff, the key of -inf), so range tests skip forced tokens
  // by value and the tail of a partial 4-token chunk (0) is never in range.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  auto lds_key = [](float x, bool f, bool& isn) -> uint32_t {
    const uint32_t k = score_key(x, isn);
    return f ? 0u : (isn ? 1u : k);
  };
  auto take_key = [&](float x, bool f) -> uint32_t {  // with the statistics
    bool isn;
    const uint32_t k = lds_key(x, f, isn);
    nan_seen |= isn;
    nf += f;
    if (!f) {
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
    return k;
  };
  const bool vec = (reinterpret_cast<uintptr_t>(sp) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(mp) & 3u) == 0;
  // load round r into LDS (store = false: statistics only, nothing written)
  auto load_round = [&](int r, bool stats, bool store) {
    const int nr = round_len(r);
    const float* spr = sp + (size_t)r * SEL_LDS_MAX;
    const uint8_t* mpr = mp ? mp + (size_t)r * SEL_LDS_MAX : nullptr;
    auto key = [&](float x, bool f) -> uint32_t {
      if (stats) return take_key(x, f);
      bool isn;
      return lds_key(x, f, isn);
    };
    if (vec) {
      // chunk g = u*1024 + tid holds tokens 4g..4g+3: the loads of a batch
      // are all issued first (one batch of 8 for a single round; rounds that
      // are reloaded inside the passes use batches of 4, fewer registers)
      constexpr int NGB = MULTI ? NG / 2 : NG;
#pragma unroll
      for (int u0 = 0; u0 < NG; u0 += NGB) {
        f32x4 xv[NGB];
        uint32_t mv[NGB];
#pragma unroll
        for (int uu = 0; uu < NGB; ++uu) {
          const int i = 4 * ((u0 + uu) * SEL_THREADS + tid);
          mv[uu] = 0u;
          if (i + 3 < nr) {
            xv[uu] = *reinterpret_cast<const f32x4*>(spr + i);
            if (mpr) mv[uu] = *reinterpret_cast<const uint32_t*>(mpr + i);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xv[uu][e] = i + e < nr ? spr[i + e] : 0.f;
              if (mpr && i + e < nr && mpr[i + e]) mv[uu] |= 1u << (8 * e);
            }
          }
        }
#pragma unroll
        for (int uu = 0; uu < NGB; ++uu) {
          const int g = (u0 + uu) * SEL_THREADS + tid, i = 4 * g;
          u32x4 kv;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            kv[e] = i + e < nr ? key(xv[uu][e], ((mv[uu] >> (8 * e)) & 0xffu) != 0) : 0u;
          if (store && i < nr) *reinterpret_cast<u32x4*>(keys + 4 * kchunk(g)) = kv;
        }
      }
    } else {
      for (int i = tid; i < ((nr + 3) & ~3); i += SEL_THREADS) {
        const uint32_t k = i < nr ? key(spr[i], mpr && mpr[i]) : 0u;
        if (store) keys[4 * kchunk(i >> 2) + (i & 3)] = k;
      }
    }
  };
  // walks over the keys of every round: a single round is loaded once (here)
  auto reload = [&](int r) {
    if (MULTI) {
      __syncthreads();  // the previous round's readers are done
      load_round(r, false, true);
      __syncthreads();
    }
  };
  for (int r = 0; r < nrounds; ++r) load_round(r, true, !MULTI);
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
        for (int rr = 0; rr < nrounds; ++rr) {
          reload(rr);
          const int ng = (round_len(rr) + 3) / 4;
          int cnt = 0;
          for (int g = tid; g < ng; g += SEL_THREADS) {
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
            for (int g = tid; g < ng; g += SEL_THREADS) {
              u32x4 kv;
              const uint32_t m = in_range4(g, kv);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if ((m >> e) & 1u) list[pos++] = kv[e];
            }
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
  // per round, thread t owns tokens [32t, 32t + 32): 32-bit masks of sure
  // keeps (forced, key 0, or key > T) and of ties (candidate key == T), one
  // block scan of the packed (sure, tie) counts, the first needT ties in
  // index order are kept, and each thread writes its kept indices in order;
  // the counts of earlier rounds carry over. T = 0 keeps every token;
  // T = 0xffffffff (no candidate slot) keeps the forced ones.
  int sure_run = 0, tie_run = 0;  // kept sure tokens and ties seen in earlier rounds
  for (int rr = 0; rr < nrounds; ++rr) {
    reload(rr);
    const int nr = round_len(rr);
    uint32_t sure = 0u, tie = 0u;
    const int i0 = 32 * tid;
    if (i0 < nr) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(keys + 4 * kchunk(8 * tid + q));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int bit = 4 * q + e;
          const bool in = i0 + bit < nr;
          const uint32_t k = kv[e];
          sure |= (uint32_t)(in && (k == 0u || k > T)) << bit;
          tie |= (uint32_t)(in && k != 0u && k == T) << bit;
        }
      }
    }
    // per-round sure and tie totals are <= 32768, so the packed halves never carry
    const uint32_t packed = (uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16);
    const uint32_t incl = (uint32_t)wave_incl_scan((int)packed);
    __syncthreads();  // red is free
    if (lane == 63) red[w] = (int)incl;
    __syncthreads();
    uint32_t excl = incl - packed, total = 0u;
#pragma unroll
    for (int v = 0; v < SEL_WAVES; ++v) {
      excl += v < w ? (uint32_t)red[v] : 0u;
      total += (uint32_t)red[v];
    }
    const int sure_before = sure_run + (int)(excl & 0xffffu), tie_before = tie_run + (int)(excl >> 16);
    const int take = min(max(needT - tie_before, 0), __popc(tie));
    uint32_t rest = tie;  // drop the lowest `take` tie bits from rest: they are kept
    for (int c = 0; c < take; ++c) rest &= rest - 1u;
    uint32_t keep = sure | (tie ^ rest);
    int pos = sure_before + min(tie_before, needT);
    const int tok0 = in0 + rr * SEL_LDS_MAX + i0;
    while (keep) {
      const int bit = __builtin_ctz(keep);
      if (pos < K) kp[pos] = tok0 + bit;  // pos < K always holds; the guard keeps a logic slip in bounds
      ++pos;
      keep &= keep - 1u;
    }
    sure_run += (int)(total & 0xffffu);
    tie_run += (int)(total >> 16);
  }
}

// MULTI: some sequence may be longer than one LDS round (max_n > SEL_LDS_MAX);
// a separate kernel, so the one-round kernel keeps its lower register count
template <bool MULTI>
__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(
    const float* __restrict__ s, const uint8_t* __restrict__ mask,
    const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
    int32_t* __restrict__ kept, int32_t* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sel_smem[];
  __shared__ uint32_t hist[SEL_LDS_BINS];
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
  if (!MULTI && n > SEL_LDS_MAX) {  // longer than the max_n the host announced
    if (threadIdx.x == 0 && st) *st = 8;  // TG_DEV_LEN_GT_MAX_N
    for (int i = threadIdx.x; i < K; i += SEL_THREADS) kept[out0 + i] = -1;
    return;
  }
  select_keys<MULTI>(sp, mp, n, K, in0, kept + out0, st, sel_smem, hist, red, list);
}

template <bool MULTI>
static hipError_t launch_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                                const int32_t* cu_kept, int B, int32_t* kept, int32_t* status,
                                hipStream_t stream) {
  constexpr size_t lds = (size_t)SEL_LDS_MAX * sizeof(uint32_t);
  {
    const hipError_t e = ensure_dynamic_lds<topk_select_kernel<MULTI>>((int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_select_kernel<MULTI>, dim3(B), dim3(SEL_THREADS), lds, stream, s, mask,
                     cu_in, cu_kept, kept, status);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int max_n, int32_t* kept,
                              int32_t* status, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  return max_n <= SEL_LDS_MAX
             ? launch_select<false>(s, mask, cu_in, cu_kept, B, kept, status, stream)
             : launch_select<true>(s, mask, cu_in, cu_kept, B, kept, status, stream);
}

}  // namespace tg
