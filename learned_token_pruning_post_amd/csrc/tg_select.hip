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
// Up to SEL_LDS_MAX tokens per sequence, one workgroup holds a sequence's keys
// in LDS (select_keys). Longer sequences run the same search and emit spread
// over many workgroups of MW_CHUNK tokens each, as a chain of short kernels
// (the "mw" kernels below).
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

// Search key of a token: 0 if forced, 1 if a NaN candidate, else its order
// key (>= 0x007fffff, the key of -inf), so range tests skip forced tokens by
// value.
__device__ __forceinline__ uint32_t sel_key(float x, bool forced, bool& is_nan) {
  const uint32_t k = score_key(x, is_nan);
  return forced ? 0u : (is_nan ? 1u : k);
}

// ---------------------------------------------------------------------------
// Keys in LDS (sequences of up to SEL_LDS_MAX tokens, loaded once).
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

__device__ __forceinline__ void select_keys(const float* __restrict__ sp, const uint8_t* __restrict__ mp, int n,
                           int K, int in0, int32_t* __restrict__ kp, int32_t* __restrict__ status_b,
                           uint32_t* keys, uint32_t* hist, int* red, uint32_t* list) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NG = SEL_LDS_MAX / 4 / SEL_THREADS;  // 4-token groups per thread

  // ---- load ----
  // LDS key of a token: sel_key; the tail of a partial 4-token chunk holds 0,
  // so it is never in range either.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  int nf = 0, nan_seen = 0;
  auto take_key = [&](float x, bool f) -> uint32_t {  // with the statistics
    bool isn;
    const uint32_t k = sel_key(x, f, isn);
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
  // load the sequence into LDS with the statistics
  {
    const int nr = n;
    const float* spr = sp;
    const uint8_t* mpr = mp;
    auto key = [&](float x, bool f) -> uint32_t { return take_key(x, f); };
    if (vec) {
      // chunk g = u*1024 + tid holds tokens 4g..4g+3: all loads are issued
      // before any is used
      constexpr int NGB = NG;
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
          if (i < nr) *reinterpret_cast<u32x4*>(keys + 4 * kchunk(g)) = kv;
        }
      }
    } else {
      for (int i = tid; i < ((nr + 3) & ~3); i += SEL_THREADS) {
        const uint32_t k = i < nr ? key(spr[i], mpr && mpr[i]) : 0u;
        keys[4 * kchunk(i >> 2) + (i & 3)] = k;
      }
    }
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
        {
          const int ng = (n + 3) / 4;
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
  // thread t owns tokens [32t, 32t + 32): 32-bit masks of sure keeps
  // (forced, key 0, or key > T) and of ties (candidate key == T), one block
  // scan of the packed (sure, tie) counts, the first needT ties in index
  // order are kept, and each thread writes its kept indices in order.
  // T = 0 keeps every token; T = 0xffffffff (no candidate slot) keeps the
  // forced ones.
  {
    const int nr = n;
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
    const int tok0 = in0 + i0;
    while (keep) {
      const int bit = __builtin_ctz(keep);
      if (pos < K) kp[pos] = tok0 + bit;  // pos < K always holds; the guard keeps a logic slip in bounds
      ++pos;
      keep &= keep - 1u;
    }
  }
}

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
  if (n > SEL_LDS_MAX) {  // longer than the max_n the host announced
    if (threadIdx.x == 0 && st) *st = 8;  // TG_DEV_LEN_GT_MAX_N
    for (int i = threadIdx.x; i < K; i += SEL_THREADS) kept[out0 + i] = -1;
    return;
  }
  select_keys(sp, mp, n, K, in0, kept + out0, st, sel_smem, hist, red, list);
}

// ---------------------------------------------------------------------------
// Sequences longer than SEL_LDS_MAX: the LDS path's range search and emit,
// spread over workgroups of MW_CHUNK consecutive tokens of one sequence, as a
// chain of kernels in which no workgroup waits for another:
//   init   clears each sequence's histogram and statistics (workspace)
//   stats  per chunk: forced count, NaN seen, candidate key min and max,
//          merged with global atomics
//   plan   per sequence: status flags and -1 slots for a rejected sequence;
//          the threshold at once when the budget takes no candidate, every
//          candidate, or the live range is one key; else [kmin, kmax]
//   3 x  { hist (per chunk: LDS histogram of the live range in 4096
//          power-of-two bins, merged with global atomics), pick (per
//          sequence: the bin that holds the threshold; clears the histogram
//          for the next pass) }: a range shrinks 2^12-fold per pass, so three
//          passes reach one key from any 32-bit span
//   count  per chunk: sure keeps (forced or key > T) and ties (key == T)
//   emit   per chunk: the earlier chunks' counts, one block scan, the first
//          needT ties of the sequence in index order, indices ascending
// Keys are formed again from the scores on every walk (sel_key), so the
// workspace holds per sequence only its state and one histogram, plus two
// counts per chunk. Thread t of a chunk owns its tokens 16t..16t+15.
// ---------------------------------------------------------------------------
constexpr int MW_THREADS = 256;
constexpr int MW_TPT = 16;                     // consecutive tokens per thread
constexpr int MW_CHUNK = MW_THREADS * MW_TPT;  // tokens per workgroup
constexpr int MW_BINS = 4096;
constexpr int MW_PICK_THREADS = MW_BINS / 4;   // 4 bins per thread
constexpr int MW_PASSES = 3;

struct MwState {
  uint32_t lo, hi;      // live key range of the search
  int need;             // candidates still to take inside [lo, hi]
  int active;           // the range search is still running
  uint32_t T;           // threshold key
  int needT;            // keys equal to T that are kept, lowest indices first
  int nf, nan_seen;     // forced tokens; some candidate score is NaN
  uint32_t kmin, kmax;  // candidate key range
  int skip;             // rejected sequence: its slots already hold -1
  int pad[5];
};
static_assert(sizeof(MwState) == 64, "64-byte per-sequence state");

struct MwWs {
  MwState* st;     // [B]
  uint32_t* hist;  // [B][MW_BINS]
  int2* counts;    // (sure, tie) per chunk; chunk c of sequence b at mw_chunk_slot(in0_b, b) + c
};

__host__ __device__ inline size_t mw_align(size_t x) { return (x + 255) & ~(size_t)255; }
// Chunk slots of sequence b start at in0_b / MW_CHUNK + b: the sequences
// before b hold sum(ceil(N / MW_CHUNK)) <= in0_b / MW_CHUNK + b chunks, so
// the ranges never overlap and T_in / MW_CHUNK + B + 1 slots cover a batch.
__device__ __forceinline__ int64_t mw_chunk_slot(int in0, int b) { return (int64_t)(in0 / MW_CHUNK) + b; }

static size_t mw_workspace_bytes(int B, int64_t T_in) {
  return mw_align((size_t)B * sizeof(MwState)) + mw_align((size_t)B * MW_BINS * sizeof(uint32_t)) +
         mw_align((size_t)(T_in / MW_CHUNK + B + 1) * sizeof(int2));
}

static MwWs mw_carve(void* ws, int B) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  MwWs w;
  w.st = reinterpret_cast<MwState*>(p);
  p += mw_align((size_t)B * sizeof(MwState));
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += mw_align((size_t)B * MW_BINS * sizeof(uint32_t));
  w.counts = reinterpret_cast<int2*>(p);
  return w;
}

// keys of the thread's tokens [i0, i0 + 16) of a sequence; returns how many
// of them exist (tokens at or past n read as key 0 and are never used);
// nan_bits marks NaN scores, forced tokens included (they set the status flag)
__device__ __forceinline__ int mw_keys(const float* __restrict__ sp, const uint8_t* __restrict__ mp,
                                       int n, int i0, bool vec, uint32_t (&k)[MW_TPT], uint32_t& nan_bits) {
  const int nv = min(max(n - i0, 0), MW_TPT);
  nan_bits = 0u;
  if (vec && nv == MW_TPT) {
    f32x4 x[MW_TPT / 4];
    u32x4 m = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < MW_TPT / 4; ++q) x[q] = *reinterpret_cast<const f32x4*>(sp + i0 + 4 * q);
    if (mp) m = *reinterpret_cast<const u32x4*>(mp + i0);
#pragma unroll
    for (int q = 0; q < MW_TPT / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool isn;
        k[4 * q + e] = sel_key(x[q][e], ((m[q] >> (8 * e)) & 0xffu) != 0u, isn);
        nan_bits |= (uint32_t)isn << (4 * q + e);
      }
  } else {
#pragma unroll
    for (int j = 0; j < MW_TPT; ++j) {
      bool isn = false;
      k[j] = j < nv ? sel_key(sp[i0 + j], mp && mp[i0 + j], isn) : 0u;
      nan_bits |= (uint32_t)isn << j;
    }
  }
  return nv;
}

// the workgroup's sequence and chunk; false if the chunk is past the sequence
struct MwChunk {
  int b, c, in0, n, i0;
  const float* sp;
  const uint8_t* mp;
  bool vec;
};
__device__ __forceinline__ bool mw_chunk(const float* s, const uint8_t* mask, const int32_t* cu_in, int nch,
                                         MwChunk& ck) {
  ck.b = blockIdx.x / nch;
  ck.c = blockIdx.x % nch;
  ck.in0 = cu_in[ck.b];
  ck.n = cu_in[ck.b + 1] - ck.in0;
  if (ck.c * MW_CHUNK >= ck.n) return false;
  ck.i0 = ck.c * MW_CHUNK + (int)threadIdx.x * MW_TPT;
  ck.sp = s + ck.in0;
  ck.mp = mask ? mask + ck.in0 : nullptr;
  ck.vec = (reinterpret_cast<uintptr_t>(ck.sp) & 15u) == 0 && (reinterpret_cast<uintptr_t>(ck.mp) & 15u) == 0;
  return true;
}

__global__ __launch_bounds__(MW_THREADS) void mw_init_kernel(MwWs ws) {
  const int b = blockIdx.x;
  uint32_t* h = ws.hist + (size_t)b * MW_BINS;
  for (int i = threadIdx.x; i < MW_BINS; i += MW_THREADS) h[i] = 0u;
  if (threadIdx.x == 0) {
    MwState z = {};
    z.kmin = 0xffffffffu;
    ws.st[b] = z;
  }
}

__global__ __launch_bounds__(MW_THREADS) void mw_stats_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                              const int32_t* __restrict__ cu_in, int nch, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, nch, ck)) return;
  uint32_t k[MW_TPT], nanb;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, k, nanb);
  int nf = 0;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < MW_TPT; ++j)
    if (j < nv) {
      nf += k[j] == 0u;
      if (k[j] != 0u) {
        kmin = min(kmin, k[j]);
        kmax = max(kmax, k[j]);
      }
    }
  int nan_seen = nanb != 0u;
  nf = lane63(wave_incl_scan(nf));
  nan_seen = lane63(wave_incl_scan(nan_seen));
  kmin = (uint32_t)lane63((int)wave_scan_u32(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }));
  kmax = (uint32_t)lane63((int)wave_scan_u32(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }));
  __shared__ uint32_t red[MW_THREADS / 64][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    red[w][0] = (uint32_t)nf;
    red[w][1] = (uint32_t)nan_seen;
    red[w][2] = kmin;
    red[w][3] = kmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0u, o = 0u, lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int v = 0; v < MW_THREADS / 64; ++v) {
      a += red[v][0];
      o |= red[v][1];
      lo = min(lo, red[v][2]);
      hi = max(hi, red[v][3]);
    }
    MwState* st = ws.st + ck.b;
    if (a) atomicAdd(&st->nf, (int)a);
    if (o) atomicOr(&st->nan_seen, 1);
    if (lo <= hi) {
      atomicMin(&st->kmin, lo);
      atomicMax(&st->kmax, hi);
    }
  }
}

// One wave per sequence: flags, rejection, or the start of the range search.
__global__ __launch_bounds__(64) void mw_plan_kernel(const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                     int max_n, int32_t* __restrict__ kept, int32_t* __restrict__ status,
                                                     MwWs ws) {
  const int b = blockIdx.x;
  const int in0 = cu_in[b], n = cu_in[b + 1] - in0;
  const int out0 = cu_kept[b], K = cu_kept[b + 1] - out0;
  MwState* st = ws.st + b;
  const int nf = st->nf, nan_seen = st->nan_seen;
  const uint32_t kmin = st->kmin, kmax = st->kmax;
  // a sequence longer than max_n has chunks outside the grid: rejected
  const int flags = n > max_n ? 8 : ((nan_seen ? 4 : 0) | (K > n ? 2 : 0) | (nf > K ? 1 : 0));
  if (threadIdx.x == 0 && status) status[b] = flags;
  if (flags & 11) {
    for (int i = threadIdx.x; i < K; i += 64) kept[out0 + i] = -1;
    if (threadIdx.x == 0) st->skip = 1;
    return;
  }
  if (threadIdx.x != 0) return;
  const int C = n - nf, r = K - nf;  // candidates, slots for them
  uint32_t T = 0u;
  int needT = 0, active = 0;
  if (r == 0) {
    T = 0xffffffffu;  // no key reaches it
  } else if (r == C) {
    needT = C;  // T = 0: every token is kept
  } else if (kmin == kmax) {
    T = kmin;
    needT = r;
  } else {
    active = 1;
  }
  st->lo = kmin;
  st->hi = kmax;
  st->need = r;
  st->T = T;
  st->needT = needT;
  st->active = active;
}

__global__ __launch_bounds__(MW_THREADS) void mw_hist_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                             const int32_t* __restrict__ cu_in, int nch, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, nch, ck)) return;
  const MwState* st = ws.st + ck.b;
  if (!st->active) return;
  const uint32_t lo = st->lo, span = st->hi - lo;
  const int bits = 32 - __clz(span);
  const int shift = bits > 12 ? bits - 12 : 0;
  const int nb = (int)(span >> shift) + 1;
  __shared__ uint32_t h[MW_BINS];
  for (int i = threadIdx.x; i < nb; i += MW_THREADS) h[i] = 0u;
  __syncthreads();
  uint32_t k[MW_TPT], nanb;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, k, nanb);
#pragma unroll
  for (int j = 0; j < MW_TPT; ++j)
    if (j < nv && k[j] - lo <= span) atomicAdd(&h[(k[j] - lo) >> shift], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)ck.b * MW_BINS;
  for (int i = threadIdx.x; i < nb; i += MW_THREADS)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Per sequence: thread t owns bins 4t'..4t'+3 with t' = 1023 - t, so an
// inclusive scan in thread order counts the keys in every bin >= 4t'.
__global__ __launch_bounds__(MW_PICK_THREADS) void mw_pick_kernel(MwWs ws) {
  const int b = blockIdx.x;
  MwState* st = ws.st + b;
  if (!st->active) return;
  const uint32_t lo = st->lo, hi = st->hi, span = hi - lo;
  const int need = st->need;
  const int bits = 32 - __clz(span);
  const int shift = bits > 12 ? bits - 12 : 0;
  const int nb = (int)(span >> shift) + 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tb = 4 * (MW_PICK_THREADS - 1 - tid);
  uint32_t* gh = ws.hist + (size_t)b * MW_BINS;
  int h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = tb + e < nb ? (int)gh[tb + e] : 0;
    gh[tb + e] = 0u;  // cleared for the next pass (only this thread reads these bins)
  }
  __shared__ int red[MW_PICK_THREADS / 64 + 3];
  const int mine = h[0] + h[1] + h[2] + h[3];
  int incl = wave_incl_scan(mine);
  if (lane == 63) red[w] = incl;
  __syncthreads();
#pragma unroll
  for (int v = 0; v < MW_PICK_THREADS / 64; ++v) incl += v < w ? red[v] : 0;
  int above = incl - mine;  // keys in bins above tb + 3
  constexpr int R = MW_PICK_THREADS / 64;
  if (above < need && incl >= need) {
    int bstar = tb;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (above + h[e] >= need) {
        bstar = tb + e;
        break;
      }
      above += h[e];
    }
    red[R] = bstar;
    red[R + 1] = above;
  }
  __syncthreads();
  if (tid != 0) return;
  const uint64_t nlo = (uint64_t)lo + ((uint64_t)red[R] << shift);
  const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
  const uint32_t lo2 = (uint32_t)nlo, hi2 = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  const int need2 = need - red[R + 1];
  st->lo = lo2;
  st->hi = hi2;
  st->need = need2;
  if (shift == 0 || lo2 == hi2) {
    st->T = lo2;
    st->needT = need2;
    st->active = 0;
  }
}

// sure keeps (forced, key 0, or key > T) and ties (candidate key == T) of the
// thread's tokens, bit j for token i0 + j
__device__ __forceinline__ void mw_keep_bits(const uint32_t (&k)[MW_TPT], int nv, uint32_t T, uint32_t& sure,
                                             uint32_t& tie) {
  sure = 0u;
  tie = 0u;
#pragma unroll
  for (int j = 0; j < MW_TPT; ++j) {
    const bool in = j < nv;
    sure |= (uint32_t)(in && (k[j] == 0u || k[j] > T)) << j;
    tie |= (uint32_t)(in && k[j] != 0u && k[j] == T) << j;
  }
}

__global__ __launch_bounds__(MW_THREADS) void mw_count_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                              const int32_t* __restrict__ cu_in, int nch, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, nch, ck)) return;
  const MwState* st = ws.st + ck.b;
  if (st->skip) return;
  uint32_t k[MW_TPT], nanb, sure, tie;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, k, nanb);
  mw_keep_bits(k, nv, st->T, sure, tie);
  // chunk totals are <= 4096, so the packed halves never carry
  const uint32_t packed = (uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16);
  const uint32_t tot = (uint32_t)lane63(wave_incl_scan((int)packed));
  __shared__ uint32_t red[MW_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tot;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0u;
#pragma unroll
    for (int v = 0; v < MW_THREADS / 64; ++v) a += red[v];
    ws.counts[mw_chunk_slot(ck.in0, ck.b) + ck.c] = make_int2((int)(a & 0xffffu), (int)(a >> 16));
  }
}

__global__ __launch_bounds__(MW_THREADS) void mw_emit_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                             const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                             int nch, int32_t* __restrict__ kept, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, nch, ck)) return;
  const MwState* st = ws.st + ck.b;
  if (st->skip) return;
  const int out0 = cu_kept[ck.b], K = cu_kept[ck.b + 1] - out0;
  const uint32_t T = st->T;
  const int needT = st->needT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // kept sure tokens and ties of the sequence's earlier chunks
  const int2* cnt = ws.counts + mw_chunk_slot(ck.in0, ck.b);
  int ps = 0, pt = 0;
  for (int c = tid; c < ck.c; c += MW_THREADS) {
    const int2 v = cnt[c];
    ps += v.x;
    pt += v.y;
  }
  ps = lane63(wave_incl_scan(ps));
  pt = lane63(wave_incl_scan(pt));
  __shared__ int red[MW_THREADS / 64][2];
  __shared__ uint32_t red2[MW_THREADS / 64];
  if (lane == 0) {
    red[w][0] = ps;
    red[w][1] = pt;
  }
  uint32_t k[MW_TPT], nanb, sure, tie;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, k, nanb);
  mw_keep_bits(k, nv, T, sure, tie);
  const uint32_t packed = (uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16);
  const uint32_t incl = (uint32_t)wave_incl_scan((int)packed);
  if (lane == 63) red2[w] = incl;
  __syncthreads();
  int sure_run = 0, tie_run = 0;
  uint32_t excl = incl - packed;
#pragma unroll
  for (int v = 0; v < MW_THREADS / 64; ++v) {
    sure_run += red[v][0];
    tie_run += red[v][1];
    excl += v < w ? red2[v] : 0u;
  }
  const int sure_before = sure_run + (int)(excl & 0xffffu), tie_before = tie_run + (int)(excl >> 16);
  const int take = min(max(needT - tie_before, 0), __popc(tie));
  uint32_t rest = tie;  // drop the lowest `take` tie bits from rest: they are kept
  for (int c = 0; c < take; ++c) rest &= rest - 1u;
  uint32_t keep = sure | (tie ^ rest);
  int pos = sure_before + min(tie_before, needT);
  int32_t* kp = kept + out0;
  const int tok0 = ck.in0 + ck.i0;
  while (keep) {
    const int bit = __builtin_ctz(keep);
    if (pos < K) kp[pos] = tok0 + bit;  // pos < K always holds; the guard keeps a logic slip in bounds
    ++pos;
    keep &= keep - 1u;
  }
}

size_t topk_select_workspace_bytes(int B, int64_t T_in, int max_n) {
  return max_n <= SEL_LDS_MAX || B <= 0 ? 0 : mw_workspace_bytes(B, T_in);
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int64_t T_in, int max_n, int32_t* kept,
                              int32_t* status, void* ws, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  if (max_n <= SEL_LDS_MAX) {
    constexpr size_t lds = (size_t)SEL_LDS_MAX * sizeof(uint32_t);
    const hipError_t e = ensure_dynamic_lds<topk_select_kernel>((int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(SEL_THREADS), lds, stream, s, mask, cu_in,
                       cu_kept, kept, status);
    return hipGetLastError();
  }
  const int nch = (int)(((int64_t)max_n + MW_CHUNK - 1) / MW_CHUNK);
  const int64_t nblk = (int64_t)nch * B;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const MwWs w = mw_carve(ws, B);
  const dim3 g((unsigned)nblk);
#define TG_MW(...)                                   \
  do {                                               \
    hipLaunchKernelGGL(__VA_ARGS__);                 \
    const hipError_t e_ = hipGetLastError();         \
    if (e_ != hipSuccess) return e_;                 \
  } while (0)
  TG_MW(mw_init_kernel, dim3(B), dim3(MW_THREADS), 0, stream, w);
  TG_MW(mw_stats_kernel, g, dim3(MW_THREADS), 0, stream, s, mask, cu_in, nch, w);
  TG_MW(mw_plan_kernel, dim3(B), dim3(64), 0, stream, cu_in, cu_kept, max_n, kept, status, w);
  for (int p = 0; p < MW_PASSES; ++p) {
    TG_MW(mw_hist_kernel, g, dim3(MW_THREADS), 0, stream, s, mask, cu_in, nch, w);
    TG_MW(mw_pick_kernel, dim3(B), dim3(MW_PICK_THREADS), 0, stream, w);
  }
  TG_MW(mw_count_kernel, g, dim3(MW_THREADS), 0, stream, s, mask, cu_in, nch, w);
  TG_MW(mw_emit_kernel, g, dim3(MW_THREADS), 0, stream, s, mask, cu_in, cu_kept, nch, kept, w);
#undef TG_MW
  return hipSuccess;
}

}  // namespace tg
