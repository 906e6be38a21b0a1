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
// chain of six kernels in which no workgroup waits for another:
//   stats      per chunk: forced count, NaN seen, candidate key min and max
//              (one record per chunk); chunk 0 also clears the sequence's
//              three histograms
//   hist 0..2  per chunk: LDS histogram of the live key range in 4096
//              power-of-two bins, merged into that pass's global histogram
//              with atomics
//   count      per chunk: sure keeps (forced or key > T) and ties (key == T)
//   emit       per chunk: the earlier chunks' counts, one block scan, the
//              first needT ties of the sequence in index order, indices
//              written ascending; chunk 0 writes the status (and -1 slots
//              for a rejected sequence)
// The per-sequence decisions (status flags, the live range, the bin of each
// pass) are not stored: every workgroup derives them again from the chunk
// records and the finished histograms (mw_resolve), which costs a
// reduction over the chunk records and one 4096-bin scan per finished pass
// and saves a launch per decision. A range shrinks 2^12-fold per pass, so
// three passes reach one key from any 32-bit span. Keys are formed again
// from the scores on every walk (sel_key). Thread t of a chunk owns its
// tokens 16t..16t+15.
// ---------------------------------------------------------------------------
constexpr int MW_THREADS = 256;
constexpr int MW_WAVES = MW_THREADS / 64;
constexpr int MW_TPT = 16;                     // consecutive tokens per thread
constexpr int MW_CHUNK = MW_THREADS * MW_TPT;  // tokens per workgroup
constexpr int MW_BINS = 4096;
constexpr int MW_PASSES = 3;
static_assert(MW_BINS == MW_THREADS * 16, "a thread scans 16 bins");

struct MwRec {                 // one per chunk
  int nf, nan_seen;            // forced tokens; some score is NaN
  uint32_t kmin, kmax;         // candidate key range (kmin > kmax: none)
  int sure, tie;               // kept sure tokens and ties (count kernel)
  int pad[2];
};
static_assert(sizeof(MwRec) == 32, "32-byte chunk record");

struct MwWs {
  uint32_t* hist;  // [B][MW_PASSES][MW_BINS]
  MwRec* rec;      // chunk c of sequence b at mw_chunk_slot(in0_b, b) + c
};

__host__ __device__ inline size_t mw_align(size_t x) { return (x + 255) & ~(size_t)255; }
// Chunk slots of sequence b start at in0_b / MW_CHUNK + b. A sequence uses
// max(ceil(N / MW_CHUNK), 1) slots (an empty one keeps slot 0 for its
// status), and floor(in0 / C) + max(ceil(N / C), 1) <= floor((in0 + N) / C) + 1,
// so the ranges never overlap and T_in / MW_CHUNK + B + 1 slots cover a batch.
__device__ __forceinline__ int64_t mw_chunk_slot(int in0, int b) { return (int64_t)(in0 / MW_CHUNK) + b; }

static size_t mw_workspace_bytes(int B, int64_t T_in) {
  return mw_align((size_t)B * MW_PASSES * MW_BINS * sizeof(uint32_t)) +
         mw_align((size_t)(T_in / MW_CHUNK + B + 1) * sizeof(MwRec));
}

static MwWs mw_carve(void* ws, int B) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  MwWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += mw_align((size_t)B * MW_PASSES * MW_BINS * sizeof(uint32_t));
  w.rec = reinterpret_cast<MwRec*>(p);
  return w;
}

// A thread's 16 scores and mask bytes, loaded with 16-byte loads when the
// sequence is aligned and all 16 tokens exist (issued before the workgroup's
// decisions are derived, so their latency overlaps that work).
struct MwRaw {
  f32x4 x[MW_TPT / 4];
  u32x4 m;
};
__device__ __forceinline__ void mw_issue(const float* __restrict__ sp, const uint8_t* __restrict__ mp, int n,
                                         int i0, bool vec, MwRaw& raw) {
  if (vec && n - i0 >= MW_TPT) {
#pragma unroll
    for (int q = 0; q < MW_TPT / 4; ++q) raw.x[q] = *reinterpret_cast<const f32x4*>(sp + i0 + 4 * q);
    raw.m = mp ? *reinterpret_cast<const u32x4*>(mp + i0) : u32x4{0u, 0u, 0u, 0u};
  }
}

// keys of the thread's tokens [i0, i0 + 16) of a sequence; returns how many
// of them exist (tokens at or past n read as key 0 and are never used);
// nan_bits marks NaN scores, forced tokens included (they set the status flag)
__device__ __forceinline__ int mw_keys(const float* __restrict__ sp, const uint8_t* __restrict__ mp,
                                       int n, int i0, bool vec, const MwRaw& raw, uint32_t (&k)[MW_TPT],
                                       uint32_t& nan_bits) {
  const int nv = min(max(n - i0, 0), MW_TPT);
  nan_bits = 0u;
  if (vec && nv == MW_TPT) {
    const f32x4* x = raw.x;
    const u32x4 m = raw.m;
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

// the workgroup's sequence and chunk; false if the chunk is past the
// sequence (chunk 0 always exists, also for an empty sequence)
struct MwChunk {
  int b, c, in0, n, K, out0, i0, nchunks;
  const float* sp;
  const uint8_t* mp;
  bool vec;
};
__device__ __forceinline__ bool mw_chunk(const float* s, const uint8_t* mask, const int32_t* cu_in,
                                         const int32_t* cu_kept, int nch, MwChunk& ck) {
  ck.b = blockIdx.x / nch;
  ck.c = blockIdx.x % nch;
  ck.in0 = cu_in[ck.b];
  ck.n = cu_in[ck.b + 1] - ck.in0;
  ck.nchunks = max((ck.n + MW_CHUNK - 1) / MW_CHUNK, 1);
  if (ck.c >= ck.nchunks) return false;
  ck.out0 = cu_kept[ck.b];
  ck.K = cu_kept[ck.b + 1] - ck.out0;
  ck.i0 = ck.c * MW_CHUNK + (int)threadIdx.x * MW_TPT;
  ck.sp = s + ck.in0;
  ck.mp = mask ? mask + ck.in0 : nullptr;
  ck.vec = (reinterpret_cast<uintptr_t>(ck.sp) & 15u) == 0 && (reinterpret_cast<uintptr_t>(ck.mp) & 15u) == 0;
  return true;
}

// Block-wide sum / or / min / max of one value per thread (all threads get
// the result). `scratch` holds MW_WAVES words; the call syncs twice.
template <class Op>
__device__ __forceinline__ uint32_t mw_block_reduce(uint32_t x, uint32_t id, Op op, uint32_t* scratch) {
  x = (uint32_t)lane63((int)wave_scan_u32(x, id, op));
  __syncthreads();  // scratch is free
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t r = id;
#pragma unroll
  for (int v = 0; v < MW_WAVES; ++v) r = op(r, scratch[v]);
  return r;
}

// Block-wide (sum, or, min, max) of four values per thread in one exchange.
__device__ __forceinline__ void mw_block_stats(uint32_t& nf, uint32_t& nan_seen, uint32_t& kmin, uint32_t& kmax,
                                               uint32_t (*scratch)[4]) {
  nf = (uint32_t)lane63((int)wave_scan_u32(nf, 0u, [](uint32_t a, uint32_t b) { return a + b; }));
  nan_seen = (uint32_t)lane63((int)wave_scan_u32(nan_seen, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
  kmin = (uint32_t)lane63((int)wave_scan_u32(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }));
  kmax = (uint32_t)lane63((int)wave_scan_u32(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }));
  __syncthreads();  // scratch is free
  if ((threadIdx.x & 63) == 0) {
    const int w = threadIdx.x >> 6;
    scratch[w][0] = nf;
    scratch[w][1] = nan_seen;
    scratch[w][2] = kmin;
    scratch[w][3] = kmax;
  }
  __syncthreads();
  nf = 0u;
  nan_seen = 0u;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int v = 0; v < MW_WAVES; ++v) {
    nf += scratch[v][0];
    nan_seen |= scratch[v][1];
    kmin = min(kmin, scratch[v][2]);
    kmax = max(kmax, scratch[v][3]);
  }
}

struct MwPlan {
  int flags;           // status flags of the sequence
  bool reject;         // flags & (1 | 2 | 8): slots hold -1
  bool active;         // the range search is still open
  uint32_t lo, hi;     // live range (active)
  int need;            // candidates still to take inside [lo, hi] (active)
  uint32_t T;          // threshold key (done)
  int needT;           // keys equal to T that are kept (done)
};

// The sequence's decisions after `npass` finished histogram passes, derived
// by the whole workgroup (uniform result). Same rules as the LDS path:
// forced tokens always kept; K - F slots to the highest keys; equal keys to
// the lowest indices.
__device__ __forceinline__ MwPlan mw_resolve(const MwChunk& ck, int max_n, const MwWs& ws, int npass) {
  __shared__ uint32_t scratch[MW_WAVES][4];
  __shared__ int pick[2];
  MwPlan P = {};
  if (ck.n > max_n) {  // chunks outside the grid: rejected without statistics
    P.flags = 8;  // TG_DEV_LEN_GT_MAX_N
    P.reject = true;
    return P;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // every load first: the chunk records, then the bins of the finished passes
  // that this thread scans (16 per pass, see below)
  const uint32_t* h0 = ws.hist + (size_t)ck.b * MW_PASSES * MW_BINS;
  const int tb = 16 * (MW_THREADS - 1 - tid);
  u32x4 hv[MW_PASSES][4];
#pragma unroll
  for (int p = 0; p < MW_PASSES; ++p)
    if (p < npass)
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[p][q] = reinterpret_cast<const u32x4*>(h0 + (size_t)p * MW_BINS + tb)[q];
  const MwRec* rec = ws.rec + mw_chunk_slot(ck.in0, ck.b);
  uint32_t nf = 0u, nan_seen = 0u, kmin = 0xffffffffu, kmax = 0u;
  for (int c = tid; c < ck.nchunks; c += MW_THREADS) {
    const MwRec r = rec[c];
    nf += (uint32_t)r.nf;
    nan_seen |= (uint32_t)r.nan_seen;
    kmin = min(kmin, r.kmin);
    kmax = max(kmax, r.kmax);
  }
  mw_block_stats(nf, nan_seen, kmin, kmax, scratch);
  const int n = ck.n, K = ck.K;
  P.flags = (nan_seen ? 4 : 0) | (K > n ? 2 : 0) | ((int)nf > K ? 1 : 0);
  if (P.flags & 3) {
    P.reject = true;
    return P;
  }
  const int C = n - (int)nf, r = K - (int)nf;  // candidates, slots for them
  if (r == 0) {
    P.T = 0xffffffffu;  // no key reaches it
    return P;
  }
  if (r == C) {
    P.T = 0u;  // every token is kept
    P.needT = C;
    return P;
  }
  uint32_t lo = kmin, hi = kmax;
  int need = r;
#pragma unroll
  for (int p = 0; p <= MW_PASSES; ++p) {
    if (lo == hi) {
      P.T = lo;
      P.needT = need;
      return P;
    }
    if (p == npass) break;
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 12 ? bits - 12 : 0;
    // thread t owns bins 16t'..16t'+15 with t' = 255 - t, so an inclusive
    // scan in thread order counts the keys in every bin >= 16t' (bins past
    // the range were never incremented)
    int h[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) h[4 * q + e] = (int)hv[p < MW_PASSES ? p : 0][q][e];
    int mine = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) mine += h[e];
    int incl = wave_incl_scan(mine);
    __syncthreads();  // scratch and pick are free
    if (lane == 63) scratch[w][0] = (uint32_t)incl;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < MW_WAVES; ++v) incl += v < w ? (int)scratch[v][0] : 0;
    int above = incl - mine;  // keys in bins above tb + 15
    if (above < need && incl >= need) {
      int bstar = tb;
#pragma unroll
      for (int e = 15; e >= 0; --e) {
        if (above + h[e] >= need) {
          bstar = tb + e;
          break;
        }
        above += h[e];
      }
      pick[0] = bstar;
      pick[1] = above;
    }
    __syncthreads();
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)pick[0] << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
    need -= pick[1];
    if (shift == 0) {
      P.T = lo;
      P.needT = need;
      return P;
    }
  }
  P.active = true;
  P.lo = lo;
  P.hi = hi;
  P.need = need;
  return P;
}

__global__ __launch_bounds__(MW_THREADS) void mw_stats_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                              const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                              int nch, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, cu_kept, nch, ck)) return;
  if (ck.c == 0) {  // the histograms of this call's passes start from zero
    u32x4* h = reinterpret_cast<u32x4*>(ws.hist + (size_t)ck.b * MW_PASSES * MW_BINS);
    for (int i = threadIdx.x; i < MW_PASSES * MW_BINS / 4; i += MW_THREADS) h[i] = u32x4{0u, 0u, 0u, 0u};
  }
  MwRaw raw;
  mw_issue(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw);
  uint32_t k[MW_TPT], nanb;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw, k, nanb);
  uint32_t nf = 0u, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < MW_TPT; ++j)
    if (j < nv) {
      nf += k[j] == 0u;
      if (k[j] != 0u) {
        kmin = min(kmin, k[j]);
        kmax = max(kmax, k[j]);
      }
    }
  __shared__ uint32_t scratch[MW_WAVES][4];
  uint32_t nan_seen = nanb != 0u;
  mw_block_stats(nf, nan_seen, kmin, kmax, scratch);
  if (threadIdx.x == 0) {
    MwRec* r = ws.rec + mw_chunk_slot(ck.in0, ck.b) + ck.c;
    r->nf = (int)nf;
    r->nan_seen = (int)nan_seen;
    r->kmin = kmin;
    r->kmax = kmax;
  }
}

template <int PASS>
__global__ __launch_bounds__(MW_THREADS) void mw_hist_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                             const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                             int nch, int max_n, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, cu_kept, nch, ck)) return;
  MwRaw raw;
  mw_issue(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw);
  const MwPlan P = mw_resolve(ck, max_n, ws, PASS);
  if (!P.active) return;
  const uint32_t lo = P.lo, span = P.hi - lo;
  const int bits = 32 - __clz(span);
  const int shift = bits > 12 ? bits - 12 : 0;
  const int nb = (int)(span >> shift) + 1;
  __shared__ uint32_t h[MW_BINS];
  for (int i = threadIdx.x; i < nb; i += MW_THREADS) h[i] = 0u;
  __syncthreads();
  uint32_t k[MW_TPT], nanb;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw, k, nanb);
#pragma unroll
  for (int j = 0; j < MW_TPT; ++j)
    if (j < nv && k[j] - lo <= span) atomicAdd(&h[(k[j] - lo) >> shift], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + ((size_t)ck.b * MW_PASSES + PASS) * MW_BINS;
  for (int i = threadIdx.x; i < nb; i += MW_THREADS)
    if (h[i]) atomicAdd(&gh[i], h[i]);
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
                                                              const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                              int nch, int max_n, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, cu_kept, nch, ck)) return;
  MwRaw raw;
  mw_issue(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw);
  const MwPlan P = mw_resolve(ck, max_n, ws, MW_PASSES);
  if (P.reject) return;
  uint32_t k[MW_TPT], nanb, sure, tie;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw, k, nanb);
  mw_keep_bits(k, nv, P.T, sure, tie);
  // chunk totals are <= 4096, so the packed halves never carry
  __shared__ uint32_t scratch[MW_WAVES];
  const uint32_t tot = mw_block_reduce((uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16), 0u,
                                       [](uint32_t a, uint32_t b) { return a + b; }, scratch);
  if (threadIdx.x == 0) {
    MwRec* r = ws.rec + mw_chunk_slot(ck.in0, ck.b) + ck.c;
    r->sure = (int)(tot & 0xffffu);
    r->tie = (int)(tot >> 16);
  }
}

__global__ __launch_bounds__(MW_THREADS) void mw_emit_kernel(const float* __restrict__ s, const uint8_t* __restrict__ mask,
                                                             const int32_t* __restrict__ cu_in, const int32_t* __restrict__ cu_kept,
                                                             int nch, int max_n, int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ status, MwWs ws) {
  MwChunk ck;
  if (!mw_chunk(s, mask, cu_in, cu_kept, nch, ck)) return;
  MwRaw raw;
  mw_issue(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw);
  const MwPlan P = mw_resolve(ck, max_n, ws, MW_PASSES);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t* kp = kept + ck.out0;
  if (ck.c == 0 && tid == 0 && status) status[ck.b] = P.flags;
  if (P.reject) {
    if (ck.c == 0)
      for (int i = tid; i < ck.K; i += MW_THREADS) kp[i] = -1;
    return;
  }
  // kept sure tokens and ties of the sequence's earlier chunks
  const MwRec* rec = ws.rec + mw_chunk_slot(ck.in0, ck.b);
  uint32_t ps = 0u, pt = 0u;
  for (int c = tid; c < ck.c; c += MW_THREADS) {
    ps += (uint32_t)rec[c].sure;
    pt += (uint32_t)rec[c].tie;
  }
  __shared__ uint32_t scratch[MW_WAVES];
  const int sure_run = (int)mw_block_reduce(ps, 0u, [](uint32_t a, uint32_t b) { return a + b; }, scratch);
  const int tie_run = (int)mw_block_reduce(pt, 0u, [](uint32_t a, uint32_t b) { return a + b; }, scratch);
  uint32_t k[MW_TPT], nanb, sure, tie;
  const int nv = mw_keys(ck.sp, ck.mp, ck.n, ck.i0, ck.vec, raw, k, nanb);
  mw_keep_bits(k, nv, P.T, sure, tie);
  const uint32_t packed = (uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16);
  const uint32_t incl = (uint32_t)wave_incl_scan((int)packed);
  __syncthreads();  // scratch is free
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  uint32_t excl = incl - packed;
#pragma unroll
  for (int v = 0; v < MW_WAVES; ++v) excl += v < w ? scratch[v] : 0u;
  const int needT = P.needT;
  const int sure_before = sure_run + (int)(excl & 0xffffu), tie_before = tie_run + (int)(excl >> 16);
  const int take = min(max(needT - tie_before, 0), __popc(tie));
  uint32_t rest = tie;  // drop the lowest `take` tie bits from rest: they are kept
  for (int c = 0; c < take; ++c) rest &= rest - 1u;
  uint32_t keep = sure | (tie ^ rest);
  int pos = sure_before + min(tie_before, needT);
  const int tok0 = ck.in0 + ck.i0;
  while (keep) {
    const int bit = __builtin_ctz(keep);
    if (pos < ck.K) kp[pos] = tok0 + bit;  // pos < K always holds; the guard keeps a logic slip in bounds
    ++pos;
    keep &= keep - 1u;
  }
}

size_t topk_select_workspace_bytes(int B, int64_t T_in, int max_n) {
  return max_n <= SEL_LDS_MAX || B <= 0 ? 0 : mw_workspace_bytes(B, T_in);
}

hipError_t launch_topk_select(const float* s, const uint8_t* mask, const int32_t* cu_in,
                              const int32_t* cu_kept, int B, int max_n, int32_t* kept,
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
  const dim3 g((unsigned)nblk), t(MW_THREADS);
#define TG_MW(...)                           \
  do {                                       \
    hipLaunchKernelGGL(__VA_ARGS__);         \
    const hipError_t e_ = hipGetLastError(); \
    if (e_ != hipSuccess) return e_;         \
  } while (0)
  TG_MW(mw_stats_kernel, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, w);
  TG_MW(mw_hist_kernel<0>, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, max_n, w);
  TG_MW(mw_hist_kernel<1>, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, max_n, w);
  TG_MW(mw_hist_kernel<2>, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, max_n, w);
  TG_MW(mw_count_kernel, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, max_n, w);
  TG_MW(mw_emit_kernel, g, t, 0, stream, s, mask, cu_in, cu_kept, nch, max_n, kept, status, w);
#undef TG_MW
  return hipSuccess;
}

}  // namespace tg
