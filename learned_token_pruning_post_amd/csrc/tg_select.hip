// Top-K selection with forced keep, and the compaction of the kept rows, in
// two data-parallel kernels.
//
// Rule (Tencent Cloud TokenGate article, section on early token filtering; the
// ai.866data article, mechanism-design section): forced tokens are always
// kept; the other K - F slots go to the highest scores, equal scores to the
// lower index, NaN below every number, -0.0 equal to +0.0. Output ascending.
// Compaction gathers the kept rows, their original positions and their
// scores in that order (only selected tokens continue above the gate: same
// article, same section).
//
// Scores map to order-preserving uint32 keys (forced tokens: key 0; NaN
// candidates: key 1, below the key of -inf). The threshold search narrows by
// the top 12 bits of the keys ("coarse bins"), then the top 16 ("fine bins"),
// then the low 16 bits inside the one fine bin that holds the threshold.
//
//  chunk kernel (one workgroup per chunk of CH tokens of a sequence):
//    the chunk's forced count, NaN flag and candidate key range; its
//    candidate keys counting-sorted by fine bin; the list of its non-empty
//    fine bins (bin << 16 | count - 1) and the list of its non-empty coarse
//    bins (bin << 20 | fine bins in it - 1 << 16 | keys in it - 1), both
//    ascending. Nothing is shared between workgroups, so nothing needs
//    clearing between calls.
//  emit kernel (workgroups share the batch's output rows evenly):
//    each workgroup derives the decisions of the sequences its rows belong
//    to from the chunk records (all workgroups of a sequence derive the same
//    ones), one thread per chunk: the coarse lists give the threshold's
//    coarse bin, the fine-list entries inside it give its fine bin, and the
//    keys of that bin (a few hundred at the workloads' score spread) are
//    resolved in LDS with two 256-bin passes into the threshold key T and the
//    number of keys equal to T to keep; per chunk the sure keeps (forced or
//    key > T) and ties (key == T) scan into output offsets (the first ties in
//    index order are kept). It then re-reads the chunks that hold its rows,
//    ranks their kept tokens and writes indices, positions, scores and (when
//    compacting) the rows.
// No workgroup waits for another; the only hand-over is the kernel boundary.
#include <algorithm>

#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace sc {

constexpr int NT = 256;         // threads per workgroup (both kernels)
constexpr int NWV = NT / 64;    // waves
constexpr int LBINS = 4096;     // LDS histogram window
constexpr int GMAX = 256;       // chunks per sequence (max): one per thread in the scans
constexpr int RMAX = 4096;      // output rows per emit workgroup held in LDS

struct Rec {  // one chunk's summary (32 bytes)
  uint32_t nf;     // forced tokens
  uint32_t nan;    // a score is NaN
  uint32_t kmin;   // candidate key range (0xffffffff / 0 when none)
  uint32_t kmax;
  uint32_t ncl;    // entries in the coarse-bin list
  uint32_t nfl;    // entries in the fine-bin list
  uint32_t ncand;  // candidate keys
  uint32_t pad;
};

// Chunk c of sequence b (input rows from in0_b) has slot in0_b / CH + b + c:
// a sequence of N tokens uses max(ceil(N / CH), 1) slots and the ranges of
// consecutive sequences never overlap, so T_in / CH + B + 1 slots cover a
// batch.
struct Ws {
  Rec* rec;         // [slots]
  uint32_t* clist;  // [slots][CH] coarse-bin list
  uint32_t* flist;  // [slots][CH] fine-bin list
  uint32_t* keys;   // [slots][CH] candidate keys sorted by fine bin
};
__device__ __forceinline__ size_t slot0(int in0, int b, int CH) { return (size_t)(in0 / CH) + (size_t)b; }

// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float x, bool& is_nan) {
  uint32_t u = __float_as_uint(x);
  is_nan = (u & 0x7fffffffu) > 0x7f800000u;
  if (is_nan) return 0u;
  if (u == 0x80000000u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// wave-wide inclusive scans on DPP row shifts and broadcasts
template <class Op>
__device__ __forceinline__ uint32_t wscan(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

// block exclusive sum scan (uniform `total`); tmp: NWV words of LDS
__device__ __forceinline__ uint32_t bscan(uint32_t x, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t incl = wscan(x, 0u, OpAdd());
  __syncthreads();
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int v = 0; v < NWV; ++v) {
    before += v < w ? tmp[v] : 0u;
    tot += tmp[v];
  }
  total = tot;
  return before + incl - x;
}

template <class Op>
__device__ __forceinline__ uint32_t breduce(uint32_t x, uint32_t id, Op op, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)wscan(x, id, op), 63);
  __syncthreads();
  if (lane == 0) tmp[w] = r;
  __syncthreads();
  uint32_t a = id;
#pragma unroll
  for (int v = 0; v < NWV; ++v) a = op(a, tmp[v]);
  return a;
}

// Block-wide (sum of nf, or of nan, min of kmin, max of kmax, sum of ncand) in
// one exchange; tmp: 5 * NWV words of LDS.
struct Stats {
  uint32_t nf, nan, kmin, kmax, ncand;
};
__device__ __forceinline__ Stats block_stats(Stats v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)wscan(v.nf, 0u, OpAdd()), 63);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)wscan(v.nan, 0u, OpMax()), 63);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)wscan(v.kmin, 0xffffffffu, OpMin()), 63);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)wscan(v.kmax, 0u, OpMax()), 63);
  const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)wscan(v.ncand, 0u, OpAdd()), 63);
  __syncthreads();
  if (lane == 0) {
    tmp[5 * w + 0] = a;
    tmp[5 * w + 1] = b;
    tmp[5 * w + 2] = c;
    tmp[5 * w + 3] = d;
    tmp[5 * w + 4] = e;
  }
  __syncthreads();
  Stats r = {0u, 0u, 0xffffffffu, 0u, 0u};
#pragma unroll
  for (int u = 0; u < NWV; ++u) {
    r.nf += tmp[5 * u + 0];
    r.nan |= tmp[5 * u + 1];
    r.kmin = min(r.kmin, tmp[5 * u + 2]);
    r.kmax = max(r.kmax, tmp[5 * u + 3]);
    r.ncand += tmp[5 * u + 4];
  }
  return r;
}

// The first min(m, 16) entries at p (m >= 1), entry k of the lane in slot
// (k + rot) mod min(m, 16): lanes that rotate by their lane id visit
// different entries at the same step, so their LDS atomics on bins that
// every chunk holds do not all collide. Loaded unconditionally, so all 16
// loads are in flight together; slots past min(m, 16) repeat entries.
__device__ __forceinline__ void load16r(const uint32_t* __restrict__ p, uint32_t m, uint32_t rot,
                                        uint32_t (&v)[16]) {
  const uint32_t mm = min(m, 16u);
  uint32_t idx = rot % mm;
#pragma unroll
  for (uint32_t k = 0; k < 16; ++k) {
    v[k] = p[idx];
    idx = idx + 1u == mm ? 0u : idx + 1u;
  }
}

// last i in [0, n) with a[i] <= x (a non-decreasing, a[0] <= x)
__device__ __forceinline__ int last_le(const uint32_t* a, int n, uint32_t x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Load the TPT consecutive tokens of one thread (local indices base..base+TPT-1
// of a sequence starting at sp / mp) and turn them into keys: forced -> 0,
// NaN candidate -> 1, else the order key. valid / cand: bit j per token.
template <int TPT>
__device__ __forceinline__ void load_keys(const float* __restrict__ sp, const uint8_t* __restrict__ mp,
                                          int n, int base, uint32_t (&key)[TPT], uint32_t& valid,
                                          uint32_t& cand, int& nf, uint32_t& nan) {
  float x[TPT];
  uint32_t m = 0u;  // forced bits
  const bool full = base + TPT <= n;
  const bool vec = full && TPT >= 4 && ((reinterpret_cast<uintptr_t>(sp + base) & 15u) == 0) &&
                   (!mp || (reinterpret_cast<uintptr_t>(mp + base) & 3u) == 0);
  if (vec) {
#pragma unroll
    for (int q = 0; q < TPT / 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sp + base + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
      if (mp) {
        const uint32_t mw = *reinterpret_cast<const uint32_t*>(mp + base + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) m |= (uint32_t)(((mw >> (8 * e)) & 0xffu) != 0u) << (4 * q + e);
      }
    }
  } else if (n > 0) {
    // every load issued unconditionally (a clamped index: no branch, so all
    // are in flight together); tokens past the end are masked below
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int i = min(base + j, n - 1);
      x[j] = sp[i];
      if (mp && mp[i]) m |= 1u << j;
    }
  } else {
#pragma unroll
    for (int j = 0; j < TPT; ++j) x[j] = 0.f;
  }
  valid = 0u;
  cand = 0u;
  nf = 0;
  nan = 0u;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const bool in = base + j < n;
    bool isn;
    const uint32_t k = score_key(x[j], isn);
    const bool f = (m >> j) & 1u;
    valid |= (uint32_t)in << j;
    cand |= (uint32_t)(in && !f) << j;
    nf += (in && f) ? 1 : 0;
    nan |= (uint32_t)(in && isn);
    key[j] = (!in || f) ? 0u : (isn ? 1u : k);
  }
}

// ---------------------------------------------------------------------------
// chunk kernel
// ---------------------------------------------------------------------------
template <int TPT>
__global__ __launch_bounds__(NT) void sc_chunk_kernel(const float* __restrict__ s,
                                                      const uint8_t* __restrict__ mask,
                                                      const int32_t* __restrict__ cu_in, int G,
                                                      int max_n, Ws ws) {
  constexpr int CH = NT * TPT;
  __shared__ uint32_t hist[LBINS];  // fine-bin counts of a window, then key cursors; coarse key counts
  __shared__ uint32_t fl[CH];       // the fine list
  __shared__ uint32_t cf[CH];       // fine bins per coarse entry
  __shared__ uint32_t tmp[5 * NWV];
  const int b = blockIdx.x / G, c = blockIdx.x % G;
  const int in0 = cu_in[b], n = cu_in[b + 1] - in0;
  if (n > max_n) return;  // flagged by the emit kernel; no chunk records
  const int Gb = n > 0 ? (n + CH - 1) / CH : 1;
  if (c >= Gb) return;
  const int t = threadIdx.x;
  const int nloc = min(n - c * CH, CH);  // tokens of this chunk (may be 0 for an empty sequence)
  uint32_t key[TPT], valid, cand, nan;
  int nf;
  load_keys<TPT>(s + in0 + c * CH, mask ? mask + in0 + c * CH : nullptr, nloc, t * TPT, key, valid,
                 cand, nf, nan);
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < TPT; ++j)
    if ((cand >> j) & 1u) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  const Stats st = block_stats(Stats{(uint32_t)nf, nan, kmin, kmax, (uint32_t)__popc(cand)}, tmp);
  const uint32_t nf_b = st.nf, nan_b = st.nan, kmin_b = st.kmin, kmax_b = st.kmax, ncand_b = st.ncand;

  const size_t slot = slot0(in0, b, CH) + c;
  uint32_t* keys = ws.keys + slot * CH;
  // fine-bin histogram in windows of KW bins, lowest first; per window:
  // the non-empty bins appended to the fine list in ascending order, and the
  // keys scattered to their bin's range of the key array
  uint32_t todo = cand;
  uint32_t wlo = kmin_b >> 16;
  uint32_t nfl = 0u, placed = 0u;
  constexpr int KW = 1024;  // window (the fine bins of a chunk of sigmoid scores span a few hundred)
  for (int round = 0; round < 64 && placed < ncand_b; ++round) {
#pragma unroll
    for (int e = 0; e < KW / NT; ++e) hist[t * (KW / NT) + e] = 0u;
    __syncthreads();
    uint32_t inwin = 0u;
#pragma unroll
    for (int j = 0; j < TPT; ++j)
      if ((todo >> j) & 1u) {
        const uint32_t d = (key[j] >> 16) - wlo;
        if (d < (uint32_t)KW) {
          inwin |= 1u << j;
          atomicAdd(&hist[d], 1u);
        }
      }
    __syncthreads();
    constexpr int BPT = KW / NT;  // bins per thread
    uint32_t h[BPT];
    uint32_t nz = 0u, cnt = 0u;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      h[e] = hist[t * BPT + e];
      nz += h[e] != 0u;
      cnt += h[e];
    }
    // both counts are <= CH <= 4096 per block: pack them (no carry)
    uint32_t tot;
    const uint32_t ex = bscan(nz | (cnt << 16), tmp, tot);
    uint32_t lpos = nfl + (ex & 0xffffu);
    uint32_t kpos = placed + (ex >> 16);
#pragma unroll
    for (int e = 0; e < BPT; ++e)
      if (h[e]) {
        fl[lpos++] = ((wlo + (uint32_t)(t * BPT + e)) << 16) | (h[e] - 1u);
        hist[t * BPT + e] = kpos;  // cursor of this bin's keys
        kpos += h[e];
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TPT; ++j)
      if ((inwin >> j) & 1u) {
        const uint32_t at = atomicAdd(&hist[(key[j] >> 16) - wlo], 1u);
        keys[at] = key[j];
      }
    todo &= ~inwin;
    nfl += tot & 0xffffu;
    placed += tot >> 16;
    // next window: the lowest bin still to place
    uint32_t nb = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < TPT; ++j)
      if ((todo >> j) & 1u) nb = min(nb, key[j] >> 16);
    wlo = placed < ncand_b ? breduce(nb, 0xffffffffu, OpMin(), tmp) : 0xffffffffu;
    __syncthreads();  // hist readers done before the next round clears it
  }
  // coarse list from the fine list: runs of fine entries with the same top
  // 12 key bits; thread t takes fine entries t*TPT .. t*TPT+TPT-1
  uint32_t heads = 0u;
  uint32_t ent[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const uint32_t i = (uint32_t)(t * TPT + j);
    ent[j] = i < nfl ? fl[i] : 0u;
    const bool head = i < nfl && (i == 0u || (fl[i - 1] >> 20) != (ent[j] >> 20));
    heads += head ? 1u : 0u;
  }
  uint32_t ncl;
  uint32_t ci = bscan(heads, tmp, ncl);  // coarse index of this thread's first head
  for (int i = t; i < (int)ncl; i += NT) {
    hist[i] = 0u;
    cf[i] = 0u;
  }
  __syncthreads();
  {
    uint32_t cur = ci;  // coarse index of the entry being visited (heads bump it)
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const uint32_t i = (uint32_t)(t * TPT + j);
      if (i < nfl) {
        const bool head = i == 0u || (fl[i - 1] >> 20) != (ent[j] >> 20);
        const uint32_t k = head ? cur++ : cur - 1u;
        atomicAdd(&hist[k], (ent[j] & 0xffffu) + 1u);
        atomicAdd(&cf[k], 1u);
        if (head) atomicOr(&cf[k], (ent[j] >> 20) << 20);  // the coarse bin rides in the top bits
      }
    }
  }
  __syncthreads();
  uint32_t* clist = ws.clist + slot * CH;
  uint32_t* flist = ws.flist + slot * CH;
  for (int i = t; i < (int)ncl; i += NT) {
    const uint32_t nfine = cf[i] & 0xfffffu;  // <= 16
    clist[i] = (cf[i] & 0xfff00000u) | ((nfine - 1u) << 16) | (hist[i] - 1u);
  }
  for (int i = t; i < (int)nfl; i += NT) flist[i] = fl[i];
  if (t == 0) {
    Rec r;
    r.nf = nf_b;
    r.nan = nan_b;
    r.kmin = kmin_b;
    r.kmax = kmax_b;
    r.ncl = ncl;
    r.nfl = nfl;
    r.ncand = ncand_b;
    r.pad = 0u;
    ws.rec[slot] = r;
  }
}

// ---------------------------------------------------------------------------
// emit kernel
// ---------------------------------------------------------------------------
constexpr int CUMAX = 1024;  // sequences whose offsets the emit kernel stages in LDS

constexpr int CW = 32;  // coarse entries per chunk staged in LDS (more: read from memory)
constexpr int FW = 16;  // fine entries of one coarse bin (a coarse bin holds at most 16 fine bins)
constexpr int KS = 16;  // keys of the threshold's fine bin per chunk staged in LDS (more: from memory)

// LDS slot of entry k of chunk c in the staged per-chunk lists: entry-major,
// with the chunk index XOR-ed by k, so that a pass where thread c reads
// entry k of its chunk and the staging where consecutive lanes write
// consecutive entries of one chunk both hit distinct banks.
__device__ __forceinline__ uint32_t slot(uint32_t c, uint32_t k) { return k * GMAX + (c ^ (k & 63u)); }

struct Smem {  // dynamic LDS of the emit kernel
  uint32_t hist[LBINS];
  uint32_t a[GMAX];      // per chunk: forced count, then output offset
  uint32_t lp[GMAX];     // per chunk: coarse-list length, then tie prefix
  uint32_t fo[GMAX];     // per chunk: fine-list length, then fine entries before the threshold's coarse bin
  uint32_t fn[GMAX];     // per chunk: fine entries in the threshold's coarse bin
  uint32_t below[GMAX];  // per chunk: keys below the threshold's fine bin (where its keys start)
  uint32_t cnt0[GMAX];   // per chunk: keys in the threshold's fine bin
  uint32_t cl[GMAX * CW];  // per chunk: its first CW coarse entries
  uint32_t fl[GMAX * FW];  // per chunk: its fine entries inside the threshold's coarse bin
  uint32_t sk[GMAX * KS];  // per chunk: its first KS keys of the threshold's fine bin
  int32_t map[RMAX];       // source row of each of this workgroup's output rows
  int32_t cui[CUMAX + 1];  // cu_in and cu_kept (batches of up to CUMAX sequences)
  int32_t cuk[CUMAX + 1];
  uint32_t tmp[5 * NWV];
  uint32_t val[8];
};

// Find, from the top of hist[0, nb), the bin where the count of keys above
// reaches `need`: returns (bin, keys in bins above it).
__device__ __forceinline__ void find_from_top(Smem& S, int nb, uint32_t need, uint32_t& bin,
                                              uint32_t& above) {
  constexpr int BPT = LBINS / NT;
  const int t = threadIdx.x;
  const int tb = BPT * (NT - 1 - t);  // thread t owns bins tb..tb+BPT-1, from the top down
  uint32_t h[BPT];
  uint32_t mine = 0u;
#pragma unroll
  for (int q = 0; q < BPT / 4; ++q) {  // 16-byte reads (a quarter of the bank conflicts)
    const u32x4 hv = *reinterpret_cast<const u32x4*>(&S.hist[tb + 4 * q]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[4 * q + e] = tb + 4 * q + e < nb ? hv[e] : 0u;
      mine += h[4 * q + e];
    }
  }
  uint32_t tot;
  uint32_t ab = bscan(mine, S.tmp, tot);  // keys in bins above tb + BPT - 1
  if (ab < need && ab + mine >= need) {
#pragma unroll
    for (int e = BPT - 1; e >= 0; --e) {
      if (ab + h[e] >= need) {
        S.val[0] = (uint32_t)(tb + e);
        S.val[1] = ab;
        break;
      }
      ab += h[e];
    }
  }
  __syncthreads();
  bin = S.val[0];
  above = S.val[1];
  __syncthreads();
}

struct Decision {
  int flags;       // TG_DEV_* of the sequence
  bool reject;     // slots get -1
  uint32_t T;      // threshold key
  uint32_t needT;  // keys == T kept (the first ones in index order)
  int Gb;          // chunks
};

// The decisions of sequence b (uniform over the workgroup). With `full`, the
// per-chunk output offsets S.a[] and tie prefixes S.lp[] are left in LDS.
// Every list is first staged into fixed-width LDS slots by element-parallel
// loads (one round trip each, all loads in flight together); the passes then
// read LDS. Entries beyond a slot's width (rare) are read from memory.
template <int TPT>
__device__ __forceinline__ Decision decide(Smem& S, const Ws& ws, int b, int in0, int n, int K, int max_n,
                                           bool full) {
  constexpr int CH = NT * TPT;
  const int t = threadIdx.x;
  Decision D = {};
  if (n > max_n) {
    D.flags = 8;  // TG_DEV_LEN_GT_MAX_N
    D.reject = true;
    return D;
  }
  const int Gb = n > 0 ? (n + CH - 1) / CH : 1;  // <= GMAX = NT: chunk t belongs to thread t
  D.Gb = Gb;
  const bool own = t < Gb;
  const size_t sl0 = slot0(in0, b, CH);
  // ---- chunk records ----
  Stats st = {0u, 0u, 0xffffffffu, 0u, 0u};
  if (own) {
    const Rec r = ws.rec[sl0 + t];
    S.a[t] = r.nf;
    S.lp[t] = r.ncl;
    S.fo[t] = r.nfl;
    st.nf = r.nf;
    st.nan = r.nan;
    st.kmin = r.kmin;
    st.kmax = r.kmax;
  }
  st = block_stats(st, S.tmp);
  D.flags = (st.nan ? 4 : 0) | (K > n ? 2 : 0) | ((int)st.nf > K ? 1 : 0);
  if (D.flags & 3) {
    D.reject = true;
    return D;
  }
  if (!full) return D;
  const uint32_t C = (uint32_t)n - st.nf, r = (uint32_t)K - st.nf;
  uint32_t tot;
  if (r == 0u || r == C) {
    // only the forced tokens, or every token
    D.T = r == 0u ? 0xffffffffu : 0u;
    D.needT = 0u;
    const uint32_t v = own ? (r == 0u ? S.a[t] : (uint32_t)min(CH, n - t * CH)) : 0u;
    const uint32_t ex = bscan(v, S.tmp, tot);
    if (own) {
      S.a[t] = ex;
      S.lp[t] = 0u;
    }
    __syncthreads();
    return D;
  }
  const uint32_t* clist = ws.clist + sl0 * CH;
  const uint32_t* flist = ws.flist + sl0 * CH;
  const uint32_t* keys = ws.keys + sl0 * CH;
  const uint32_t ncl = own ? S.lp[t] : 0u;
  const uint32_t blo = st.kmin >> 20, nbc = (st.kmax >> 20) - blo + 1u;  // live coarse bins
  for (uint32_t i = t; i < nbc; i += NT) S.hist[i] = 0u;
  __syncthreads();
  // ---- stage the coarse lists (slot (c, k) = entry k of chunk c) and count
  // the keys per coarse bin (top 12 key bits) on the way ----
  const uint32_t ncw = (uint32_t)Gb * CW;
  for (uint32_t i0 = 0; i0 < ncw; i0 += 8u * NT) {
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {  // clamped indices: every load issued unconditionally
      const uint32_t i = min(i0 + (uint32_t)(q * NT + t), ncw - 1u), c = i / CW, k = i % CW;
      const uint32_t m = S.lp[c];
      v[q] = clist[c * CH + (m > 0u ? min(k, m - 1u) : 0u)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = i0 + (uint32_t)(q * NT + t), c = i / CW, k = i % CW;
      if (i < ncw && k < S.lp[c]) {
        S.cl[slot(c, k)] = v[q];
        atomicAdd(&S.hist[(v[q] >> 20) - blo], (v[q] & 0xffffu) + 1u);
      }
    }
  }
  for (uint32_t k = CW; k < ncl; ++k) {  // a chunk's entries beyond its slot (rare)
    const uint32_t e = clist[(uint32_t)t * CH + k];
    atomicAdd(&S.hist[(e >> 20) - blo], (e & 0xffffu) + 1u);
  }
  __syncthreads();
  uint32_t T0c, above;
  find_from_top(S, (int)nbc, r, T0c, above);
  T0c += blo;
  const uint32_t rc = r - above;  // keys needed from coarse bin T0c (>= 1)
  // per chunk: keys above / below T0c, fine entries before and in it
  uint32_t ab = 0u, bl = 0u, fo = 0u, fnn = 0u;
  auto classify = [&](uint32_t e) {
    const uint32_t cb = e >> 20, kc = (e & 0xffffu) + 1u, fc = ((e >> 16) & 15u) + 1u;
    if (cb > T0c) {
      ab += kc;
    } else if (cb < T0c) {
      bl += kc;
      fo += fc;
    } else {
      fnn = fc;
    }
  };
  {
    // every slot read issued at once (unconditional; slots past the chunk's
    // entries hold stale words that the mask drops)
    uint32_t e[CW];
#pragma unroll
    for (int k = 0; k < CW; ++k) e[k] = S.cl[slot(t, k)];
#pragma unroll
    for (int k = 0; k < CW; ++k)
      if ((uint32_t)k < ncl) classify(e[k]);
  }
  for (uint32_t k = CW; k < ncl; ++k) classify(clist[(uint32_t)t * CH + k]);
  if (own) {
    S.fo[t] = fo;
    S.fn[t] = fnn;
  }
  if (t < 16) S.hist[t] = 0u;
  __syncthreads();
  // ---- stage the fine entries inside T0c (slot (c, k) = entry k of chunk c)
  // and count the keys of its 16 fine bins (top 16 key bits) ----
  const uint32_t nfw = (uint32_t)Gb * FW;
  for (uint32_t i0 = 0; i0 < nfw; i0 += 8u * NT) {
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = min(i0 + (uint32_t)(q * NT + t), nfw - 1u), c = i / FW, k = i % FW;
      const uint32_t m = S.fn[c];  // none: read the chunk's first entry (in its slot), dropped below
      v[q] = flist[c * CH + (m > 0u ? S.fo[c] + min(k, m - 1u) : 0u)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = i0 + (uint32_t)(q * NT + t), c = i / FW, k = i % FW;
      if (i < nfw && k < S.fn[c]) {
        S.fl[slot(c, k)] = v[q];
        atomicAdd(&S.hist[(v[q] >> 16) & 15u], (v[q] & 0xffffu) + 1u);
      }
    }
  }
  __syncthreads();
  uint32_t sub0, ab2;
  find_from_top(S, 16, rc, sub0, ab2);
  const uint32_t T0 = (T0c << 4) | sub0;  // fine bin of the threshold
  const uint32_t r0 = rc - ab2;           // keys needed from it (>= 1)
  uint32_t c0 = 0u;
  {
    uint32_t e[FW];
#pragma unroll
    for (int k = 0; k < FW; ++k) e[k] = S.fl[slot(t, k)];
#pragma unroll
    for (int k = 0; k < FW; ++k) {
      const uint32_t sub = (e[k] >> 16) & 15u, cnt = (uint32_t)k < fnn ? (e[k] & 0xffffu) + 1u : 0u;
      ab += sub > sub0 ? cnt : 0u;
      bl += sub < sub0 ? cnt : 0u;
      c0 += sub == sub0 ? cnt : 0u;
    }
  }
  if (own) {
    S.below[t] = bl;  // the chunk's keys are sorted by fine bin: T0's keys start here
    S.cnt0[t] = c0;
  }
  S.hist[t] = 0u;  // 256 bins, one per thread
  __syncthreads();
  // ---- stage the keys of fine bin T0 (slot (c, k) = key k of chunk c) and
  // count them by key bits 15..8 ----
  const uint32_t nkw = (uint32_t)Gb * KS;
  for (uint32_t i0 = 0; i0 < nkw; i0 += 8u * NT) {
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = min(i0 + (uint32_t)(q * NT + t), nkw - 1u), c = i / KS, k = i % KS;
      const uint32_t m = S.cnt0[c];  // none: read the chunk's first key (in its slot), dropped below
      v[q] = keys[c * CH + (m > 0u ? S.below[c] + min(k, m - 1u) : 0u)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = i0 + (uint32_t)(q * NT + t), c = i / KS, k = i % KS;
      if (i < nkw && k < S.cnt0[c]) {
        S.sk[slot(c, k)] = v[q];
        atomicAdd(&S.hist[(v[q] >> 8) & 255u], 1u);
      }
    }
  }
  for (uint32_t k = KS; k < c0; ++k)  // a chunk's keys beyond its slot (rare)
    atomicAdd(&S.hist[(keys[(uint32_t)t * CH + bl + k] >> 8) & 255u], 1u);
  __syncthreads();
  // ---- exact threshold inside fine bin T0: key bits 15..8, then 7..0 ----
  uint32_t b1, a1, b2, a2;
  find_from_top(S, 256, r0, b1, a1);
  S.hist[t] = 0u;
  __syncthreads();
  uint32_t tk[KS];  // this chunk's staged keys of fine bin T0, read at once
#pragma unroll
  for (int k = 0; k < KS; ++k) tk[k] = S.sk[slot(t, k)];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    if ((uint32_t)k < c0 && ((tk[k] >> 8) & 255u) == b1) atomicAdd(&S.hist[tk[k] & 255u], 1u);
  for (uint32_t k = KS; k < c0; ++k) {
    const uint32_t kk = keys[(uint32_t)t * CH + bl + k];
    if (((kk >> 8) & 255u) == b1) atomicAdd(&S.hist[kk & 255u], 1u);
  }
  __syncthreads();
  find_from_top(S, 256, r0 - a1, b2, a2);
  D.T = (T0 << 16) | (b1 << 8) | b2;
  D.needT = r0 - a1 - a2;
  // ---- per chunk: keys > T and == T inside fine bin T0 ----
  uint32_t eq = 0u;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const bool in = (uint32_t)k < c0;
    ab += in && tk[k] > D.T ? 1u : 0u;
    eq += in && tk[k] == D.T ? 1u : 0u;
  }
  for (uint32_t k = KS; k < c0; ++k) {
    const uint32_t kk = keys[(uint32_t)t * CH + bl + k];
    ab += kk > D.T ? 1u : 0u;
    eq += kk == D.T ? 1u : 0u;
  }
  // ---- tie prefix, kept counts, output offsets ----
  const uint32_t tex = bscan(eq, S.tmp, tot);  // ties in earlier chunks
  // ties kept in this chunk, written without a guarded subtraction (a form
  // the compiler has been seen to miscompile: speculated with a no-wrap
  // flag that then folded a neighbouring min)
  const uint32_t take = min(D.needT, tex + eq) - min(D.needT, tex);
  const uint32_t kv = own ? S.a[t] + ab + take : 0u;  // forced + keys > T + kept ties
  const uint32_t kex = bscan(kv, S.tmp, tot);
  if (own) {
    S.a[t] = kex;
    S.lp[t] = tex;
  }
  __syncthreads();
  return D;
}

template <int TPT, bool GATHER, bool SMALLB>
__global__ __launch_bounds__(NT) void sc_emit_kernel(
    const float* __restrict__ s, const uint8_t* __restrict__ mask, const int32_t* __restrict__ cu_in,
    const int32_t* __restrict__ cu_kept, int B, int max_n, Ws ws, int32_t* __restrict__ kept,
    int32_t* __restrict__ status, const uint8_t* __restrict__ h, const int32_t* __restrict__ pos,
    uint32_t row_bytes, uint8_t* __restrict__ h_out, int32_t* __restrict__ pos_out,
    float* __restrict__ s_out) {
  constexpr int CH = NT * TPT;
  extern __shared__ __attribute__((aligned(16))) unsigned char sc_smem[];
  Smem& S = *reinterpret_cast<Smem*>(sc_smem);
  const int t = threadIdx.x;
  const int W = gridDim.x, w = blockIdx.x;
  // the batch offsets: staged in LDS in one round trip for batches of up to
  // CUMAX sequences (SMALLB), else read from memory
  if (SMALLB) {
    for (int i = t; i <= B; i += NT) {
      S.cuk[i] = cu_kept[i];
      S.cui[i] = cu_in[i];
    }
    __syncthreads();
  }
  auto cuk = [&](int i) -> int { return SMALLB ? S.cuk[i] : cu_kept[i]; };
  auto cui = [&](int i) -> int { return SMALLB ? S.cui[i] : cu_in[i]; };
  const int Tt = cuk(B);
  const int R = (Tt + W - 1) / W;
  const int j0 = min(Tt, w * R), j1 = min(Tt, j0 + R);
  // sequences whose rows meet [j0, j1), and those whose status this
  // workgroup writes (owner of b: the workgroup holding row cuk(b), the
  // last workgroup for sequences that start at Tt)
  auto owner = [&](int b) { const int o = cuk(b); return (o < Tt && R > 0) ? o / R : W - 1; };
  int b_lo = B, b_hi = -1;
  if (j0 < j1) {
    int lo = 0, hi = B;  // last b with cuk(b) <= j0 (and a row there)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cuk(mid) <= j0) lo = mid; else hi = mid;
    }
    b_lo = lo;
    lo = 0;
    hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cuk(mid) <= j1 - 1) lo = mid; else hi = mid;
    }
    b_hi = lo;
  }
  {  // status duty: owner(b) == w, a contiguous run of b
    int lo = -1, hi = B;  // first b with owner(b) >= w
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (owner(mid) >= w) hi = mid; else lo = mid;
    }
    for (int b = hi; b < B && owner(b) == w; ++b) {
      b_lo = min(b_lo, b);
      b_hi = max(b_hi, b);
    }
  }
  for (int b = b_lo; b <= b_hi; ++b) {
    const int in0 = cui(b), n = cui(b + 1) - in0;
    const int out0 = cuk(b), K = cuk(b + 1) - out0;
    const int e0 = max(j0, out0) - out0, e1 = min(j1, out0 + K) - out0;  // this workgroup's rows of b
    const bool duty = owner(b) == w;
    if (!duty && e0 >= e1) continue;
    const Decision D = decide<TPT>(S, ws, b, in0, n, K, max_n, e0 < e1);
    if (duty && t == 0 && status) status[b] = D.flags;
    if (e0 >= e1) continue;
    if (D.reject) {
      for (int j = e0 + t; j < e1; j += NT) {
        kept[out0 + j] = -1;
        if (GATHER) {
          pos_out[out0 + j] = -1;
          if (s_out) s_out[out0 + j] = 0.f;
        }
      }
      if (GATHER)
        for (int j = e0; j < e1; ++j) {
          uint8_t* dp = h_out + (size_t)(out0 + j) * row_bytes;
          for (uint32_t o = 2u * t; o < row_bytes; o += 2u * NT) *reinterpret_cast<uint16_t*>(dp + o) = 0;
        }
      __syncthreads();
      continue;
    }
    if (GATHER) {
      for (int r = t; r < RMAX; r += NT) S.map[r] = -1;
      __syncthreads();
    }
    // chunks holding rows e0..e1-1: S.a[] are their output offsets
    const int c_lo = last_le(S.a, D.Gb, (uint32_t)e0);
    const int c_hi = last_le(S.a, D.Gb, (uint32_t)(e1 - 1));
    for (int c = c_lo; c <= c_hi; ++c) {
      const int nloc = min(n - c * CH, CH);
      uint32_t key[TPT], valid, cand, nan;
      int nf;
      const float* sp = s + in0 + c * CH;
      load_keys<TPT>(sp, mask ? mask + in0 + c * CH : nullptr, nloc, t * TPT, key, valid, cand, nf,
                     nan);
      uint32_t sure = 0u, tie = 0u;
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const bool f = ((valid & ~cand) >> j) & 1u;
        const bool cj = (cand >> j) & 1u;
        sure |= (uint32_t)(f || (cj && key[j] > D.T)) << j;
        tie |= (uint32_t)(cj && key[j] == D.T) << j;
      }
      // sure and tie counts of a chunk are <= CH <= 4096: pack them
      uint32_t tot;
      const uint32_t ex = bscan((uint32_t)__popc(sure) | ((uint32_t)__popc(tie) << 16), S.tmp, tot);
      const uint32_t tie_before = S.lp[c] + (ex >> 16);  // ties of the sequence before this thread's
      const uint32_t take = min(D.needT, tie_before + (uint32_t)__popc(tie)) - min(D.needT, tie_before);
      uint32_t rest = tie;  // drop the lowest `take` tie bits: those are kept
      for (uint32_t q = 0; q < take; ++q) rest &= rest - 1u;
      uint32_t keep = sure | (tie ^ rest);
      const uint32_t kept_before_chunk_ties = min(D.needT, S.lp[c] + (ex >> 16)) - min(D.needT, S.lp[c]);
      int o = (int)(S.a[c] + (ex & 0xffffu) + kept_before_chunk_ties);
      while (keep) {
        const int j = __builtin_ctz(keep);
        keep &= keep - 1u;
        if (o >= e0 && o < e1) {
          const int li = c * CH + t * TPT + j;  // index in the sequence
          kept[out0 + o] = in0 + li;
          if (GATHER) {
            pos_out[out0 + o] = pos ? pos[in0 + li] : li;
            if (s_out) s_out[out0 + o] = sp[t * TPT + j];
            if (o - e0 < RMAX) S.map[o - e0] = in0 + li;
          }
        }
        ++o;
      }
      __syncthreads();  // S.tmp reuse by the next chunk's scan
    }
    if (GATHER) {
      __syncthreads();
      const int nr = min(e1 - e0, RMAX);
      // every row has its source by now; one without (which a consistent
      // decision never leaves) is written as zeros instead of read from
      // outside the input
      const int64_t T_in = cu_in[B];
      for (int r = t; r < nr; r += NT)
        if (S.map[r] < 0 || S.map[r] >= T_in) S.map[r] = -1;
      __syncthreads();
      const uint8_t* hb = h;
      uint8_t* ob = h_out + (size_t)(out0 + e0) * row_bytes;
      if ((row_bytes & 15u) == 0u && ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(h_out)) & 15u) == 0u) {
        // 16-byte pieces; each wave takes whole rows, 4 rows at a time in flight
        const int lane = t & 63, wv = t >> 6;
        const int npc = (int)(row_bytes >> 4);
        for (int r0 = wv * 4; r0 < nr; r0 += NWV * 4) {
          u32x4 buf[4][4];
          // every load issued unconditionally (a missing row reads row 0 and
          // is stored as zeros; pieces past the row repeat its last one)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = r0 + rr;
            const int src_row = r < nr ? S.map[r] : -1;
            const u32x4* src = reinterpret_cast<const u32x4*>(hb + (size_t)max(src_row, 0) * row_bytes);
#pragma unroll
            for (int q = 0; q < 4; ++q) buf[rr][q] = __builtin_nontemporal_load(src + min(lane + 64 * q, npc - 1));
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (src_row < 0) buf[rr][q] = u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = r0 + rr;
            u32x4* dst = reinterpret_cast<u32x4*>(ob + (size_t)r * row_bytes);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int pc = lane + 64 * q;
              if (r < nr && pc < npc) __builtin_nontemporal_store(buf[rr][q], dst + pc);
            }
          }
          // rows wider than 4 KB: the rest of each row
          for (int pc = lane + 256; pc < npc; pc += 64)
            for (int rr = 0; rr < 4; ++rr) {
              const int r = r0 + rr;
              if (r < nr)
                reinterpret_cast<u32x4*>(ob + (size_t)r * row_bytes)[pc] =
                    S.map[r] >= 0 ? reinterpret_cast<const u32x4*>(hb + (size_t)S.map[r] * row_bytes)[pc]
                                  : u32x4{0u, 0u, 0u, 0u};
            }
        }
      } else {
        for (int r = 0; r < nr; ++r) {
          const int src_row = S.map[r];
          const uint8_t* src = hb + (size_t)max(src_row, 0) * row_bytes;
          uint8_t* dst = ob + (size_t)r * row_bytes;
          for (uint32_t o = 2u * t; o < row_bytes; o += 2u * NT)
            *reinterpret_cast<uint16_t*>(dst + o) =
                src_row >= 0 ? *reinterpret_cast<const uint16_t*>(src + o) : (uint16_t)0;
        }
      }
      __syncthreads();  // S.map reuse
    }
  }
}

}  // namespace sc

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
inline size_t sc_align(size_t x) { return (x + 255) & ~(size_t)255; }

// tokens per thread of a chunk: the smallest power of two from 2 that keeps
// a sequence of max_n tokens within GMAX = 256 chunks, at most 16 (4096-token
// chunks: sequences of up to 1M tokens). At least 512-token chunks: fewer
// chunk records for every emit workgroup to stage (measured: N = 32768 36.7
// -> 35.3 us, 8 x 16384 88 -> 77 us; 1024-token chunks 39.5 us at N = 32768).
int sc_tpt(int max_n) {
  int tpt = 2;
  while (tpt < 16 && (int64_t)sc::NT * tpt * 256 < (int64_t)max_n) tpt <<= 1;
  return tpt;
}
}  // namespace

bool select_supported(int max_n) {
  const int64_t ch = (int64_t)sc::NT * sc_tpt(max_n);
  return (int64_t)max_n <= ch * sc::GMAX;
}

size_t select_workspace_bytes(int B, int64_t T_in, int max_n) {
  if (B <= 0) return 0;
  const int64_t CH = (int64_t)sc::NT * sc_tpt(max_n);
  const size_t slots = (size_t)(T_in / CH) + (size_t)B + 1;
  return sc_align(slots * sizeof(sc::Rec)) + 3 * sc_align(slots * (size_t)CH * sizeof(uint32_t));
}

size_t select_workspace_bound(int B, int64_t T_in) {
  size_t m = 0;
  for (int tpt = 1; tpt <= 16; tpt <<= 1)  // every chunk size the selection may pick
    m = std::max(m, select_workspace_bytes(B, T_in, sc::NT * tpt * 256 / 2 + 1));
  return m;
}

template <int TPT>
static hipError_t sc_launch(const float* s, const uint8_t* mask, const int32_t* cu_in,
                            const int32_t* cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                            int32_t* kept, int32_t* status, void* ws, const void* h,
                            const int32_t* pos, size_t row_bytes, void* h_out, int32_t* pos_out,
                            float* s_out, hipStream_t stream) {
  constexpr int CH = sc::NT * TPT;
  const int G = max_n > 0 ? (max_n + CH - 1) / CH : 1;
  const size_t slots = (size_t)(T_in / CH) + (size_t)B + 1;
  unsigned char* p = static_cast<unsigned char*>(ws);
  sc::Ws w;
  w.rec = reinterpret_cast<sc::Rec*>(p);
  p += sc_align(slots * sizeof(sc::Rec));
  w.clist = reinterpret_cast<uint32_t*>(p);
  p += sc_align(slots * (size_t)CH * sizeof(uint32_t));
  w.flist = reinterpret_cast<uint32_t*>(p);
  p += sc_align(slots * (size_t)CH * sizeof(uint32_t));
  w.keys = reinterpret_cast<uint32_t*>(p);
  const int64_t nblk = (int64_t)B * G;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sc::sc_chunk_kernel<TPT>, dim3((unsigned)nblk), dim3(sc::NT), 0, stream, s, mask,
                     cu_in, G, max_n, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // output rows shared evenly: enough workgroups for every CU, every row range
  // within RMAX rows, and about one per sequence for many short ones
  const int cus = device_cu_count();
  int64_t W = std::max<int64_t>(std::max<int64_t>(cus, 2 * (int64_t)B), (T + sc::RMAX - 1) / sc::RMAX);
  W = std::min<int64_t>(W, 65535);
  if ((T + W - 1) / W > sc::RMAX) return hipErrorInvalidValue;
  constexpr int lds = (int)sizeof(sc::Smem);
#define TG_SC_EMIT(G_, SB_)                                                                        \
  do {                                                                                             \
    e = ensure_dynamic_lds<sc::sc_emit_kernel<TPT, G_, SB_>>(lds);                                 \
    if (e != hipSuccess) return e;                                                                 \
    hipLaunchKernelGGL((sc::sc_emit_kernel<TPT, G_, SB_>), dim3((unsigned)W), dim3(sc::NT), lds,   \
                       stream, s, mask, cu_in, cu_kept, B, max_n, w, kept, status,                 \
                       static_cast<const uint8_t*>(h), pos, (uint32_t)row_bytes,                   \
                       static_cast<uint8_t*>(h_out), pos_out, s_out);                              \
  } while (0)
  const bool smallb = B <= sc::CUMAX;
  if (h_out) {
    if (smallb) TG_SC_EMIT(true, true); else TG_SC_EMIT(true, false);
  } else {
    if (smallb) TG_SC_EMIT(false, true); else TG_SC_EMIT(false, false);
  }
#undef TG_SC_EMIT
  return hipGetLastError();
}

hipError_t launch_select_compact(const float* s, const uint8_t* mask, const int32_t* cu_in,
                                 const int32_t* cu_kept, int B, int64_t T_in, int64_t T, int max_n,
                                 int32_t* kept, int32_t* status, void* ws, const void* h,
                                 const int32_t* pos, size_t row_bytes, void* h_out,
                                 int32_t* pos_out, float* s_out, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  switch (sc_tpt(max_n)) {
    case 1: return sc_launch<1>(s, mask, cu_in, cu_kept, B, T_in, T, max_n, kept, status, ws, h, pos, row_bytes, h_out, pos_out, s_out, stream);
    case 2: return sc_launch<2>(s, mask, cu_in, cu_kept, B, T_in, T, max_n, kept, status, ws, h, pos, row_bytes, h_out, pos_out, s_out, stream);
    case 4: return sc_launch<4>(s, mask, cu_in, cu_kept, B, T_in, T, max_n, kept, status, ws, h, pos, row_bytes, h_out, pos_out, s_out, stream);
    case 8: return sc_launch<8>(s, mask, cu_in, cu_kept, B, T_in, T, max_n, kept, status, ws, h, pos, row_bytes, h_out, pos_out, s_out, stream);
    default: return sc_launch<16>(s, mask, cu_in, cu_kept, B, T_in, T, max_n, kept, status, ws, h, pos, row_bytes, h_out, pos_out, s_out, stream);
  }
}

}  // namespace tg
