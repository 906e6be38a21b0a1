// Backward of the gate scorer s = sigmoid(w2 . GELU(W1 h + b1) + b2).
//
// Tencent Cloud TokenGate article, gradient-path section: the gate gives the
// scoring network a gradient path, so it trains with the model. Given the
// forward's scores s and their gradient ds (the attention backward's ds
// scattered back through the compaction):
//   z = W1 h + b1;  du = ds s (1 - s);  dw2 = sum_t du_t GELU(z_t);  db2 = sum_t du_t
//   dz = du w2 GELU'(z);  db1 = sum_t dz_t;  dW1 = sum_t dz_t h_t^T;  dh = dz W1
// (GELU in the exact erf form, GELU'(x) = Phi(x) + x phi(x)).
//
// Passes (bf16 operands, fp32 sums):
//  1. W1 h^T by the library's bf16 GEMM (the scorer's hidden pre-activations);
//  2. one thread per hidden unit over a block of tokens: dz (bf16, the
//     operand of the two products below) and the block's partial sums of
//     dw2, db1, db2;
//  3. dh = dz W1 by the same GEMM on a transposed copy of W1;
//  4. dW1 = dz^T h: a split-K MFMA kernel over token chunks (the reduction
//     runs over tokens, so both operands come from transposing reads of LDS
//     slabs with padded rows, double-buffered), fp32 partials per chunk;
//  5. fixed-order sums of the partials (deterministic).
#include "tg_common.hpp"
#include "tg_internal.hpp"

namespace tg {
namespace sbwd {

constexpr int NT = 256;
constexpr int ROWS_PER_BLOCK = 64;  // tokens per block of pass 2
constexpr int CHUNK = 2048;         // tokens per split of pass 4
constexpr int TILE = 128;           // output tile of pass 4 (m and n)
constexpr int SLAB = 32;            // tokens per LDS slab
constexpr int PADW = TILE + 32;     // padded LDS row (elements): 320 bytes, so the four rows of one
                                    // transposing read start 64 bytes apart modulo the 256-byte bank width

__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.f + erf_fast(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad(float x) {
  return 0.5f * (1.f + erf_fast(x * 0.70710678118654752f)) +
         x * 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.5f * TG_LOG2E * x * x);
}

// pass 2: thread k of a block handles hidden unit k (and k + NT, ...) over ROWS_PER_BLOCK tokens
__global__ __launch_bounds__(NT) void dz_kernel(const bf16* __restrict__ z, const bf16* __restrict__ b1,
                                                const bf16* __restrict__ w2, const float* __restrict__ s,
                                                const float* __restrict__ ds, int64_t T, int H1,
                                                bf16* __restrict__ dz, float* __restrict__ part) {
  const int64_t r0 = (int64_t)blockIdx.x * ROWS_PER_BLOCK;
  const int r1 = (int)min((int64_t)ROWS_PER_BLOCK, T - r0);
  float* pb = part + (size_t)blockIdx.x * (2 * H1 + 1);
  float du_sum = 0.f;
  for (int k = threadIdx.x; k < H1; k += NT) {
    const float bk = bf2f(b1[k]), wk = bf2f(w2[k]);
    float dw2 = 0.f, db1 = 0.f;
    for (int r = 0; r < r1; ++r) {
      const int64_t t = r0 + r;
      const float st = s[t];
      const float du = ds[t] * st * (1.f - st);
      const float x = bf2f(z[(size_t)t * H1 + k]) + bk;
      const float g = du * wk * gelu_grad(x);
      dz[(size_t)t * H1 + k] = f2bf(g);
      dw2 = fmaf(du, gelu(x), dw2);
      db1 += g;
      if (k == 0) du_sum += du;
    }
    pb[k] = dw2;
    pb[H1 + k] = db1;
  }
  if (threadIdx.x == 0) pb[2 * H1] = du_sum;
}

// sums over the pass-2 blocks: dw2, db1 [H1], db2. A workgroup takes 32 of
// the 2*H1+1 entries; 8 lanes per entry sum every 8th block (four loads in
// flight each), then the 8 partial sums combine in a fixed order.
__global__ __launch_bounds__(NT) void small_reduce_kernel(const float* __restrict__ part, int nblk, int H1,
                                                          float* __restrict__ dw2, float* __restrict__ db1,
                                                          float* __restrict__ db2) {
  const int ne = 2 * H1 + 1;
  const int e = blockIdx.x * 32 + threadIdx.x / 8, j = threadIdx.x % 8;
  const int ec = min(e, ne - 1);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int b = j;
  for (; b + 24 < nblk; b += 32) {
    a0 += part[(size_t)b * ne + ec];
    a1 += part[(size_t)(b + 8) * ne + ec];
    a2 += part[(size_t)(b + 16) * ne + ec];
    a3 += part[(size_t)(b + 24) * ne + ec];
  }
  for (; b < nblk; b += 8) a0 += part[(size_t)b * ne + ec];
  float acc = (a0 + a1) + (a2 + a3);
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (j != 0 || e >= ne) return;
  if (e < H1)
    dw2[e] = acc;
  else if (e < 2 * H1)
    db1[e - H1] = acc;
  else
    db2[0] = acc;
}

// out[c][r] = in[r][c] for a [R][C] bf16 matrix, 64 x 64 tiles through LDS
__global__ __launch_bounds__(NT) void transpose_kernel(const bf16* __restrict__ in, bf16* __restrict__ out,
                                                       int R, int C) {
  __shared__ bf16 tile[64][66];
  const int tc = blockIdx.x % ((C + 63) / 64), tr = blockIdx.x / ((C + 63) / 64);
  for (int i = threadIdx.x; i < 64 * 64; i += NT) {
    const int r = i / 64, c = i % 64;
    const int gr = tr * 64 + r, gc = tc * 64 + c;
    tile[r][c] = (gr < R && gc < C) ? in[(size_t)gr * C + gc] : f2bf(0.f);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += NT) {
    const int c = i / 64, r = i % 64;
    const int gr = tr * 64 + r, gc = tc * 64 + c;
    if (gr < R && gc < C) out[(size_t)gc * R + gr] = tile[r][c];
  }
}

// 8 rows (k-slots) x 1 column (lane) of a [SLAB][PADW] bf16 slab as an MFMA
// operand: lane l takes column c0 + l%32 and rows 16*ks + {0..3, 8..11} +
// 4*(l/32) (the same row order for both operands, so it cancels); two
// ds_read_tr16_b64: within 16 lanes, lane 4e+m addresses row e, columns
// 4m .. 4m+3, and lane i receives column i of rows 0..3.
__device__ __forceinline__ bf16x8 slab_frag(const bf16 (*slab)[PADW], int ks, int c0, int lane) {
  const int vg = (lane >> 4) & 3, vs = lane & 15;
  const int r = 16 * ks + 4 * (vg >> 1) + (vs >> 2);
  const int c = c0 + 16 * (vg & 1) + 4 * (vs & 3);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(&slab[r][c]));
  const bf16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(&slab[r + 8][c]));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// pass 4: part[split][m][n] = sum over the split's tokens t of A[t][m] B[t][n]
// (A = dz [T, M], B = h [T, N]); 4 waves of 64 x 64 on a 128 x 128 tile; the
// next slab's rows are loaded into registers while the current one is
// multiplied, then written to the other LDS buffer (one barrier per slab).
// Two waves per SIMD at most: the MFMAs then accumulate in vector registers
// instead of being copied to and from the accumulation registers.
__global__ __launch_bounds__(NT, 2) void tn_kernel(const bf16* __restrict__ A, const bf16* __restrict__ Bm,
                                                int64_t T, int M, int N, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) bf16 sa[2][SLAB][PADW];
  __shared__ __attribute__((aligned(16))) bf16 sb[2][SLAB][PADW];
  constexpr int PPT = SLAB * TILE / 8 / NT;  // 16-byte pieces per thread and operand
  const int ntn = (N + TILE - 1) / TILE, ntm = (M + TILE - 1) / TILE;
  const int bid = blockIdx.x;
  const int tn = bid % ntn, tm = (bid / ntn) % ntm, split = bid / (ntn * ntm);
  const int m0 = tm * TILE, n0 = tn * TILE;
  const int64_t t0 = (int64_t)split * CHUNK, t1 = min(t0 + CHUNK, T);
  const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, grp = lane >> 5;
  const int w = tid >> 6, wm = w >> 1, wn = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero_f32x16();
  u32x4 pa[PPT], pb[PPT];
  auto load = [&](int64_t ts) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int q = tid + i * NT, r = q / (TILE / 8), c = (q % (TILE / 8)) * 8;
      const int64_t t = ts + r;
      pa[i] = u32x4{0u, 0u, 0u, 0u};
      pb[i] = u32x4{0u, 0u, 0u, 0u};
      if (t < t1 && m0 + c < M) pa[i] = *reinterpret_cast<const u32x4*>(A + (size_t)t * M + m0 + c);
      if (t < t1 && n0 + c < N) pb[i] = *reinterpret_cast<const u32x4*>(Bm + (size_t)t * N + n0 + c);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int q = tid + i * NT, r = q / (TILE / 8), c = (q % (TILE / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sa[buf][r][c]) = pa[i];
      *reinterpret_cast<u32x4*>(&sb[buf][r][c]) = pb[i];
    }
  };
  load(t0);
  put(0);
  __syncthreads();
  int buf = 0;
  for (int64_t ts = t0; ts < t1; ts += SLAB, buf ^= 1) {
    const bool more = ts + SLAB < t1;
    if (more) load(ts + SLAB);
#pragma unroll
    for (int ks = 0; ks < SLAB / 16; ++ks) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = slab_frag(sa[buf], ks, wm * 64 + 32 * i, lane);
        bf[i] = slab_frag(sb[buf], ks, wn * 64 + 32 * i, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (more) put(buf ^ 1);
    __syncthreads();
  }
  // acc[i][j]: lane l holds column n = n0 + wn*64 + 32j + l31, rows m = m0 + wm*64 + 32i + row(r)
  float* pp = part + (size_t)split * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + 32 * j + l31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * grp + (r & 3);
        if (m < M && n < N) pp[(size_t)m * N + n] = acc[i][j][r];
      }
    }
}

// dW1[i] = sum over splits of part[split][i], four elements per thread
__global__ __launch_bounds__(NT) void split_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                          int64_t n, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * NT + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int c = 1; c < nsplit; ++c) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)c * n + i);
    acc += v;
  }
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t z, dz, w1t, part2, part4, total;
  int nblk, nsplit;
};

inline WsLayout layout(int64_t T, int D, int H1) {
  WsLayout L{};
  L.nblk = (int)((T + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK);
  L.nsplit = (int)((T + CHUNK - 1) / CHUNK);
  size_t off = 0;
  L.z = off;
  off += al256((size_t)T * H1 * 2);
  L.dz = off;
  off += al256((size_t)T * H1 * 2);
  L.w1t = off;
  off += al256((size_t)D * H1 * 2);
  L.part2 = off;
  off += al256((size_t)L.nblk * (2 * H1 + 1) * 4);
  L.part4 = off;
  off += al256((size_t)L.nsplit * H1 * D * 4);
  L.total = off;
  return L;
}

}  // namespace sbwd

size_t score_bwd_workspace_bytes(int64_t T, int D, int H1) { return sbwd::layout(T, D, H1).total; }

hipError_t launch_score_bwd(const void* h, int64_t T, int D, int H1, const void* W1, const void* b1,
                            const void* w2, const float* s, const float* ds, void* dh, float* dW1,
                            float* db1, float* dw2, float* db2, void* ws, hipStream_t stream) {
  using namespace sbwd;
  const WsLayout L = layout(T, D, H1);
  char* base = static_cast<char*>(ws);
  bf16* z = reinterpret_cast<bf16*>(base + L.z);
  bf16* dz = reinterpret_cast<bf16*>(base + L.dz);
  bf16* w1t = reinterpret_cast<bf16*>(base + L.w1t);
  float* part2 = reinterpret_cast<float*>(base + L.part2);
  float* part4 = reinterpret_cast<float*>(base + L.part4);
  hipError_t e = gemm_bf16_plain(static_cast<const bf16*>(h), static_cast<const bf16*>(W1), nullptr, z, (int)T,
                                 H1, D, stream);
  if (e != hipSuccess) return e;
  dz_kernel<<<dim3((unsigned)L.nblk), dim3(NT), 0, stream>>>(z, static_cast<const bf16*>(b1),
                                                            static_cast<const bf16*>(w2), s, ds, T, H1, dz, part2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  small_reduce_kernel<<<dim3((unsigned)((2 * H1 + 1 + 31) / 32)), dim3(NT), 0, stream>>>(part2, L.nblk, H1, dw2,
                                                                                          db1, db2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  transpose_kernel<<<dim3((unsigned)(((H1 + 63) / 64) * ((D + 63) / 64))), dim3(NT), 0, stream>>>(
      static_cast<const bf16*>(W1), w1t, H1, D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = gemm_bf16_plain(dz, w1t, nullptr, static_cast<bf16*>(dh), (int)T, D, H1, stream);
  if (e != hipSuccess) return e;
  const int ntn = (D + TILE - 1) / TILE, ntm = (H1 + TILE - 1) / TILE;
  tn_kernel<<<dim3((unsigned)(ntn * ntm * L.nsplit)), dim3(NT), 0, stream>>>(dz, static_cast<const bf16*>(h), T, H1,
                                                                            D, part4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = (int64_t)H1 * D;
  split_reduce_kernel<<<dim3((unsigned)((n / 4 + NT - 1) / NT)), dim3(NT), 0, stream>>>(part4, L.nsplit, n, dW1);
  return hipGetLastError();
}

}  // namespace tg
