/*
 * tokengate.h — C ABI of libtokengate.so: the TokenGate gated-prefill path
 * (gate scorer, Top-K selection with forced keep, compaction, token-gated
 * attention, upper decoder layer) as hand-written HIP kernels for gfx950.
 *
 * Method sources (web pages about "Token-Gated Language Models"):
 *   [TC] Tencent Cloud developer article on TokenGate, sections
 *        "TokenGate 提前筛选 Token" (early token filtering),
 *        "门控机制为评分网络建立梯度路径" (gradient path through the gate),
 *        "TokenGate 的工程验证仍有限" (engineering validation);
 *   [FW] farwalk.ai summary, section "论文的方法" (the method);
 *   [AI] ai.866data.com article, section "可学习剪枝的机制设计" (mechanism).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: the caller owns every buffer. The library never allocates or
 *    frees device memory and keeps no mutable global state; scratch memory is
 *    passed in as (ws, ws_bytes), sized by the matching *_workspace_size().
 *    Calls on different streams with different workspaces may run
 *    concurrently.
 *  - Pointers: all tensor pointers are DEVICE pointers unless stated. Layouts
 *    are dense row-major with the last dimension contiguous.
 *  - Execution: every call validates its arguments on the host, enqueues its
 *    kernels on `stream` and returns without synchronising.
 *  - Errors: the return value reports argument errors synchronously (nothing
 *    is enqueued then) and launch errors (hipGetLastError after the launch).
 *    Per-sequence data errors that only the device can see are reported in a
 *    device status array (see tg_topk_select).
 *  - Dtypes: activations and weights are TG_BF16 (bf16 storage, fp32
 *    accumulation) or TG_F32. Scores, t, g, s_c and lse are always fp32;
 *    indices, positions and offsets are int32.
 *  - Batches are packed ("varlen"): sequence b owns rows
 *    [cu_in[b], cu_in[b+1]) of the input and rows [cu_kept[b], cu_kept[b+1])
 *    of every kept-token tensor; K_b = cu_kept[b+1] - cu_kept[b].
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int tg_status;
#define TG_OK              0  /* enqueued */
#define TG_ERR_INVALID_ARG 1  /* null required pointer, bad size, Hq % Hkv != 0, ... */
#define TG_ERR_UNSUPPORTED 2  /* dtype, head_dim or shape outside what the kernels handle, or not gfx950 */
#define TG_ERR_WORKSPACE   3  /* ws too small (or null while a workspace is needed) */
#define TG_ERR_LAUNCH      4  /* a HIP runtime error while enqueuing */

/* Per-sequence device status flags written by tg_topk_select. */
#define TG_DEV_FORCED_GT_BUDGET 1 /* more forced tokens than K_b: kept slots of b are -1 */
#define TG_DEV_BUDGET_GT_LEN    2 /* K_b > N_b: kept slots of b are -1 */
#define TG_DEV_NAN_SCORE        4 /* a score of b is NaN (informational; NaN ranks lowest) */
#define TG_DEV_LEN_GT_MAX_N     8 /* N_b > max_n passed by the host: kept slots of b are -1 */

typedef enum tg_dtype { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* Text for a status code (static storage; never NULL). */
const char* tg_status_string(tg_status s);

/* ABI version of this header: (major << 16) | minor. */
int tg_abi_version(void);

/* -------------------------------------------------------------------------
 * Gate scorer — [TC] early token filtering, [AI] mechanism design: after
 * layer L's attention a lightweight MLP reads every token's post-attention
 * residual and gives it an importance score. Form:
 *     s_j = sigmoid( w2 . GELU_erf(W1 h_j + b1) + b2 )
 *
 *  h   [T_in, D]  dtype   post-attention residual of layer L (not normalised)
 *  W1  [H1, D]    dtype   (nn.Linear layout), b1 [H1] dtype
 *  w2  [H1]       dtype,  b2 [1] dtype (biases may be zeros, never NULL)
 *  s_out [T_in]   fp32
 * bf16 needs D % 64 == 0 and H1 % 4 == 0 (H1 > 256 needs a workspace for
 * the partial row sums); fp32 accepts any D and H1 (workspace T_in*H1 fp32).
 * T_in == 0 is a no-op.
 * ------------------------------------------------------------------------- */
size_t tg_gate_score_workspace_size(int64_t T_in, int D, int H1, tg_dtype dtype);
tg_status tg_gate_score(const void* h, int64_t T_in, int D, int H1,
                        const void* W1, const void* b1, const void* w2, const void* b2,
                        tg_dtype dtype, float* s_out,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Top-K selection with forced keep — [TC] early token filtering: a Top-K
 * selector keeps K of the N tokens and designated tokens (the question) are
 * never pruned; [AI] mechanism design: only the document body is prunable.
 * Per sequence b: every token with keep_mask = 1 is kept, and the remaining
 * K_b - F_b slots go to the highest-scoring other tokens, ranked by
 * (score descending, index ascending); -0.0 equals +0.0 and NaN ranks below
 * every number. The kept set is therefore unique.
 *
 *  s         [T_in]   fp32 scores
 *  keep_mask [T_in]   uint8, 1 = unprunable; NULL = nothing forced
 *  d_cu_in   [B+1]    int32 device, prefix sums of N_b (d_cu_in[0] = 0, d_cu_in[B] = T_in)
 *  d_cu_kept [B+1]    int32 device, prefix sums of K_b (d_cu_kept[B] = T)
 *  max_n              an upper bound of every N_b. Up to 32768 one workgroup
 *                     per sequence holds its keys in LDS (no workspace); above,
 *                     every sequence is searched by workgroups of 4096 tokens
 *                     in a chain of short kernels, with a workspace of
 *                     tg_topk_select_workspace_size bytes (256-byte aligned).
 *                     A sequence longer than max_n gets TG_DEV_LEN_GT_MAX_N
 *                     and -1 slots.
 *  kept_idx  [T]      int32 out: GLOBAL row indices into s/h, ascending inside
 *                     each sequence, at that sequence's cu_kept offsets
 *  d_status  [B]      int32 device out, TG_DEV_* flags of each sequence
 *                     (overwritten, 0 when fine); may be NULL
 *  ws, ws_bytes       scratch for max_n > 32768 (three 4096-bin histograms
 *                     per sequence, a 32-byte record per 4096-token chunk:
 *                     about B * 48 KB + T_in / 128 bytes); NULL / 0 otherwise.
 *                     Too small: TG_ERR_WORKSPACE; misaligned: TG_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------- */
size_t tg_topk_select_workspace_size(int B, int64_t T_in, int max_n);
tg_status tg_topk_select(const float* s, const uint8_t* keep_mask,
                         const int32_t* d_cu_in, const int32_t* d_cu_kept,
                         int B, int64_t T_in, int64_t T, int max_n,
                         int32_t* kept_idx, int32_t* d_status,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Compaction — [TC] early token filtering: only the selected tokens go on
 * into layer L's FFN and the layers above; [FW] the method: above the gate
 * only the K kept tokens are processed.
 *   h_out[k] = h[kept_idx[k]], pos_out[k] = pos[kept_idx[k]],
 *   s_out[k] = s[kept_idx[k]]   for k < T.
 *  h [T_in, D] dtype; pos [T_in] int32 or NULL (then the position of a token
 *  is its index inside its own sequence: kept_idx[k] - cu_in[b]);
 *  s [T_in] fp32; kept_idx [T] int32 (from tg_topk_select).
 *  h_out [T, D] dtype, pos_out [T] int32, s_out [T] fp32 (s_out may be NULL).
 * Rows are copied bit for bit. A negative kept_idx entry (a slot of a
 * sequence the selection rejected) or one past d_cu_in[B] yields a zero row,
 * position -1 and score 0.
 * ------------------------------------------------------------------------- */
tg_status tg_compact(const void* h, const int32_t* pos, const float* s,
                     const int32_t* kept_idx, const int32_t* d_cu_in,
                     const int32_t* d_cu_kept, int B, int64_t T, int D, tg_dtype dtype,
                     void* h_out, int32_t* pos_out, float* s_out, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Token-gated attention — [TC] gradient-path section: the kept tokens' gate
 * scores enter the upper layers' attention, with a learnable gain and
 * temperature per head; [TC] engineering section: as a bias on the logit of
 * each key. Causal GQA over each sequence of the packed batch, in compacted
 * (ascending position) order:
 *   L_ij = t_h * (q_i,h . k_j,h') / sqrt(d) + g_h * s_c[j],  j <= i,
 *   h' = h / (Hq / Hkv);   o_i,h = sum_j softmax_j(L_ij) v_j,h'.
 *  q [T, Hq, d], k/v [T, Hkv, d] dtype; s_c [T] fp32; t/g [Hq] fp32.
 *  o [T, Hq, d] dtype out; lse [Hq, T] fp32 out (natural log) or NULL.
 *  max_k: an upper bound of every K_b.
 * bf16: d in {64, 128}, Hq / Hkv in {1, 2, 4}. fp32: d in {64, 128}.
 * ------------------------------------------------------------------------- */
size_t tg_gated_attn_workspace_size(int B, int max_k, int Hq, int Hkv, int d, tg_dtype dtype);
tg_status tg_gated_attn_fwd(const void* q, const void* k, const void* v,
                            const float* s_c, const float* t, const float* g,
                            const int32_t* d_cu_kept, int B, int max_k,
                            int Hq, int Hkv, int d, tg_dtype dtype,
                            void* o, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* -------------------------------------------------------------------------
 * One upper decoder layer on the kept tokens — [TC] early token filtering:
 * the FFN and every later layer run on kept tokens only and no KV is made for
 * pruned ones. Qwen3-shaped pre-norm layer:
 *   n1 = RMSNorm(x) * attn_norm;  q,k,v = n1 Wq^T, n1 Wk^T, n1 Wv^T;
 *   rotate-half RoPE on q and k at pos_c (theta_i = pos * rope_base^(-2i/d));
 *   o = token-gated attention (as tg_gated_attn_fwd, with t and g of the layer);
 *   x1 = x + o Wo^T;  n2 = RMSNorm(x1) * ffn_norm;
 *   x_out = x1 + (silu(n2 Wg^T) * (n2 Wu^T)) Wd^T.
 * kcache/vcache [T, Hkv, d] receive the post-RoPE k and v of the kept tokens
 * only. x_out may alias x_in. Every pointer in tg_layer_weights is a device
 * pointer of `dims.dtype` except t and g (fp32).
 * bf16 needs D, I, Hq*d multiples of 64, d in {64, 128}, Hq/Hkv in {1,2,4}.
 * ------------------------------------------------------------------------- */
typedef struct tg_layer_weights {
  const void* attn_norm;  /* [D]        */
  const void* wq;         /* [Hq*d, D]  */
  const void* wk;         /* [Hkv*d, D] */
  const void* wv;         /* [Hkv*d, D] */
  const void* wo;         /* [D, Hq*d]  */
  const void* ffn_norm;   /* [D]        */
  const void* wg;         /* [I, D]     */
  const void* wu;         /* [I, D]     */
  const void* wd;         /* [D, I]     */
  const float* t;         /* [Hq] per-head temperature */
  const float* g;         /* [Hq] per-head gain        */
} tg_layer_weights;

typedef struct tg_layer_dims {
  int D, Hq, Hkv, d, I;
  float rope_base;        /* e.g. 1e6 */
  float rms_eps;          /* e.g. 1e-6 */
  tg_dtype dtype;
  int flags;              /* TG_LAYER_* below; 0 by default */
} tg_layer_dims;

/* tg_layer_dims.flags: the workspace's RoPE table region (layout.rope)
 * already holds the table for this call's pos_c, T, d and rope_base,
 * written by an earlier tg_upper_layer_fwd on the same workspace and stream
 * (the layers of one stack share positions), so the call does not rebuild
 * it. With any other content the layer's RoPE is wrong: the flag is the
 * caller's promise, the library does not check it. */
#define TG_LAYER_ROPE_READY 1

/* tg_layer_dims.flags, bf16 only: both RMSNorms are fused into the
 * projections that consume them. The caller has folded the norm weights
 * into the input columns of those projections (tg_fold_norm_weights: wq, wk
 * and wv by attn_norm, wg and wu by ffn_norm); attn_norm and ffn_norm are
 * then ignored and may be NULL. The QKV and gate/up GEMMs read the raw x and
 * x1 and scale each token row of their products by
 * 1 / sqrt(mean(row^2) + rms_eps), formed from per-64-feature sums of
 * squares: the O and down projections write those of x1 and x_out in their
 * epilogues (layout.ssq), x_in's come from a small kernel unless
 * TG_LAYER_INPUT_SSQ is set. Same layer up to rounding: the normalised
 * activations are never rounded to the dtype. fp32 layers return
 * TG_ERR_UNSUPPORTED with this flag. */
#define TG_LAYER_NORMS_FOLDED 2

/* tg_layer_dims.flags, with TG_LAYER_NORMS_FOLDED: the first half of the
 * workspace's ssq region already holds x_in's sums of squares, written by
 * the previous NORMS_FOLDED call on the same workspace and stream whose
 * x_out is this call's x_in (consecutive layers of a stack), so the call
 * does not recompute them. The caller's promise, unchecked; without
 * TG_LAYER_NORMS_FOLDED the call returns TG_ERR_INVALID_ARG. */
#define TG_LAYER_INPUT_SSQ 4

/* Fold an RMSNorm weight into a projection for TG_LAYER_NORMS_FOLDED, in
 * place on the stream: W[r, c] = W[r, c] * norm_w[c], the product taken in
 * fp32 and rounded to the dtype (nearest even). W [rows, cols] and
 * norm_w [cols] are device pointers of `dtype`. Errors: TG_ERR_INVALID_ARG
 * for NULL pointers or negative sizes; rows or cols == 0 is a no-op. */
tg_status tg_fold_norm_weights(const void* norm_w, void* W, int64_t rows, int cols,
                               tg_dtype dtype, hipStream_t stream);

/* Byte offsets of the layer's intermediates inside its workspace (valid
 * after the call returns and the stream has run): RMSNorm output n2 (n1 is
 * overwritten; unused with TG_LAYER_NORMS_FOLDED), q after RoPE [T,Hq,d],
 * attention output o [T,Hq,d], x1 [T,D], SwiGLU activation [T,I] (all
 * dtype), RoPE table [T, d] fp32 (cos for i < d/2, then sin), and with
 * TG_LAYER_NORMS_FOLDED the row sums of squares [2][T][D/64] fp32 (sum over
 * features 64s..64s+63 of row t at [., t, s]): x_out's in the first half
 * (x_in's until the down projection overwrites them), x1's in the second. */
typedef struct tg_layer_ws_layout {
  size_t norm, q, attn, x1, act, rope, ssq, total;
} tg_layer_ws_layout;

tg_status tg_upper_layer_ws_layout(const tg_layer_dims* dims, int64_t T, tg_layer_ws_layout* out);
size_t tg_upper_layer_workspace_size(const tg_layer_dims* dims, int64_t T, int B, int max_k);
tg_status tg_upper_layer_fwd(const tg_layer_weights* w, const tg_layer_dims* dims,
                             const void* x_in, void* x_out,
                             const int32_t* pos_c, const float* s_c,
                             const int32_t* d_cu_kept, int B, int64_t T, int max_k,
                             void* kcache, void* vcache,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* A stack of upper layers on the same kept tokens — [TC] early token
 * filtering: every layer above the gate runs on the K kept tokens only.
 * Runs tg_upper_layer_fwd for l = 0 .. n_layers-1 in order on x in place
 * (x [T, D] holds the input and receives the last layer's output), with
 * layer l's weights w[l] and its K/V caches at element offset l*T*Hkv*d of
 * kcache / vcache ([n_layers, T, Hkv, d], dtype). Layers after the first
 * reuse the RoPE table (TG_LAYER_ROPE_READY) and, when dims->flags holds
 * TG_LAYER_NORMS_FOLDED, their input's row sums of squares
 * (TG_LAYER_INPUT_SSQ) from the shared workspace; dims->flags may hold
 * only TG_LAYER_NORMS_FOLDED. Workspace: tg_upper_layer_workspace_size()
 * (one layer's). Argument errors are checked for every layer before the
 * first launch; n_layers = 0 is a no-op. */
tg_status tg_upper_layer_stack_fwd(const tg_layer_weights* w, int n_layers,
                                   const tg_layer_dims* dims, void* x,
                                   const int32_t* pos_c, const float* s_c,
                                   const int32_t* d_cu_kept, int B, int64_t T, int max_k,
                                   void* kcache, void* vcache,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * One gated prefill step above layer L, the whole path in one call — [FW]
 * the method: score after layer L, keep K tokens, run the layers above on
 * them; [TC] early token filtering. In order on `stream`: tg_gate_score on h,
 * tg_topk_select, tg_compact (pos NULL: a token's position is its index in
 * its sequence), tg_upper_layer_stack_fwd on the compacted rows.
 *  h [T_in, D] dtype (D = dims->D); gate: the scorer's weights (W1 [H1, D],
 *  b1 [H1], w2 [H1], b2 [1], dtype); layers [n_layers], dims as for the
 *  stack (flags 0 or TG_LAYER_NORMS_FOLDED).
 *  Outputs: s [T_in] fp32, kept_idx [T] int32, d_status [B] int32 (may be
 *  NULL), x [T, D] dtype (the compacted rows, then the last layer's output),
 *  pos_c [T] int32, s_c [T] fp32, kcache / vcache [n_layers, T, Hkv, d].
 * Workspace: tg_gated_prefill_workspace_size() (the larger of the scorer's
 * and one layer's). The first failing stage's status is returned; stages
 * before it have been enqueued.
 * ------------------------------------------------------------------------- */
typedef struct tg_gate_weights {
  const void* W1;  /* [H1, D] */
  const void* b1;  /* [H1]    */
  const void* w2;  /* [H1]    */
  const void* b2;  /* [1]     */
  int H1;
} tg_gate_weights;

size_t tg_gated_prefill_workspace_size(const tg_layer_dims* dims, int H1, int64_t T_in, int64_t T,
                                       int B, int max_k);
tg_status tg_gated_prefill(const void* h, const int32_t* pos, const uint8_t* keep_mask,
                           const int32_t* d_cu_in, const int32_t* d_cu_kept, int B,
                           int64_t T_in, int64_t T, int max_n, int max_k,
                           const tg_gate_weights* gate, const tg_layer_weights* layers,
                           int n_layers, const tg_layer_dims* dims,
                           float* s, int32_t* kept_idx, int32_t* d_status,
                           void* x, int32_t* pos_c, float* s_c, void* kcache, void* vcache,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Instrumentation: exactly tg_upper_layer_fwd, and in addition records
 * events[i] on `stream` right before stage i of the layer and
 * events[TG_LAYER_STAGES] after the last one, so hipEventElapsedTime gives each
 * stage's GPU time. Stages: 0 RoPE table, 1 RMSNorm, 2 QKV projection (+RoPE,
 * KV-cache write), 3 gated attention, 4 O projection (+residual), 5 RMSNorm,
 * 6 gate/up projection (+SwiGLU), 7 down projection (+residual). In bf16 each
 * stage is one kernel; with TG_LAYER_NORMS_FOLDED stage 1 is the sums of
 * squares of x_in (empty with TG_LAYER_INPUT_SSQ) and stage 5 is empty. events: TG_LAYER_STAGES + 1 handles created by the
 * caller with hipEventCreate (none may be NULL). */
#define TG_LAYER_STAGES 8
tg_status tg_upper_layer_fwd_timed(const tg_layer_weights* w, const tg_layer_dims* dims,
                                   const void* x_in, void* x_out,
                                   const int32_t* pos_c, const float* s_c,
                                   const int32_t* d_cu_kept, int B, int64_t T, int max_k,
                                   void* kcache, void* vcache,
                                   void* ws, size_t ws_bytes, hipStream_t stream,
                                   hipEvent_t* events);

#ifdef __cplusplus
}
#endif
#endif /* TOKENGATE_H */
