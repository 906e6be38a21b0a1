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
 *    frees device memory; scratch memory is passed in as (ws, ws_bytes),
 *    sized by the matching *_workspace_size(). Calls on different streams
 *    with different workspaces may run concurrently. Host-side state is
 *    limited to per-device caches that are idempotent and thread-safe (the
 *    gfx950 check, kernels' raised LDS limits, the address of the scratch of
 *    tg_topk_select_noalloc); the one device-side state is that scratch,
 *    which the library defines as a static device array.
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
 *  - Size limit (bf16): the kernels address every operand through 32-bit
 *    buffer ranges, so each activation or weight matrix a bf16 call reads
 *    (and one sequence's K or V) must be smaller than 4 GiB; larger calls
 *    return TG_ERR_UNSUPPORTED before anything is enqueued.
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

/* Element type of activations and weights. A plain 32-bit integer (not an
 * enum) so that any value a caller passes is well defined inside the library,
 * which refuses codes other than these with TG_ERR_UNSUPPORTED. */
typedef int32_t tg_dtype;
#define TG_F32  0
#define TG_BF16 1

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
 *  max_n              an upper bound of every N_b, at most 1048576 (else
 *                     TG_ERR_UNSUPPORTED). A sequence longer than max_n gets
 *                     TG_DEV_LEN_GT_MAX_N and -1 slots.
 *  kept_idx  [T]      int32 out: GLOBAL row indices into s/h, ascending inside
 *                     each sequence, at that sequence's cu_kept offsets
 *  d_status  [B]      int32 device out, TG_DEV_* flags of each sequence
 *                     (overwritten, 0 when fine); may be NULL
 *  ws, ws_bytes       scratch of tg_topk_select_workspace_size(B, T_in, max_n)
 *                     bytes, 256-byte aligned, contents irrelevant (about 12
 *                     bytes per input token: per chunk of the sequences a
 *                     record, two lists of its score bins and its keys sorted
 *                     by bin). Too small or NULL: TG_ERR_WORKSPACE; misaligned:
 *                     TG_ERR_INVALID_ARG.
 * Two kernels: per chunk of up to 4096 tokens a summary (forced count, NaN
 * flag, key range, the non-empty bins of the keys' top 16 bits, the keys
 * sorted by bin); then workgroups that share the output rows derive the
 * threshold key from the summaries and emit their rows.
 * ------------------------------------------------------------------------- */
size_t tg_topk_select_workspace_size(int B, int64_t T_in, int max_n);
tg_status tg_topk_select(const float* s, const uint8_t* keep_mask,
                         const int32_t* d_cu_in, const int32_t* d_cu_kept,
                         int B, int64_t T_in, int64_t T, int max_n,
                         int32_t* kept_idx, int32_t* d_status,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Selection and compaction in one pass — [TC] early token filtering: only the
 * selected tokens go on above the gate. Exactly tg_topk_select followed by
 * tg_compact on the same arguments (same outputs, bit for bit), but the
 * workgroups that emit a share of the kept indices copy those rows, positions
 * and scores at once, so the row gather is spread over the whole GPU and the
 * kept indices are not read back.
 *  h [T_in, D] dtype, pos [T_in] int32 or NULL (then a token's position is its
 *  index inside its sequence); h_out [T, D] dtype, pos_out [T] int32,
 *  s_out [T] fp32 or NULL; the rest as tg_topk_select (same workspace). Rows
 *  of a rejected sequence are zeros, its positions -1 and its scores 0.
 * ------------------------------------------------------------------------- */
tg_status tg_select_compact(const float* s, const uint8_t* keep_mask,
                            const int32_t* d_cu_in, const int32_t* d_cu_kept,
                            int B, int64_t T_in, int64_t T, int max_n,
                            const void* h, const int32_t* pos, int D, tg_dtype dtype,
                            int32_t* kept_idx, int32_t* d_status,
                            void* h_out, int32_t* pos_out, float* s_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* The same selection for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no ws argument. In place of the workspace this call uses a
 * scratch array of TG_SELECT_NOALLOC_SCRATCH_BYTES that the library holds in
 * device memory, one per GPU for the life of the process, and calls no
 * allocating routine (about 340 thousand input tokens per call).
 * Arguments, outputs and results are those of tg_topk_select. Errors: as
 * tg_topk_select, plus TG_ERR_WORKSPACE when
 * tg_topk_select_workspace_size(B, T_in, max_n) exceeds the scratch size
 * (nothing is enqueued then). Every call on a GPU shares that GPU's scratch,
 * which keeps the last call's contents (each call writes everything it reads
 * before reading it): calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller. */
#define TG_SELECT_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
tg_status tg_topk_select_noalloc(const float* s, const uint8_t* keep_mask,
                                 const int32_t* d_cu_in, const int32_t* d_cu_kept,
                                 int B, int64_t T_in, int64_t T, int max_n,
                                 int32_t* kept_idx, int32_t* d_status, hipStream_t stream);

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

/* tg_layer_dims.flags: one half of the layer only, for a gate layer L whose
 * FFN runs on the kept tokens alone ([TC] early token filtering: pruned
 * tokens skip layer L's FFN; the scorer reads layer L's post-attention
 * residual). TG_LAYER_ATTN_ONLY runs stages 0-4: x_out receives the
 * post-attention residual x1 = x_in + o Wo^T (x_out may alias x_in).
 * TG_LAYER_FFN_ONLY runs stages 5-7 on x_in as that residual:
 * x_out = x_in + SwiGLU(...) Wd^T; pos_c, s_c, d_cu_kept, kcache and vcache
 * are not used and may be NULL, and with TG_LAYER_NORMS_FOLDED the row sums
 * of squares of x_in are computed by the call. Both at once:
 * TG_ERR_INVALID_ARG. */
#define TG_LAYER_ATTN_ONLY 8
#define TG_LAYER_FFN_ONLY 16

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
 * tg_select_compact (pos NULL: a token's position is its index in its
 * sequence), tg_upper_layer_stack_fwd on the compacted rows.
 *  h [T_in, D] dtype (D = dims->D); gate: the scorer's weights (W1 [H1, D],
 *  b1 [H1], w2 [H1], b2 [1], dtype); layers [n_layers], dims as for the
 *  stack (flags 0 or TG_LAYER_NORMS_FOLDED).
 *  Outputs: s [T_in] fp32, kept_idx [T] int32, d_status [B] int32 (may be
 *  NULL), x [T, D] dtype (the compacted rows, then the last layer's output),
 *  pos_c [T] int32, s_c [T] fp32, kcache / vcache [n_layers, T, Hkv, d].
 * Workspace: tg_gated_prefill_workspace_size() (the largest of the
 * scorer's, the selection's for any max_n and one layer's). The first
 * failing stage's status is returned; stages
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

/* -------------------------------------------------------------------------
 * The whole three-stage prefill with the gate at layer L = n_below — [FW]
 * the method: the forward splits in three; [TC] early token filtering: all
 * prompt tokens run through the layers below the gate and through layer L's
 * attention, with the full prompt's K/V kept there ([TC] engineering
 * section); the scorer reads layer L's post-attention residual, the selector
 * keeps K_b tokens per sequence, and only those go on into layer L's FFN and
 * the layers above (token-gated attention). In order on `stream`:
 *   below[l], l < n_below: whole layers on all T_in rows, plain causal
 *     attention (t = 1, g = 0: their t and g are not read);
 *   gate_layer: attention half on all T_in rows (plain), x_full = x1;
 *   tg_gate_score on x_full -> s; tg_select_compact of x_full's rows -> x,
 *   pos_c, s_c; gate_layer's FFN half on x; tg_upper_layer_stack_fwd of
 *   above[] on x.
 *  h [T_in, D] dtype: the rows entering layer 0 (not modified);
 *  pos [T_in] int32: every token's original position (its index in its
 *  sequence for a plain prompt);
 *  x_full [T_in, D] dtype out: layer L's post-attention residual;
 *  kcache_full / vcache_full [n_below + 1, T_in, Hkv, d] out: K/V of every
 *  token in layers 0 .. L; max_n bounds the N_b (the attention and selection
 *  of the full rows), max_k the K_b;
 *  s, kept_idx, d_status, x, pos_c, s_c, kcache, vcache [n_above, T, Hkv, d]:
 *  as tg_gated_prefill; with T = 0 (nothing kept) kept_idx, x, pos_c, s_c,
 *  kcache and vcache may be NULL and the call ends after the selection.
 *  dims->flags: 0 or TG_LAYER_NORMS_FOLDED.
 * Workspace: tg_full_prefill_workspace_size(). The first failing stage's
 * status is returned; stages before it have been enqueued.
 * ------------------------------------------------------------------------- */
size_t tg_full_prefill_workspace_size(const tg_layer_dims* dims, int H1, int64_t T_in, int64_t T,
                                      int B, int max_n, int max_k);
tg_status tg_full_prefill(const void* h, const int32_t* pos, const uint8_t* keep_mask,
                          const int32_t* d_cu_in, const int32_t* d_cu_kept, int B,
                          int64_t T_in, int64_t T, int max_n, int max_k,
                          const tg_gate_weights* gate,
                          const tg_layer_weights* below, int n_below,
                          const tg_layer_weights* gate_layer,
                          const tg_layer_weights* above, int n_above,
                          const tg_layer_dims* dims,
                          void* x_full, void* kcache_full, void* vcache_full,
                          float* s, int32_t* kept_idx, int32_t* d_status,
                          void* x, int32_t* pos_c, float* s_c, void* kcache, void* vcache,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Backward of the token-gated attention — [TC] gradient-path section: the
 * kept tokens' scores enter the upper layers' attention logits, so the loss
 * reaches the scorer through them, and the per-head gain and temperature are
 * learned. For the forward of tg_gated_attn_fwd and an upstream gradient dO:
 *   dv_j = sum_i P_ij dO_i;  dL_ij = P_ij (dO_i.v_j - dO_i.o_i);
 *   dq_i = t_h/sqrt(d) sum_j dL_ij k_j;  dk_j = t_h/sqrt(d) sum_i dL_ij q_i;
 *   ds_j = sum_h g_h sum_i dL_ij;  dg_h = sum_ij dL_ij s_c[j];
 *   dt_h = sum_ij dL_ij q_i.k_j / sqrt(d)
 * (dk, dv of a kv head sum over the query heads of its group). P is
 * recomputed from the forward's log-sum-exp.
 *  q [T, Hq, d], k, v [T, Hkv, d], o [T, Hq, d] (the forward's output), dO
 *  [T, Hq, d]: bf16; s_c [T], t, g [Hq], lse [Hq, T] (the forward's, natural
 *  log): fp32; d_cu_kept [B+1] (device); T = cu_kept[B] (host); max_k bounds
 *  the K_b.
 *  Outputs, fp32: dq [T, Hq, d], dk, dv [T, Hkv, d], ds [T] (gradient of the
 *  kept tokens' scores), dt, dg [Hq]. Every element is written (none is
 *  accumulated into), and the results do not depend on timing.
 * Supported: bf16, d in {64, 128}, Hq / Hkv in {1, 2, 4}, one sequence's q
 * rows below 4 GiB (max_k * Hq * d * 2 bytes, else TG_ERR_UNSUPPORTED); q, k,
 * v, o, dO, dq, dk, dv 16-byte aligned. Workspace:
 * tg_gated_attn_bwd_workspace_size() bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t tg_gated_attn_bwd_workspace_size(int B, int64_t T, int max_k, int Hq, int Hkv, int d,
                                        tg_dtype dtype);
tg_status tg_gated_attn_bwd(const void* q, const void* k, const void* v, const float* s_c,
                            const float* t, const float* g, const int32_t* d_cu_kept, int B,
                            int64_t T, int max_k, int Hq, int Hkv, int d, tg_dtype dtype,
                            const void* o, const float* lse, const void* dO,
                            float* dq, float* dk, float* dv, float* ds, float* dt, float* dg,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Backward of the gate scorer — [TC] gradient-path section: the gate gives
 * the scoring network a gradient path, so it trains with the model. For
 * s = sigmoid(w2 . GELU(W1 h + b1) + b2) (tg_gate_score) and ds per token:
 *   du = ds s (1 - s); dw2 = sum_t du_t GELU(z_t); db2 = sum_t du_t;
 *   dz = du w2 GELU'(z) with z = W1 h + b1; db1 = sum_t dz_t;
 *   dW1 = sum_t dz_t h_t^T; dh = dz W1   (erf GELU).
 *  h [T_in, D], W1 [H1, D], b1, w2 [H1]: bf16 (the forward's inputs);
 *  s [T_in] fp32: the forward's scores (b2 enters only through them);
 *  ds [T_in] fp32; dh [T_in, D] bf16 out; dW1 [H1, D], db1, dw2 [H1], db2 [1]
 *  fp32 out (all written; zero when T_in = 0). Sums run in a fixed order
 *  (deterministic).
 * Supported: bf16, D % 64 == 0, H1 % 64 == 0; h, W1, dh, dW1 16-byte
 * aligned. Workspace: tg_gate_score_bwd_workspace_size() bytes, 256-byte
 * aligned (none when T_in = 0).
 * ------------------------------------------------------------------------- */
size_t tg_gate_score_bwd_workspace_size(int64_t T_in, int D, int H1, tg_dtype dtype);
tg_status tg_gate_score_bwd(const void* h, int64_t T_in, int D, int H1, const void* W1,
                            const void* b1, const void* w2, tg_dtype dtype, const float* s,
                            const float* ds, void* dh, float* dW1, float* db1, float* dw2,
                            float* db2, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gradient of the prompt scores through the compaction — [TC] early token
 * filtering: pruned tokens stop at the gate layer and never reach the layers
 * whose attention reads the scores. ds[kept_idx[r]] = ds_c[r] for r < T and
 * ds[i] = 0 for every other i < T_in (a kept slot of -1, written for a
 * rejected sequence, carries nothing). kept_idx [T] int32 as written by
 * tg_topk_select; ds_c [T], ds [T_in] fp32. */
tg_status tg_compact_scores_bwd(const float* ds_c, const int32_t* kept_idx, int64_t T, int64_t T_in,
                                float* ds, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Gated DeltaNet mixer of the hybrid variant — [TC] section on the gate
 * position: in a hybrid model (Qwen3.5-2B) only some layers use full
 * attention and the rest are Gated DeltaNet; the scorer reads hidden states,
 * so the gate can sit on a GDN layer, and a GDN layer above the gate has no
 * attention logits to bias: it runs on the kept tokens (the rows compacted
 * by tg_select_compact, packed by d_cu). Per sequence and head, state S
 * [dv, dk] (state_in's, or zero), for each token in order:
 *   k^ = k / sqrt(|k|^2 + 1e-6),  q^ = q / (sqrt(|q|^2 + 1e-6) sqrt(dk))
 *   S <- alpha S;  S <- S + beta (v - S k^) k^T;  o = S q^
 *  q, k [T, H, dk], v [T, H, dv], o [T, H, dv] out: dtype; alpha, beta
 *  [T, H] fp32 (decay and write strength of each token and head; alpha in
 *  [0, 1]); d_cu [B+1] int32 (device), with d_cu[B] <= T (rows at or past T
 *  are never read or written; with T = 0 the row operands may be NULL); state_in / state_out [B, H, dv, dk] fp32,
 *  optional (NULL: start from zero / do not write), 16-byte aligned.
 * bf16 runs the chunked form of the recurrence on the matrix cores (chunks of
 * 64 tokens; a decay below e^-80 counts as e^-80 inside a chunk); its
 * workspace is tg_gdn_workspace_size() bytes, 256-byte aligned (0 when T is
 * 0). fp32 runs the token recurrence itself and takes no workspace (ws may
 * be NULL). Splitting a sequence over calls at a multiple of 64 tokens, with
 * the state carried, gives the same bits as one call.
 * Supported: dk in {64, 128}, dv % 32 == 0; q, k, v and o 16-byte aligned.
 * ------------------------------------------------------------------------- */
size_t tg_gdn_workspace_size(int64_t T, int B, int H, int dk, int dv, tg_dtype dtype);
tg_status tg_gdn_fwd(const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta, const int32_t* d_cu, int64_t T, int B, int H, int dk,
                     int dv, tg_dtype dtype, const float* state_in, void* o, float* state_out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Decode attention over the pruned K/V cache — [TC] engineering section:
 * once prefill has fixed the gate bias, decoding folds it into the attention
 * mask and runs ordinary attention over the cache; [TC] early token
 * filtering: generated tokens are never gated out and join the cache. One
 * new token per sequence attends to every cached key of its sequence (all of
 * them precede it, so no causal mask) with the prefill's logit
 *   L_j = t_h * (q_h . k_j,h') / sqrt(d) + g_h * s_j,  h' = h / (Hq / Hkv).
 * The cache has two segments per sequence:
 *  A: the kept prompt tokens where the prefill wrote them: kA, vA
 *     [rows, Hkv, d] dtype (post-RoPE), sA [rows] fp32 their scores, d_cuA
 *     [B+1] int32 (device) sequence b's rows cuA[b] .. cuA[b+1]-1 (the
 *     prefill's d_cu_kept, kcache, vcache and s_c). Required even when empty.
 *  B: the generated tokens: kB, vB [B, capB, Hkv, d] dtype, sB [B, capB]
 *     fp32, d_lenB [B] int32 (device): sequence b uses rows 0 .. lenB[b]-1 of
 *     its capB (the caller appends each new token's k, v and score before the
 *     call that attends from it). May be NULL when capB == 0.
 * The key scores are the caller's: the library reads sA / sB as given (the
 * tests and the benchmark give a generated token its own scorer score, as a
 * forced prompt token keeps its own).
 *  q [B, Hq, d] dtype (post-RoPE at the new token's position); t, g [Hq]
 *  fp32; max_len (host) bounds (cuA[b+1]-cuA[b]) + lenB[b] over b;
 *  o [B, Hq, d] dtype out; lse [B, Hq] fp32 out (natural log; optional);
 *  d_status [B] int32 out (optional): TG_DEV_LEN_GT_MAX_N when a sequence's
 *  segment lengths are negative, lenB[b] > capB, or the total exceeds
 *  max_len; that sequence's o and lse are then NaN. A sequence with no keys
 *  gets o = 0, lse = -inf.
 * Supported: d in {64, 128}, Hq / Hkv in {1, 2, 4, 8}; q, k, v and o 16-byte
 * aligned. Workspace: tg_decode_attn_workspace_size() bytes (0 when every
 * sequence fits one key chunk), 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t tg_decode_attn_workspace_size(int B, int max_len, int Hq, int Hkv, int d, tg_dtype dtype);
tg_status tg_decode_attn_fwd(const void* q, const void* kA, const void* vA, const float* sA,
                             const int32_t* d_cuA, const void* kB, const void* vB,
                             const float* sB, const int32_t* d_lenB, int capB,
                             const float* t, const float* g, int B, int max_len,
                             int Hq, int Hkv, int d, tg_dtype dtype,
                             void* o, float* lse, int32_t* d_status,
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
