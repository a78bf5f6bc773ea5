/*
 * mha.h -- C ABI of libmha, multi-head scaled dot-product attention (forward
 * and backward) for AMD Instinct MI355X (gfx950).
 *
 * The operation ("Attention Is All You Need" as explained on the pages cited
 * below; trishampatil.com = [TP], aicassindra.com = [AC], alexdo.xyz = [AD],
 * zeroshotmind.com = [ZS]):
 *
 *   out_i = sum_j softmax_j(scale * q_i . k_j over the visible keys j) * v_j
 *
 * per batch entry b and head h ([TP] "Scaled Dot-Product Attention: Step by
 * Step"; [ZS] "Scaled dot-product attention").  A key j is visible to query i
 * unless it is padding (j >= key_lens[b], [AD] "Two masks, not one") or, under
 * the causal mask, in the future (j > i, [TP] "Why Masking Is Required").
 * Masked keys get weight exactly 0.  The three roles of [ZS] "Where attention
 * is used three ways" map onto the arguments: encoder self-attention
 * (MHA_MASK_NONE, keys = queries' sequence), decoder masked self-attention
 * (MHA_MASK_CAUSAL) and encoder-decoder cross-attention (MHA_MASK_NONE,
 * Nq != Nk, keys/values from the encoder; [AD] "Multi-Head Attention (middle) -
 * cross-attention").
 *
 * Conventions shared by every entry point:
 *   - Pointers are device memory owned by the caller unless stated otherwise;
 *     the library never allocates, frees or keeps them.
 *   - All tensors are dense row-major with the stated shapes; element type is
 *     given by `dtype` (MHA_F32, MHA_BF16, MHA_F16), the same for every
 *     floating-point tensor of a call.  bf16/f16 math accumulates in fp32;
 *     outputs are rounded to nearest-even into the input type.
 *   - `key_lens` is a device int32[B] or NULL (no padding).  Values are clamped
 *     to [0, Nk] on the device; the host never reads them.  A query with no
 *     visible key (key length 0) gets an output row of zeros.
 *   - `scale` is the factor applied to q.k; pass 1/sqrt(d_k) for the pages'
 *     scaling ([TP] "Why the sqrt(d_k) Scaling Exists").  It must be finite.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Argument errors are detected on the host before any HIP call
 *     and return a negative status with nothing launched; launch failures
 *     return MHA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation.  mha_last_error_message() gives a message for the last failure
 *     on the calling thread.
 *   - Entry points keep no state between calls and may be called from several
 *     threads at once.
 */
#ifndef MHA_H_
#define MHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* mask_kind */
#define MHA_MASK_NONE 0   /* every key below key_lens[b] is visible */
#define MHA_MASK_CAUSAL 1 /* additionally j <= i; requires Nq == Nk (decoding: see
                             mha_decode_forward) */

/* dtype */
#define MHA_F32 0
#define MHA_BF16 1
#define MHA_F16 2

/* kernel plans of mha_proj_forward_timed */
#define MHA_PLAN_AUTO 0    /* what mha_proj_forward does (see mha_proj_fused) */
#define MHA_PLAN_UNFUSED 1 /* projection GEMM, attention kernel, output GEMM */
#define MHA_PLAN_FUSED 2   /* fused projection+attention kernel, output GEMM */

/* status codes */
#define MHA_OK 0
#define MHA_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad enum, ... */
#define MHA_ERR_UNSUPPORTED (-2) /* valid request the library has no kernel for */
#define MHA_ERR_WORKSPACE (-3)   /* workspace missing, too small or misaligned */
#define MHA_ERR_HIP (-4)         /* the HIP runtime refused a launch */

/*
 * mha_forward -- attention on per-head tensors ([TP] "Scaled Dot-Product
 * Attention: Step by Step", applied per head as in [TP] "Multi-Head Attention").
 *
 *   q   [B, H, Nq, d_k]     k [B, H, Nk, d_k]     v [B, H, Nk, d_v]
 *   out [B, H, Nq, d_v]     written; may not overlap the inputs
 *
 * Sizes: B, H, Nq, Nk >= 0 (zero-sized problems return MHA_OK; with Nk == 0
 * every output row is zero); d_k, d_v >= 1.  Supported: MHA_F32 with
 * d_k, d_v <= 128; MHA_BF16 and MHA_F16 with d_k == d_v == 64.  bf16/f16
 * tensors must be 16-byte aligned.  Returns MHA_OK or a negative status.
 */
int mha_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                int dtype, void* stream);

/*
 * mha_proj_workspace_bytes -- device workspace mha_proj_forward needs for these
 * sizes (the projected Q, K, V and the concatenated head outputs, each 256-byte
 * aligned).  Returns 0 for invalid sizes.
 */
size_t mha_proj_workspace_bytes(int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int dtype);

/*
 * mha_proj_forward -- multi-head attention with its projections ([TP] "Query /
 * Key / Value Roles", "Multi-Head Attention", "The Output Projection W^O"; the
 * layer of [AC] "A faithful layer in code"):
 *
 *   Q = x_q W_Q^T + b_Q,  K = x_kv W_K^T + b_K,  V = x_kv W_V^T + b_V
 *   head h attends with feature columns [h*d, (h+1)*d) of Q, K and V
 *   out = Concat(head_0 .. head_{H-1}) W_O^T + b_O
 *
 *   x_q  [B, Nq, D]      decoder/query side
 *   x_kv [B, Nk, D]      encoder/key-value side, or NULL for self-attention
 *                        (keys and values from x_q; then Nk must equal Nq)
 *   W_Q, W_K [H*d_k, D]  W_V [H*d_v, D]  W_O [D, H*d_v]
 *                        -- the [out_features, in_features] layout of the
 *                        nn.Linear layers in [AC]'s listing, i.e. the transpose
 *                        of the X*W matrices in [TP]'s formulas
 *   b_Q, b_K [H*d_k], b_V [H*d_v], b_O [D]   nullable (no bias)
 *   out  [B, Nq, D]      written
 *   workspace            device memory of at least
 *                        mha_proj_workspace_bytes(...) bytes, 256-byte aligned,
 *                        owned by the caller; its contents are scratch.
 *
 * Supported: MHA_BF16 and MHA_F16 with d_k == d_v == 64, D a multiple of 8,
 * all tensors 16-byte aligned.  The projected Q, K, V and the head outputs are
 * rounded to the input type (in the workspace, or in on-chip memory when the
 * call is fused -- see mha_proj_fused; the results are the same).  Returns
 * MHA_OK or a negative status.
 */
int mha_proj_forward(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                     const void* W_V, const void* W_O, const void* b_Q, const void* b_K,
                     const void* b_V, const void* b_O, void* out, int B, int Nq, int Nk, int D,
                     int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mha_proj_forward_gqa -- mha_proj_forward with the key and value projections
 * shared by groups of query heads ([TP] "Limitations of the Original Design":
 * multi-query and grouped-query attention keep a query projection per head and
 * share the key/value projections; [ZS] "Many heads, many subspaces").  W_K is
 * [H_kv*d_k, D], W_V [H_kv*d_v, D], b_K, b_V [H_kv*d] (nullable); query head h
 * attends with key/value head h / (H / H_kv), so each run of H / H_kv
 * consecutive query heads shares one.  Everything else as mha_proj_forward;
 * H_kv == H is mha_proj_forward (same plan, same results), H_kv == 1
 * multi-query attention.  1 <= H_kv <= H with H a multiple of H_kv, else
 * MHA_ERR_INVALID_ARG.  The plan is mha_proj_forward's for the same sizes
 * (mha_proj_fused): fused, each query head's workgroup projects its group's K
 * and V itself; unfused, the projections write K and V once per key/value
 * head and the attention kernel reads them for the whole group.  `workspace`:
 * at least mha_proj_gqa_workspace_bytes(...) bytes (0 for invalid sizes).
 */
size_t mha_proj_gqa_workspace_bytes(int B, int Nq, int Nk, int D, int H, int H_kv, int d_k, int d_v, int dtype);

int mha_proj_forward_gqa(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K, const void* W_V,
                         const void* W_O, const void* b_Q, const void* b_K, const void* b_V, const void* b_O,
                         void* out, int B, int Nq, int Nk, int D, int H, int H_kv, int d_k, int d_v, int mask_kind,
                         const int32_t* key_lens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                         void* stream);

/* mha_proj_forward_gqa_timed -- as mha_proj_forward_gqa, plus 6 events as for
 * mha_proj_forward_timed (whose plan is MHA_PLAN_AUTO). */
int mha_proj_forward_gqa_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                               const void* W_V, const void* W_O, const void* b_Q, const void* b_K, const void* b_V,
                               const void* b_O, void* out, int B, int Nq, int Nk, int D, int H, int H_kv, int d_k,
                               int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                               void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * Timed variants, for profiling.  Same arguments, validation and results as the
 * entry point they extend, plus `events`: caller-created hipEvent_t handles
 * (hipEventCreate; the caller owns them) that receive the start and end
 * timestamps of each kernel the call launches, taken by the dispatch itself
 * (hipExtLaunchKernel), so hipEventElapsedTime(events[2k], events[2k+1]) is
 * kernel k's own duration.  NULL records nothing.
 *
 * mha_forward_timed: 2 events -- the attention kernel.
 * mha_proj_forward_timed: 6 events -- the Q/K/V projection, the attention
 * kernel and the output projection, in that order.  A fused call launches two
 * kernels: events[0..1] time the fused projection+attention kernel,
 * events[4..5] the output projection, and events[2..3] are left untouched.
 * Its last argument selects the kernel plan: MHA_PLAN_AUTO (the plan
 * mha_proj_forward takes), MHA_PLAN_UNFUSED, or MHA_PLAN_FUSED (returns
 * MHA_ERR_UNSUPPORTED when the fused kernel does not take these sizes -- see
 * mha_proj_fused); an unknown
 * value is MHA_ERR_INVALID_ARG.  Both plans compute the same function; they
 * agree bit for bit when every sequence has at most 64 keys.
 */
int mha_forward_timed(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                      int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                      int dtype, void* stream, void* const* events);

int mha_proj_forward_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                           const void* W_V, const void* W_O, const void* b_Q, const void* b_K,
                           const void* b_V, const void* b_O, void* out, int B, int Nq, int Nk,
                           int D, int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens,
                           float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events, int plan);

/*
 * mha_forward_strided -- mha_forward on strided views, so that layouts such as
 * the [B, N, H, d] of a projection's output ([TP] "Multi-Head Attention": head
 * h is a block of d columns of the projected rows) need no copy.  Element
 * (b, h, n, c) of q lives at q + b*q_strides[0] + h*q_strides[1] +
 * n*q_strides[2] + c (strides in elements, host arrays of 3, c contiguous);
 * likewise k and v (n over keys) and out.  lse: NULL, or as for
 * mha_forward_lse (dense [B, H, Nq] fp32).
 *
 * Strides must be >= 0 (zero strides broadcast an input); bf16/f16 strides
 * must be multiples of 8 elements and the tensors 16-byte aligned (fp32:
 * 4-byte aligned).  Output rows must not overlap (out strides of a dimension
 * with more than one entry at least d_v) and out must not overlap the inputs.
 * bf16/f16 rows of one head, with their stride, must span less than 2^31
 * bytes (including 128 rows past the end).  Otherwise as mha_forward; with
 * dense strides it is mha_forward (or mha_forward_lse).
 */
int mha_forward_strided(const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
                        const void* v, const int64_t* v_strides, void* out, const int64_t* out_strides, float* lse,
                        int B, int H, int Nq, int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens,
                        float scale, int dtype, void* stream);

/*
 * Training ([TP] "Training (Teacher Forcing + Masking)": one parallel forward
 * pass over the whole target sequence, then gradients back through it; [AD]
 * "One forward pass covers the whole sequence").  The pages give no gradient
 * formulas; the backward pass computes the exact derivatives of the
 * mha_forward definition for a scalar loss whose gradient with respect to
 * `out` is `dout`:
 *
 *   P_ij  = weight of key j in row i (0 for masked keys)
 *   dv_j  = sum_i P_ij dout_i                  dP_ij = dout_i . v_j
 *   dS_ij = P_ij (dP_ij - D_i),  D_i = dout_i . out_i
 *   dq_i  = scale sum_j dS_ij k_j              dk_j  = scale sum_i dS_ij q_i
 *
 * Masked keys (padding, the future under the causal mask) receive exactly
 * zero gradient, and a row with no visible key contributes nothing.
 *
 * mha_forward_lse -- mha_forward that also writes the row statistic the
 * backward pass needs:
 *
 *   lse [B, H, Nq] fp32   ln(sum over visible j of exp(scale q_i . k_j));
 *                         -inf for a row with no visible key
 *
 * lse must be non-null and 4-byte aligned (MHA_ERR_INVALID_ARG otherwise) and
 * must not overlap the other tensors.  Supported types and sizes as for
 * mha_forward.
 */
int mha_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                    int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                    void* stream);

/*
 * mha_backward -- gradients of mha_forward with respect to q, k and v.
 *
 *   q, k, v, key_lens, mask_kind, scale   as passed to the forward call
 *   out  [B, H, Nq, d_v]   the forward output
 *   lse  [B, H, Nq] fp32   the forward's row statistic (mha_forward_lse)
 *   dout [B, H, Nq, d_v]   gradient of the loss with respect to out
 *   dq   [B, H, Nq, d_k]   written
 *   dk   [B, H, Nk, d_k]   written (zero rows for padded keys)
 *   dv   [B, H, Nk, d_v]   written (zero rows for padded keys)
 *
 * The weights P are recomputed from q, k and lse tile by tile; no Nq x Nk
 * matrix is stored.  Supported types and head sizes as for mha_forward
 * (MHA_F32 with d_k, d_v <= 128; MHA_BF16 and MHA_F16 with d_k == d_v == 64);
 * bf16/f16 tensors 16-byte aligned, fp32 tensors and lse 4-byte aligned;
 * outputs must not overlap inputs or each other; bf16/f16 sequences below
 * 2^24 rows.  Pointers of a side with zero rows may be NULL.  `workspace`: device
 * memory of at least mha_backward_workspace_bytes(...) bytes, 256-byte
 * aligned, owned by the caller, contents scratch (it holds D); calls sharing a
 * workspace must not run concurrently.  Two kernels run in stream order (dq,
 * which also forms D; then dk and dv).  Returns MHA_OK or a negative status.
 */
size_t mha_backward_workspace_bytes(int B, int H, int Nq, int Nk, int d_k, int d_v, int dtype);

/*
 * mha_backward_single_launch -- 1 when a backward call with these sizes
 * (bf16/f16, d_k == d_v == 64, at most 64 queries and 64 keys, H_kv == H) runs
 * as one kernel, whose workgroup per (b, h) forms dq and then, from D kept in
 * LDS, dk and dv; 0 otherwise (two kernels).  A pure function of the sizes;
 * both plans give the same results bit for bit.
 */
int mha_backward_single_launch(int B, int H, int H_kv, int Nq, int Nk, int d_k, int d_v, int dtype);

int mha_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d_k, int d_v, int mask_kind,
                 const int32_t* key_lens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream);

/* mha_backward_timed -- as mha_backward, plus 4 events (see the timed variants
 * above): events[0..1] time the dq kernel, events[2..3] the dk/dv kernel; when
 * mha_backward_single_launch is 1 for the sizes, events[0..1] time the one
 * kernel and events[2..3] are left untouched. */
int mha_backward_timed(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d_k,
                       int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* events);

/*
 * Shared key/value heads in training (grouped-query attention, H_kv key/value
 * heads serving H query heads; [TP] "Limitations of the Original Design"; [ZS]
 * "Many heads, many subspaces"; [TP] "Training (Teacher Forcing + Masking)").
 * Query head h reads key/value head h / (H / H_kv); H_kv == H is mha_forward,
 * H_kv == 1 multi-query attention.  k and v (and dk, dv) are dense
 * [B, H_kv, Nk, d]; q, out, lse, dout and dq are as in mha_forward_lse and
 * mha_backward.  1 <= H_kv <= H with H a multiple of H_kv, else
 * MHA_ERR_INVALID_ARG.
 *
 * mha_forward_gqa -- the forward pass; lse may be NULL (not written), else as
 * for mha_forward_lse.
 *
 * mha_backward_gqa -- its gradients: dk and dv of a shared head are the sums,
 * over the H / H_kv query heads that read it, of the per-head gradients of
 * mha_backward.  `workspace`: at least mha_backward_gqa_workspace_bytes(...)
 * bytes (0 when H_kv does not divide H), 256-byte aligned, scratch, not shared
 * by concurrent calls; the other requirements as mha_backward.  A dk/dv
 * workgroup owns a key block of one shared head and loops over the query heads
 * that read it, so the sums form in registers in a fixed order, without
 * atomics.  When that leaves too few workgroups to fill the chip (bf16/f16),
 * the group's query heads are split into equal runs whose fp32 sums go to the
 * workspace and a third kernel adds them in order; results are deterministic
 * either way.
 */
size_t mha_backward_gqa_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d_k, int d_v, int dtype);

int mha_forward_gqa(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int H_kv,
                    int Nq, int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                    void* stream);

int mha_backward_gqa(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk,
                     int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* mha_backward_gqa_timed -- as mha_backward_gqa, plus 4 events (as for
 * mha_backward_timed; events[2..3] span the dk/dv kernel and the kernel that
 * adds the runs, when there is one). */
int mha_backward_gqa_timed(const void* q, const void* k, const void* v, const void* out, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk,
                           int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * mha_proj_ln_forward -- the attention sublayer with its residual connection and
 * layer normalisation ([TP] "Residual Connections and Layer Normalization":
 * LayerNorm(x + Sublayer(x)), the normalisation after the residual addition;
 * [AD] "Add & Norm": normalised across each token's features; [AC] "A faithful
 * layer in code": x is the sublayer's query-side input):
 *
 *   z = x_q + mha_proj_forward(...)            per token, D features
 *   out = (z - mean(z)) / sqrt(var(z) + ln_eps) * ln_gamma + ln_beta
 *
 * with the biased variance (divided by D).  Arguments as mha_proj_forward,
 * plus ln_gamma, ln_beta [D] (nullable: 1 and 0; 16-byte aligned) and ln_eps
 * (finite, >= 0; nn.LayerNorm's default is 1e-5); b_O must then be 8-byte
 * aligned; the workspace must hold mha_proj_ln_workspace_bytes(...) bytes.
 * Supported: as mha_proj_forward.  The residual addition and the row
 * statistics run in the epilogue of the output projection (each output tile
 * keeps its share of every row's statistics in fp32 and the rows as fp16
 * differences from its own mean, scaled by a power of two that keeps them
 * inside fp16's range, in `out`); one more light kernel merges the
 * statistics and normalises the rows in place.  Range: the statistics are
 * fp32 sums of squares about each tile's mean, so rows whose features differ
 * from that mean by more than ~1e18 overflow them.  Returns MHA_OK or a
 * negative status.
 */
int mha_proj_ln_forward(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K, const void* W_V,
                        const void* W_O, const void* b_Q, const void* b_K, const void* b_V, const void* b_O,
                        const void* ln_gamma, const void* ln_beta, float ln_eps, void* out, int B, int Nq, int Nk,
                        int D, int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mha_proj_ln_forward_timed -- as mha_proj_ln_forward, plus 8 events and a plan:
 * events[0..5] and the plan as mha_proj_forward_timed (events[4..5] time the
 * output projection with the residual and statistics), events[6..7] the
 * normalisation pass.
 */
int mha_proj_ln_forward_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                              const void* W_V, const void* W_O, const void* b_Q, const void* b_K, const void* b_V,
                              const void* b_O, const void* ln_gamma, const void* ln_beta, float ln_eps, void* out,
                              int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int mask_kind,
                              const int32_t* key_lens, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream, void* const* events, int plan);

/*
 * mha_proj_ln_workspace_bytes -- device workspace mha_proj_ln_forward needs:
 * mha_proj_workspace_bytes plus per-row tile statistics (a 256-byte aligned
 * region of B*Nq*ceil(D/64) fp32 pairs).  Returns 0 for invalid sizes.
 */
size_t mha_proj_ln_workspace_bytes(int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int dtype);

/*
 * mha_proj_fused -- 1 if mha_proj_forward with these sizes runs as two
 * kernels (the Q/K/V projections fused with attention, then the output
 * projection), 0 if it runs as three (projections, attention, output
 * projection).  self_attention: nonzero when x_kv is NULL or equal to x_q.
 * The fused kernel takes D a multiple of 64, d_k == d_v == 64 (bf16 or
 * f16), and either self-attention with Nq == Nk <= 128 or cross-attention
 * with Nq <= 64 and Nk <= 128 -- sentence-length encoder, decoder and
 * encoder-decoder layers.  mha_proj_forward uses it for these except where
 * the three-kernel plan measured faster: cross-attention with D >= 768 over
 * 65..96 keys, and small batches, whose fused grid -- one workgroup per head
 * (taken as D / 64 heads) and per 128 token rows (self-attention) or two
 * sequences (cross-attention) -- has fewer than D / 8 (self) or 256 (cross)
 * workgroups.  MHA_PLAN_FUSED still runs the fused kernel there.  Pure
 * function of its arguments; no device access.
 */
int mha_proj_fused(int B, int Nq, int Nk, int D, int d_k, int d_v, int self_attention);

/*
 * mha_forward_block_queries -- queries per workgroup of the attention kernel
 * that mha_forward (and the attention step of mha_forward_lse,
 * mha_forward_gqa, mha_forward_strided, the three-kernel projection plan and
 * decoding with more rows than the decoding kernel takes) runs for B
 * sequences of H query heads with Nq queries: 4 for MHA_F32 (vector ALUs);
 * for MHA_BF16 / MHA_F16, 32 (one wave per workgroup, each wave reading its
 * own key/value tiles), 256 or 512 (four or eight waves sharing each
 * key/value tile staged in LDS).  The three give the same results bit for
 * bit; the choice follows how well each would use the chip ([TP] "The
 * Trade-Off: Quadratic Cost": the longer the sequence, the more the shared
 * tiles pay): at most 64 queries take 32; from 4096 queries with well-filled
 * 512-query blocks, 512; where 256-query blocks are well filled, 256; else 32
 * up to 2048 queries and 256 beyond.  The environment variable
 * MHA_ATTENTION_BLOCK=32, =256 or =512, read on every call, forces one of
 * them (for tests and measurement).  0 for invalid arguments.  Pure function
 * of its arguments and that variable; no device access.
 */
int mha_forward_block_queries(int B, int H, int Nq, int mask_kind, int dtype);

/*
 * Decoding against a key/value cache ([AD] "How predictions are generated, per
 * downstream task", "Translation and summarization (encoder-decoder)": during
 * generation the keys and values of the positions already produced are kept
 * and only the newest position is computed, and the cross-attention keys and
 * values are computed once from the encoder output; [TP] "Inference
 * (Autoregressive Loop)").  Query heads may share cache heads: multi-query and
 * grouped-query attention ([TP] "Limitations of the Original Design"; [ZS]
 * "Many heads, many subspaces").
 *
 *   q       [B, H, Nq, d_k]      the Nq newest positions of each sequence
 *   k_cache [B, H_kv, S, d_k]    key cache: S slots per (sequence, cache head)
 *   v_cache [B, H_kv, S, d_v]    value cache
 *   out     [B, H, Nq, d_v]      written; may not overlap the inputs
 *   cache_lens                   device int32[B] or NULL: sequence b has
 *                                L_b = clamp(cache_lens[b], 0, S) filled slots
 *                                (NULL: S), already including the Nq new
 *                                positions; slots >= L_b are never read
 *   mask_kind  MHA_MASK_CAUSAL   decoder self-attention: query i sits at
 *                                position L_b - Nq + i and sees the slots
 *                                j <= L_b - Nq + i (a query whose position is
 *                                negative sees none and gets zeros)
 *              MHA_MASK_NONE     cross-attention against a source's cache:
 *                                every query sees the L_b filled slots
 *
 * Query head h reads cache head h / (H / H_kv): each run of H / H_kv
 * consecutive query heads shares one cache head.  H_kv == H is ordinary
 * multi-head attention, H_kv == 1 multi-query attention.  Sizes: B, Nq,
 * S >= 0; 1 <= H_kv <= H with H a multiple of H_kv (else MHA_ERR_INVALID_ARG);
 * supported types and head sizes as for mha_forward, and S + 1024 slots of one
 * cache head must span less than 2^31 bytes.  Nq need not equal S and the
 * causal mask needs no Nq == S.
 *
 * The filled slots of all caches are shared out evenly over the GPU, so that
 * a step over few sequences or caches of unequal length still keeps every
 * compute unit busy; caches cut between several workers are merged by a
 * second kernel, which needs `workspace`: device memory of at least
 * mha_decode_workspace_bytes(...) bytes, 256-byte aligned, owned by the
 * caller, contents scratch (may be NULL when that size is 0).  Calls that
 * share a workspace must not run concurrently.  Returns MHA_OK or a negative
 * status.
 */
size_t mha_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int S, int d_k, int d_v, int dtype);

int mha_decode_forward(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                       int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                       float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mha_decode_forward_timed -- as mha_decode_forward, plus 4 events (see the
 * timed variants above): events[0..1] time the decoding kernel, events[2..3]
 * the merging kernel (left untouched when mha_decode_split is 0: then
 * events[0..1] time the attention kernel).
 */
int mha_decode_forward_timed(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                             int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events);

/*
 * mha_decode_forward_noalloc -- mha_decode_forward without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid hipMalloc.  The call itself
 * allocates nothing.  The scratch the decoding kernels need (the partial
 * softmax states and the wave spans of caches cut between workers, sized as
 * mha_decode_workspace_bytes reports) comes from an array of 16 MiB
 * (16777216 bytes) compiled into the library, one per GPU, held from the
 * library's first use on that GPU until the process ends; its address is
 * looked up once per device, on the first call with that device current.
 * Steps whose mha_decode_workspace_bytes exceeds 16 MiB are rejected with
 * MHA_ERR_UNSUPPORTED before anything is launched (at one new token per
 * sequence and H_kv == H that is above ~60,000 caches; use
 * mha_decode_forward with a workspace for those).  Nothing in the array
 * needs to start at zero: each call writes every state it reads.  All calls
 * on one GPU share that GPU's array, so calls that may overlap on one GPU
 * (different streams, or different threads without ordering) race and must
 * be serialised by the caller.  Arguments, validation, kernels and results
 * are otherwise those of mha_decode_forward; plans without the split kernel
 * (mha_decode_split == 0) use no scratch.
 */
int mha_decode_forward_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                               int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                               float scale, int dtype, void* stream);

/*
 * mha_decode_split -- how mha_decode_forward runs these sizes: the number of
 * workers (one wave each) the filled cache slots are shared out over by the
 * decoding kernel (bf16/f16, d_k == d_v == 64, at most 64 query rows
 * (H / H_kv) * Nq per cache head), or 0 when the call runs on the attention
 * kernels instead (fp32, or more query rows per cache head).  Pure function of
 * its arguments; 0 for invalid sizes.
 */
int mha_decode_split(int B, int H, int H_kv, int Nq, int S, int d_k, int d_v, int dtype);

/* Static description of a status code; never NULL. */
const char* mha_status_string(int status);

/* Message for the last failed call on the calling thread ("" if none): the
 * argument that was rejected, the workspace size that was needed, or the HIP
 * runtime's text for MHA_ERR_HIP.  The string is thread-local and stays valid
 * until that thread's next call into the library. */
const char* mha_last_error_message(void);

/* Same as mha_last_error_message (the name earlier versions exported). */
const char* mha_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H_ */
