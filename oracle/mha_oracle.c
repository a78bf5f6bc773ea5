/*
 * mha_oracle.c -- plain, slow, fp64 CPU oracle for multi-head scaled
 * dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the GPU
 * library, and the GPU library never calls it.
 *
 * Sources (web pages on "Attention Is All You Need"; section names as printed
 * on each page):
 *   [TP]  trishampatil.com, "Attention Is All You Need" (engineering explainer)
 *   [AC]  aicassindra.com, "Attention Is All You Need, in depth: ..."
 *   [ACI] aicomputerinstitute.com, grade-12 chapter "attention-all-you-need"
 *   [ZS]  zeroshotmind.com, "Attention Is All You Need"
 *   [AD]  alexdo.xyz, "Attention Is All You Need: The Transformer" (notes)
 *
 * What is computed, for every batch entry b, head h and query row i:
 *   1. raw score of query i against key j: the dot product q_i . k_j
 *      ([TP] "Scaled Dot-Product Attention: Step by Step", step 1);
 *   2. the score times `scale` (the caller passes 1/sqrt(d_k) for the pages'
 *      scaling, [TP] step 2 and "Why the sqrt(d_k) Scaling Exists");
 *   3. keys that may not be seen get a logit of -infinity, hence weight
 *      exactly 0: future keys j > i under the causal mask ([TP] "Why Masking
 *      Is Required"; [AD] "Masked Multi-Head Attention") and padded keys
 *      j >= len_b ([AD] "Two masks, not one"; [AC] "Pitfalls when reproducing
 *      the paper": padding masks keys, not queries);
 *   4. row-wise softmax over the visible keys ([TP] step 3);
 *   5. output row = sum_j weight_j * v_j ([TP] step 4).
 * Multi-head projection path ([TP] "Query / Key / Value Roles",
 * "Multi-Head Attention", "The Output Projection W^O"; [AC] code listing
 * "A faithful layer in code"): Q = x_q W_Q^T + b_Q, K = x_kv W_K^T + b_K,
 * V = x_kv W_V^T + b_V, head h uses feature columns [h*d, (h+1)*d), the head
 * outputs are concatenated head-major and out = O_cat W_O^T + b_O.  Weights use
 * the [out_features, in_features] layout of the listing's nn.Linear layers.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - softmax subtracts the row maximum before exponentiating (same value in
 *     exact arithmetic, avoids overflow);
 *   - a masked logit of -infinity is realised by leaving that key out of the
 *     sum, which gives the same weight (exactly 0) without -inf arithmetic;
 *   - a row with no visible key (only possible when len_b == 0) returns 0
 *     instead of the NaN the pages warn about ([AC] "Pitfalls");
 *   - key lengths are clamped to [0, Nk]; padded query rows are ordinary rows;
 *   - the causal mask is defined only for Nq == Nk (self-attention).
 *   - decoding against a cache (oracle_decode): the new queries are the last
 *     Nq positions of the filled cache, and a run of H / Hkv consecutive query
 *     heads shares one cache head.
 *   - residual + layer normalisation (oracle_mha_proj_ln): biased variance,
 *     eps an argument, inference (no dropout).
 *
 * Everything is fp64; inputs arrive as fp64 (bf16 and fp32 values convert
 * exactly).  Sums run in index order.  Threads split independent (b, h) pairs
 * or independent rows and never change the arithmetic of a single output.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

#define ORACLE_MASK_NONE 0
#define ORACLE_MASK_CAUSAL 1

/* ------------------------------------------------------------------------ */
/* Parallel loop over independent units.                                     */

typedef void (*unit_fn)(void *ctx, long unit, double *scratch);

struct pool_job {
    unit_fn fn;
    void *ctx;
    long nunits;
    int nthreads;
    int tid;
    long scratch_len;
    int failed;
};

static void *pool_worker(void *arg) {
    struct pool_job *job = (struct pool_job *)arg;
    double *scratch = NULL;
    if (job->scratch_len > 0) {
        scratch = (double *)malloc(sizeof(double) * (size_t)job->scratch_len);
        if (!scratch) {
            job->failed = 1;
            return NULL;
        }
    }
    for (long u = job->tid; u < job->nunits; u += job->nthreads) job->fn(job->ctx, u, scratch);
    free(scratch);
    return NULL;
}

static int parallel_for(long nunits, int nthreads, long scratch_len, unit_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nunits) nthreads = (int)(nunits > 0 ? nunits : 1);
    struct pool_job jobs[256];
    pthread_t threads[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct pool_job){fn, ctx, nunits, nthreads, t, scratch_len, 0};
        started[t] = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&threads[t], NULL, pool_worker, &jobs[t]) == 0;
    for (int t = 1; t < nthreads; ++t)
        if (!started[t]) pool_worker(&jobs[t]); /* run it inline instead */
    pool_worker(&jobs[0]);
    int failed = jobs[0].failed;
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(threads[t], NULL);
        failed |= jobs[t].failed;
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The method, one query row at a time.                                      */

/* Effective key length of batch entry b: key_lens[b] clamped to [0, Nk], or
 * Nk when no lengths are given. */
static int key_length(const int32_t *key_lens, int b, int Nk) {
    if (!key_lens) return Nk;
    int L = key_lens[b];
    if (L < 0) L = 0;
    if (L > Nk) L = Nk;
    return L;
}

/* May query i see key j?  Padding hides keys j >= L; the causal mask also
 * hides future keys j > i. */
static int key_visible(int i, int j, int L, int mask_kind) {
    if (j >= L) return 0;
    if (mask_kind == ORACLE_MASK_CAUSAL && j > i) return 0;
    return 1;
}

/* Steps 1 and 2: scale * (q . k), summed in index order. */
static double scaled_score(const double *q, const double *k, int dk, double scale) {
    double dot = 0.0;
    for (int c = 0; c < dk; ++c) dot += q[c] * k[c];
    return dot * scale;
}

/* Steps 1-5 for one query row.
 *   q      : d_k values of query i
 *   kbase  : key j starts at kbase + j*ldk (d_k values)
 *   vbase  : value j starts at vbase + j*ldv (d_v values)
 *   out    : d_v outputs
 *   w      : Nk slots; receives the attention weights of this row (0 where
 *            masked); may be scratch */
static void attend_row(const double *q, const double *kbase, long ldk, const double *vbase, long ldv,
                       int i, int Nk, int L, int mask_kind, int dk, int dv, double scale, double *out,
                       double *w) {
    int any = 0;
    double m = 0.0;
    for (int j = 0; j < Nk; ++j) {
        if (!key_visible(i, j, L, mask_kind)) {
            w[j] = 0.0;
            continue;
        }
        w[j] = scaled_score(q, kbase + (long)j * ldk, dk, scale);
        if (!any || w[j] > m) m = w[j];
        any = 1;
    }
    for (int c = 0; c < dv; ++c) out[c] = 0.0;
    if (!any) return; /* no visible key: output 0 (see header) */

    /* Step 3: softmax over the visible keys (row maximum subtracted). */
    double z = 0.0;
    for (int j = 0; j < Nk; ++j) {
        if (!key_visible(i, j, L, mask_kind)) continue;
        w[j] = exp(w[j] - m);
        z += w[j];
    }
    for (int j = 0; j < Nk; ++j)
        if (key_visible(i, j, L, mask_kind)) w[j] /= z;

    /* Step 4: weighted sum of the value rows. */
    for (int j = 0; j < Nk; ++j) {
        if (!key_visible(i, j, L, mask_kind)) continue;
        const double *vj = vbase + (long)j * ldv;
        for (int c = 0; c < dv; ++c) out[c] += w[j] * vj[c];
    }
}

static int check_dims(int B, int H, int Nq, int Nk, int dk, int dv, int mask_kind) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
    if (mask_kind != ORACLE_MASK_NONE && mask_kind != ORACLE_MASK_CAUSAL) return ORACLE_EINVAL;
    if (mask_kind == ORACLE_MASK_CAUSAL && Nq != Nk) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention on per-head tensors q [B,H,Nq,dk], k [B,H,Nk,dk], v [B,H,Nk,dv]. */

struct attn_ctx {
    const double *q, *k, *v;
    double *out, *weights;
    int B, H, Nq, Nk, dk, dv, mask_kind;
    const int32_t *key_lens;
    double scale;
};

static void attn_unit(void *vctx, long unit, double *scratch) {
    struct attn_ctx *c = (struct attn_ctx *)vctx;
    int b = (int)(unit / c->H);
    const double *qbh = c->q + unit * (long)c->Nq * c->dk;
    const double *kbh = c->k + unit * (long)c->Nk * c->dk;
    const double *vbh = c->v + unit * (long)c->Nk * c->dv;
    double *obh = c->out + unit * (long)c->Nq * c->dv;
    int L = key_length(c->key_lens, b, c->Nk);
    for (int i = 0; i < c->Nq; ++i) {
        double *w = c->weights ? c->weights + (unit * (long)c->Nq + i) * c->Nk : scratch;
        attend_row(qbh + (long)i * c->dk, kbh, c->dk, vbh, c->dv, i, c->Nk, L, c->mask_kind, c->dk,
                   c->dv, c->scale, obh + (long)i * c->dv, w);
    }
}

/* out [B,H,Nq,dv]; weights (nullable) [B,H,Nq,Nk] receives the softmax rows. */
int oracle_attention(const double *q, const double *k, const double *v, double *out, int B, int H,
                     int Nq, int Nk, int dk, int dv, int mask_kind, const int32_t *key_lens,
                     double scale, double *weights, int nthreads) {
    int st = check_dims(B, H, Nq, Nk, dk, dv, mask_kind);
    if (st) return st;
    if (!q || !k || !v || !out) return ORACLE_EINVAL;
    struct attn_ctx ctx = {q, k, v, out, weights, B, H, Nq, Nk, dk, dv, mask_kind, key_lens, scale};
    return parallel_for((long)B * H, nthreads, Nk > 0 ? Nk : 1, attn_unit, &ctx);
}

/* Steps 1-3 only: s [B,H,Nq,Nk] = scale * q.k for visible keys, -inf where
 * masked (the logits the pages feed to the softmax). */
int oracle_scores(const double *q, const double *k, double *s, int B, int H, int Nq, int Nk,
                  int dk, int mask_kind, const int32_t *key_lens, double scale) {
    int st = check_dims(B, H, Nq, Nk, dk, 1, mask_kind);
    if (st) return st;
    if (!q || !k || !s) return ORACLE_EINVAL;
    for (long unit = 0; unit < (long)B * H; ++unit) {
        int b = (int)(unit / H);
        int L = key_length(key_lens, b, Nk);
        for (int i = 0; i < Nq; ++i)
            for (int j = 0; j < Nk; ++j) {
                double *dst = s + (unit * Nq + i) * (long)Nk + j;
                if (key_visible(i, j, L, mask_kind))
                    *dst = scaled_score(q + (unit * Nq + i) * (long)dk,
                                        k + (unit * Nk + j) * (long)dk, dk, scale);
                else
                    *dst = -INFINITY;
            }
    }
    return ORACLE_OK;
}

/* Selected rows only: rows[3*r .. 3*r+2] = (b, h, i); out [nrows, dv]. */
struct rows_ctx {
    struct attn_ctx a;
    const int32_t *rows;
};

static void rows_unit(void *vctx, long r, double *scratch) {
    struct rows_ctx *c = (struct rows_ctx *)vctx;
    const struct attn_ctx *a = &c->a;
    int b = c->rows[3 * r], h = c->rows[3 * r + 1], i = c->rows[3 * r + 2];
    long bh = (long)b * a->H + h;
    int L = key_length(a->key_lens, b, a->Nk);
    attend_row(a->q + (bh * a->Nq + i) * (long)a->dk, a->k + bh * a->Nk * (long)a->dk, a->dk,
               a->v + bh * a->Nk * (long)a->dv, a->dv, i, a->Nk, L, a->mask_kind, a->dk, a->dv,
               a->scale, a->out + r * (long)a->dv, scratch);
}

int oracle_attention_rows(const double *q, const double *k, const double *v, double *out, int B,
                          int H, int Nq, int Nk, int dk, int dv, int mask_kind,
                          const int32_t *key_lens, double scale, int nrows, const int32_t *rows,
                          int nthreads) {
    int st = check_dims(B, H, Nq, Nk, dk, dv, mask_kind);
    if (st) return st;
    if (!q || !k || !v || !out || (nrows > 0 && !rows) || nrows < 0) return ORACLE_EINVAL;
    for (int r = 0; r < nrows; ++r)
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= H ||
            rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Nq)
            return ORACLE_EINVAL;
    struct rows_ctx ctx = {{q, k, v, out, NULL, B, H, Nq, Nk, dk, dv, mask_kind, key_lens, scale},
                           rows};
    return parallel_for(nrows, nthreads, Nk > 0 ? Nk : 1, rows_unit, &ctx);
}

/* ------------------------------------------------------------------------ */
/* Multi-head attention with projections.                                     */

/* y[m, r] = sum_c x[m, c] * W[r, c] (+ bias[r]) for m < M, r < R, c < D. */
struct linear_ctx {
    const double *x, *W, *bias;
    double *y;
    int R, D;
};

static void linear_unit(void *vctx, long m, double *scratch) {
    (void)scratch;
    struct linear_ctx *c = (struct linear_ctx *)vctx;
    const double *xm = c->x + m * (long)c->D;
    for (int r = 0; r < c->R; ++r) {
        const double *wr = c->W + (long)r * c->D;
        double acc = 0.0;
        for (int d = 0; d < c->D; ++d) acc += xm[d] * wr[d];
        if (c->bias) acc += c->bias[r];
        c->y[m * (long)c->R + r] = acc;
    }
}

static int linear(const double *x, const double *W, const double *bias, double *y, long M, int R,
                  int D, int nthreads) {
    struct linear_ctx ctx = {x, W, bias, y, R, D};
    return parallel_for(M, nthreads, 0, linear_unit, &ctx);
}

/* Per (b, h): attention over the head's column block of the projected rows.
 * Q [B*Nq, H*dk], K [B*Nk, H*dk], V [B*Nk, H*dv] row-major; O [B*Nq, H*dv]. */
struct heads_ctx {
    const double *Q, *K, *V;
    double *O;
    int H, Nq, Nk, dk, dv, mask_kind;
    const int32_t *key_lens;
    double scale;
};

static void heads_unit(void *vctx, long unit, double *scratch) {
    struct heads_ctx *c = (struct heads_ctx *)vctx;
    int b = (int)(unit / c->H), h = (int)(unit % c->H);
    long ldq = (long)c->H * c->dk, ldv = (long)c->H * c->dv;
    const double *kb = c->K + (long)b * c->Nk * ldq + (long)h * c->dk;
    const double *vb = c->V + (long)b * c->Nk * ldv + (long)h * c->dv;
    int L = key_length(c->key_lens, b, c->Nk);
    for (int i = 0; i < c->Nq; ++i) {
        const double *qi = c->Q + ((long)b * c->Nq + i) * ldq + (long)h * c->dk;
        double *oi = c->O + ((long)b * c->Nq + i) * ldv + (long)h * c->dv;
        attend_row(qi, kb, ldq, vb, ldv, i, c->Nk, L, c->mask_kind, c->dk, c->dv, c->scale, oi,
                   scratch);
    }
}

/* x_q [B,Nq,D]; x_kv [B,Nk,D] or NULL (self-attention: keys and values come
 * from x_q, Nk must equal Nq); W_Q, W_K [H*dk, D]; W_V [H*dv, D];
 * W_O [D, H*dv]; biases nullable; out [B,Nq,D]. */
int oracle_mha_proj(const double *x_q, const double *x_kv, const double *W_Q, const double *W_K,
                    const double *W_V, const double *W_O, const double *b_Q, const double *b_K,
                    const double *b_V, const double *b_O, double *out, int B, int Nq, int Nk, int D,
                    int H, int dk, int dv, int mask_kind, const int32_t *key_lens, double scale,
                    int nthreads) {
    int st = check_dims(B, H, Nq, Nk, dk, dv, mask_kind);
    if (st) return st;
    if (D <= 0 || !x_q || !W_Q || !W_K || !W_V || !W_O || !out) return ORACLE_EINVAL;
    if (!x_kv) {
        if (Nk != Nq) return ORACLE_EINVAL;
        x_kv = x_q;
    }
    size_t nq = (size_t)B * Nq, nk = (size_t)B * Nk;
    double *Q = (double *)malloc(sizeof(double) * (nq * H * dk + 1));
    double *K = (double *)malloc(sizeof(double) * (nk * H * dk + 1));
    double *V = (double *)malloc(sizeof(double) * (nk * H * dv + 1));
    double *O = (double *)malloc(sizeof(double) * (nq * H * dv + 1));
    if (!Q || !K || !V || !O) {
        free(Q);
        free(K);
        free(V);
        free(O);
        return ORACLE_ENOMEM;
    }
    st = linear(x_q, W_Q, b_Q, Q, (long)nq, H * dk, D, nthreads);
    if (!st) st = linear(x_kv, W_K, b_K, K, (long)nk, H * dk, D, nthreads);
    if (!st) st = linear(x_kv, W_V, b_V, V, (long)nk, H * dv, D, nthreads);
    if (!st) {
        struct heads_ctx hc = {Q, K, V, O, H, Nq, Nk, dk, dv, mask_kind, key_lens, scale};
        st = parallel_for((long)B * H, nthreads, Nk > 0 ? Nk : 1, heads_unit, &hc);
    }
    if (!st) st = linear(O, W_O, b_O, out, (long)nq, D, H * dv, nthreads);
    free(Q);
    free(K);
    free(V);
    free(O);
    return st;
}

/* ------------------------------------------------------------------------ */
/* One decoding step against a key/value cache.                               */
/*
 * [AD] "How predictions are generated, per downstream task", "Translation and
 * summarization (encoder-decoder)": during generation the keys and values of
 * the positions already produced are kept (the KV cache) and only the newest
 * position is computed; the cross-attention keys and values are computed once
 * from the encoder output.  [TP] "Inference (Autoregressive Loop)": one new
 * token per step; [AD] "This parallelism is a training-time property": the
 * cache saves recomputing past keys and values, it does not change the result.
 *
 * q [B,H,Nq,dk]      the Nq newest positions of each sequence;
 * k [B,Hkv,S,dk]     key cache, S slots per (b, cache head);
 * v [B,Hkv,S,dv]     value cache;
 * cache_lens [B]     filled slots L_b = clamp(cache_lens[b], 0, S) (NULL: S);
 *                    slots >= L_b are never read.
 * mask_kind CAUSAL   decoder self-attention: the cache already holds the new
 *                    positions, query i sits at position p = L_b - Nq + i and
 *                    sees keys j <= p; a query with p < 0 sees none (output 0).
 * mask_kind NONE     cross-attention against a source's cache: every query
 *                    sees the keys j < L_b.
 * Shared key/value heads ([TP] "Limitations of the Original Design", on the
 * quadratic parameter count: multi-query and grouped-query attention share the
 * key/value projections across heads; [ZS] "Many heads, many subspaces": they
 * are multi-head attention with key/value heads shared): H must be a multiple
 * of Hkv and query head h reads cache head h / (H / Hkv), so each run of
 * H / Hkv consecutive query heads shares one cache head.  Hkv == H is ordinary
 * multi-head attention, Hkv == 1 multi-query attention.
 */
struct decode_ctx {
    const double *q, *k, *v;
    double *out;
    int B, H, Hkv, Nq, S, dk, dv, mask_kind;
    const int32_t *cache_lens;
    double scale;
};

/* Number of cache slots query i may see when the cache holds L entries: all
 * of them for cross-attention, those up to its own position when causal. */
static int decode_visible_keys(int i, int Nq, int L, int mask_kind) {
    if (mask_kind != ORACLE_MASK_CAUSAL) return L;
    int p = L - Nq + i; /* position of query i in its sequence */
    if (p < 0) return 0;
    return p + 1;
}

static void decode_unit(void *vctx, long unit, double *scratch) {
    struct decode_ctx *c = (struct decode_ctx *)vctx;
    int b = (int)(unit / c->H), h = (int)(unit % c->H);
    int g = h / (c->H / c->Hkv); /* cache head shared by query head h */
    long bg = (long)b * c->Hkv + g;
    const double *kc = c->k + bg * c->S * (long)c->dk;
    const double *vc = c->v + bg * c->S * (long)c->dv;
    int L = key_length(c->cache_lens, b, c->S);
    for (int i = 0; i < c->Nq; ++i) {
        int n = decode_visible_keys(i, c->Nq, L, c->mask_kind);
        /* keys 0..n-1 are exactly the visible ones: attend to all of them */
        attend_row(c->q + (unit * c->Nq + i) * (long)c->dk, kc, c->dk, vc, c->dv, i, n, n,
                   ORACLE_MASK_NONE, c->dk, c->dv, c->scale, c->out + (unit * c->Nq + i) * (long)c->dv,
                   scratch);
    }
}

/* out [B,H,Nq,dv]. */
int oracle_decode(const double *q, const double *k, const double *v, double *out, int B, int H,
                  int Hkv, int Nq, int S, int dk, int dv, int mask_kind, const int32_t *cache_lens,
                  double scale, int nthreads) {
    if (B < 0 || H < 0 || Nq < 0 || S < 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
    if (mask_kind != ORACLE_MASK_NONE && mask_kind != ORACLE_MASK_CAUSAL) return ORACLE_EINVAL;
    if (Hkv <= 0 || Hkv > H || H % Hkv != 0) return ORACLE_EINVAL;
    if (!q || !k || !v || !out) return ORACLE_EINVAL;
    struct decode_ctx ctx = {q, k, v, out, B, H, Hkv, Nq, S, dk, dv, mask_kind, cache_lens, scale};
    return parallel_for((long)B * H, nthreads, S > 0 ? S : 1, decode_unit, &ctx);
}

/* ------------------------------------------------------------------------ */
/* Residual connection and layer normalisation after the attention sublayer.  */
/*
 * [TP] "Residual Connections and Layer Normalization": every sublayer is
 * wrapped as LayerNorm(x + Sublayer(x)), the normalisation after the residual
 * addition (post-LN); layer normalisation normalises each token on its own,
 * across its feature dimension.  [AD] "Add & Norm": add is the residual
 * connection, norm normalises across the feature dimension of each token.
 * [AC] "A faithful layer in code": the encoder layer applies the norm to
 * x + attention(x), x being the sublayer's (query-side) input; its counting
 * section gives each norm a scale and a shift per feature.
 *
 * Readings (the pages give no formula for the normalisation itself): the row
 * z of D features becomes (z - mean) / sqrt(var + eps) * gamma + beta with the
 * mean and the biased variance (divided by D) of the row, as the listing's
 * nn.LayerNorm layers compute; eps is an argument (that layer's default is
 * 1e-5); gamma and beta NULL mean 1 and 0; dropout is the identity (inference).
 *
 * x_q, W_*, b_*, mask, lengths and scale as in oracle_mha_proj; out [B,Nq,D]
 * = LayerNorm(x_q + MHA(x_q, x_kv)).
 */
static void layer_norm_row(const double *z, const double *gamma, const double *beta, double eps, int D,
                           double *y) {
    double mean = 0.0;
    for (int c = 0; c < D; ++c) mean += z[c];
    mean /= D;
    double var = 0.0;
    for (int c = 0; c < D; ++c) var += (z[c] - mean) * (z[c] - mean);
    var /= D;
    const double rstd = 1.0 / sqrt(var + eps);
    for (int c = 0; c < D; ++c) {
        const double g = gamma ? gamma[c] : 1.0, b = beta ? beta[c] : 0.0;
        y[c] = (z[c] - mean) * rstd * g + b;
    }
}

int oracle_mha_proj_ln(const double *x_q, const double *x_kv, const double *W_Q, const double *W_K,
                       const double *W_V, const double *W_O, const double *b_Q, const double *b_K,
                       const double *b_V, const double *b_O, const double *gamma, const double *beta,
                       double eps, double *out, int B, int Nq, int Nk, int D, int H, int dk, int dv,
                       int mask_kind, const int32_t *key_lens, double scale, int nthreads) {
    if (!(eps >= 0.0)) return ORACLE_EINVAL;
    int st = oracle_mha_proj(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H, dk,
                             dv, mask_kind, key_lens, scale, nthreads);
    if (st) return st;
    double *z = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    if (!z) return ORACLE_ENOMEM;
    for (long m = 0; m < (long)B * Nq; ++m) {
        for (int c = 0; c < D; ++c) z[c] = x_q[m * D + c] + out[m * D + c]; /* the residual connection */
        layer_norm_row(z, gamma, beta, eps, D, out + m * D);
    }
    free(z);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Training: the row statistics of the forward pass and the backward pass.    */
/*
 * [TP] "Training (Teacher Forcing + Masking)": the pages' main use of the path is
 * parallel training, in which gradients flow back through every layer; [AD]
 * "One forward pass covers the whole sequence".  The pages give no gradient
 * formulas; these are the derivatives of the forward definition above,
 * written out: with P the softmax weights of a row (0 at masked keys) and dO
 * the gradient of a scalar loss with respect to the output rows,
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - D_i),   D_i = sum_j P_ij dP_ij = dO_i . out_i
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_i dS_ij q_i
 * (the chain rule through out = P V, the softmax Jacobian
 * diag(P) - P P^T, and s = scale q.k).  Masked keys have P = 0, so they get no
 * gradient, and a row with no visible key contributes nothing.
 *
 * oracle_attention_lse: lse [B,H,Nq] = log sum_j exp(scale q_i.k_j) over the
 * visible keys (natural logarithm; -inf for a row with no visible key), the
 * row statistic from which the backward pass recomputes P = exp(s - lse).
 */
struct lse_ctx {
    const double *q, *k;
    double *lse;
    int H, Nq, Nk, dk, mask_kind;
    const int32_t *key_lens;
    double scale;
};

static void lse_unit(void *vctx, long unit, double *scratch) {
    (void)scratch;
    struct lse_ctx *c = (struct lse_ctx *)vctx;
    int b = (int)(unit / c->H);
    int L = key_length(c->key_lens, b, c->Nk);
    for (int i = 0; i < c->Nq; ++i) {
        const double *qi = c->q + (unit * c->Nq + i) * (long)c->dk;
        double m = -INFINITY;
        for (int j = 0; j < c->Nk; ++j)
            if (key_visible(i, j, L, c->mask_kind)) {
                double s = scaled_score(qi, c->k + (unit * c->Nk + j) * (long)c->dk, c->dk, c->scale);
                if (s > m) m = s;
            }
        double z = 0.0;
        for (int j = 0; j < c->Nk; ++j)
            if (key_visible(i, j, L, c->mask_kind))
                z += exp(scaled_score(qi, c->k + (unit * c->Nk + j) * (long)c->dk, c->dk, c->scale) - m);
        c->lse[unit * c->Nq + i] = (m == -INFINITY) ? -INFINITY : m + log(z);
    }
}

int oracle_attention_lse(const double *q, const double *k, double *lse, int B, int H, int Nq, int Nk, int dk,
                         int mask_kind, const int32_t *key_lens, double scale, int nthreads) {
    int st = check_dims(B, H, Nq, Nk, dk, 1, mask_kind);
    if (st) return st;
    if (!q || !k || !lse) return ORACLE_EINVAL;
    struct lse_ctx ctx = {q, k, lse, H, Nq, Nk, dk, mask_kind, key_lens, scale};
    return parallel_for((long)B * H, nthreads, 0, lse_unit, &ctx);
}

/* Gradients of a scalar loss with respect to q, k, v, given dout = dLoss/dout,
 * per (b, h) on per-head tensors as in oracle_attention. */
struct bwd_ctx {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    int H, Nq, Nk, dkd, dvd, mask_kind;
    const int32_t *key_lens;
    double scale;
};

static void bwd_unit(void *vctx, long unit, double *scratch) {
    struct bwd_ctx *c = (struct bwd_ctx *)vctx;
    int b = (int)(unit / c->H);
    int L = key_length(c->key_lens, b, c->Nk);
    const int Nq = c->Nq, Nk = c->Nk, dkd = c->dkd, dvd = c->dvd;
    const double *q = c->q + unit * (long)Nq * dkd, *k = c->k + unit * (long)Nk * dkd;
    const double *v = c->v + unit * (long)Nk * dvd, *dout = c->dout + unit * (long)Nq * dvd;
    double *dq = c->dq + unit * (long)Nq * dkd, *dk = c->dk + unit * (long)Nk * dkd;
    double *dv = c->dv + unit * (long)Nk * dvd;
    double *w = scratch;             /* Nk weights of the current row */
    double *out = scratch + Nk;      /* dvd outputs of the current row */
    for (long x = 0; x < (long)Nq * dkd; ++x) dq[x] = 0.0;
    for (long x = 0; x < (long)Nk * dkd; ++x) dk[x] = 0.0;
    for (long x = 0; x < (long)Nk * dvd; ++x) dv[x] = 0.0;
    for (int i = 0; i < Nq; ++i) {
        /* forward for row i: weights P_i. and out_i */
        attend_row(q + (long)i * dkd, k, dkd, v, dvd, i, Nk, L, c->mask_kind, dkd, dvd, c->scale, out, w);
        double D = 0.0;
        for (int e = 0; e < dvd; ++e) D += dout[(long)i * dvd + e] * out[e];
        for (int j = 0; j < Nk; ++j) {
            if (!key_visible(i, j, L, c->mask_kind)) continue;
            const double p = w[j];
            double dp = 0.0;
            for (int e = 0; e < dvd; ++e) {
                dv[(long)j * dvd + e] += p * dout[(long)i * dvd + e];
                dp += dout[(long)i * dvd + e] * v[(long)j * dvd + e];
            }
            const double ds = p * (dp - D);
            for (int e = 0; e < dkd; ++e) {
                dq[(long)i * dkd + e] += c->scale * ds * k[(long)j * dkd + e];
                dk[(long)j * dkd + e] += c->scale * ds * q[(long)i * dkd + e];
            }
        }
    }
}

int oracle_attention_backward(const double *q, const double *k, const double *v, const double *dout, double *dq,
                              double *dk, double *dv, int B, int H, int Nq, int Nk, int dkd, int dvd,
                              int mask_kind, const int32_t *key_lens, double scale, int nthreads) {
    int st = check_dims(B, H, Nq, Nk, dkd, dvd, mask_kind);
    if (st) return st;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORACLE_EINVAL;
    struct bwd_ctx ctx = {q, k, v, dout, dq, dk, dv, H, Nq, Nk, dkd, dvd, mask_kind, key_lens, scale};
    return parallel_for((long)B * H, nthreads, (long)Nk + dvd + 1, bwd_unit, &ctx);
}
