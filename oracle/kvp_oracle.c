/*
 * kvp_oracle.c -- plain, slow, fp64 reference for attention against a key-value cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * file; only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * do.  It shares no header, helper, table or constant with the HIP path.
 *
 * Every function is the plain definition written out in scalar double loops, summing in
 * index order.  No blocking, fusion or reordering beyond what each definition states.
 *
 * Pages cited (by title and section):
 *   [CHAP]  "Tornar a inferencia barata: KV cache, batching e quantizacao" (neuralialabs
 *           chapter, pt; ja translation alongside) -- KV cache, prefill vs decode,
 *           cache-size formula, grouped-query attention.
 *   [KVES]  "La cache de claves y valores: cuanto cuesta cada token" (gustavoai lesson) --
 *           sections "Las claves y los valores de una posicion no cambian" and
 *           "Lo que cuesta un token, con cache y sin ella".
 *   [XF]    chatgpz.de "Aufmerksamkeit" feed, xformers demo: "4. Variable-length packed
 *           batch" and "5. Grouped-query attention (5-D BMGHK format)".
 *   [LIN]   same feed, linear-attention post: the TraditionalAttention module
 *           (softmax(Q K^T / sqrt(d_k)) V).
 *   [FLASH] same feed, FlashAttention post: "Was ist der mathematische Aspekt von Softmax?"
 *           (partial softmax blocks merged by rescaling with e^(m_local - m_global)).
 *   [PAGED] same feed, paged-attention article: SECTION 3 "Copy-on-Write: Shared System
 *           Prompts".
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------------------
 * One attention row, the plain definition.  [LIN] TraditionalAttention: scores are the
 * dot products q.k_j divided by sqrt(d_k) (here: multiplied by `scale`), a softmax over
 * the row, then the weighted sum of the value rows.  [KVES] "Las claves y los valores ...":
 * the output row of position t uses its own query against the t cached keys and values.
 *
 *   s_j = scale * sum_c q_c k_{j,c}
 *   m   = max_j s_j,  e_j = exp(s_j - m),  Z = sum_j e_j,  p_j = e_j / Z
 *   o_c = sum_j p_j v_{j,c}
 *
 * K row j starts at K + j*kstride, V row j at V + j*vstride.  n >= 1.
 * If p_out is not NULL it receives the n probabilities.
 * ------------------------------------------------------------------------------------- */
void orc_attention_row(int d, int n, const double *q, const double *K, long kstride,
                       const double *V, long vstride, double scale, double *out,
                       double *p_out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += q[c] * K[(long)j * kstride + c];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    double Z = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    for (int j = 0; j < n; ++j)
        s[j] = s[j] / Z;
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
            acc += s[j] * V[(long)j * vstride + c];
        out[c] = acc;
    }
    if (p_out)
        for (int j = 0; j < n; ++j)
            p_out[j] = s[j];
    free(s);
}

/* Grouped-query head map.  [CHAP] GQA passage: each key-value head serves a group of
 * query heads; [XF] section 5 lays q out as (B, M, G, Hq/G, K) with k/v (B, M, G, 1, K),
 * so flattened query head h = g*(Hq/G) + i reads key-value head g = h / (Hq/Hkv). */
int orc_kv_head(int h, int Hq, int Hkv)
{
    return h / (Hq / Hkv);
}

/* ---------------------------------------------------------------------------------------
 * Decode against a cache.  [CHAP] decode loop: the model is fed one token and its query
 * attends over every cached key; [KVES] four-step token recipe: k_t, v_t are appended to
 * the end of each head's cache (step 2) before the attention row over the whole cache
 * (step 3), so the new position looks at all earlier positions and at itself.
 *
 * The caller has already placed the new token's k, v at position ctx[b]-1, so the row for
 * request b attends over positions 0 .. ctx[b]-1.
 *   q   [B][Hq][d]          K, V  [B][Hkv][Lmax][d]        out [B][Hq][d]
 * ------------------------------------------------------------------------------------- */
void orc_decode_gqa(int B, int Hq, int Hkv, int d, int Lmax, const int *ctx,
                    const double *q, const double *K, const double *V, double scale,
                    double *out)
{
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int g = orc_kv_head(h, Hq, Hkv);
            long base = (((long)b * Hkv + g) * Lmax) * d;
            orc_attention_row(d, ctx[b], q + ((long)b * Hq + h) * d, K + base, d, V + base, d,
                              scale, out + ((long)b * Hq + h) * d, NULL);
        }
}

/* ---------------------------------------------------------------------------------------
 * Full recompute, the slow path.  [CHAP] opening: re-run the whole sequence for every
 * token, building the n x n attention matrix; [KVES] "Lo que cuesta un token": the code
 * computes the whole t x t grid of scores and masks it afterwards.  The causal mask puts
 * -inf on column j > i of row i.  Here the n x n matrix is formed in full, then masked,
 * then each row goes through the softmax and the value product.
 *   q [n][Hq][d]   k, v [n][Hkv][d]   out [n][Hq][d]
 * ------------------------------------------------------------------------------------- */
void orc_full_causal(int n, int Hq, int Hkv, int d, const double *q, const double *k,
                     const double *v, double scale, double *out)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)n * (size_t)n);
    for (int h = 0; h < Hq; ++h) {
        int g = orc_kv_head(h, Hq, Hkv);
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += q[((long)i * Hq + h) * d + c] * k[((long)j * Hkv + g) * d + c];
                S[(long)i * n + j] = scale * acc;
            }
        for (int i = 0; i < n; ++i)
            for (int j = i + 1; j < n; ++j)
                S[(long)i * n + j] = -INFINITY;
        for (int i = 0; i < n; ++i) {
            double *row = S + (long)i * n;
            double m = -INFINITY;
            for (int j = 0; j < n; ++j)
                if (row[j] > m)
                    m = row[j];
            double Z = 0.0;
            for (int j = 0; j < n; ++j) {
                row[j] = exp(row[j] - m); /* exp(-inf) = 0 on masked entries */
                Z += row[j];
            }
            for (int j = 0; j < n; ++j)
                row[j] /= Z;
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j)
                    acc += row[j] * v[((long)j * Hkv + g) * d + c];
                out[((long)i * Hq + h) * d + c] = acc;
            }
        }
    }
    free(S);
}

/* ---------------------------------------------------------------------------------------
 * Several new query rows per request against its cache (chunked prefill into an existing
 * prefix; verification of gamma drafted tokens).  [CHAP] speculative-decoding section:
 * checking a proposed run of gamma tokens is one forward pass over gamma positions, a
 * matrix-matrix product; [KVES] prompt paragraph: the rows of a stretch of known tokens
 * are computed in one pass, each by the same causal mask, and leave one cached row per
 * token; [PAGED] copy-on-write section: requests continue from shared prefix blocks with
 * their own tokens.  Reading: the m new rows of request b are the last m positions of its
 * context, ctx[b] - m .. ctx[b] - 1, already in the cache, and each attends to every
 * position up to and including its own -- row i over positions 0 .. ctx[b] - m + i.
 *   q   [T][Hq][d] packed, request b's rows cu[b] .. cu[b+1]-1
 *   K, V  [B][Hkv][Lmax][d]        out [T][Hq][d]
 * ------------------------------------------------------------------------------------- */
void orc_chunk_attention(int B, int Hq, int Hkv, int d, int Lmax, const int *ctx,
                         const int *cu, const double *q, const double *K, const double *V,
                         double scale, double *out)
{
    for (int b = 0; b < B; ++b) {
        int m = cu[b + 1] - cu[b];
        int first = ctx[b] - m; /* position of the first new row */
        for (int i = 0; i < m; ++i)
            for (int h = 0; h < Hq; ++h) {
                int g = orc_kv_head(h, Hq, Hkv);
                long base = (((long)b * Hkv + g) * Lmax) * d;
                long row = (long)cu[b] + i;
                orc_attention_row(d, first + i + 1, q + (row * Hq + h) * d, K + base, d, V + base, d,
                                  scale, out + (row * Hq + h) * d, NULL);
            }
    }
}

/* ---------------------------------------------------------------------------------------
 * Packed variable-length prefill.  [XF] section 4: sequences of different lengths are
 * packed into one token axis with no padding; a block-diagonal mask lets a token attend
 * only inside its own sequence, and the causal variant additionally hides later tokens of
 * that sequence.  Segment s covers packed rows cu[s] .. cu[s+1]-1.
 *   q [T][Hq][d]   k, v [T][Hkv][d]   out [T][Hq][d]     causal: 1 or 0
 * ------------------------------------------------------------------------------------- */
void orc_varlen_prefill(int T, int Hq, int Hkv, int d, const double *q, const double *k,
                        const double *v, const int *cu, int nseg, int causal, double scale,
                        double *out)
{
    (void)T;
    for (int s = 0; s < nseg; ++s) {
        int a = cu[s], n = cu[s + 1] - cu[s];
        for (int i = 0; i < n; ++i)
            for (int h = 0; h < Hq; ++h) {
                int g = orc_kv_head(h, Hq, Hkv);
                int nk = causal ? i + 1 : n;
                orc_attention_row(d, nk, q + ((long)(a + i) * Hq + h) * d,
                                  k + ((long)a * Hkv + g) * d, (long)Hkv * d,
                                  v + ((long)a * Hkv + g) * d, (long)Hkv * d, scale,
                                  out + ((long)(a + i) * Hq + h) * d, NULL);
            }
    }
}

/* ---------------------------------------------------------------------------------------
 * Softmax over a block of keys, kept unnormalised.  [FLASH] "Was ist der mathematische
 * Aspekt von Softmax?": each block's softmax is computed on its own while the block's
 * row maximum and its sum of exponentials are kept.
 *   m = max_{j in [j0,j1)} s_j,  l = sum_j e^(s_j - m),  o_c = sum_j e^(s_j - m) v_{j,c}
 * ------------------------------------------------------------------------------------- */
void orc_partial(int d, int j0, int j1, const double *q, const double *K, long kstride,
                 const double *V, long vstride, double scale, double *m_out, double *l_out,
                 double *o_out)
{
    int n = j1 - j0;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += q[c] * K[(long)(j0 + j) * kstride + c];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
            acc += s[j] * V[(long)(j0 + j) * vstride + c];
        o_out[c] = acc;
    }
    *m_out = m;
    *l_out = l;
    free(s);
}

/* Merge of block partials.  [FLASH] same section: when two blocks are merged, numerator
 * and denominator of each are scaled by e^(block max - global max), then summed.
 *   M = max_i m_i,   L = sum_i l_i e^(m_i - M),   out_c = (sum_i o_{i,c} e^(m_i - M)) / L
 * Partials are merged in index order i = 0 .. nparts-1.   o is [nparts][d]. */
void orc_merge(int d, int nparts, const double *m, const double *l, const double *o,
               double *out)
{
    double M = -INFINITY;
    for (int i = 0; i < nparts; ++i)
        if (m[i] > M)
            M = m[i];
    double L = 0.0;
    for (int i = 0; i < nparts; ++i)
        L += l[i] * exp(m[i] - M);
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = 0; i < nparts; ++i)
            acc += o[(long)i * d + c] * exp(m[i] - M);
        out[c] = acc / L;
    }
}

/* [CHAP] cache-size passage: per token, every layer stores one key and one value vector
 * per key-value head, hence 2 * L * H_kv * d * bytes per element. */
long long orc_kv_bytes_per_token(int L, int Hkv, int d, int elem_bytes)
{
    return 2LL * L * Hkv * d * elem_bytes;
}
