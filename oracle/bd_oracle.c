/*
 * CPU oracle for one block-diffusion denoising step and its speculative
 * verify / append companion.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that
 * the GPU library is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may build, load or call it;
 * the GPU library never does, and the two share no code.
 *
 * Everything is computed in double precision with plain loops: no BLAS,
 * no intrinsics, no fast-math.  bf16 inputs (raw 16-bit patterns) and
 * fp32 inputs are widened to double exactly.
 *
 * Sources (web pages, cited by title and section):
 *  [FD]  "Fast-dVLM: block diffusion ..." write-up (itsolotime.com),
 *        section 4.1 (causal-context attention: noisy block attends to
 *        itself bidirectionally and to every earlier clean position incl.
 *        vision; clean tokens stay causal), section 5.1 (each block opens
 *        with an AR step), section 5.3 (linear self-speculative decoding:
 *        bidirectional draft, causal verify, accept the longest matching
 *        prefix, crop the KV cache).
 *  [FD2] Fast-dVLM summary page (signal-papers), Fig. 3 caption
 *        (M_N2N is block-diagonal; vision tokens only in the clean stream).
 *  [DV]  "DiffusionVL" notes (papernotes.org), "cached block decoding"
 *        design item and Algorithm 1 as restated there: confidence is the
 *        model probability of the chosen token; static commit takes the
 *        k = min(ceil(D/S), |M|) most confident masked positions; the
 *        dynamic rule also commits every masked position whose confidence
 *        is greater than tau; committed tokens stay as context; a finished
 *        block joins the KV cache.
 *
 * Readings where the pages are silent (each also listed in the design
 * notes): scale 1/sqrt(d) is passed in; GQA head h uses KV head
 * h / (Hq/Hkv); Q and K are already position-encoded; the greedy token is
 * the argmax with the lowest index on ties; "greater than tau" is strict;
 * positions are ranked by (confidence desc, index asc).  The commit decision
 * is taken on the fp64 confidences themselves (the rule is stated on the
 * model's probabilities); tau is compared as given, in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define BDO_F32 0
#define BDO_BF16 1
#define BDO_BIDIR 0
#define BDO_CAUSAL 1
#define BDO_QUAD 2  /* quadratic self-speculative block: B draft slots + B groups of mask slots */

#define BDO_FP8 2  /* OCP FP8 E4M3 ("e4m3fn") */

/* OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities. */
static double fp8_e4m3(uint8_t b) {
    const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

static double widen(const void *base, int dtype, size_t idx) {
    if (dtype == BDO_F32) return (double)((const float *)base)[idx];
    if (dtype == BDO_FP8) return fp8_e4m3(((const uint8_t *)base)[idx]);
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int bdo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (>= 1). */
void bdo_set_num_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}

/*
 * Block attention ([FD] 4.1, 5.3; [FD2] Fig. 3).
 *
 * Key sequence of item n: positions 0..P-1 come from the frozen cache,
 * positions P..P+D-1 are this step's block slots 0..D-1.
 * Query (slot i, head h) may attend to key position j when
 *   j < P                      (every earlier clean position, vision included), or
 *   BIDIR:  P <= j < P + D     (the whole current block), or
 *   CAUSAL: P <= j <= P + i    (the block up to and including itself).
 * o = sum_j w_j v_j / sum_j w_j,  w_j = exp(s_j - max s),  s_j = scale * <q, k_j>.
 *
 * Layouts: q [n][D][Hq][d], k_blk/v_blk [n][D][Hkv][d],
 * k_cache and v_cache [n][Hkv][cap][d],
 * out [n][D][Hq][d] double.
 */
static void attention_impl(int n, int D, int Hq, int Hkv, int d, int cap, int q_dtype, int kv_dtype,
                           int mode, int B, double scale, const void *q, const void *k_blk, const void *v_blk,
                           const void *k_cache, const void *v_cache, const float *k_scale,
                           const float *v_scale, const int32_t *prefix_len, double *out);

void bdo_attention(int n, int D, int Hq, int Hkv, int d, int cap, int dtype, int mode,
                   double scale, const void *q, const void *k_blk, const void *v_blk,
                   const void *k_cache, const void *v_cache, const int32_t *prefix_len,
                   double *out) {
    attention_impl(n, D, Hq, Hkv, d, cap, dtype, dtype, mode, 0, scale, q, k_blk, v_blk, k_cache, v_cache,
                   NULL, NULL, prefix_len, out);
}

/*
 * The same block attention with an FP8 KV cache: queries bf16, every key and
 * value (cache and block) an OCP E4M3 byte times the fp32 scale of its
 * (item, KV head), k_scale / v_scale [n][Hkv]:
 *   k_j = e4m3(K_j) * k_scale[n][g],  v_j = e4m3(V_j) * v_scale[n][g].
 */
void bdo_attention_fp8kv(int n, int D, int Hq, int Hkv, int d, int cap, int mode, double scale,
                         const void *q, const void *k_blk, const void *v_blk, const void *k_cache,
                         const void *v_cache, const float *k_scale, const float *v_scale,
                         const int32_t *prefix_len, double *out) {
    attention_impl(n, D, Hq, Hkv, d, cap, BDO_BF16, BDO_FP8, mode, 0, scale, q, k_blk, v_blk, k_cache, v_cache,
                   k_scale, v_scale, prefix_len, out);
}

static int quad_slots(int B);

/* The quadratic self-speculative mask (bdo_attention_quad) over an FP8 KV cache. */
void bdo_attention_quad_fp8kv(int n, int B, int Hq, int Hkv, int d, int cap, double scale, const void *q,
                              const void *k_blk, const void *v_blk, const void *k_cache, const void *v_cache,
                              const float *k_scale, const float *v_scale, const int32_t *prefix_len,
                              double *out) {
    attention_impl(n, quad_slots(B), Hq, Hkv, d, cap, BDO_BF16, BDO_FP8, BDO_QUAD, B, scale, q, k_blk, v_blk,
                   k_cache, v_cache, k_scale, v_scale, prefix_len, out);
}

/*
 * Quadratic self-speculative attention ([FD] 5.3, the quadratic variant;
 * [FD] Fig. 6 and section 9.3 on its kernel).  One forward pass both
 * verifies a block of B draft tokens and proposes the next block for every
 * possible acceptance length: the B drafts are expanded into B groups of B
 * tokens, group g holding draft tokens 0..g-1 (the hypothesis that they are
 * accepted) followed by B - g mask tokens that draft what comes next.
 * Within a group the drafts attend causally and the mask tokens attend to
 * the whole group; groups do not see each other; everything sees the
 * cache.  (The pages state the B x B expansion and a non-standard mask;
 * this mask is the reading of that expansion: causal verify plus
 * bidirectional draft, per hypothesis.)
 *
 * A draft token's keys and values are the same in every group that holds
 * it (its context, the cache and the drafts before it, is the same), so
 * the slots here hold each draft once: slot t < B is draft token t, then
 * group g's mask tokens t = g..B-1 follow in group order (B - g slots per
 * group, B (B + 3) / 2 slots in all).  Visibility of block slot b from
 * query slot i:
 *   draft t     : draft slots t' <= t;
 *   mask of g   : draft slots t' < g, and every mask slot of group g.
 * Cache positions 0..P-1 are visible to every slot.
 */
static int quad_slots(int B) { return B * (B + 3) / 2; }

/* Group of block slot i: -1 for a draft slot, else g with its mask tokens. */
static int quad_group(int B, int i) {
    if (i < B) return -1;
    int rest = i - B;
    for (int g = 0; g < B; ++g) {
        if (rest < B - g) return g;
        rest -= B - g;
    }
    return B; /* not reached for i < quad_slots(B) */
}

static int quad_visible(int B, int i, int b) {
    const int gi = quad_group(B, i), gb = quad_group(B, b);
    if (gi < 0) return gb < 0 && b <= i; /* draft query: causal over the drafts */
    if (gb < 0) return b < gi;           /* mask query: the drafts its group assumes */
    return gb == gi;                     /* ... and its own group's mask tokens */
}

void bdo_attention_quad(int n, int B, int Hq, int Hkv, int d, int cap, int dtype, double scale,
                        const void *q, const void *k_blk, const void *v_blk, const void *k_cache,
                        const void *v_cache, const int32_t *prefix_len, double *out) {
    attention_impl(n, quad_slots(B), Hq, Hkv, d, cap, dtype, dtype, BDO_QUAD, B, scale, q, k_blk, v_blk,
                   k_cache, v_cache, NULL, NULL, prefix_len, out);
}

static void attention_impl(int n, int D, int Hq, int Hkv, int d, int cap, int q_dtype, int kv_dtype,
                           int mode, int B, double scale, const void *q, const void *k_blk, const void *v_blk,
                           const void *k_cache, const void *v_cache, const float *k_scale,
                           const float *v_scale, const int32_t *prefix_len, double *out) {
    const int group = Hq / Hkv;
    long total = (long)n * D * Hq;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long u = 0; u < total; ++u) {
        const int it = (int)(u / ((long)D * Hq));
        const int i = (int)((u / Hq) % D);
        const int h = (int)(u % Hq);
        const int g = h / group;
        const int P = prefix_len[it];
        const int nkeys = P + D;
        double *s = (double *)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
        const size_t qoff = (((size_t)it * D + i) * Hq + h) * (size_t)d;
        double m = -INFINITY;
        for (int j = 0; j < nkeys; ++j) {
            int allowed = (j < P) || (mode == BDO_BIDIR) || (mode == BDO_CAUSAL && j - P <= i) ||
                          (mode == BDO_QUAD && quad_visible(B, i, j - P));
            if (!allowed) { s[j] = -INFINITY; continue; }
            double acc = 0.0;
            for (int t = 0; t < d; ++t) {
                double kv;
                if (j < P)
                    kv = widen(k_cache, kv_dtype, (((size_t)it * Hkv + g) * cap + j) * (size_t)d + t);
                else
                    kv = widen(k_blk, kv_dtype, (((size_t)it * D + (j - P)) * Hkv + g) * (size_t)d + t);
                if (k_scale) kv *= (double)k_scale[(size_t)it * Hkv + g];
                acc += widen(q, q_dtype, qoff + t) * kv;
            }
            s[j] = scale * acc;
            if (s[j] > m) m = s[j];
        }
        double denom = 0.0;
        for (int j = 0; j < nkeys; ++j) {
            s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
            denom += s[j];
        }
        for (int t = 0; t < d; ++t) {
            double acc = 0.0;
            for (int j = 0; j < nkeys; ++j) {
                if (s[j] == 0.0) continue;
                double vv;
                if (j < P)
                    vv = widen(v_cache, kv_dtype, (((size_t)it * Hkv + g) * cap + j) * (size_t)d + t);
                else
                    vv = widen(v_blk, kv_dtype, (((size_t)it * D + (j - P)) * Hkv + g) * (size_t)d + t);
                if (v_scale) vv *= (double)v_scale[(size_t)it * Hkv + g];
                acc += s[j] * vv;
            }
            out[qoff + t] = acc / denom;
        }
        free(s);
    }
}

/*
 * Confidence of one row of logits ([DV] cached block decoding: the
 * confidence of a position is the model probability of the token chosen
 * for it).  Greedy choice a = first index of the maximum (values compared
 * exactly); conf = 1 / sum_v exp(x_v - x_a); lse = x_a + log(sum).
 * p2 = probability of the best token other than a (diagnostic).
 */
void bdo_confidence_row(int V, const float *x, double *conf, int32_t *argmax, double *lse,
                        double *p2) {
    int a = 0;
    for (int v = 1; v < V; ++v)
        if (x[v] > x[a]) a = v;
    double m = (double)x[a];
    double z = 0.0;
    for (int v = 0; v < V; ++v) z += exp((double)x[v] - m);
    double second = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (v != a && (double)x[v] > second) second = (double)x[v];
    *argmax = a;
    *conf = 1.0 / z;
    if (lse) *lse = m + log(z);
    if (p2) *p2 = exp(second - m) / z;
}

/* k = min(ceil(D / S), |M|)  ([DV] Algorithm 1 as restated in the notes). */
int bdo_commit_k(int D, int S, int n_masked) {
    int k = (D + S - 1) / S;
    return k < n_masked ? k : n_masked;
}

/* a ranks before b: higher confidence first, lower index on equal confidence. */
static int ranks_before(double ca, int ia, double cb, int ib) {
    return (ca > cb) || (ca == cb && ia < ib);
}

/*
 * One denoising step's confidence + commit for n_req requests ([DV]
 * cached block decoding; Algorithm 1; dynamic rule).
 *   M = masked positions; for i in M: (conf_i, a_i) from the row's logits.
 *   k = min(ceil(D/S), |M|); T = the k positions of M ranked first;
 *   H = { i in M : conf_i > tau };  commit C = T u H:
 *   tokens[i] = a_i, masked[i] = 0, committed[i] = 1.
 * Positions outside M are not read and never change.
 * conf_out (NaN outside M) and argmax_out (-1 outside M) report the values
 * the ranking and the threshold were decided on.
 */
void bdo_confidence_commit(int n_req, int D, int V, int S, double tau, const float *logits,
                           uint8_t *masked, int32_t *tokens, double *conf_out,
                           int32_t *argmax_out, uint8_t *committed_out,
                           int32_t *n_committed_out) {
    double *conf = (double *)malloc(sizeof(double) * (size_t)D);
    int32_t *amax = (int32_t *)malloc(sizeof(int32_t) * (size_t)D);
    uint8_t *take = (uint8_t *)malloc((size_t)D);
    for (int r = 0; r < n_req; ++r) {
        int n_m = 0;
        for (int i = 0; i < D; ++i) {
            conf[i] = NAN;
            amax[i] = -1;
            take[i] = 0;
            if (masked[(size_t)r * D + i]) {
                ++n_m;
                bdo_confidence_row(V, logits + ((size_t)r * D + i) * (size_t)V, &conf[i], &amax[i],
                                   NULL, NULL);
            }
        }
        int k = bdo_commit_k(D, S, n_m);
        for (int i = 0; i < D; ++i) {
            if (!masked[(size_t)r * D + i]) continue;
            int rank = 0;
            for (int j = 0; j < D; ++j)
                if (j != i && masked[(size_t)r * D + j] && ranks_before(conf[j], j, conf[i], i)) ++rank;
            if (rank < k || conf[i] > tau) take[i] = 1;
        }
        int cnt = 0;
        for (int i = 0; i < D; ++i) {
            size_t o = (size_t)r * D + i;
            if (conf_out) conf_out[o] = conf[i];
            if (argmax_out) argmax_out[o] = amax[i];
            if (committed_out) committed_out[o] = take[i];
            if (take[i]) {
                tokens[o] = amax[i];
                masked[o] = 0;
                ++cnt;
            }
        }
        if (n_committed_out) n_committed_out[r] = cnt;
    }
    free(conf);
    free(amax);
    free(take);
}

/*
 * Speculative verify ([FD] 5.3, linear variant): row i of the causal
 * pass gives the AR prediction for draft slot i (greedy, lowest index on
 * ties); L = first i whose prediction differs from draft[i], or D if all
 * agree.
 */
void bdo_spec_verify(int n_req, int D, int V, const float *logits, const int32_t *draft,
                     int32_t *accepted_len, int32_t *argmax_out) {
    for (int r = 0; r < n_req; ++r) {
        int L = D;
        for (int i = 0; i < D; ++i) {
            const float *x = logits + ((size_t)r * D + i) * (size_t)V;
            int a = 0;
            for (int v = 1; v < V; ++v)
                if (x[v] > x[a]) a = v;
            if (argmax_out) argmax_out[(size_t)r * D + i] = a;
            if (L == D && a != draft[(size_t)r * D + i]) L = i;
        }
        accepted_len[r] = L;
    }
}

/*
 * Append the accepted block K/V to the frozen cache ([FD] 5.3: crop the
 * cache to the accepted prefix; [DV] a finished block joins the history
 * cache).  For item it with L = n_accept[it] (D when n_accept is NULL):
 * cache slots P..P+L-1 receive block slots 0..L-1 bit for bit and
 * prefix_len[it] becomes P+L.  If P+L exceeds cap the item is left
 * untouched and *err is set to 1.
 */
void bdo_kv_append(int n, int D, int Hkv, int d, int cap, int dtype, void *k_cache, void *v_cache,
                   int32_t *prefix_len, const void *k_blk, const void *v_blk,
                   const int32_t *n_accept, int32_t *err) {
    size_t es = dtype == BDO_F32 ? 4 : dtype == BDO_FP8 ? 1 : 2;
    for (int it = 0; it < n; ++it) {
        int P = prefix_len[it];
        int L = n_accept ? n_accept[it] : D;
        if (L < 0 || L > D || P + L > cap) {
            if (err) *err = 1;
            continue;
        }
        for (int t = 0; t < L; ++t)
            for (int g = 0; g < Hkv; ++g)
                for (int e = 0; e < d; ++e) {
                    size_t src = (((size_t)it * D + t) * Hkv + g) * (size_t)d + e;
                    size_t dst = (((size_t)it * Hkv + g) * cap + (P + t)) * (size_t)d + e;
                    memcpy((char *)k_cache + dst * es, (const char *)k_blk + src * es, es);
                    memcpy((char *)v_cache + dst * es, (const char *)v_blk + src * es, es);
                }
        prefix_len[it] = P + L;
    }
}

/*
 * Split-K softmax partial over one key range (online normaliser: Milakov and
 * Gimelshein, "Online normalizer calculation for softmax", 2018):
 *   m = max_j s_j,  l = sum_j exp(s_j - m),  o = sum_j exp(s_j - m) v_j / l.
 * s[nk] are the range's scores, v[nk][d] its values.  An empty range gives
 * m = -inf, l = 0 and o = 0.
 */
void bdo_softmax_partial(int nk, int d, const double *s, const double *v, double *m, double *l,
                         double *o) {
    double mx = -INFINITY;
    for (int j = 0; j < nk; ++j)
        if (s[j] > mx) mx = s[j];
    double sum = 0.0;
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int j = 0; j < nk; ++j) {
        double w = exp(s[j] - mx);
        sum += w;
        for (int e = 0; e < d; ++e) o[e] += w * v[(size_t)j * d + e];
    }
    if (sum > 0.0)
        for (int e = 0; e < d; ++e) o[e] /= sum;
    *m = mx;
    *l = sum;
}

/*
 * Merge of np partials in the given order (the same source):
 *   M = max_p m_p,  c_p = exp(m_p - M) l_p,  out = sum_p c_p o_p / sum_p c_p.
 * Partials of empty ranges (l = 0) contribute nothing.
 */
void bdo_merge_partials(int np, int d, const double *m, const double *l, const double *o,
                        double *out) {
    double M = -INFINITY;
    for (int p = 0; p < np; ++p)
        if (m[p] > M) M = m[p];
    double L = 0.0;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (int p = 0; p < np; ++p) {
        double c = l[p] > 0.0 ? exp(m[p] - M) * l[p] : 0.0;
        L += c;
        for (int e = 0; e < d; ++e) out[e] += c * o[(size_t)p * d + e];
    }
    for (int e = 0; e < d; ++e) out[e] /= L;
}

/*
 * Logits of the block's masked-token predictions: the language model's
 * vocabulary projection applied to the final hidden state of every block
 * slot, logits[r][v] = sum_h hidden[r][h] * weight[v][h] (hidden bf16
 * [R][H], weight bf16 [V][H], out fp64 [R][V]).  These are the logits whose
 * softmax gives the confidence of [DV]'s cached block decoding.
 */
void bdo_lm_head_logits(int R, int V, int H, const uint16_t *hidden, const uint16_t *weight,
                        double *out) {
#pragma omp parallel for schedule(static)
    for (long v = 0; v < V; ++v)
        for (int r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += widen(hidden, BDO_BF16, (size_t)r * H + h) * widen(weight, BDO_BF16, (size_t)v * H + h);
            out[(size_t)r * V + v] = acc;
        }
}

/* Decode OCP FP8 E4M3 bytes (the definition used by the FP8-KV attention). */
void bdo_fp8_e4m3_decode(int n, const uint8_t *b, double *out) {
    for (int i = 0; i < n; ++i) out[i] = fp8_e4m3(b[i]);
}

/*
 * Two-stream training attention ([FD] section 4.1, causal-context attention;
 * section 4.3, auto-truncation; section 4.4, vision-efficient concatenation;
 * [FD2] Fig. 3).
 *
 * Sequence s is the clean stream x (Lc tokens: vision, prompts and responses
 * in order) followed by the noisy stream w (Ln tokens).  Only response text is
 * corrupted, so w holds the response tokens alone, in order: response r is the
 * span (start c_r, length len_r) of x and occupies w[o_r .. o_r + len_r),
 * o_r = len_0 + ... + len_{r-1}.  Vision tokens appear only in x.  Each
 * response is cut into blocks of D tokens from its start; its last block ends
 * at the response boundary (auto-truncation), so no block reaches into the
 * next prompt.  Keys are the positions of [x ; w]:
 *   clean query at position p           : clean keys 0..p            (M_C2C, token causal)
 *   noisy query in the block of response r covering x[b0, b1):
 *                                          clean keys 0..b0-1        (M_N2C: every earlier clean
 *                                                                      position, vision included)
 *                                          the noisy keys of its own  (M_N2N: bidirectional in the
 *                                          block, w[o_r + b0 - c_r .. o_r + b1 - c_r)   block)
 *   clean queries never see noisy keys; noisy positions past the last
 *   response see nothing and their output is 0.
 *
 * Layouts: q, out [n][L][Hq][d] with L = Lc + Ln (clean positions first);
 * k and v [n][Hkv][cap][d] over the same L positions;
 * spans int32 [n][max_spans][2] = (c_r, len_r), n_spans int32 [n].
 */
static int ts_noisy_block(const int32_t *sp, int ns, int D, int i, int *b0, int *b1, int *w0) {
    int o = 0;
    for (int r = 0; r < ns; ++r) {
        const int c = sp[2 * r], len = sp[2 * r + 1];
        if (i < o + len) {
            const int k = (i - o) / D;
            *b0 = c + k * D;
            *b1 = c + (k + 1) * D < c + len ? c + (k + 1) * D : c + len;
            *w0 = o + k * D;
            return 1;
        }
        o += len;
    }
    return 0;
}

static int ts_visible(int Lc, const int32_t *sp, int ns, int D, int i, int j) {
    if (i < Lc) return j <= i; /* clean query: causal over the clean stream */
    int b0, b1, w0;
    if (!ts_noisy_block(sp, ns, D, i - Lc, &b0, &b1, &w0)) return 0;
    if (j < Lc) return j < b0;                     /* earlier clean positions */
    return j - Lc >= w0 && j - Lc < w0 + (b1 - b0); /* its own noisy block */
}

void bdo_two_stream_attention(int n, int Lc, int Ln, int cap, int D, int Hq, int Hkv, int d, int dtype,
                              double scale, int max_spans, const void *q, const void *k, const void *v,
                              const int32_t *spans, const int32_t *n_spans, double *out) {
    const int L = Lc + Ln, group = Hq / Hkv;
    const long total = (long)n * L * Hq;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (long u = 0; u < total; ++u) {
        const int it = (int)(u / ((long)L * Hq));
        const int i = (int)((u / Hq) % L);
        const int h = (int)(u % Hq);
        const int g = h / group;
        const int32_t *sp = spans + (size_t)it * max_spans * 2;
        const int ns = n_spans[it];
        const size_t qoff = (((size_t)it * L + i) * Hq + h) * (size_t)d;
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        double m = -INFINITY;
        for (int j = 0; j < L; ++j) {
            s[j] = -INFINITY;
            if (!ts_visible(Lc, sp, ns, D, i, j)) continue;
            double acc = 0.0;
            for (int t = 0; t < d; ++t)
                acc += widen(q, dtype, qoff + t) * widen(k, dtype, (((size_t)it * Hkv + g) * cap + j) * (size_t)d + t);
            s[j] = scale * acc;
            if (s[j] > m) m = s[j];
        }
        double denom = 0.0;
        for (int j = 0; j < L; ++j) {
            s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
            denom += s[j];
        }
        for (int t = 0; t < d; ++t) {
            double acc = 0.0;
            for (int j = 0; j < L; ++j)
                if (s[j] != 0.0) acc += s[j] * widen(v, dtype, (((size_t)it * Hkv + g) * cap + j) * (size_t)d + t);
            out[qoff + t] = denom > 0.0 ? acc / denom : 0.0;
        }
        free(s);
    }
}
