/*
 * sdm_oracle.c -- plain, slow CPU oracle for the Sparse Delta Memory (SDM)
 * hot path: product-key top-k addressing, softmax weights and the sparse
 * gated delta-rule scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP kernels.
 *
 * Sources (web pages on the method; cited by title and section):
 *   [P]  "Sparse Delta Memory: Scaling the State of Linear RNNs through
 *        Sparsity" -- the paper text.
 *          Sec. 2  (Product-Key Memories): scores of the N = n_sub^2 slots are
 *                  the outer sum of two half-score vectors; the top-k can be
 *                  found without materialising all N scores.
 *          Sec. 3.1, step 1 (Sparse Key Selection): keys/queries are split in
 *                  two halves; top-W of the write scores and top-R of the read
 *                  scores select the slots.
 *          Sec. 3.1, step 2 (Gated Delta Write, Eq. 4): selected rows only;
 *                  unselected slots stay unchanged.
 *          Sec. 3.1, step 3 (Sparse Read): weighted sum of the selected read
 *                  rows, after the write.
 *          Sec. 3.1, "Learned Initial State": M0 copied into every sequence.
 *          Sec. 4 (SDM Configuration): read and write activations use
 *                  softmax normalisation.
 *   [B]  "Sparse Delta Memory: Scaling Linear RNN States to 1M Tokens via
 *        Sparsity" -- blog summary, "Methodology", item 2 (Gated Delta
 *        Updates): M_t[i] <- a_t M_{t-1}[i] + b_t k^(i) (v_t - a_t M_{t-1}^T k_t).
 *
 * Readings where the pages are silent or garbled (each is also listed in the
 * design notes of the repository):
 *   - The prediction is M_{t-1}^T k_t = sum over the W selected slots of
 *     w_j M_{t-1}[slot_j], formed on the pre-write state before any row is
 *     written (this is what makes W = N reduce to the Gated DeltaNet rule of
 *     [P] Sec. 2, Eq. 2, as [P] Sec. 3.1 states).
 *   - The read uses the post-write state of the same token.
 *   - Decay applies to the written rows only.
 *   - Each half is scored against its own sub-key codebook C[h][c] of shape
 *     [n_sub, d_k/2]; slot = i1 * n_sub + i2 with i1 from the first half.
 *   - Weights are a softmax over the selected slot scores, no temperature.
 *   - Scores are fp32 values (the kernel's precision for the selection):
 *     a half score is the fp32 rounding of the exact (fp64) dot product, and
 *     a slot score is the fp32 sum of its two half scores.  Every order is by
 *     score descending, ties to the lower index (sub-key index in the halves,
 *     flat slot index in the merge).
 *   - Memory state is fp32; the scan accumulates in fp64 and rounds each
 *     stored row element and each output element once to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T, H, d_k, n_sub, d_v, k_prime, W, R;
    int32_t in_bf16; /* 1: k, q, v and codebooks are bf16 bit patterns; 0: fp32 */
    int32_t pad_;
} orc_dims;

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2, ORC_EINDEX = -3, ORC_ENONFINITE = -4 };

/* ---- input decoding (bf16 -> fp64 is exact) ------------------------------ */
static double dec_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_in(const void *p, int bf16, int64_t i)
{
    return bf16 ? dec_bf16(((const uint16_t *)p)[i]) : (double)((const float *)p)[i];
}

static int check_dims(const orc_dims *d)
{
    if (!d) return ORC_EINVAL;
    if (d->B < 0 || d->T < 0 || d->H < 1 || d->d_k < 2 || (d->d_k & 1) || d->n_sub < 1 ||
        d->d_v < 1 || d->k_prime < 1 || d->k_prime > d->n_sub || d->W < 1 || d->R < 1 ||
        d->W > d->k_prime * d->k_prime || d->R > d->k_prime * d->k_prime)
        return ORC_EINVAL;
    if (d->n_sub > 46340) return ORC_EINVAL; /* N must fit in int32 */
    return ORC_OK;
}

/* ---- scores -------------------------------------------------------------- */
/* Half scores of one token-head row for half c: s[u] = fp32(<x_c, C[h][c][u]>),
 * the dot product taken in fp64.  [P] Sec. 2 (PKM) and Sec. 3.1 step 1. */
static int half_scores(const void *x, const void *C, const orc_dims *d, int64_t row, int64_t h,
                       int c, float *s)
{
    const int64_t half = d->d_k / 2;
    const int bf = d->in_bf16;
    for (int64_t u = 0; u < d->n_sub; ++u) {
        double acc = 0.0;
        const int64_t cbase = ((h * 2 + c) * d->n_sub + u) * half;
        const int64_t xbase = row * d->d_k + (int64_t)c * half;
        for (int64_t e = 0; e < half; ++e)
            acc += load_in(x, bf, xbase + e) * load_in(C, bf, cbase + e);
        if (!isfinite(acc)) return ORC_ENONFINITE;
        s[u] = (float)acc;
    }
    return ORC_OK;
}

typedef struct {
    float s;
    int32_t i;
} scored;

/* score descending, then index ascending: a total order on distinct indices */
static int cmp_scored(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* One addressing problem: top-n slots of x against codebook C, with weights.
 * Step order of [P] Sec. 2: top-k' per half, then the k' x k' outer-sum
 * candidates, then top-n of those.  Then the softmax of [P] Sec. 4. */
static int address_one(const void *x, const void *C, const orc_dims *d, int64_t row, int64_t h,
                       int64_t n, scored *work, int32_t *idx_out, float *wt_out, float *sc_out)
{
    const int64_t ns = d->n_sub, kp = d->k_prime;
    scored *h0 = work, *h1 = work + ns, *cand = work + 2 * ns;
    float *tmp = (float *)(work + 2 * ns + kp * kp);
    int rc;
    for (int c = 0; c < 2; ++c) {
        scored *hc = c ? h1 : h0;
        if ((rc = half_scores(x, C, d, row, h, c, tmp)) != ORC_OK) return rc;
        for (int64_t u = 0; u < ns; ++u) {
            hc[u].s = tmp[u];
            hc[u].i = (int32_t)u;
        }
        qsort(hc, (size_t)ns, sizeof(scored), cmp_scored); /* first k' are the top-k' */
    }
    for (int64_t a = 0; a < kp; ++a)
        for (int64_t b = 0; b < kp; ++b) {
            scored *e = &cand[a * kp + b];
            e->s = h0[a].s + h1[b].s; /* fp32 addition */
            e->i = (int32_t)(h0[a].i * ns + h1[b].i);
        }
    qsort(cand, (size_t)(kp * kp), sizeof(scored), cmp_scored);
    double z = 0.0;
    const double m = (double)cand[0].s;
    for (int64_t j = 0; j < n; ++j) z += exp((double)cand[j].s - m);
    for (int64_t j = 0; j < n; ++j) {
        idx_out[j] = cand[j].i;
        wt_out[j] = (float)(exp((double)cand[j].s - m) / z);
        if (sc_out) sc_out[j] = cand[j].s;
    }
    return ORC_OK;
}

/* Addressing for every token-head row of k (write) and q (read).
 *   k, q   [B,T,H,d_k]; C_w, C_r [H,2,n_sub,d_k/2]
 *   widx, wwt [B,T,H,W]; ridx, rwt [B,T,H,R]; wsc, rsc optional selected scores */
int orc_address(const void *k, const void *q, const void *C_w, const void *C_r, const orc_dims *d,
                int32_t *widx, float *wwt, int32_t *ridx, float *rwt, float *wsc, float *rsc,
                int nthreads)
{
    int rc = check_dims(d);
    if (rc) return rc;
    const int64_t rows = d->B * d->T * d->H;
    const int64_t kp = d->k_prime, ns = d->n_sub;
    const size_t wbytes = sizeof(scored) * (size_t)(2 * ns + kp * kp) + sizeof(float) * (size_t)ns;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        scored *work = (scored *)malloc(wbytes + 16);
        if (!work) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < rows; ++r) {
            if (!work || err) continue;
            const int64_t h = r % d->H;
            int e1 = address_one(k, C_w, d, r, h, d->W, work, widx + r * d->W, wwt + r * d->W,
                                 wsc ? wsc + r * d->W : NULL);
            int e2 = address_one(q, C_r, d, r, h, d->R, work, ridx + r * d->R, rwt + r * d->R,
                                 rsc ? rsc + r * d->R : NULL);
            if (e1 || e2) {
#pragma omp atomic write
                err = e1 ? e1 : e2;
            }
        }
        free(work);
    }
    return err;
}

/* Half scores for every row and both halves: out [rows, 2, n_sub]. */
int orc_half_scores(const void *x, const void *C, const orc_dims *d, float *out, int nthreads)
{
    int rc = check_dims(d);
    if (rc) return rc;
    const int64_t rows = d->B * d->T * d->H;
    int err = ORC_OK;
#pragma omp parallel for num_threads(nthreads > 0 ? nthreads : 1) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int c = 0; c < 2; ++c) {
            int e = half_scores(x, C, d, r, r % d->H, c, out + (r * 2 + c) * d->n_sub);
            if (e) {
#pragma omp atomic write
                err = e;
            }
        }
    }
    return err;
}

/* fp32 slot score fp32(s1[i1]) + fp32(s2[i2]) of given (row, slot) pairs. */
int orc_slot_scores(const void *x, const void *C, const orc_dims *d, int64_t nq,
                    const int64_t *rows, const int32_t *slots, float *out)
{
    int rc = check_dims(d);
    if (rc) return rc;
    float *s = (float *)malloc(sizeof(float) * (size_t)(2 * d->n_sub));
    if (!s) return ORC_ENOMEM;
    const int64_t N = d->n_sub * d->n_sub;
    for (int64_t i = 0; i < nq; ++i) {
        if (slots[i] < 0 || slots[i] >= N || rows[i] < 0 || rows[i] >= d->B * d->T * d->H) {
            free(s);
            return ORC_EINDEX;
        }
        const int64_t h = rows[i] % d->H;
        if ((rc = half_scores(x, C, d, rows[i], h, 0, s)) ||
            (rc = half_scores(x, C, d, rows[i], h, 1, s + d->n_sub))) {
            free(s);
            return rc;
        }
        out[i] = s[slots[i] / d->n_sub] + s[d->n_sub + slots[i] % d->n_sub];
    }
    free(s);
    return ORC_OK;
}

/* ---- the scan ------------------------------------------------------------ */
/* Sequence-serial sparse gated delta rule, [P] Sec. 3.1 steps 2-3 and [B]
 * item 2.  For every (b, h), tokens in order:
 *     p   = sum_j w_j M[widx_j]                  (pre-write rows, fp64)
 *     u   = v_t - a_t p
 *     M[widx_j] = fp32(a_t M[widx_j] + b_t w_j u)    for all j at once
 *     o_t = fp32(sum_j r_j M[ridx_j])              (post-write rows)
 * Rows not in widx are untouched.
 *   M [B,H,N,d_v] fp32 in/out; widx, wwt [B,T,H,W]; ridx, rwt [B,T,H,R];
 *   v [B,T,H,d_v]; a, b [B,T,H]; o [B,T,H,d_v] */
int orc_scan(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx, const float *rwt,
             const void *v, const float *a, const float *b, float *o, const orc_dims *d,
             int nthreads)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->n_sub < 1 || d->d_v < 1 || d->W < 1 ||
        d->R < 1 || d->n_sub > 46340)
        return ORC_EINVAL;
    const int64_t N = d->n_sub * d->n_sub, dv = d->d_v, W = d->W, R = d->R;
    const int64_t chains = d->B * d->H;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(2 * dv));
        if (!p) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ch = 0; ch < chains; ++ch) {
            if (!p || err) continue;
            double *u = p + dv;
            const int64_t bb = ch / d->H, h = ch % d->H;
            float *Mc = M + ch * N * dv;
            for (int64_t t = 0; t < d->T && !err; ++t) {
                const int64_t row = (bb * d->T + t) * d->H + h;
                const int32_t *wi = widx + row * W, *ri = ridx + row * R;
                const float *ww = wwt + row * W, *rw = rwt + row * R;
                int bad = 0;
                for (int64_t j = 0; j < W; ++j) {
                    if (wi[j] < 0 || wi[j] >= N) bad = 1;
                    for (int64_t jj = 0; jj < j; ++jj)
                        if (wi[jj] == wi[j]) bad = 1; /* write slots must be distinct */
                }
                for (int64_t j = 0; j < R; ++j)
                    if (ri[j] < 0 || ri[j] >= N) bad = 1;
                if (bad) {
#pragma omp atomic write
                    err = ORC_EINDEX;
                    break;
                }
                const double at = (double)a[row], bt = (double)b[row];
                for (int64_t c = 0; c < dv; ++c) p[c] = 0.0;
                for (int64_t j = 0; j < W; ++j) {
                    const float *Mr = Mc + (int64_t)wi[j] * dv;
                    for (int64_t c = 0; c < dv; ++c) p[c] += (double)ww[j] * (double)Mr[c];
                }
                for (int64_t c = 0; c < dv; ++c)
                    u[c] = load_in(v, d->in_bf16, row * dv + c) - at * p[c];
                for (int64_t j = 0; j < W; ++j) {
                    float *Mr = Mc + (int64_t)wi[j] * dv;
                    const double bw = bt * (double)ww[j];
                    for (int64_t c = 0; c < dv; ++c)
                        Mr[c] = (float)(at * (double)Mr[c] + bw * u[c]);
                }
                for (int64_t c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < R; ++j)
                        acc += (double)rw[j] * (double)Mc[(int64_t)ri[j] * dv + c];
                    o[row * dv + c] = (float)acc;
                }
            }
        }
        free(p);
    }
    return err;
}

/* Learned initial state copied into every sequence, [P] Sec. 3.1:
 * M[b][h] = M0[h].  M [B,H,N,d_v], M0 [H,N,d_v]. */
int orc_state_init(float *M, const float *M0, const orc_dims *d)
{
    if (!d || d->B < 0 || d->H < 1 || d->n_sub < 1 || d->d_v < 1) return ORC_EINVAL;
    const size_t per_seq = (size_t)(d->H * d->n_sub * d->n_sub * d->d_v);
    for (int64_t b = 0; b < d->B; ++b) memcpy(M + (size_t)b * per_seq, M0, per_seq * sizeof(float));
    return ORC_OK;
}

/* ---- around the path: the gates before it, the output norm after it ------ */
/* The gates of one token-head, [P] Sec. 3.1 step 2 (a per-head forget gate
 * a_t with a learnable decay A, and an input gate b_t) in the Gated DeltaNet
 * parameterisation that [P] Sec. 4 says the decay and the time-step bias are
 * initialised for (the pages print no formula; this is the reading):
 *     a = exp(-A[h] * softplus(a_raw + dt_bias[h])),  softplus(z) = ln(1 + e^z)
 *     b = 1 / (1 + e^(-b_raw))
 * in fp64, each result rounded once to fp32.
 *   a_raw, b_raw, a, b [B,T,H] fp32; A (>= 0), dt_bias [H] fp32. */
static double softplus(double z)
{
    /* ln(1 + e^z) = z + ln(1 + e^-z): the form whose exponential cannot overflow */
    return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
}

int orc_gates(const float *a_raw, const float *b_raw, const float *A, const float *dt_bias,
              const orc_dims *d, float *a, float *b)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1) return ORC_EINVAL;
    for (int64_t h = 0; h < d->H; ++h)
        if (!isfinite(A[h]) || A[h] < 0.0f || !isfinite(dt_bias[h])) return ORC_ENONFINITE;
    const int64_t n = d->B * d->T * d->H;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t h = i % d->H;
        if (!isfinite(a_raw[i]) || !isfinite(b_raw[i])) return ORC_ENONFINITE;
        a[i] = (float)exp(-(double)A[h] * softplus((double)a_raw[i] + (double)dt_bias[h]));
        b[i] = (float)(1.0 / (1.0 + exp(-(double)b_raw[i])));
    }
    return ORC_OK;
}

/* The read-out's norm and output gate, [P] Sec. 3.1 step 4: each token-head's
 * o row is RMS-normalised over its d_v features with the learned gain gamma,
 * then multiplied element-wise by the gate activation of g (reading: the
 * Gated DeltaNet output gate, silu(g) = g / (1 + e^-g)):
 *     y[c] = o[c] / sqrt(mean_c' o[c']^2 + eps) * gamma[c] * silu(g[c])
 * The exact value in fp64 (the caller rounds it to the output precision).
 *   o [B,T,H,d_v] fp32; g [B,T,H,d_v] (bf16 bits or fp32); gamma [d_v] fp32;
 *   y [B,T,H,d_v] fp64. */
int orc_output_norm_gate(const float *o, const void *g, const float *gamma, double eps, const orc_dims *d,
                         double *y)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->d_v < 1 || !(eps >= 0.0)) return ORC_EINVAL;
    const int64_t rows = d->B * d->T * d->H, dv = d->d_v;
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < dv; ++c) ss += (double)o[r * dv + c] * (double)o[r * dv + c];
        const double inv = 1.0 / sqrt(ss / (double)dv + eps);
        for (int64_t c = 0; c < dv; ++c) {
            const double gc = load_in(g, d->in_bf16, r * dv + c);
            y[r * dv + c] = (double)o[r * dv + c] * inv * (double)gamma[c] * (gc / (1.0 + exp(-gc)));
        }
    }
    return ORC_OK;
}

/* ---- the dense Gated DeltaNet recurrence (every slot selected) ----------- */
/* [P] Sec. 2, Eq. 2 (Gated DeltaNet), the rule that Sec. 3.1 ("Connection to
 * GDN") says SDM reduces to when every slot is selected with a dense key:
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 * with S_t in R^{d_v x d_k}.  Stored transposed, like the SDM memory with
 * N = d_k slots: S [B,H,d_k,d_v], row j = the state's column for key
 * dimension j.  Expanding the product, row j of the new state is
 *     a S[j] + b k_j (v - a sum_l k_l S[l])
 * (the prediction sum_l k_l S[l] is formed from the old state, before any
 * row changes).  fp64 arithmetic, each stored state element and each output
 * rounded once to fp32.
 *   k, q [B,T,H,d_k] and v [B,T,H,d_v] (bf16 bits or fp32); a, b [B,T,H];
 *   S [B,H,d_k,d_v] fp32 in/out; o [B,T,H,d_v] fp32. */
int orc_gdn_dense(float *S, const void *k, const void *q, const void *v, const float *a, const float *b,
                  float *o, const orc_dims *d, int nthreads)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->d_k < 1 || d->d_v < 1) return ORC_EINVAL;
    const int64_t dk = d->d_k, dv = d->d_v, chains = d->B * d->H;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(2 * dv + 2 * dk));
        if (!p) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ch = 0; ch < chains; ++ch) {
            if (!p || err) continue;
            double *u = p + dv, *kk = u + dv, *qq = kk + dk;
            const int64_t bb = ch / d->H, h = ch % d->H;
            float *Sc = S + ch * dk * dv;
            for (int64_t t = 0; t < d->T; ++t) {
                const int64_t row = (bb * d->T + t) * d->H + h;
                const double at = (double)a[row], bt = (double)b[row];
                for (int64_t j = 0; j < dk; ++j) {
                    kk[j] = load_in(k, d->in_bf16, row * dk + j);
                    qq[j] = load_in(q, d->in_bf16, row * dk + j);
                }
                for (int64_t c = 0; c < dv; ++c) p[c] = 0.0;
                for (int64_t j = 0; j < dk; ++j)
                    for (int64_t c = 0; c < dv; ++c) p[c] += kk[j] * (double)Sc[j * dv + c];
                for (int64_t c = 0; c < dv; ++c) u[c] = load_in(v, d->in_bf16, row * dv + c) - at * p[c];
                for (int64_t j = 0; j < dk; ++j)
                    for (int64_t c = 0; c < dv; ++c)
                        Sc[j * dv + c] = (float)(at * (double)Sc[j * dv + c] + bt * kk[j] * u[c]);
                for (int64_t c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < dk; ++j) acc += qq[j] * (double)Sc[j * dv + c];
                    o[row * dv + c] = (float)acc;
                }
            }
        }
        free(p);
    }
    return err;
}

/* ---- gradients of the scan ---------------------------------------------- */
/* Reverse-mode derivative of orc_scan for a loss L with given dL/do_t (dout)
 * and dL/dM_T (dM on entry; zeros if the loss does not see the final state).
 * [P] Sec. 3.1 steps 2-3 (Eq. 4) differentiated; the pages print no
 * backward pass (its appendix is not among them), so this is the plain
 * chain rule of the forward above, token by token in reverse:
 *   forward:  X_j = M[s_j] (before),  p = sum_j w_j X_j,  u = v - a p,
 *             M[s_j] = Y_j = a X_j + b w_j u,  Z_i = M[r_i] (after),
 *             o = sum_i r_i Z_i
 *   reverse, with G = dL/dM after the token:
 *     dr_i = <do, Z_i>;  G[r_i] += r_i do
 *     dY_j = G[s_j];  du = b sum_j w_j dY_j;  dv = du;  dp = -a du
 *     da = sum_j <dY_j, X_j> - <p, du>;  db = sum_j w_j <dY_j, u>
 *     dw_j = b <dY_j, u> + <dp, X_j>;  G[s_j] = a dY_j + w_j dp
 *   and on exit G = dL/dM before the first token.
 * The forward is re-run here (fp32 state, as orc_scan) to obtain X, p, u
 * and Z; all gradient arithmetic is fp64, rounded once on output.
 *   M [B,H,N,d_v] fp32: the state before the call (read only);
 *   dM [B,H,N,d_v] fp32 in/out; dout [B,T,H,d_v] fp32;
 *   dv [B,T,H,d_v], da, db [B,T,H], dw [B,T,H,W], dr [B,T,H,R] fp32 out. */
int orc_scan_backward(const float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                      const float *rwt, const void *v, const float *a, const float *b, const float *dout,
                      float *dM, float *dv, float *da, float *db, float *dw, float *dr, const orc_dims *d,
                      int nthreads)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->n_sub < 1 || d->d_v < 1 || d->W < 1 || d->R < 1 ||
        d->n_sub > 46340)
        return ORC_EINVAL;
    const int64_t N = d->n_sub * d->n_sub, dvv = d->d_v, W = d->W, R = d->R, T = d->T;
    const int64_t chains = d->B * d->H;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        /* per chain: the forward state (fp32), the saved rows, G (fp64) */
        float *Mc = (float *)malloc(sizeof(float) * (size_t)(N * dvv));
        double *G = (double *)malloc(sizeof(double) * (size_t)(N * dvv));
        float *X = (float *)malloc(sizeof(float) * (size_t)((T > 0 ? T : 1) * W * dvv));
        float *Z = (float *)malloc(sizeof(float) * (size_t)((T > 0 ? T : 1) * R * dvv));
        double *tmp = (double *)malloc(sizeof(double) * (size_t)(4 * dvv));
        if (!Mc || !G || !X || !Z || !tmp) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ch = 0; ch < chains; ++ch) {
            if (!Mc || !G || !X || !Z || !tmp || err) continue;
            const int64_t bb = ch / d->H, h = ch % d->H;
            double *p = tmp, *u = tmp + dvv, *du = tmp + 2 * dvv, *dp = tmp + 3 * dvv;
            memcpy(Mc, M + ch * N * dvv, sizeof(float) * (size_t)(N * dvv));
            /* forward, saving the pre-write write rows and the post-write read rows */
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (bb * T + t) * d->H + h;
                const int32_t *wi = widx + row * W, *ri = ridx + row * R;
                const float *ww = wwt + row * W;
                for (int64_t j = 0; j < W; ++j) {
                    if (wi[j] < 0 || wi[j] >= N) err = ORC_EINDEX;
                    for (int64_t jj = 0; jj < j; ++jj)
                        if (wi[jj] == wi[j]) err = ORC_EINDEX; /* write slots must be distinct */
                }
                for (int64_t j = 0; j < R; ++j)
                    if (ri[j] < 0 || ri[j] >= N) err = ORC_EINDEX;
                if (err) break;
                const double at = (double)a[row], bt = (double)b[row];
                for (int64_t c = 0; c < dvv; ++c) p[c] = 0.0;
                for (int64_t j = 0; j < W; ++j) {
                    memcpy(X + (t * W + j) * dvv, Mc + (int64_t)wi[j] * dvv, sizeof(float) * (size_t)dvv);
                    for (int64_t c = 0; c < dvv; ++c) p[c] += (double)ww[j] * (double)Mc[(int64_t)wi[j] * dvv + c];
                }
                for (int64_t c = 0; c < dvv; ++c) u[c] = load_in(v, d->in_bf16, row * dvv + c) - at * p[c];
                for (int64_t j = 0; j < W; ++j) {
                    float *Mr = Mc + (int64_t)wi[j] * dvv;
                    const double bw = bt * (double)ww[j];
                    for (int64_t c = 0; c < dvv; ++c) Mr[c] = (float)(at * (double)Mr[c] + bw * u[c]);
                }
                for (int64_t i = 0; i < R; ++i)
                    memcpy(Z + (t * R + i) * dvv, Mc + (int64_t)ri[i] * dvv, sizeof(float) * (size_t)dvv);
            }
            if (err) continue;
            /* reverse */
            for (int64_t e = 0; e < N * dvv; ++e) G[e] = (double)dM[ch * N * dvv + e];
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t row = (bb * T + t) * d->H + h;
                const int32_t *wi = widx + row * W, *ri = ridx + row * R;
                const float *ww = wwt + row * W, *rw = rwt + row * R;
                const float *dov = dout + row * dvv;
                const double at = (double)a[row], bt = (double)b[row];
                for (int64_t i = 0; i < R; ++i) {
                    double s = 0.0;
                    double *Gr = G + (int64_t)ri[i] * dvv;
                    const float *Zi = Z + (t * R + i) * dvv;
                    for (int64_t c = 0; c < dvv; ++c) {
                        s += (double)dov[c] * (double)Zi[c];
                        Gr[c] += (double)rw[i] * (double)dov[c];
                    }
                    dr[row * R + i] = (float)s;
                }
                for (int64_t c = 0; c < dvv; ++c) { p[c] = 0.0; du[c] = 0.0; }
                for (int64_t j = 0; j < W; ++j) {
                    const float *Xj = X + (t * W + j) * dvv;
                    const double *Gw = G + (int64_t)wi[j] * dvv;
                    for (int64_t c = 0; c < dvv; ++c) {
                        p[c] += (double)ww[j] * (double)Xj[c];
                        du[c] += (double)ww[j] * Gw[c];
                    }
                }
                double sa = 0.0, sb = 0.0;
                for (int64_t c = 0; c < dvv; ++c) {
                    du[c] *= bt;
                    u[c] = load_in(v, d->in_bf16, row * dvv + c) - at * p[c];
                    dp[c] = -at * du[c];
                    sa -= p[c] * du[c];
                    dv[row * dvv + c] = (float)du[c];
                }
                for (int64_t j = 0; j < W; ++j) {
                    const float *Xj = X + (t * W + j) * dvv;
                    double *Gw = G + (int64_t)wi[j] * dvv;
                    double yu = 0.0, px = 0.0, yx = 0.0;
                    for (int64_t c = 0; c < dvv; ++c) {
                        yu += Gw[c] * u[c];
                        px += dp[c] * (double)Xj[c];
                        yx += Gw[c] * (double)Xj[c];
                        Gw[c] = at * Gw[c] + (double)ww[j] * dp[c];
                    }
                    dw[row * W + j] = (float)(bt * yu + px);
                    sa += yx;
                    sb += (double)ww[j] * yu;
                }
                da[row] = (float)sa;
                db[row] = (float)sb;
            }
            for (int64_t e = 0; e < N * dvv; ++e) dM[ch * N * dvv + e] = (float)G[e];
        }
        free(Mc); free(G); free(X); free(Z); free(tmp);
    }
    return err;
}

/* ---- gradients of the addressing ------------------------------------------ */
/* Reverse-mode derivative of orc_address for given gradients of the weights
 * (dw [B,T,H,W] for the write lists, dr [B,T,H,R] for the read lists), with
 * the selected slots held fixed (the selection is piecewise constant).  The
 * chain rule through [P] Sec. 4's softmax and Sec. 2's two-half scores:
 *   weights = softmax(sc),  sc_j = s_0[i1_j] + s_1[i2_j]  (slot_j = i1_j n_sub + i2_j)
 *   dsc_j  = wt_j (dwt_j - sum_k wt_k dwt_k)
 *   s_c[u] = <x_c, C[h][c][u]>:  dx_c += dsc_j C[h][c][i_c j];  dC[h][c][i_c j] += dsc_j x_c
 * for each kind (write: x = k with C_w; read: x = q with C_r).  fp64, each
 * output rounded once.  dk, dq [B,T,H,d_k]; dCw, dCr [H,2,n_sub,d_k/2]
 * (written; sums over every token). */
int orc_address_backward(const void *k, const void *q, const void *C_w, const void *C_r, const int32_t *widx,
                         const float *wwt, const int32_t *ridx, const float *rwt, const float *dw, const float *dr,
                         const orc_dims *d, float *dk, float *dq, float *dCw, float *dCr)
{
    int err = check_dims(d);
    if (err) return err;
    const int64_t half = d->d_k / 2, ns = d->n_sub, N = ns * ns;
    const int64_t rows = d->B * d->T * d->H;
    const int64_t csz = d->H * 2 * ns * half;
    double *acc = (double *)calloc((size_t)(2 * csz), sizeof(double));
    double *dx = (double *)malloc(sizeof(double) * (size_t)d->d_k);
    if (!acc || !dx) {
        free(acc); free(dx);
        return ORC_ENOMEM;
    }
    for (int kind = 0; kind < 2 && !err; ++kind) {
        const void *X = kind ? q : k, *C = kind ? C_r : C_w;
        const int32_t *idx = kind ? ridx : widx;
        const float *wt = kind ? rwt : wwt, *dwt = kind ? dr : dw;
        float *dX = kind ? dq : dk;
        double *dC = acc + kind * csz;
        const int64_t n = kind ? d->R : d->W;
        for (int64_t r = 0; r < rows && !err; ++r) {
            const int64_t h = r % d->H;
            double g = 0.0;
            for (int64_t j = 0; j < n; ++j) g += (double)wt[r * n + j] * (double)dwt[r * n + j];
            for (int64_t e = 0; e < d->d_k; ++e) dx[e] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const int32_t s = idx[r * n + j];
                if (s < 0 || s >= N) {
                    err = ORC_EINDEX;
                    break;
                }
                const double dsc = (double)wt[r * n + j] * ((double)dwt[r * n + j] - g);
                const int64_t iu[2] = {s / ns, s % ns};
                for (int c = 0; c < 2; ++c) {
                    const int64_t cb = ((h * 2 + c) * ns + iu[c]) * half;
                    for (int64_t e = 0; e < half; ++e) {
                        dx[c * half + e] += dsc * load_in(C, d->in_bf16, cb + e);
                        dC[cb + e] += dsc * load_in(X, d->in_bf16, r * d->d_k + c * half + e);
                    }
                }
            }
            for (int64_t e = 0; e < d->d_k; ++e) dX[r * d->d_k + e] = (float)dx[e];
        }
    }
    if (!err)
        for (int64_t e = 0; e < csz; ++e) {
            dCw[e] = (float)acc[e];
            dCr[e] = (float)acc[csz + e];
        }
    free(acc);
    free(dx);
    return err;
}

/* ---- gradients of the gates and of the output norm and gate -------------- */
/* Reverse mode of orc_gates: with z = a_raw + dt_bias[h], a = exp(-A sp(z)),
 * sp' = sigmoid, b = sigmoid(b_raw):
 *   da_raw = da * a * (-A[h]) * sigmoid(z);  ddt_bias[h] = sum of da_raw over (b, t)
 *   dA[h] = sum over (b, t) of da * a * (-sp(z));  db_raw = db * b (1 - b)
 * fp64, each output rounded once.  1 - sigmoid(x) is taken as sigmoid(-x), the
 * same number without the cancellation that loses it when x is large. */
int orc_gates_backward(const float *a_raw, const float *b_raw, const float *A, const float *dt_bias, const float *da,
                       const float *db, const orc_dims *d, float *da_raw, float *db_raw, float *dA, float *ddt)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1) return ORC_EINVAL;
    double *acc = (double *)calloc((size_t)(2 * d->H), sizeof(double));
    if (!acc) return ORC_ENOMEM;
    const int64_t n = d->B * d->T * d->H;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t h = i % d->H;
        const double z = (double)a_raw[i] + (double)dt_bias[h];
        const double sp = softplus(z), sg = 1.0 / (1.0 + exp(-z));
        const double a = exp(-(double)A[h] * sp);
        const double g = (double)da[i] * a * (-(double)A[h]) * sg;
        da_raw[i] = (float)g;
        acc[d->H + h] += g;
        acc[h] += (double)da[i] * a * (-sp);
        const double b = 1.0 / (1.0 + exp(-(double)b_raw[i])), nb = 1.0 / (1.0 + exp((double)b_raw[i]));
        db_raw[i] = (float)((double)db[i] * b * nb);
    }
    for (int64_t h = 0; h < d->H; ++h) {
        dA[h] = (float)acc[h];
        ddt[h] = (float)acc[d->H + h];
    }
    free(acc);
    return ORC_OK;
}

/* Reverse mode of orc_output_norm_gate, per row with inv = (mean o^2 + eps)^-1/2,
 * n = o inv, s = sigmoid(g), q = dy gamma g s:
 *   do = inv (q - n <q, n> / d_v);  dg = dy gamma n s (1 + g (1 - s));
 *   dgamma = sum over rows of dy n g s.
 * fp64; do, dg [B,T,H,d_v] and dgamma [d_v] rounded once to fp32. */
int orc_output_norm_gate_backward(const float *o, const void *g, const float *gamma, double eps, const float *dy,
                                  const orc_dims *d, float *dout, float *dg, float *dgamma)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->d_v < 1 || !(eps >= 0.0)) return ORC_EINVAL;
    const int64_t rows = d->B * d->T * d->H, dv = d->d_v;
    double *acc = (double *)calloc((size_t)dv, sizeof(double));
    double *q = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!acc || !q) {
        free(acc); free(q);
        return ORC_ENOMEM;
    }
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < dv; ++c) ss += (double)o[r * dv + c] * (double)o[r * dv + c];
        const double inv = 1.0 / sqrt(ss / (double)dv + eps);
        double qn = 0.0;
        for (int64_t c = 0; c < dv; ++c) {
            const double gc = load_in(g, d->in_bf16, r * dv + c), s = 1.0 / (1.0 + exp(-gc)),
                         ns = 1.0 / (1.0 + exp(gc));   /* 1 - s */
            const double n = (double)o[r * dv + c] * inv, y = (double)dy[r * dv + c];
            q[c] = y * (double)gamma[c] * gc * s;
            qn += q[c] * n;
            dg[r * dv + c] = (float)(y * (double)gamma[c] * n * s * (1.0 + gc * ns));
            acc[c] += y * n * gc * s;
        }
        for (int64_t c = 0; c < dv; ++c)
            dout[r * dv + c] = (float)(inv * (q[c] - (double)o[r * dv + c] * inv * qn / (double)dv));
    }
    for (int64_t c = 0; c < dv; ++c) dgamma[c] = (float)acc[c];
    free(acc);
    free(q);
    return ORC_OK;
}
