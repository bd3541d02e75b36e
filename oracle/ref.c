/*
 * ref.c -- CPU oracle (test infrastructure only; see ref.h for the contract,
 * the sources each function follows and the readings taken where the pages
 * are silent).  Plain C, double precision, single thread, no blocking or
 * fusion: each function is the definition written out.
 */
#include "ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ Philox */

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 * as 1, 2, 3", SC'11).  One round: two 32x32->64 products of counter words 0
 * and 2 with the round multipliers; the high halves are xor-ed with the other
 * counter words and the key, the low halves are carried; the key is bumped by
 * the golden-ratio Weyl constants before the next round. */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void ref_draw(uint64_t seed, uint64_t round, int32_t req, int32_t k, uint32_t out[4])
{
    uint32_t ctr[4] = {(uint32_t)k, (uint32_t)req, (uint32_t)round, (uint32_t)(round >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    ref_philox4x32_10(ctr, key, out);
}

void ref_philox_words(uint64_t seed, uint64_t round, uint64_t n, uint32_t* out)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t ctr[4] = {(uint32_t)(i % 65536u), (uint32_t)(i / 65536u), (uint32_t)round,
                                 (uint32_t)(round >> 32)};
        ref_philox4x32_10(ctr, key, out + 4 * i);
    }
}

double ref_u24(uint32_t w)
{
    return (double)(w >> 8) * (1.0 / 16777216.0);
}

/* ----------------------------------------------------------------- helpers */

static double weight_at(const void* W, int w_dtype, size_t idx)
{
    if (w_dtype == REF_F32)
        return (double)((const float*)W)[idx];
    /* bf16: the upper half of an IEEE binary32; decoding is exact. */
    uint32_t bits = (uint32_t)((const uint16_t*)W)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Markov bias of the DSpark page, section 4: B(x, .) = W1[x] W2. */
void ref_bias(const void* W1, const void* W2, int w_dtype, int r, int V,
              int32_t xprev, double* B)
{
    for (int v = 0; v < V; ++v) {
        double acc = 0.0;
        for (int i = 0; i < r; ++i)
            acc += weight_at(W1, w_dtype, (size_t)xprev * r + i) *
                   weight_at(W2, w_dtype, (size_t)v * r + i);
        B[v] = acc;
    }
}

int32_t ref_inverse_cdf(const double* w, int V, double u, double* margin)
{
    double total = 0.0;
    for (int v = 0; v < V; ++v)
        total += w[v];
    double target = u * total;
    double run = 0.0, prev = 0.0;
    int32_t pick = -1;
    for (int v = 0; v < V; ++v) {
        prev = run;
        run += w[v];
        if (run > target) {
            pick = v;
            break;
        }
    }
    if (pick < 0) {
        /* rounding left the total at or below the target */
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) { pick = v; break; }
        if (margin) *margin = 0.0;
        return pick;
    }
    if (margin) {
        double hi = run / total - u, lo = u - prev / total;
        *margin = hi < lo ? hi : lo;
    }
    return pick;
}

int32_t ref_argmax(const double* z, int V, double* margin)
{
    int32_t best = 0;
    for (int v = 1; v < V; ++v)
        if (z[v] > z[best]) best = v;
    if (margin) {
        double second = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (v != best && z[v] > second) second = z[v];
        *margin = V > 1 ? z[best] - second : INFINITY;
    }
    return best;
}

/* softmax(z / T) over V entries: p[v] = exp((z[v] - M) / T) / S. */
static void softmax_T(const double* z, int V, double T, double* p, double* M_out, double* S_out)
{
    double M = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (z[v] > M) M = z[v];
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        p[v] = exp((z[v] - M) / T);
        S += p[v];
    }
    for (int v = 0; v < V; ++v)
        p[v] /= S;
    if (M_out) *M_out = M;
    if (S_out) *S_out = S;
}

/* Base logits plus Markov bias for request row `row`, draft position k (1-based). */
static void draft_logits(const float* U, const void* W1, const void* W2, int w_dtype,
                         int row, int k, int gamma, int r, int V, int32_t xprev, double* z)
{
    ref_bias(W1, W2, w_dtype, r, V, xprev, z);
    const float* u = U + ((size_t)row * gamma + (size_t)(k - 1)) * (size_t)V;
    for (int v = 0; v < V; ++v)
        z[v] = (double)u[v] + z[v];
}

static int bad_common(const float* U, const void* W1, const void* W2, int w_dtype,
                      const int32_t* x0, int R, int gamma, int r, int V, float T)
{
    if (!U || !W1 || !W2 || !x0) return 1;
    if (w_dtype != REF_F32 && w_dtype != REF_BF16) return 1;
    if (R < 0 || gamma < 1 || r < 1 || V < 1) return 1;
    if (!(T > 0.0f) || isinf(T)) return 1;
    return 0;
}

/* ----------------------------------------------------------------- propose */

/* DSpark page, section 3: x_k ~ p_k = softmax(U_k + B_k) with B_k from
 * x_{k-1} (section 4); the anchor x_0 conditions position 1.  Temperature T
 * divides the logits. */
int ref_markov_propose(const float* U, const void* W1, const void* W2, int w_dtype,
                       const int32_t* x0, int R, int gamma, int r, int V, float T,
                       int greedy, uint64_t seed, uint64_t round,
                       const int32_t* req_ids, const int32_t* x_cond,
                       int32_t* x, double* pd_x, double* pd_stats, double* margin)
{
    if (bad_common(U, W1, W2, w_dtype, x0, R, gamma, r, V, T) || !x) return -1;
    const double Td = (double)T;
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    if (!z || !p) { free(z); free(p); return -1; }
    int status = 0;
    for (int row = 0; row < R; ++row) {
        int32_t rid = req_ids ? req_ids[row] : row;
        int32_t xprev = x0[row];
        for (int k = 1; k <= gamma; ++k) {
            size_t o = (size_t)row * gamma + (size_t)(k - 1);
            if (xprev < 0 || xprev >= V) {
                /* no previous token (an anchor outside [0, V), or a row
                 * without a sample): the rest of the chain is undefined */
                x[o] = -1;
                if (pd_x) pd_x[o] = NAN;
                if (pd_stats) { pd_stats[2 * o] = NAN; pd_stats[2 * o + 1] = NAN; }
                if (margin) margin[o] = INFINITY;
                status = 1;
                xprev = -1;
                continue;
            }
            draft_logits(U, W1, W2, w_dtype, row, k, gamma, r, V, xprev, z);
            double M, S, mg;
            softmax_T(z, V, Td, p, &M, &S);
            if (!(S > 0.0) || isnan(S) || isinf(M)) {
                /* every logit -inf (or NaN): softmax is 0/0, there is no
                 * distribution to draw from */
                x[o] = -1;
                if (pd_x) pd_x[o] = NAN;
                if (pd_stats) { pd_stats[2 * o] = NAN; pd_stats[2 * o + 1] = NAN; }
                if (margin) margin[o] = INFINITY;
                status = 1;
                xprev = x_cond ? x_cond[o] : -1;
                continue;
            }
            int32_t tok;
            if (greedy) {
                tok = ref_argmax(z, V, &mg);
            } else {
                uint32_t w[4];
                ref_draw(seed, round, rid, k, w);
                tok = ref_inverse_cdf(p, V, ref_u24(w[0]), &mg);
            }
            x[o] = tok;
            if (pd_x) pd_x[o] = p[tok];
            if (pd_stats) { pd_stats[2 * o] = M; pd_stats[2 * o + 1] = S; }
            if (margin) margin[o] = mg;
            xprev = x_cond ? x_cond[o] : tok;
        }
    }
    free(z);
    free(p);
    return status;
}

/* ------------------------------------------------------------------ verify */

/* The draft distribution of one drafted position: fills pd[0..V) for row
 * `row`, position k (1-based), previous token xprev; returns 0, or -1 when
 * the inputs name a token outside [0, V). */
typedef int (*draft_pd_fn)(const void* ctx, int row, int k, int32_t xprev, double* pd);

struct markov_ctx {
    const float* U; const void* W1; const void* W2; int w_dtype;
    int gamma, r, V; double T; double* z;
};

static int markov_pd(const void* vctx, int row, int k, int32_t xprev, double* pd)
{
    const struct markov_ctx* c = (const struct markov_ctx*)vctx;
    if (xprev < 0 || xprev >= c->V) return -1;
    draft_logits(c->U, c->W1, c->W2, c->w_dtype, row, k, c->gamma, c->r, c->V, xprev, c->z);
    softmax_T(c->z, c->V, c->T, pd, NULL, NULL);
    return 0;
}

/* Lossless verification (standard rejection rule; see ref.h): accept x_k with
 * probability min(1, p_t(x_k)/p_d(x_k)); at the first rejection draw from
 * normalize(max(0, p_t - p_d)) (p_t itself if that mass is zero); after a
 * full accept draw the bonus token from the next target row.  c*_k follows
 * the DSpark page, section 5, for every verified position.  The draft
 * distribution comes from draft_pd; x0 (may be NULL) starts the chain of
 * previous tokens it receives. */
static int verify_core(draft_pd_fn draft_pd, const void* ctx,
                       const int32_t* x0, const int32_t* x, const float* Lt, const int32_t* ell,
                       int R, int gamma, int V, float T, int greedy,
                       uint64_t seed, uint64_t round, const int32_t* req_ids,
                       int32_t* n_acc, int32_t* y, double* pt_x, double* pd_x, double* c_star,
                       int32_t* acc, double* acc_margin, int32_t* y_alt, double* y_margin)
{
    const double Td = (double)T;
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    double* lt = (double*)malloc(sizeof(double) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    double* res = (double*)malloc(sizeof(double) * (size_t)V);
    if (!pd || !lt || !pt || !res) {
        free(pd); free(lt); free(pt); free(res);
        return -1;
    }
    int status = 0;
    for (int row = 0; row < R && status == 0; ++row) {
        int32_t rid = req_ids ? req_ids[row] : row;
        int L = ell ? ell[row] : gamma;
        if (L < 0 || L > gamma) { status = -1; break; }
        for (int k = 1; k <= gamma; ++k) {
            size_t o = (size_t)row * gamma + (size_t)(k - 1);
            if (pt_x) pt_x[o] = NAN;
            if (pd_x) pd_x[o] = NAN;
            if (c_star) c_star[o] = NAN;
            if (acc) acc[o] = -1;
            if (acc_margin) acc_margin[o] = NAN;
        }
        for (int k = 0; k <= gamma; ++k) {
            size_t o = (size_t)row * (gamma + 1) + (size_t)k;
            y[o] = -1;
            if (y_alt) y_alt[o] = -1;
            if (y_margin) y_margin[o] = NAN;
        }
        int first_reject = 0; /* 1-based; 0 = none */
        int32_t residual_tok = -1;
        int32_t xprev = x0 ? x0[row] : -1;
        for (int k = 1; k <= L; ++k) {
            size_t o = (size_t)row * gamma + (size_t)(k - 1);
            int32_t xk = x[o];
            if (xk < 0 || xk >= V || draft_pd(ctx, row, k, xprev, pd) != 0) { status = -1; break; }
            const float* lrow = Lt + ((size_t)row * (gamma + 1) + (size_t)(k - 1)) * (size_t)V;
            for (int v = 0; v < V; ++v)
                lt[v] = (double)lrow[v];
            softmax_T(lt, V, Td, pt, NULL, NULL);

            double l1 = 0.0;
            for (int v = 0; v < V; ++v)
                l1 += fabs(pd[v] - pt[v]);
            double cs = 1.0 - 0.5 * l1;
            if (cs < 0.0) cs = 0.0;
            if (cs > 1.0) cs = 1.0;
            if (c_star) c_star[o] = cs;
            if (pt_x) pt_x[o] = pt[xk];
            if (pd_x) pd_x[o] = pd[xk];

            uint32_t w[4];
            ref_draw(seed, round, rid, k, w);
            int accept;
            double am, ym;
            int32_t yk;
            if (greedy) {
                int32_t best = ref_argmax(lt, V, &am);
                accept = (xk == best);
                yk = best;
                ym = am;
            } else {
                double u1 = ref_u24(w[1]);
                double ratio;
                if (pd[xk] > 0.0)
                    ratio = pt[xk] / pd[xk];
                else
                    ratio = pt[xk] > 0.0 ? INFINITY : 0.0;
                accept = u1 < ratio;
                double lim = ratio < 1.0 ? ratio : 1.0;
                am = fabs(u1 - lim);
                double Z = 0.0;
                for (int v = 0; v < V; ++v) {
                    double d = pt[v] - pd[v];
                    res[v] = d > 0.0 ? d : 0.0;
                    Z += res[v];
                }
                yk = ref_inverse_cdf(Z > 0.0 ? res : pt, V, ref_u24(w[2]), &ym);
            }
            if (acc) acc[o] = accept;
            if (acc_margin) acc_margin[o] = am;
            if (y_alt) y_alt[(size_t)row * (gamma + 1) + (size_t)(k - 1)] = yk;
            if (y_margin) y_margin[(size_t)row * (gamma + 1) + (size_t)(k - 1)] = ym;
            if (!accept && first_reject == 0) {
                first_reject = k;
                residual_tok = yk;
            }
            xprev = xk;
        }
        if (status) break;

        /* bonus draw from target row L (checks nothing; follows x_1..x_L) */
        const float* brow = Lt + ((size_t)row * (gamma + 1) + (size_t)L) * (size_t)V;
        for (int v = 0; v < V; ++v)
            lt[v] = (double)brow[v];
        int32_t bonus;
        double bm;
        if (greedy) {
            bonus = ref_argmax(lt, V, &bm);
        } else {
            softmax_T(lt, V, Td, pt, NULL, NULL);
            uint32_t w[4];
            ref_draw(seed, round, rid, L + 1, w);
            bonus = ref_inverse_cdf(pt, V, ref_u24(w[2]), &bm);
        }
        if (y_alt) y_alt[(size_t)row * (gamma + 1) + (size_t)L] = bonus;
        if (y_margin) y_margin[(size_t)row * (gamma + 1) + (size_t)L] = bm;

        int na = first_reject ? first_reject - 1 : L;
        n_acc[row] = na;
        for (int k = 0; k < na; ++k)
            y[(size_t)row * (gamma + 1) + (size_t)k] = x[(size_t)row * gamma + (size_t)k];
        y[(size_t)row * (gamma + 1) + (size_t)na] = first_reject ? residual_tok : bonus;
    }
    free(pd); free(lt); free(pt); free(res);
    return status;
}

int ref_verify(const float* U, const void* W1, const void* W2, int w_dtype,
               const int32_t* x0, const int32_t* x, const float* Lt, const int32_t* ell,
               int R, int gamma, int r, int V, float T, int greedy,
               uint64_t seed, uint64_t round, const int32_t* req_ids,
               int32_t* n_acc, int32_t* y, double* pt_x, double* pd_x, double* c_star,
               int32_t* acc, double* acc_margin, int32_t* y_alt, double* y_margin)
{
    if (bad_common(U, W1, W2, w_dtype, x0, R, gamma, r, V, T) || !x || !Lt || !n_acc || !y)
        return -1;
    struct markov_ctx c = {U, W1, W2, w_dtype, gamma, r, V, (double)T, NULL};
    c.z = (double*)malloc(sizeof(double) * (size_t)V);
    if (!c.z) return -1;
    int st = verify_core(markov_pd, &c, x0, x, Lt, ell, R, gamma, V, T, greedy, seed, round, req_ids,
                         n_acc, y, pt_x, pd_x, c_star, acc, acc_margin, y_alt, y_margin);
    free(c.z);
    return st;
}

/* -------------------------------------------------------------- confidence */

/* DSpark page, section 5 (c*) and section 5/6 (prefix survival as a product). */
int ref_confidence(const float* U, const void* W1, const void* W2, int w_dtype,
                   const int32_t* x0, const int32_t* x, const float* Lt,
                   int R, int gamma, int r, int V, float T,
                   double* c_star, double* a_star)
{
    if (bad_common(U, W1, W2, w_dtype, x0, R, gamma, r, V, T) || !x || !Lt || !c_star)
        return -1;
    const double Td = (double)T;
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    double* lt = (double*)malloc(sizeof(double) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    if (!z || !pd || !lt || !pt) {
        free(z); free(pd); free(lt); free(pt);
        return -1;
    }
    int status = 0;
    for (int row = 0; row < R && status == 0; ++row) {
        int32_t xprev = x0[row];
        double run = 1.0;
        for (int k = 1; k <= gamma; ++k) {
            size_t o = (size_t)row * gamma + (size_t)(k - 1);
            if (xprev < 0 || xprev >= V) { status = -1; break; }
            draft_logits(U, W1, W2, w_dtype, row, k, gamma, r, V, xprev, z);
            softmax_T(z, V, Td, pd, NULL, NULL);
            const float* lrow = Lt + ((size_t)row * (gamma + 1) + (size_t)(k - 1)) * (size_t)V;
            for (int v = 0; v < V; ++v)
                lt[v] = (double)lrow[v];
            softmax_T(lt, V, Td, pt, NULL, NULL);
            double l1 = 0.0;
            for (int v = 0; v < V; ++v)
                l1 += fabs(pd[v] - pt[v]);
            double cs = 1.0 - 0.5 * l1;
            if (cs < 0.0) cs = 0.0;
            if (cs > 1.0) cs = 1.0;
            c_star[o] = cs;
            run *= cs;
            if (a_star) a_star[o] = run;
            xprev = x[o];
        }
    }
    free(z); free(pd); free(lt); free(pt);
    return status;
}

/* ------------------------------------------------------------ training loss */

/* Training-side loss over the drafted positions (DSpark page, section 9, the
 * weighted sum of a cross-entropy, an L1/TV and a confidence term with
 * position weights; the coefficients of DeepSpec's configuration, section 8,
 * are the caller's alphas).  Teacher-forced: the bias of position k uses the
 * label y_{k-1} (y_0 = the anchor).  Per position (r, k):
 *   ce  = -log p_d(y_k)
 *   l1  = sum_v |p_d(v) - p_t(v)|               (twice the TV distance)
 *   c*  = clamp(1 - l1 / 2, 0, 1)                 (section 5)
 *   bce = BCE-with-logits(q, c*) = max(q, 0) - q c* + log(1 + exp(-|q|))
 *   w_k = exp(-(k - 1) / gamma)
 * loss = sum_{r,k} w_k (a_ce ce + a_tv l1 + a_conf bce) / sum_{r,k} w_k, and
 * dq = d loss / d q = w_k a_conf (sigmoid(q) - c*) / sum w (c* is a label). */
int ref_draft_loss(const float* U, const void* W1, const void* W2, int w_dtype,
                   const int32_t* x0, const int32_t* y, const float* Lt, const float* q,
                   int R, int gamma, int r, int V, float T, float a_ce, float a_tv, float a_conf,
                   double* loss, double* terms, double* dq)
{
    if (bad_common(U, W1, W2, w_dtype, x0, R, gamma, r, V, T) || !y || !Lt || !q || !loss)
        return -1;
    const double Td = (double)T;
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    double* lt = (double*)malloc(sizeof(double) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    if (!z || !pd || !lt || !pt) {
        free(z); free(pd); free(lt); free(pt);
        return -1;
    }
    int status = 0;
    double wsum = 0.0, total = 0.0;
    for (int k = 1; k <= gamma; ++k)
        wsum += (double)R * exp(-(double)(k - 1) / (double)gamma);
    for (int row = 0; row < R && status == 0; ++row) {
        int32_t yprev = x0[row];
        for (int k = 1; k <= gamma; ++k) {
            size_t o = (size_t)row * gamma + (size_t)(k - 1);
            const int32_t yk = y[o];
            if (yprev < 0 || yprev >= V || yk < 0 || yk >= V) { status = -1; break; }
            draft_logits(U, W1, W2, w_dtype, row, k, gamma, r, V, yprev, z);
            softmax_T(z, V, Td, pd, NULL, NULL);
            const float* lrow = Lt + ((size_t)row * (gamma + 1) + (size_t)(k - 1)) * (size_t)V;
            for (int v = 0; v < V; ++v)
                lt[v] = (double)lrow[v];
            softmax_T(lt, V, Td, pt, NULL, NULL);
            double l1 = 0.0;
            for (int v = 0; v < V; ++v)
                l1 += fabs(pd[v] - pt[v]);
            double cs = 1.0 - 0.5 * l1;
            if (cs < 0.0) cs = 0.0;
            if (cs > 1.0) cs = 1.0;
            const double ce = -log(pd[yk]);
            const double qv = (double)q[o];
            const double bce = (qv > 0.0 ? qv : 0.0) - qv * cs + log1p(exp(-fabs(qv)));
            const double wk = exp(-(double)(k - 1) / (double)gamma);
            total += wk * ((double)a_ce * ce + (double)a_tv * l1 + (double)a_conf * bce);
            if (terms) {
                terms[3 * o] = ce;
                terms[3 * o + 1] = l1;
                terms[3 * o + 2] = bce;
            }
            if (dq) dq[o] = wk * (double)a_conf * (1.0 / (1.0 + exp(-qv)) - cs) / wsum;
            yprev = yk;
        }
    }
    *loss = total / wsum;
    free(z); free(pd); free(lt); free(pt);
    return status;
}

/* ---------------------------------------------------------------- schedule */

typedef struct {
    double a;
    int32_t r, j;
} ref_entry;

/* order: a descending, then request ascending, then position ascending */
static int entry_cmp(const void* pa, const void* pb)
{
    const ref_entry* x = (const ref_entry*)pa;
    const ref_entry* y = (const ref_entry*)pb;
    if (x->a > y->a) return -1;
    if (x->a < y->a) return 1;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->j != y->j) return x->j < y->j ? -1 : 1;
    return 0;
}

/* DSpark page, section 6: a_{r,j} = prod_{i<=j} c_{r,i};  B = sum_r (1 + l_r);
 * tau = sum_r (1 + sum_{j<=l_r} a_{r,j});  maximise Theta = tau * SPS(B) by
 * ranking every candidate extension by a, highest first (prefix-safe because
 * a does not increase along j).  For each total K of verified drafts the best
 * set is the top K of that ranking; the oracle scans every feasible K. */
int ref_schedule(const float* c, int R, int gamma, const float* sps, int B_max,
                 int32_t* ell, double* a, int32_t* K_star, double* theta_star,
                 double* theta_margin, double* a_gap)
{
    if (!c || !sps || !ell || !K_star || !theta_star) return -1;
    if (R < 1 || gamma < 1 || B_max < R) return -1;
    size_t n = (size_t)R * (size_t)gamma;
    for (size_t i = 0; i < n; ++i)
        if (!(c[i] >= 0.0f && c[i] <= 1.0f)) return -1;
    ref_entry* e = (ref_entry*)malloc(sizeof(ref_entry) * n);
    double* P = (double*)malloc(sizeof(double) * (n + 1));
    if (!e || !P) { free(e); free(P); return -1; }
    for (int r = 0; r < R; ++r) {
        double run = 1.0;
        for (int j = 1; j <= gamma; ++j) {
            size_t o = (size_t)r * gamma + (size_t)(j - 1);
            run *= (double)c[o];
            e[o].a = run;
            e[o].r = r;
            e[o].j = j;
            if (a) a[o] = run;
        }
    }
    qsort(e, n, sizeof(ref_entry), entry_cmp);
    P[0] = 0.0;
    for (size_t K = 1; K <= n; ++K)
        P[K] = P[K - 1] + e[K - 1].a;
    size_t Kmax = n;
    if ((size_t)(B_max - R) < Kmax) Kmax = (size_t)(B_max - R);
    size_t best = 0;
    double best_theta = -INFINITY;
    for (size_t K = 0; K <= Kmax; ++K) {
        double theta = ((double)R + P[K]) * (double)sps[R + K - 1];
        if (theta > best_theta) { best_theta = theta; best = K; }
    }
    if (theta_margin) {
        double second = -INFINITY;
        for (size_t K = 0; K <= Kmax; ++K) {
            if (K == best) continue;
            double theta = ((double)R + P[K]) * (double)sps[R + K - 1];
            if (theta > second) second = theta;
        }
        *theta_margin = Kmax > 0 ? (best_theta - second) / fabs(best_theta) : INFINITY;
    }
    if (a_gap) {
        if (best == 0 || best == n) {
            *a_gap = INFINITY;
        } else {
            double hi = e[best - 1].a, lo = e[best].a;
            *a_gap = hi > 0.0 ? (hi - lo) / hi : 0.0;
        }
    }
    for (int r = 0; r < R; ++r)
        ell[r] = 0;
    for (size_t K = 0; K < best; ++K)
        ell[e[K].r] += 1;
    *K_star = (int32_t)best;
    *theta_star = best_theta;
    free(e);
    free(P);
    return 0;
}

/* The asynchronous variant: K from the history ring, ranking from the
 * current survival products (both orders as in ref_schedule). */
int ref_schedule_async(const float* c, int R, int gamma, const float* sps, int B_max, int32_t* K_hist,
                       int32_t* ell, double* a, int32_t* K_used, int32_t* K_star, double* theta_star,
                       double* theta_margin)
{
    if (!K_hist || !K_used) return -1;
    /* the current optimum (also validates the arguments) */
    if (ref_schedule(c, R, gamma, sps, B_max, ell, a, K_star, theta_star, theta_margin, NULL) != 0) return -1;
    size_t n = (size_t)R * (size_t)gamma;
    long K = K_hist[0] >= 0 ? (long)K_hist[0] : (long)*K_star;
    if (K > (long)n) K = (long)n;
    /* rank the current products again and count the first K */
    ref_entry* e = (ref_entry*)malloc(sizeof(ref_entry) * n);
    if (!e) return -1;
    for (int r = 0; r < R; ++r) {
        double run = 1.0;
        for (int j = 1; j <= gamma; ++j) {
            size_t o = (size_t)r * gamma + (size_t)(j - 1);
            run *= (double)c[o];
            e[o].a = run;
            e[o].r = r;
            e[o].j = j;
        }
    }
    qsort(e, n, sizeof(ref_entry), entry_cmp);
    for (int r = 0; r < R; ++r)
        ell[r] = 0;
    for (long i = 0; i < K; ++i)
        ell[e[i].r] += 1;
    *K_used = (int32_t)K;
    K_hist[0] = K_hist[1];
    K_hist[1] = *K_star;
    free(e);
    return 0;
}

/* ---------------------------------------------------- clustered draft head */

/* cl_off/cl_tok partition [0, V) into non-empty clusters: offsets strictly
 * increasing from 0 to V, and every token listed exactly once. */
static int cluster_partition_ok(const int32_t* cl_off, const int32_t* cl_tok, int N_c, int V)
{
    if (cl_off[0] != 0 || cl_off[N_c] != V) return 0;
    for (int c = 0; c < N_c; ++c)
        if (cl_off[c + 1] <= cl_off[c]) return 0;  /* every cluster holds a token */
    unsigned char* seen = (unsigned char*)calloc((size_t)V, 1);
    if (!seen) return 0;
    int ok = 1;
    for (int i = 0; i < V && ok; ++i) {
        int32_t v = cl_tok[i];
        if (v < 0 || v >= V || seen[v]) ok = 0;
        else seen[v] = 1;
    }
    free(seen);
    return ok;
}

/* h . M[row] over d entries, in fp64. */
static double dot_row(const void* Hm, size_t hoff, const void* M, size_t row, int w_dtype, int d)
{
    double acc = 0.0;
    for (int i = 0; i < d; ++i)
        acc += weight_at(Hm, w_dtype, hoff + (size_t)i) * weight_at(M, w_dtype, row * (size_t)d + (size_t)i);
    return acc;
}

/* The K_c clusters of largest coarse logit (ties: smaller index), returned in
 * ascending cluster order; *cut = s of the last one taken minus the largest
 * s left out (infinite when nothing is left out). */
static void cluster_select(const void* H, size_t hoff, const void* C, int w_dtype, int d, int N_c, int K_c,
                           double* s, unsigned char* taken, int32_t* sel, double* cut)
{
    for (int c = 0; c < N_c; ++c) {
        s[c] = dot_row(H, hoff, C, (size_t)c, w_dtype, d);
        taken[c] = 0;
    }
    double last = INFINITY;
    for (int j = 0; j < K_c; ++j) {
        int best = -1;
        for (int c = 0; c < N_c; ++c)
            if (!taken[c] && (best < 0 || s[c] > s[best])) best = c;
        taken[best] = 1;
        last = s[best];
    }
    double out_best = -INFINITY;
    int n = 0;
    for (int c = 0; c < N_c; ++c) {
        if (taken[c]) sel[n++] = c;
        else if (s[c] > out_best) out_best = s[c];
    }
    if (cut) *cut = K_c < N_c ? last - out_best : INFINITY;
}

/* Expansion of the selected clusters: ids and fine logits z = h . E[id] in
 * expansion order; returns the count. */
static int cluster_expand(const void* H, size_t hoff, const void* E, int w_dtype, int d,
                          const int32_t* cl_off, const int32_t* cl_tok, const int32_t* sel, int K_c,
                          int32_t* ids, double* z)
{
    int n = 0;
    for (int j = 0; j < K_c; ++j)
        for (int i = cl_off[sel[j]]; i < cl_off[sel[j] + 1]; ++i) {
            ids[n] = cl_tok[i];
            z[n] = dot_row(H, hoff, E, (size_t)cl_tok[i], w_dtype, d);
            ++n;
        }
    return n;
}

static int bad_cluster(const void* H, const void* E, int w_dtype, const int32_t* cl_off, const int32_t* cl_tok,
                       int R, int gamma, int d, int N_c, int K_c, int V, float T)
{
    if (!H || !E || !cl_off || !cl_tok) return 1;
    if (w_dtype != REF_F32 && w_dtype != REF_BF16) return 1;
    if (R < 0 || gamma < 1 || d < 1 || N_c < 1 || K_c < 1 || K_c > N_c || V < 1) return 1;
    if (!(T > 0.0f) || isinf(T)) return 1;
    return !cluster_partition_ok(cl_off, cl_tok, N_c, V);
}

int ref_cluster_propose(const void* H, const void* C, const void* E, int w_dtype,
                        const int32_t* cl_off, const int32_t* cl_tok,
                        int R, int gamma, int d, int N_c, int K_c, int V, float T,
                        int greedy, uint64_t seed, uint64_t round,
                        int32_t* x, double* pd_x, int32_t* sel, double* pd_stats,
                        double* cut, double* margin)
{
    if (bad_cluster(H, E, w_dtype, cl_off, cl_tok, R, gamma, d, N_c, K_c, V, T) || !C || !x || !sel)
        return -1;
    const double Td = (double)T;
    double* s = (double*)malloc(sizeof(double) * (size_t)N_c);
    unsigned char* taken = (unsigned char*)malloc((size_t)N_c);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    if (!s || !taken || !ids || !z || !p) {
        free(s); free(taken); free(ids); free(z); free(p);
        return -1;
    }
    for (int row = 0; row < R; ++row)
        for (int k = 1; k <= gamma; ++k) {
            const size_t o = (size_t)row * gamma + (size_t)(k - 1);
            const size_t hoff = o * (size_t)d;
            int32_t* so = sel + o * (size_t)K_c;
            cluster_select(H, hoff, C, w_dtype, d, N_c, K_c, s, taken, so, cut ? cut + o : NULL);
            const int n = cluster_expand(H, hoff, E, w_dtype, d, cl_off, cl_tok, so, K_c, ids, z);
            double M, Z, mg;
            softmax_T(z, n, Td, p, &M, &Z);
            int pick;
            if (greedy) {
                /* the largest z; ties to the smaller token id */
                pick = 0;
                for (int i = 1; i < n; ++i)
                    if (z[i] > z[pick] || (z[i] == z[pick] && ids[i] < ids[pick])) pick = i;
                double second = -INFINITY;
                for (int i = 0; i < n; ++i)
                    if (i != pick && z[i] > second) second = z[i];
                mg = n > 1 ? z[pick] - second : INFINITY;
            } else {
                uint32_t w[4];
                ref_draw(seed, round, row, k, w);
                pick = ref_inverse_cdf(p, n, ref_u24(w[0]), &mg);
            }
            x[o] = ids[pick];
            if (pd_x) pd_x[o] = p[pick];
            if (pd_stats) { pd_stats[2 * o] = M; pd_stats[2 * o + 1] = Z; }
            if (margin) margin[o] = mg;
        }
    free(s); free(taken); free(ids); free(z); free(p);
    return 0;
}

struct cluster_ctx {
    const void* H; const void* E; int w_dtype;
    const int32_t* cl_off; const int32_t* cl_tok; const int32_t* sel;
    int gamma, d, N_c, K_c, V; double T;
    int32_t* ids; double* z; double* p;
};

static int cluster_pd(const void* vctx, int row, int k, int32_t xprev, double* pd)
{
    const struct cluster_ctx* c = (const struct cluster_ctx*)vctx;
    (void)xprev;
    const size_t o = (size_t)row * c->gamma + (size_t)(k - 1);
    const int32_t* so = c->sel + o * (size_t)c->K_c;
    for (int j = 0; j < c->K_c; ++j)
        if (so[j] < 0 || so[j] >= c->N_c || (j > 0 && so[j] <= so[j - 1])) return -1;
    const int n = cluster_expand(c->H, o * (size_t)c->d, c->E, c->w_dtype, c->d, c->cl_off, c->cl_tok, so,
                                 c->K_c, c->ids, c->z);
    softmax_T(c->z, n, c->T, c->p, NULL, NULL);
    for (int v = 0; v < c->V; ++v)
        pd[v] = 0.0;
    for (int i = 0; i < n; ++i)
        pd[c->ids[i]] = c->p[i];
    return 0;
}

int ref_cluster_verify(const void* H, const void* E, int w_dtype,
                       const int32_t* cl_off, const int32_t* cl_tok, const int32_t* sel,
                       const int32_t* x, const float* Lt, const int32_t* ell,
                       int R, int gamma, int d, int N_c, int K_c, int V, float T, int greedy,
                       uint64_t seed, uint64_t round,
                       int32_t* n_acc, int32_t* y, double* pt_x, double* pd_x, double* c_star,
                       int32_t* acc, double* acc_margin, int32_t* y_alt, double* y_margin)
{
    if (bad_cluster(H, E, w_dtype, cl_off, cl_tok, R, gamma, d, N_c, K_c, V, T) || !sel || !x || !Lt ||
        !n_acc || !y)
        return -1;
    struct cluster_ctx c = {H, E, w_dtype, cl_off, cl_tok, sel, gamma, d, N_c, K_c, V, (double)T, NULL, NULL, NULL};
    c.ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
    c.z = (double*)malloc(sizeof(double) * (size_t)V);
    c.p = (double*)malloc(sizeof(double) * (size_t)V);
    int st = -1;
    if (c.ids && c.z && c.p)
        st = verify_core(cluster_pd, &c, NULL, x, Lt, ell, R, gamma, V, T, greedy, seed, round, NULL,
                         n_acc, y, pt_x, pd_x, c_star, acc, acc_margin, y_alt, y_margin);
    free(c.ids); free(c.z); free(c.p);
    return st;
}
