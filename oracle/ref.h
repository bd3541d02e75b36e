/*
 * ref.h -- CPU oracle for the output side of one speculative-decoding step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library (no headers, helpers, constants or generated tables).
 *
 * Everything is plain single-threaded C in double precision, loops in
 * ascending index order, written from the equations of the DSpark blog page
 * ("[DeepSeek-6] DSpark", xutianle.me):
 *   - draft distribution p_k = softmax(U_k + B_k)           (section 3, eq. for p_k)
 *   - Markov bias B(x_{k-1}, .) = W1[x_{k-1}] W2             (section 4, eq. for B)
 *   - confidence label c*_k = 1 - 1/2 ||p_d - p_t||_1         (section 5, eq. for c*)
 *   - survival a_{r,j} = prod_{i<=j} c_{r,i}                   (section 6, eq. for a)
 *   - batch B = sum_r (1 + l_r), tau = sum_r (1 + sum_j a_rj),
 *     Theta = tau * SPS(B), sort-greedy over a                  (section 6, eqs. + text)
 * and the standard lossless rejection rule the page relies on (section 3 says
 * the exact per-position draft probability is what rejection sampling needs;
 * the section 1 diagram keeps the longest accepted prefix and adds one bonus
 * token from the target).  The verify window [bonus, d_1..d_gamma] giving gamma+1 target rows
 * follows the SGLang walk-through page ("DeepSeek-V4 MTP/NextN ...", section 3).
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes): temperature T divides both logit sets; uniforms come from
 * Philox4x32-10 with key = seed, counter = (k, request, round_lo, round_hi),
 * word 0 = draft sample, word 1 = accept test, word 2 = residual / bonus draw,
 * u = (w >> 8) * 2^-24; the inverse CDF picks the smallest v whose running
 * sum exceeds u * total; argmax ties go to the lowest index.
 *
 * Layouts (row-major, all sizes in elements):
 *   U   [R, gamma, V]   fp32 base logits
 *   Lt  [R, gamma+1, V] fp32 target logits (row k-1 checks x_k, row l_r is the bonus row)
 *   W1  [V, r]          embedding of the previous token (fp32 or bf16 bits)
 *   W2  [V, r]          weight of the bias-free projection r -> V (out x in
 *                       storage), so B[v] = sum_i W1[x, i] * W2[v, i]; this is
 *                       the transpose of the r x V matrix in the page's formula.
 */
#ifndef SPEC_ORACLE_REF_H
#define SPEC_ORACLE_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { REF_F32 = 0, REF_BF16 = 1 };

/* Philox4x32-10 block (Salmon et al., SC'11): 10 rounds, bumping the key by
 * the Weyl constants between rounds. */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
/* The four words for (seed, round, request id, position k). */
void ref_draw(uint64_t seed, uint64_t round, int32_t req, int32_t k, uint32_t out[4]);
/* out[4i .. 4i+3] = the block at counter (i mod 2^16, i / 2^16, round_lo,
 * round_hi), key = seed, for i < n (a bulk form for comparisons). */
void ref_philox_words(uint64_t seed, uint64_t round, uint64_t n, uint32_t* out);
/* 24-bit uniform in [0, 1 - 2^-24]. */
double ref_u24(uint32_t w);

/* B[v] = sum_i W1[xprev, i] * W2[v, i], accumulated in double, i ascending. */
void ref_bias(const void* W1, const void* W2, int w_dtype, int r, int V,
              int32_t xprev, double* B);
/* Inverse CDF on non-negative weights w[0..V): smallest v with
 * sum_{i<=v} w_i > u * sum_i w_i; if rounding leaves none, the largest v with
 * w_v > 0.  *margin = min(F(v) - u, u - F(v-1)) on the normalised CDF. */
int32_t ref_inverse_cdf(const double* w, int V, double u, double* margin);
/* Lowest index of the maximum of z[0..V); *margin = top1 - top2 (0 on ties). */
int32_t ref_argmax(const double* z, int V, double* margin);

/* Markov-head proposal over gamma positions.
 *   req_ids  : Philox request index of each row (NULL -> 0..R-1)
 *   x_cond   : NULL for free running; else [R,gamma] tokens whose prefix
 *              conditions each position (conditioned mode)
 * Outputs (all [R,gamma], stats [R,gamma,2]):
 *   x       : drafted tokens
 *   pd_x    : p_d(x_k)
 *   pd_stats: (M, S) with M = max_v (U+B)(v), S = sum_v exp(((U+B)(v) - M)/T)
 *   margin  : decision margin (CDF margin when sampled, top1-top2 logit when greedy)
 * A row whose logits are all -inf (or NaN) has no distribution: its x is -1,
 * pd_x and pd_stats NaN, and so are the later positions of that request
 * (free running); an anchor outside [0, V) blanks the whole request.
 * Returns 0; 1 if some request was blanked that way; -1 on a bad argument. */
int ref_markov_propose(const float* U, const void* W1, const void* W2, int w_dtype,
                       const int32_t* x0, int R, int gamma, int r, int V, float T,
                       int greedy, uint64_t seed, uint64_t round,
                       const int32_t* req_ids, const int32_t* x_cond,
                       int32_t* x, double* pd_x, double* pd_stats, double* margin);

/* Lossless verification of the drafts x against the target rows Lt.
 *   ell      : verified length per request (NULL -> gamma for every request)
 * Outputs:
 *   n_acc    [R]          accepted drafts (bonus excluded)
 *   y        [R,gamma+1]  x_1..x_{n_acc}, then the correction/bonus token, then -1
 *   pt_x, pd_x, c_star [R,gamma]   per verified position (NaN past ell)
 * Per-position instrumentation for the conditioned comparison (any may be NULL):
 *   acc      [R,gamma]    accept decision at k (1/0; -1 past ell)
 *   acc_margin [R,gamma]  |u - min(1, p_t/p_d)| (greedy: top1-top2 of the target row)
 *   y_alt    [R,gamma+1]  token drawn if k were the first rejection (index k-1),
 *                         and the bonus draw at index ell
 *   y_margin [R,gamma+1]  decision margin of each y_alt draw
 * Returns 0 or -1. */
int ref_verify(const float* U, const void* W1, const void* W2, int w_dtype,
               const int32_t* x0, const int32_t* x, const float* Lt, const int32_t* ell,
               int R, int gamma, int r, int V, float T, int greedy,
               uint64_t seed, uint64_t round, const int32_t* req_ids,
               int32_t* n_acc, int32_t* y, double* pt_x, double* pd_x, double* c_star,
               int32_t* acc, double* acc_margin, int32_t* y_alt, double* y_margin);

/* Confidence labels c*_{r,k} for every drafted position, and their running
 * products a*_{r,j} = prod_{i<=j} c*_{r,i}. */
int ref_confidence(const float* U, const void* W1, const void* W2, int w_dtype,
                   const int32_t* x0, const int32_t* x, const float* Lt,
                   int R, int gamma, int r, int V, float T,
                   double* c_star, double* a_star);

/* Training-side loss over the drafted positions (DSpark section 9),
 * teacher-forced on the labels y [R,gamma] (the bias of position k uses
 * y_{k-1}, y_0 = x0); q [R,gamma] confidence logits.  Per position
 * ce = -log p_d(y_k), l1 = ||p_d - p_t||_1, bce = BCE-with-logits(q, c*),
 * weights w_k = exp(-(k-1)/gamma):
 *   *loss = sum w_k (a_ce ce + a_tv l1 + a_conf bce) / sum w_k
 * Optional: terms [R,gamma,3] = (ce, l1, bce); dq [R,gamma] = d loss / dq.
 * Returns 0, or -1 on a bad argument or token. */
int ref_draft_loss(const float* U, const void* W1, const void* W2, int w_dtype,
                   const int32_t* x0, const int32_t* y, const float* Lt, const float* q,
                   int R, int gamma, int r, int V, float T, float a_ce, float a_tv, float a_conf,
                   double* loss, double* terms, double* dq);

/* Hardware-aware prefix scheduler.
 *   c   [R,gamma] confidences in [0,1];  sps[B-1] = SPS(B) for B = 1..B_max
 * Outputs: ell [R], a [R,gamma] (may be NULL), *K_star, *theta_star,
 *   *theta_margin = (Theta(K*) - max_{K != K*} Theta(K)) / Theta(K*)  (may be NULL)
 *   *a_gap = relative gap between the K*-th and (K*+1)-th sorted a (may be NULL)
 * Returns 0, or -1 on a bad argument (c outside [0,1], B_max < R, ...). */
int ref_schedule(const float* c, int R, int gamma, const float* sps, int B_max,
                 int32_t* ell, double* a, int32_t* K_star, double* theta_star,
                 double* theta_margin, double* a_gap);

/* Production (asynchronous) variant of the scheduler (DSpark blog page,
 * section 7): the candidates are ranked by the current confidences, while
 * the number verified, K, is the scheduler's optimum from two calls earlier
 * (a dynamic top-K; the capacity comes from history, so the choice does not
 * look at the current tokens).
 *   K_hist [2] in/out: K* of the two previous calls, oldest first; a
 *   negative entry means "none yet", and the current call's own optimum is
 *   used instead.  On return K_hist = {K_hist[1], K*} (the ring advanced).
 * Outputs: ell [R] = counts per request among the first K_used entries of
 * the ranking (a descending, then request, then position); a [R,gamma]
 * (may be NULL); *K_used = min(K, R*gamma); *K_star, *theta_star,
 * *theta_margin as ref_schedule for the current confidences.
 * Returns 0, or -1 on a bad argument. */
int ref_schedule_async(const float* c, int R, int gamma, const float* sps, int B_max, int32_t* K_hist,
                       int32_t* ell, double* a, int32_t* K_used, int32_t* K_star, double* theta_star,
                       double* theta_margin);

/* Clustered draft head (the MTP survey page, zdszero.github.io "spec_mtp":
 * its Gemma 4 assistant section -- 2048 cluster centres give coarse logits,
 * the top clusters are expanded to cut the LM-head cost -- and the
 * FROZEN_KV_MTP path of its SGLang section, which expands the top 32 by
 * default).  Per drafted row (r, k) with hidden h = H[r,k,:]:
 *   s_c = h . C[c]            coarse logit of cluster c (c = 0..N_c-1)
 *   A   = the K_c clusters with the largest s_c (ties: smaller index),
 *         listed in ascending cluster index                     -> sel
 *   S   = the tokens of the clusters in A, in that order, each cluster's
 *         tokens in its listed (CSR) order: the expansion order
 *   z_v = h . E[v] for v in S;  p_d(v) = exp((z_v - M)/T) / Z on S, 0 elsewhere
 *   x   = inverse CDF over S in expansion order with u from Philox word 0
 *         (counter (k, request, round)); greedy: the largest z_v, ties to
 *         the smaller token id.
 * Positions are independent (no Markov bias: the clustered head replaces
 * the LM head that produces the base logits).
 * Layouts: H [R,gamma,d], C [N_c,d], E [V,d] (fp32 or bf16 bits, one dtype);
 * cl_off [N_c+1], cl_tok [V]: a partition of the vocabulary into non-empty
 * clusters (CSR).
 * Outputs: x, pd_x, sel [R,gamma,K_c], pd_stats [R,gamma,2] = (M, Z);
 * optional cut [R,gamma] = s_(K_c) - s_(K_c+1) (infinite when K_c = N_c) and
 * margin [R,gamma] (sampled: the inverse-CDF margin over the expanded
 * tokens; greedy: top1 - top2 logit).
 * Returns 0, or -1 on a bad argument or a cl_off/cl_tok that is not a
 * partition. */
int ref_cluster_propose(const void* H, const void* C, const void* E, int w_dtype,
                        const int32_t* cl_off, const int32_t* cl_tok,
                        int R, int gamma, int d, int N_c, int K_c, int V, float T,
                        int greedy, uint64_t seed, uint64_t round,
                        int32_t* x, double* pd_x, int32_t* sel, double* pd_stats,
                        double* cut, double* margin);

/* Verification of drafts from the clustered head: the same rule as
 * ref_verify with p_d the sparse distribution above, built from the given
 * selection sel (conditioned on the GPU's clusters as on its tokens).
 * The residual max(0, p_t - p_d) and the bonus are drawn over the whole
 * vocabulary in ascending id order; c* = clamp(1 - 1/2 ||p_d - p_t||_1).
 * Outputs and margins as ref_verify (pd_x may be NULL). */
int ref_cluster_verify(const void* H, const void* E, int w_dtype,
                       const int32_t* cl_off, const int32_t* cl_tok, const int32_t* sel,
                       const int32_t* x, const float* Lt, const int32_t* ell,
                       int R, int gamma, int d, int N_c, int K_c, int V, float T, int greedy,
                       uint64_t seed, uint64_t round,
                       int32_t* n_acc, int32_t* y, double* pt_x, double* pd_x, double* c_star,
                       int32_t* acc, double* acc_margin, int32_t* y_alt, double* y_margin);

#ifdef __cplusplus
}
#endif
#endif
