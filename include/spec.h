/*
 * spec.h -- C ABI of libspec: the vocabulary-sized output side of one
 * speculative-decoding step on an MI355X (gfx950) GPU.
 *
 * Four operations, in the notation of the DSpark blog page ("[DeepSeek-6]
 * DSpark", xutianle.me) and the SGLang MTP/NextN walk-through page
 * ("DeepSeek-V4 MTP/NextN ...", akiyangdev):
 *   spec_markov_propose  draft x_1..x_gamma from p_k = softmax((U_k + B_k)/T),
 *                        B_k = W1[x_{k-1}] W2            (DSpark sections 3-4)
 *   spec_verify          lossless verification against target logits: accept,
 *                        residual resample, bonus token  (DSpark section 1
 *                        diagram; the verify window of gamma+1 target rows,
 *                        SGLang page section 3), with the confidence label
 *                        c* fused in                       (DSpark section 5)
 *   spec_confidence      c*_k = 1 - 1/2 ||p_d - p_t||_1 and a*_j = prod c*_i
 *                                                          (DSpark sections 5-6)
 *   spec_schedule        per-request verify lengths l_r maximising
 *                        Theta = tau * SPS(B), B = sum_r (1 + l_r),
 *                        tau = sum_r (1 + sum_{j<=l_r} a_{r,j}) (DSpark section 6)
 *   spec_draft_loss      training-side loss over the same rows: CE, L1/TV
 *                        and confidence BCE, position-weighted (section 9)
 *   spec_schedule_async  the production step: the same ranking, with the
 *                        verified count taken from the optimum two calls
 *                        earlier (a dynamic top-K)          (DSpark section 7)
 *   spec_cluster_propose a clustered draft head: coarse logits over cluster
 *                        centres, the top K_c clusters expanded through the
 *                        LM head, drafts from the softmax over their tokens
 *   spec_cluster_verify  lossless verification of those sparse drafts
 *                        (the MTP survey page, zdszero.github.io "spec_mtp":
 *                        Gemma 4 assistant section; FROZEN_KV_MTP in its
 *                        SGLang section expands the top 32 by default)
 *
 * Conventions shared by every entry point
 *   Memory      Every pointer argument is DEVICE memory unless its comment says
 *               host.  The caller allocates and frees everything, including
 *               the workspace; the library never allocates, frees or retains
 *               caller memory and keeps no per-call state outside `ws`.
 *   Layout      Row-major, vocabulary index fastest.  U [R,gamma,V] and
 *               Lt [R,gamma+1,V] are fp32.  W1 and W2 are [V,r]: W1 row x is
 *               the embedding of token x; W2 row v holds the weights of output
 *               v of the bias-free projection r -> V, so
 *               B_k[v] = sum_i W1[x_{k-1}, i] * W2[v, i]  (the transpose of the
 *               r x V matrix in the page's formula, i.e. the usual storage of
 *               a linear layer's weight).  The hot-path calls take W2 after
 *               spec_pack_w2 has rearranged it once (W2p): the same values in
 *               the order the kernels stream them.  Target row k-1 of a
 *               request checks draft x_k; target row l_r gives the bonus token.
 *   Alignment   U, Lt, W1, W2, W2p must be 16-byte aligned; r % 16 == 0.
 *   Asynchrony  Calls only validate on the host and enqueue kernels on
 *               `stream` (a hipStream_t; NULL = the null stream).  Outputs are
 *               valid once the caller synchronises that stream.
 *   Randomness  Every uniform is Philox4x32-10 with key = seed and counter =
 *               (k, request, round_lo, round_hi); word 0 draws x_k (the Markov
 *               head's and the clustered head's draft), word 1 is the accept
 *               test at k, word 2 the residual draw at k or the bonus draw at
 *               k = l_r + 1; u = (w >> 8) * 2^-24.  Every draw is by inverse
 *               CDF in vocabulary order (smallest v whose running sum exceeds
 *               u * total), so results are a pure function of (inputs, seed,
 *               round).
 *   Greedy      greedy != 0 replaces every draw by the lowest-index argmax of
 *               the same logits (draft: U+B; accept iff x_k equals the target
 *               argmax).  Probabilities and c* are still reported at T.
 *   Errors      Return SPEC_OK or an error code.  All argument checks happen
 *               on the host before anything is enqueued; nothing is coerced.
 *               Token ids, lengths and confidences that live in device memory
 *               are checked by the kernels: the request's outputs become -1 /
 *               NaN and a bit is OR-ed into the workspace status word, read by
 *               spec_device_status().
 *   Threads     Calls with distinct workspaces may run concurrently.
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* spec_stream_t; /* identical to hipStream_t */

enum spec_status {
    SPEC_OK = 0,
    SPEC_EINVAL = 1,      /* bad scalar, NULL required pointer, misalignment    */
    SPEC_EDTYPE = 2,      /* unknown weight dtype                               */
    SPEC_EWORKSPACE = 3,  /* ws NULL or smaller than spec_workspace_bytes()     */
    SPEC_ELAUNCH = 4,     /* the HIP runtime reported an error at launch        */
    SPEC_EDEVICE = 5,     /* spec_device_status(): a kernel saw bad device data */
    SPEC_EUNSUPPORTED = 6 /* size beyond what the kernels handle (see limits)   */
};

enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 };

enum spec_op {
    SPEC_OP_PROPOSE = 0,
    SPEC_OP_VERIFY = 1,
    SPEC_OP_CONFIDENCE = 2,
    SPEC_OP_SCHEDULE = 3,
    SPEC_OP_ROUNDS = 4, /* spec_decode_rounds */
    SPEC_OP_LOSS = 5    /* spec_draft_loss */
};

/* Bits of the device status word. */
enum spec_device_flag {
    SPEC_DEV_BAD_TOKEN = 1,       /* an anchor or draft id outside [0, V)          */
    SPEC_DEV_BAD_LENGTH = 2,      /* an l_r outside [0, gamma]                     */
    SPEC_DEV_BAD_CONFIDENCE = 4,  /* a confidence outside [0, 1] (or NaN)          */
    SPEC_DEV_BAD_CLUSTER = 16,    /* a clustering that is not a partition into
                                     non-empty clusters of at most max_cl tokens,
                                     or a selection naming a cluster outside it */
    SPEC_DEV_WAIT_FAILED = 8      /* the fused propose gave up waiting for another
                                     of its workgroups (not all of them could run
                                     at once: e.g. two fused calls on different
                                     streams of one GPU); that call's outputs are
                                     undefined                                    */
};

/* Limits: 1 <= R <= 65536, 1 <= gamma <= 64, 16 <= r <= 512 (r % 16 == 0;
 * r <= 256 for SPEC_F32 weights), 1 <= V <= 2^24, R*(gamma+1)*V < 2^40;
 * spec_schedule: R*gamma <= 8192. */

/* Bytes of workspace `op` needs for these sizes (B_max only for schedule).
 * Returns 0 for sizes the entry point would reject. */
size_t spec_workspace_bytes(int op, int R, int gamma, int r, int V, int B_max);

/* Zero all ws_bytes of a freshly allocated workspace (enqueued on stream):
 * the status word, the fused propose's call counter and its hand-over words.
 * Call once after allocating a workspace, and again if the memory was used
 * for anything else in between (a workspace is only ever valid for the
 * library after this call).  Returns SPEC_EWORKSPACE if ws is NULL or
 * ws_bytes < 256. */
int spec_workspace_init(void* ws, size_t ws_bytes, spec_stream_t stream);

/* Bytes of the packed W2 for these sizes (0 if rejected). */
size_t spec_packed_w2_bytes(int w_dtype, int r, int V);

/* Rearrange W2 [V,r] (w_dtype) into W2p, the layout the kernels stream: the
 * vocabulary is cut into blocks of 32 ids; within a block, for each step of
 * the rank dimension (16 for bf16, 8 for fp32), the 64 lanes' matrix-core
 * operands are contiguous (lane n + 32h holds row 32b + n, rank slice h of
 * the step), so every load is one coalesced 1 KB chunk.  Ids past V are
 * zero.  Run once per weight (e.g. at model load); W2p is caller-owned,
 * spec_packed_w2_bytes() long.  Enqueued on stream. */
int spec_pack_w2(const void* W2, int w_dtype, int r, int V, void* W2p, spec_stream_t stream);

/* spec_pack_w2 for W2 held as the page's r x V matrix (DSpark section 4,
 * B = W1[x] W2): W2_rv [r,V] row-major, W2_rv[i*V + v] = W2[v,i].  Same W2p.
 * W2_rv needs only its element alignment. */
int spec_pack_w2_rv(const void* W2_rv, int w_dtype, int r, int V, void* W2p, spec_stream_t stream);

/* Kernel-path choices of one call (the `path` argument of the _ex entry
 * points; 0 = the library picks).  Every path computes the same function;
 * they exist so that tests can run each kernel on any shape. */
enum spec_path {
    SPEC_PATH_AUTO = 0,
    SPEC_PATH_NO_FUSED_PROPOSE = 1,  /* per-position propose kernels even where the fused launch fits */
    SPEC_PATH_NO_PIPELINED_SWEEP = 2 /* staged verify sweep even where the pipelined one applies      */
};

/* Synchronise `stream`, then return the status word of `ws` in *flags (host
 * pointer; SPEC_DEV_* bits, sticky across calls).  clear != 0 zeroes it.
 * Returns SPEC_OK, or SPEC_EDEVICE when a bit is set. */
int spec_device_status(void* ws, spec_stream_t stream, int clear, int* flags);

/* Draft gamma tokens per request with the Markov head (DSpark sections 3-4):
 *   x_0 = x0[r];  for k = 1..gamma:
 *     z_k = U[r,k-1,:] + W1[x_{k-1}] W2^T        (raw draft logits)
 *     p_k = softmax(z_k / T);  x_k ~ p_k (word 0), or argmax z_k if greedy
 * The sample is one inverse CDF over the whole row in vocabulary order: the
 * smallest v whose running sum of p_k exceeds u = (w0 >> 8) 2^-24, w0 =
 * word 0 of Philox4x32-10 (key = seed) at counter (k, r, round_lo,
 * round_hi).  A row whose logits are all -inf (or NaN) has no sample: its
 * x_k is -1, p_d(x) and (M, S) are NaN, and the next position of that
 * request raises SPEC_DEV_BAD_TOKEN (its later outputs are -1 / NaN too).
 * In:  U [R,gamma,V] fp32; W1 [V,r] (w_dtype); W2p = spec_pack_w2(W2);
 *      x0 [R] int32.
 * Out: x [R,gamma] int32; pd_x [R,gamma] fp32 = p_k(x_k);
 *      pd_stats [R,gamma,2] fp32 = (M, S) with M = max_v z_k(v) and
 *      S = sum_v exp((z_k(v) - M)/T), so p_k(v) = exp((z_k(v)-M)/T)/S.
 * The gamma positions run serially on the device; nothing returns to the
 * host in between. */
int spec_markov_propose(const float* U, const void* W1, const void* W2p, int w_dtype,
                        const int32_t* x0, int R, int gamma, int r, int V, float T,
                        int greedy, uint64_t seed, uint64_t round,
                        int32_t* x, float* pd_x, float* pd_stats,
                        void* ws, size_t ws_bytes, spec_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * spec_markov_propose with its workspace in a static device array of
 * SPEC_NOALLOC_BYTES (8 MiB) that the library holds on every GPU it runs on
 * until the process ends, instead of a caller buffer.  Inputs, outputs and
 * their layouts are those of spec_markov_propose; the kernel path is the
 * default one.  flags (device, uint32 [1]) receives the SPEC_DEV_* bits this
 * call raised (the call clears them first).  Sizes whose propose workspace
 * (spec_workspace_bytes(SPEC_OP_PROPOSE, ...)) exceeds SPEC_NOALLOC_BYTES
 * return SPEC_EUNSUPPORTED before anything is enqueued (R*ceil(V/128) up to
 * about 230000 for R <= 32, about 690000 beyond).  The first call on a GPU
 * also enqueues one zero fill of the array on `stream`.  Every call on one
 * GPU shares that GPU's array and it keeps the last call's contents: calls
 * that overlap in time on one GPU (other streams or threads) race and must
 * not be issued.  Calls no hipMalloc, hipFree or allocating library routine. */
#define SPEC_NOALLOC_BYTES ((size_t)8 << 20)
int spec_markov_propose_noalloc(const float* U, const void* W1, const void* W2p, int w_dtype,
                                const int32_t* x0, int R, int gamma, int r, int V, float T,
                                int greedy, uint64_t seed, uint64_t round,
                                int32_t* x, float* pd_x, float* pd_stats, uint32_t* flags,
                                spec_stream_t stream);

/* spec_markov_propose with an explicit kernel path (SPEC_PATH_* bits; other
 * bits: SPEC_EINVAL).  Propose runs in one of two ways; tokens agree except
 * at decisions within fp32 rounding of a boundary (the logits are computed
 * with the same operands, the sums in a different order).
 * Fused: one launch for all gamma positions; each workgroup keeps the W2
 * columns of one 128-id granule in registers for the whole call, so W2 is
 * read from HBM once, and workgroups hand partials and tokens to each other
 * through the workspace.  It is taken when every granule's workgroup fits on
 * the device at once, r fills the matrix-core k-steps exactly (r = 64, 128,
 * 256 or 512 for bf16; 16, 64 or 256 for fp32), R <= 32 and path does not
 * hold SPEC_PATH_NO_FUSED_PROPOSE.  Its workgroups wait for one another, so
 * they must all run at once: a fused call shares the GPU safely with work
 * queued before or after it on its stream, but kernels running at the same
 * time on other streams or in other processes can take the slots some of
 * its workgroups need.  Every wait is bounded: after about 2^20 polls (a
 * second or more) the call gives up, its workgroups exit, its outputs are
 * undefined and SPEC_DEV_WAIT_FAILED is raised; the next call on the same
 * workspace is unaffected; a caller that sees the flag reruns the call with
 * SPEC_PATH_NO_FUSED_PROPOSE, whose kernels never wait for one another.
 * Otherwise: two kernels per position (partials, then the pick), W2 streamed
 * about once per position. */
int spec_markov_propose_ex(const float* U, const void* W1, const void* W2p, int w_dtype,
                           const int32_t* x0, int R, int gamma, int r, int V, float T,
                           int greedy, uint64_t seed, uint64_t round,
                           int32_t* x, float* pd_x, float* pd_stats, int path,
                           void* ws, size_t ws_bytes, spec_stream_t stream);

/* Several speculative rounds back to back on the device: the loop around
 * one step.  Round i (Philox round round0 + i) drafts gamma tokens from the
 * anchors a_i (spec_markov_propose), verifies all of them (spec_verify,
 * every position, c* optional), and the next anchor of each request is the
 * token it emitted last, y_i[r][n_acc_i[r]]: the correction after a
 * rejection or the bonus after a full accept (the bonus token is the next
 * round's first prediction position; DSpark section 1 cycle, section 3
 * anchor).  U and Lt are the same every round (they stand in for the
 * per-round backbone and target logits).  Nothing returns to the host
 * between rounds and the enqueued work contains no synchronisation, host
 * copy or memset, so the whole sequence can be captured in a HIP graph.
 * In:  U, W1, W2p, w_dtype, Lt, sizes, T, greedy, seed as for the two calls;
 *      x0 [R] the first anchors; n_rounds >= 1.
 * Out: anchors [n_rounds + 1, R] (anchors[0] = x0; -1 after an invalid
 *      token); x [n_rounds, R, gamma]; n_acc [n_rounds, R];
 *      y [n_rounds, R, gamma + 1]; c_star [n_rounds, R, gamma] or NULL.
 * ws: spec_workspace_bytes(SPEC_OP_ROUNDS, ...) bytes (it also holds each
 * round's p_d(x) and (M, S)). */
int spec_decode_rounds(const float* U, const void* W1, const void* W2p, int w_dtype,
                       const int32_t* x0, const float* Lt, int R, int gamma, int r, int V,
                       float T, int greedy, uint64_t seed, uint64_t round0, int n_rounds,
                       int32_t* anchors, int32_t* x, int32_t* n_acc, int32_t* y, float* c_star,
                       void* ws, size_t ws_bytes, spec_stream_t stream);
/* spec_decode_rounds with an explicit kernel path (SPEC_PATH_* bits). */
int spec_decode_rounds_ex(const float* U, const void* W1, const void* W2p, int w_dtype,
                          const int32_t* x0, const float* Lt, int R, int gamma, int r, int V,
                          float T, int greedy, uint64_t seed, uint64_t round0, int n_rounds,
                          int32_t* anchors, int32_t* x, int32_t* n_acc, int32_t* y, float* c_star,
                          int path, void* ws, size_t ws_bytes, spec_stream_t stream);

/* Verify drafts against target logits (standard lossless rule):
 *   for k = 1..l_r: accept x_k iff u1 < p_t,k(x_k) / p_k(x_k) (greedy: iff
 *   x_k == argmax Lt[r,k-1,:]); at the first rejection emit a draw from
 *   normalize(max(0, p_t,k - p_k)) (word 2 at k; p_t,k if that mass is 0;
 *   greedy: the target argmax); after l_r accepts emit the bonus draw from
 *   p_t,l_r+1 (word 2 at k = l_r + 1).  p_t,k = softmax(Lt[r,k-1,:] / T).
 * In:  U, W1, W2p, x0 as for propose; x [R,gamma] drafts; pd_stats from
 *      propose for the same drafts; Lt [R,gamma+1,V] fp32;
 *      ell [R] int32 verify lengths in [0,gamma], or NULL = gamma for all.
 * Out: n_acc [R] int32 accepted drafts (bonus excluded);
 *      y [R,gamma+1] int32 = x_1..x_{n_acc}, correction or bonus, then -1;
 *      pt_x [R,gamma] fp32 = p_t,k(x_k) (optional, NULL to skip);
 *      c_star [R,gamma] fp32 = 1 - 1/2 ||p_k - p_t,k||_1 clamped to [0,1]
 *      (optional; the sweep that forms the residual masses forms the TV
 *      masses too, so NULL only skips writing them).
 * Entries past l_r are NaN (pt_x, c_star). */
int spec_verify(const float* U, const void* W1, const void* W2p, int w_dtype,
                const int32_t* x0, const int32_t* x, const float* pd_stats,
                const float* Lt, const int32_t* ell,
                int R, int gamma, int r, int V, float T, int greedy,
                uint64_t seed, uint64_t round,
                int32_t* n_acc, int32_t* y, float* pt_x, float* c_star,
                void* ws, size_t ws_bytes, spec_stream_t stream);

/* spec_verify with an explicit kernel path (SPEC_PATH_* bits).  The sweep
 * recomputes the Markov bias of every verified row in 32-row blocks.  For
 * bf16 weights with r = 128 or 256 (every position verified, or lengths
 * ell) it runs as a software pipeline, one workgroup per compute unit: a
 * third of each workgroup computes the bias tiles on the matrix cores, with
 * the W1 rows of the next block loaded through registers one block ahead;
 * the rest streams U and target rows two blocks ahead and finishes each
 * block.  Otherwise (r = 512, fp32 weights, or with
 * SPEC_PATH_NO_PIPELINED_SWEEP) one workgroup does each block start to end.
 * Both compute the same products in the same order (identical results). */
int spec_verify_ex(const float* U, const void* W1, const void* W2p, int w_dtype,
                   const int32_t* x0, const int32_t* x, const float* pd_stats,
                   const float* Lt, const int32_t* ell,
                   int R, int gamma, int r, int V, float T, int greedy,
                   uint64_t seed, uint64_t round,
                   int32_t* n_acc, int32_t* y, float* pt_x, float* c_star, int path,
                   void* ws, size_t ws_bytes, spec_stream_t stream);

/* Confidence labels of every drafted position (DSpark section 5) and their
 * running products (section 6):
 *   c_star [R,gamma] fp32 = clamp(1 - 1/2 ||p_k - p_t,k||_1, 0, 1)
 *   a_star [R,gamma] fp64 = prod_{i<=k} c*_i, left to right (optional).
 * pd_stats may be NULL (the draft normalisers are then recomputed). */
int spec_confidence(const float* U, const void* W1, const void* W2p, int w_dtype,
                    const int32_t* x0, const int32_t* x, const float* pd_stats,
                    const float* Lt, int R, int gamma, int r, int V, float T,
                    float* c_star, double* a_star,
                    void* ws, size_t ws_bytes, spec_stream_t stream);
/* spec_confidence with an explicit kernel path (SPEC_PATH_* bits). */
int spec_confidence_ex(const float* U, const void* W1, const void* W2p, int w_dtype,
                       const int32_t* x0, const int32_t* x, const float* pd_stats,
                       const float* Lt, int R, int gamma, int r, int V, float T,
                       float* c_star, double* a_star, int path,
                       void* ws, size_t ws_bytes, spec_stream_t stream);

/* Hardware-aware prefix scheduler (DSpark section 6):
 *   a_{r,j} = prod_{i<=j} c_{r,i} in fp64, left to right;
 *   rank all (a, r, j) by a descending, then r, then j ascending;
 *   P_K = sum of the first K;  Theta(K) = (R + P_K) * SPS(R + K) for
 *   K = 0..min(R*gamma, B_max - R);  K* = smallest maximiser;
 *   l_r = number of request-r entries among the first K*.
 * Ranking by a is prefix-safe because a does not increase along j, and the
 * top-K set maximises tau for each batch size, so this is the exact optimum.
 * In:  c [R,gamma] fp32 confidences in [0,1]; sps [B_max] fp32 with
 *      sps[B-1] = SPS(B).  B_max >= R.
 * Out: ell [R] int32; a [R,gamma] fp64 (optional); K_star [1] int32;
 *      theta_star [1] fp64. */
int spec_schedule(const float* c, int R, int gamma, const float* sps, int B_max,
                  int32_t* ell, double* a, int32_t* K_star, double* theta_star,
                  void* ws, size_t ws_bytes, spec_stream_t stream);

/* Training-side loss of the draft over the same rows (DSpark section 9: a
 * cross-entropy, an L1/TV distribution-matching term and the confidence BCE
 * against the soft label c*, with position weights; DeepSpec's configuration
 * in section 8 uses a_ce = 0.1, a_tv = 0.9, a_conf = 1.0).  Teacher-forced:
 * position k's bias uses the label y_{k-1} (y_0 = x0), p_d = softmax((U_k +
 * B_k)/T), p_t = softmax(Lt[r,k-1,:]/T).  Per position
 *   ce = -log p_d(y_k),  l1 = ||p_d - p_t||_1 (= 2 TV),
 *   c* = clamp(1 - l1/2, 0, 1),  bce = BCE-with-logits(q_k, c*),
 *   w_k = exp(-(k-1)/gamma),
 *   *loss (fp64) = sum w_k (a_ce ce + a_tv l1 + a_conf bce) / sum w_k over
 *   all R*gamma positions;
 * terms [R,gamma,3] fp32 (optional) = (ce, l1, bce); dq [R,gamma] fp32
 * (optional) = d loss / d q (c* is a label: no gradient flows into it).
 * In: U, W1, W2 (packed), x0 as spec_markov_propose; y [R,gamma] int32 labels;
 * Lt [R,gamma+1,V] (rows 0..gamma-1 used); q [R,gamma] fp32.  R >= 1.
 * A label chain with an id outside [0, V) raises SPEC_DEV_BAD_TOKEN; those
 * positions get NaN terms and add nothing to the sum (the denominator is
 * unchanged). */
int spec_draft_loss(const float* U, const void* W1, const void* W2, int w_dtype,
                    const int32_t* x0, const int32_t* y, const float* Lt, const float* q,
                    int R, int gamma, int r, int V, float T,
                    float a_ce, float a_tv, float a_conf,
                    double* loss, float* terms, float* dq,
                    void* ws, size_t ws_bytes, spec_stream_t stream);

/* ---- Clustered draft head (the MTP survey page, zdszero.github.io
 * "spec_mtp": its Gemma 4 assistant section -- coarse logits from 2048
 * cluster centres, then only the top clusters go through the LM head -- and
 * the FROZEN_KV_MTP path of its SGLang section, top 32 by default).
 *
 * The vocabulary is partitioned into N_c non-empty clusters, given in CSR
 * form: cluster c holds tokens cl_tok[cl_off[c] .. cl_off[c+1]) in that
 * listed order (cl_off [N_c+1], cl_tok [V], int32).  Per drafted row (r, k)
 * with hidden h = H[r,k,:]:
 *   s_c = h . C[c]                 coarse logit of every cluster
 *   sel = the K_c clusters of largest s_c (ties: smaller index), ascending
 *   z_v = h . E[v]                 for the tokens v of the selected clusters
 *   p_d = softmax(z / T) over those tokens, 0 on every other token
 *   x_k = inverse CDF over them in expansion order (clusters ascending, each
 *         in its listed order) with Philox word 0 of counter (k, r, round);
 *         greedy: the largest z_v, ties to the smaller token id.
 * Positions are independent (no Markov bias; the clustered head replaces
 * the LM head that would produce the base logits).
 * Limits: bf16 H, C, E only; d % 16 == 0, 16 <= d <= 16384; N_c <= 8192;
 * K_c <= 256; max_cl <= 65536; K_c * max_cl <= 65536; R * gamma <= 2^20. */

/* Workspace bytes for spec_cluster_propose and spec_cluster_verify at these
 * sizes (0 if rejected).  The status word is the workspace's. */
size_t spec_cluster_workspace_bytes(int R, int gamma, int d, int N_c, int K_c, int max_cl, int V);

/* tok_slot [V] int32 = (c << 16) | i for cl_tok[cl_off[c] + i] = v: where
 * each token sits in the clustering (once per clustering, for
 * spec_cluster_verify).  Checks on the device that cl_off/cl_tok partition
 * [0, V) into non-empty clusters of at most 65536 tokens; otherwise raises
 * SPEC_DEV_BAD_CLUSTER (tok_slot is then unusable).  ws: any workspace of at
 * least 256 bytes (its status word). */
int spec_cluster_index(const int32_t* cl_off, const int32_t* cl_tok, int N_c, int V, int32_t* tok_slot,
                       void* ws, size_t ws_bytes, spec_stream_t stream);

/* Draft with the clustered head.
 * In:  H [R,gamma,d], C [N_c,d], E [V,d] (bf16, w_dtype = SPEC_BF16, 16-byte
 *      aligned); cl_off, cl_tok as above; max_cl >= the largest selected
 *      cluster (a larger one raises SPEC_DEV_BAD_CLUSTER and blanks the row).
 * Out: x [R,gamma] int32; pd_x [R,gamma] = p_d(x); sel [R,gamma,K_c]
 *      ascending cluster ids; zf [R,gamma,K_c,max_cl] fp32 fine logits of the
 *      expanded tokens (slot i of the j-th selected cluster; -inf past its
 *      size); pd_stats [R,gamma,2] = (M, Z) with M the largest z and
 *      Z = sum exp((z - M)/T) over the expanded tokens.
 * A row whose clusters break the limits or the partition gets x = -1, NaN
 * statistics and SPEC_DEV_BAD_CLUSTER. */
int spec_cluster_propose(const void* H, const void* C, const void* E, int w_dtype,
                         const int32_t* cl_off, const int32_t* cl_tok,
                         int R, int gamma, int d, int N_c, int K_c, int max_cl, int V, float T,
                         int greedy, uint64_t seed, uint64_t round,
                         int32_t* x, float* pd_x, int32_t* sel, float* zf, float* pd_stats,
                         void* ws, size_t ws_bytes, spec_stream_t stream);

/* Verify drafts of the clustered head: the rule of spec_verify (accept with
 * min(1, p_t/p_d), residual max(0, p_t - p_d) drawn over the whole
 * vocabulary in ascending id order, bonus from target row l_r) with p_d the
 * sparse distribution given by sel, zf and pd_stats from
 * spec_cluster_propose, found per token through tok_slot
 * (spec_cluster_index).  Outputs as spec_verify: n_acc [R], y [R,gamma+1],
 * pt_x [R,gamma] (optional), c_star [R,gamma] (optional; c* = clamp(1 -
 * 1/2 ||p_d - p_t||_1, 0, 1)).  ell [R] (optional) limits the verified
 * positions.  Lt [R,gamma+1,V] fp32, 16-byte aligned. */
int spec_cluster_verify(const int32_t* tok_slot, const int32_t* sel, const float* zf, const float* pd_stats,
                        const int32_t* x, const float* Lt, const int32_t* ell,
                        int R, int gamma, int N_c, int K_c, int max_cl, int V, float T,
                        int greedy, uint64_t seed, uint64_t round,
                        int32_t* n_acc, int32_t* y, float* pt_x, float* c_star,
                        void* ws, size_t ws_bytes, spec_stream_t stream);

/* Production step of the scheduler (DSpark section 7): the candidates are
 * ranked by the current confidences exactly as in spec_schedule, but the
 * number verified is the optimum K* that the scheduler found two calls
 * earlier -- a dynamic top-K whose size comes from history, so it is known
 * a step ahead (graph replay) and does not depend on the current tokens.
 *   K_hist [2] int32, device, in/out: K* of the previous two calls, oldest
 *     first; a negative entry means "none yet" (the current K* is used).
 *     The call reads K_hist[0] and leaves {K_hist[1], K*} (initialise both
 *     to -1; one ring per decode loop; calls on one ring must be ordered).
 *   K_used [1] int32 = min(K_hist[0], R*gamma), or K* when K_hist[0] < 0.
 *   ell [R] = number of request-r entries among the first K_used of the
 *     ranking (a descending, then request, then position).
 *   a, K_star, theta_star: as spec_schedule, for the current confidences.
 * A confidence outside [0,1] raises SPEC_DEV_BAD_CONFIDENCE, writes -1 to
 * ell, K_used and K_star and leaves K_hist unchanged.  Limits as
 * spec_schedule. */
int spec_schedule_async(const float* c, int R, int gamma, const float* sps, int B_max,
                        int32_t* K_hist, int32_t* ell, double* a, int32_t* K_used,
                        int32_t* K_star, double* theta_star,
                        void* ws, size_t ws_bytes, spec_stream_t stream);

/* Name of a status code (static string). */
const char* spec_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_H */
