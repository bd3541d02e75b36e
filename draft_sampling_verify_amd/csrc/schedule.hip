// schedule.hip -- hardware-aware prefix scheduler (DSpark blog page, section 6)
// and its production step with a two-call lag on the verified count
// (section 7).
//
// One workgroup of 1024 threads does the whole problem in LDS (R*gamma <=
// 8192 entries):
//   1. a_{r,j} = prod_{i<=j} c_{r,i} in fp64, left to right, per request;
//   2. the R per-request runs (already in order, a not increasing along j)
//      merged pairwise into the order a descending, then request, then
//      position ascending (log2 R merge levels);
//   3. fp64 prefix sums P_K of the sorted a;
//   4. Theta(K) = (R + P_K) * SPS(R + K) for K = 0..min(R*gamma, B_max - R),
//      K* = the smallest maximiser;
//   5. l_r = number of request-r entries among the first K*.
// Because a does not increase along j, the first K entries of that order
// are prefix-closed per request and carry the largest expected accepted
// mass among all allocations of K drafts; scanning every K is exact.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace spec {

constexpr int SCHED_THREADS = 1024;

// K_hist == NULL: the synchronous scheduler (l from the first K* entries).
// Otherwise the production step: l from the first K entries, K = K_hist[0]
// (the optimum two calls earlier; negative: none, use K*), capped at
// R*gamma; K_used = K, and the ring advances to {K_hist[1], K*}.
__global__ __launch_bounds__(SCHED_THREADS) void k_schedule(const float* c, int R, int gamma,
                                                            const float* sps, int B_max, int32_t* ell,
                                                            double* a_out, int32_t* K_star,
                                                            double* theta_star, int32_t* K_hist,
                                                            int32_t* K_used, uint32_t* status)
{
    // survival products by entry (o = r*gamma + j - 1), and the ranking as a
    // permutation of entries, ping-ponged between two index buffers while
    // the runs are merged; the spare buffer holds the per-request counts
    __shared__ double sa[SCHED_MAX_ENTRIES];
    __shared__ int ibuf[2][SCHED_MAX_ENTRIES];
    __shared__ double wsum[SCHED_THREADS / WAVE];
    __shared__ double best_th[SCHED_THREADS / WAVE];
    __shared__ int best_k[SCHED_THREADS / WAVE];
    __shared__ int bad;

    const int t = threadIdx.x;
    const int lane = t & (WAVE - 1), w = t / WAVE;
    const int n = R * gamma;
    if (t == 0) bad = 0;
    __syncthreads();

    // 1. survival products; each request's run is already in ranking order
    //    (a does not increase along j: a factor in [0,1] cannot round above
    //    the running product, and ties keep j ascending).  The confidences
    //    are first read coalesced into sa, then multiplied along each row.
    for (int o = t; o < n; o += SCHED_THREADS) {
        const float cv = c[o];
        if (!(cv >= 0.0f && cv <= 1.0f)) bad = 1;
        sa[o] = (double)cv;
        ibuf[0][o] = o;
    }
    __syncthreads();
    for (int r = t; r < R; r += SCHED_THREADS) {
        double run = 1.0;
        for (int j = 0; j < gamma; ++j) {
            const int o = r * gamma + j;
            run *= sa[o];
            sa[o] = run;
        }
    }
    __syncthreads();
    if (a_out)
        for (int o = t; o < n; o += SCHED_THREADS) a_out[o] = sa[o];
    if (bad) {
        if (t == 0) {
            raise_flag(status, 4u);
            *K_star = -1;
            *theta_star = NAN;
            if (K_used) *K_used = -1;  // the ring is left as it was
        }
        for (int r = t; r < R; r += SCHED_THREADS) ell[r] = -1;
        return;
    }

    // 2. merge runs pairwise, gamma -> 2 gamma -> ... -> n, into the order
    //    a descending, then entry (request, position) ascending.  Each thread
    //    writes a contiguous chunk of the output; where a chunk starts (or a
    //    new pair of runs begins) its split between the two runs is found by
    //    binary search on the merge path.
    auto ranks_first = [&](int x, int y) { return sa[x] > sa[y] || (sa[x] == sa[y] && x < y); };
    const int per = (n + SCHED_THREADS - 1) / SCHED_THREADS;
    int cur = 0;
    for (int run = gamma; run < n; run *= 2, cur ^= 1) {
        const int* src = ibuf[cur];
        int* dst = ibuf[cur ^ 1];
        const int p0 = min(t * per, n), p1 = min(p0 + per, n);
        int i = 0, j = 0, base = -1, la = 0, lb = 0;
        for (int p = p0; p < p1; ++p) {
            const int pb = p - p % (2 * run);
            if (pb != base) {
                base = pb;
                la = min(run, n - base);
                lb = min(run, n - base - la);
                const int q = p - base;
                int lo = max(0, q - lb), hi = min(q, la);
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (ranks_first(src[base + mid], src[base + la + q - mid - 1])) lo = mid + 1;
                    else hi = mid;
                }
                i = lo;
                j = q - lo;
            }
            const bool take_a = j >= lb || (i < la && ranks_first(src[base + i], src[base + la + j]));
            dst[p] = take_a ? src[base + i++] : src[base + la + j++];
        }
        __syncthreads();
    }
    const int* idx = ibuf[cur];
    int* cnt = ibuf[cur ^ 1];

    // 3. inclusive prefix sums over the first n sorted values, in place;
    //    each thread owns a contiguous run of `per` entries
    const int i0 = min(t * per, n), i1 = min(i0 + per, n);
    double local = 0.0;
    for (int i = i0; i < i1; ++i) local += sa[idx[i]];
    // block exclusive scan of `local` (fp64)
    double incl = local;
    for (int o = 1; o < WAVE; o <<= 1) {
        const double v = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += v;
    }
    double ex = __shfl_up(incl, 1, WAVE);
    if (lane == 0) ex = 0.0;
    if (lane == WAVE - 1) wsum[w] = incl;
    __syncthreads();
    double before = 0.0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    double run = before + ex;

    // 4. Theta(K) and its argmax (smallest K on ties)
    const int Kmax = min(n, B_max - R);
    double bth = -INFINITY;
    int bk = 0x7fffffff;
    if (t == 0) {
        bth = (double)R * (double)sps[R - 1];
        bk = 0;
    }
    for (int i = i0; i < i1; ++i) {
        run += sa[idx[i]];
        const int K = i + 1;
        if (K <= Kmax) {
            const double th = ((double)R + run) * (double)sps[R + K - 1];
            if (th > bth) { bth = th; bk = K; }
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const double ot = __shfl_xor(bth, o, WAVE);
        const int ok = __shfl_xor(bk, o, WAVE);
        if (ot > bth || (ot == bth && ok < bk)) { bth = ot; bk = ok; }
    }
    if (lane == 0) {
        best_th[w] = bth;
        best_k[w] = bk;
    }
    __syncthreads();
    double th_star = best_th[0];
    int k_star = best_k[0];
    for (int i = 1; i < SCHED_THREADS / WAVE; ++i)
        if (best_th[i] > th_star || (best_th[i] == th_star && best_k[i] < k_star)) {
            th_star = best_th[i];
            k_star = best_k[i];
        }

    // 5. per-request counts among the first K* (production step: the first
    //    K of the history)
    int k_use = k_star;
    if (K_hist) {
        const int h = K_hist[0];
        k_use = h >= 0 ? min(h, n) : k_star;
    }
    for (int r = t; r < R; r += SCHED_THREADS) cnt[r] = 0;
    __syncthreads();
    for (int i = t; i < k_use; i += SCHED_THREADS) atomicAdd(&cnt[idx[i] / gamma], 1);
    __syncthreads();
    for (int r = t; r < R; r += SCHED_THREADS) ell[r] = cnt[r];
    if (t == 0) {
        *K_star = k_star;
        *theta_star = th_star;
        if (K_hist) {
            *K_used = k_use;
            K_hist[0] = K_hist[1];
            K_hist[1] = k_star;
        }
    }
}

hipError_t launch_schedule(const float* c, int R, int gamma, const float* sps, int B_max, int32_t* ell,
                           double* a, int32_t* K_star, double* theta_star, int32_t* K_hist, int32_t* K_used,
                           uint32_t* status, hipStream_t s)
{
    {
        ProfScope ps("schedule", s);
        hipLaunchKernelGGL(k_schedule, dim3(1), dim3(SCHED_THREADS), 0, s, c, R, gamma, sps, B_max, ell, a,
                           K_star, theta_star, K_hist, K_used, status);
    }
    return hipGetLastError();
}

}  // namespace spec
