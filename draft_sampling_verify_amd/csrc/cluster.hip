// cluster.hip -- the clustered draft head (the MTP survey page,
// zdszero.github.io "spec_mtp": its Gemma 4 assistant section, where cluster
// centres give coarse logits and only the top clusters are expanded through
// the LM head, and the FROZEN_KV_MTP path of its SGLang section, which
// expands the top 32 by default).
//
// Per drafted row with hidden h (bf16, d wide):
//   coarse   s_c = h . C[c] for every cluster: one [rows, d] x [d, N_c]
//            contraction on MFMA, split over d so that the launch fills the
//            chip; the partial products are summed in a fixed order;
//   select   the K_c clusters of largest s (ties to the smaller index) by a
//            four-pass radix select on the order-preserving key of s, then
//            listed in ascending cluster index;
//   fine     z_v = h . E[v] for the tokens of the selected clusters: one
//            workgroup per (cluster, 32-row block) multiplies the cluster's
//            E rows by the block's hidden rows on MFMA, so a cluster's rows
//            of E are read once for all rows of the block that chose it,
//            and unselected clusters cost nothing;
//   sample   per row, softmax over the expanded tokens in expansion order
//            (cluster, then the cluster's listed order) and the inverse CDF
//            with the row's Philox word 0, or the largest logit (ties to the
//            smaller token id).
// Positions are independent: there is no serial chain.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spec {

constexpr int CL_THREADS = 256;
constexpr uint32_t DEV_BAD_CLUSTER = 16u;

// ---------------------------------------------------------------- index

__global__ void k_fill_i32(int32_t* p, int n, int32_t v)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// One workgroup per cluster: tok_slot[cl_tok[cl_off[c] + i]] = (c << 16) | i.
__global__ __launch_bounds__(CL_THREADS) void k_cluster_scatter(const int32_t* cl_off, const int32_t* cl_tok,
                                                                int N_c, int V, int32_t* tok_slot, uint32_t* status)
{
    const int c = blockIdx.x;
    const int c0 = cl_off[c], c1 = cl_off[c + 1];
    const bool ok = c0 >= 0 && c1 > c0 && c1 <= V && c1 - c0 <= CL_MAX_SIZE && (c > 0 || c0 == 0) &&
                    (c < N_c - 1 || c1 == V);
    if (!ok) {
        if (threadIdx.x == 0) raise_flag(status, DEV_BAD_CLUSTER);
        return;
    }
    for (int i = threadIdx.x; i < c1 - c0; i += CL_THREADS) {
        const int v = cl_tok[c0 + i];
        if (v < 0 || v >= V) raise_flag(status, DEV_BAD_CLUSTER);
        else tok_slot[v] = (int32_t)(((uint32_t)c << 16) | (uint32_t)i);
    }
}

// Every token must have been written exactly once: V slots and no -1 left
// means no token was listed twice.
__global__ void k_cluster_check(const int32_t* tok_slot, int V, uint32_t* status)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < V && tok_slot[i] < 0) raise_flag(status, DEV_BAD_CLUSTER);
}

hipError_t launch_cluster_index(const int32_t* cl_off, const int32_t* cl_tok, int N_c, int V, int32_t* tok_slot,
                                uint32_t* status, hipStream_t s)
{
    const int nb = (V + CL_THREADS - 1) / CL_THREADS;
    hipLaunchKernelGGL(k_fill_i32, dim3(nb), dim3(CL_THREADS), 0, s, tok_slot, V, -1);
    hipLaunchKernelGGL(k_cluster_scatter, dim3(N_c), dim3(CL_THREADS), 0, s, cl_off, cl_tok, N_c, V, tok_slot,
                       status);
    hipLaunchKernelGGL(k_cluster_check, dim3(nb), dim3(CL_THREADS), 0, s, tok_slot, V, status);
    return hipGetLastError();
}

// ------------------------------------------------------ MFMA row products
//
// acc_w[m][n] = sum_k A[arow[32 w + m]][k] * B[brow[n]][k] for the 128 A rows
// and 32 B rows of a workgroup (wave w takes A rows 32 w .. 32 w + 31) on
// v_mfma_f32_32x32x16_bf16.  The rows are gathered (token or cluster ids),
// so the operands are staged through LDS: per batch of 64 reduction
// elements every thread loads 16-byte pieces such that eight consecutive
// threads read one row's 128 contiguous bytes (whole cache lines), and the
// tiles are stored with a padded row stride (72 elements: the 32 rows of an
// MFMA operand read fall on distinct bank groups).  The next batch's loads
// are in flight during the current batch's products.  MFMA operand lane
// l = n + 32h reads row (l & 31), elements 16 s + 8h .. +7 of step s; the
// result lane l = n + 32h holds B row n and A rows m = 8 (j >> 2) + 4h +
// (j & 3).  Rows whose id is negative read row 0; their results are never
// stored.  All threads of the workgroup call this (it holds barriers).
constexpr int TS = 72;  // LDS row stride (elements) of a staged tile

struct TileStage {
    uint4 a[4];
    uint4 b;
};

__device__ inline void tile_load(TileStage& st, const bf16w* A, const int* s_arow, const bf16w* B, const int* s_brow,
                                 int d, int kb, int k1)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = t + CL_THREADS * u, row = q >> 3, part = q & 7;
        const int ar = s_arow[row];
        const int k = kb + 8 * part;
        st.a[u] = k < k1 ? *reinterpret_cast<const uint4*>(A + (size_t)(ar >= 0 ? ar : 0) * d + k)
                         : make_uint4(0, 0, 0, 0);
    }
    const int row = t >> 3, part = t & 7;
    const int br = s_brow[row];
    const int k = kb + 8 * part;
    st.b = k < k1 ? *reinterpret_cast<const uint4*>(B + (size_t)(br >= 0 ? br : 0) * d + k) : make_uint4(0, 0, 0, 0);
}

__device__ inline void tile_store(const TileStage& st, uint16_t* sA, uint16_t* sB)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = t + CL_THREADS * u;
        *reinterpret_cast<uint4*>(sA + (q >> 3) * TS + 8 * (q & 7)) = st.a[u];
    }
    *reinterpret_cast<uint4*>(sB + (t >> 3) * TS + 8 * (t & 7)) = st.b;
}

__device__ inline f32x16 tile_dot(const bf16w* A, const int* s_arow, const bf16w* B, const int* s_brow, int d, int k0,
                                  int k1, uint16_t* sA, uint16_t* sB)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE, h = lane >> 5;
    f32x16 acc = {};
    TileStage st;
    if (k0 < k1) tile_load(st, A, s_arow, B, s_brow, d, k0, k1);
    for (int kb = k0; kb < k1; kb += 64) {
        tile_store(st, sA, sB);
        __syncthreads();
        if (kb + 64 < k1) tile_load(st, A, s_arow, B, s_brow, d, kb + 64, k1);
        const uint16_t* pa = sA + (32 * w + (lane & 31)) * TS + 8 * h;
        const uint16_t* pb = sB + (lane & 31) * TS + 8 * h;
        const int steps = min(4, (k1 - kb) / 16);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            if (s2 < steps) {
                const uint4 av = *reinterpret_cast<const uint4*>(pa + 16 * s2);
                const uint4 bv = *reinterpret_cast<const uint4*>(pb + 16 * s2);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                              __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }
    return acc;
}

// ---------------------------------------------------------------- coarse

// Workgroup (column block cb of 128 clusters, row block rb of 32 rows,
// reduction split q): the 128 x 32 tile of coarse logits over the split's
// part of d, stored as part[q][row][cluster].
__global__ __launch_bounds__(CL_THREADS) void k_cluster_coarse(const bf16w* H, const bf16w* C, int N, int N_c, int d,
                                                               int nsplit, float* part)
{
    __shared__ __align__(16) uint16_t sA[128 * TS];
    __shared__ __align__(16) uint16_t sB[32 * TS];
    __shared__ int s_arow[128], s_brow[32];
    const int cb = blockIdx.x, rb = blockIdx.y, q = blockIdx.z;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE, h = lane >> 5;
    if (t < 128) s_arow[t] = cb * 128 + t < N_c ? cb * 128 + t : -1;
    if (t < 32) s_brow[t] = rb * 32 + t < N ? rb * 32 + t : -1;
    __syncthreads();
    const int ks = d / 16;
    const int k0 = 16 * (int)((long)q * ks / nsplit), k1 = 16 * (int)((long)(q + 1) * ks / nsplit);
    const f32x16 acc = tile_dot(C, s_arow, H, s_brow, d, k0, k1, sA, sB);
    const int row = rb * 32 + (lane & 31);
    if (row >= N) return;
    float* out = part + ((size_t)q * N + row) * N_c;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int m = cb * 128 + 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
        if (m < N_c) out[m] = acc[j];
    }
}

// ---------------------------------------------------------------- select

__device__ inline uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one int per thread over the workgroup (CL_THREADS).
__device__ inline int block_incl_scan(int v, int* s_tmp)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    int x = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) s_tmp[w] = x;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += s_tmp[i];
    __syncthreads();
    return base + x;
}

// One workgroup per row: s_c summed over the splits in order, then the
// K_c largest by radix select (8 bits a pass, most significant first) on
// the order-preserving key; keys equal to the K_c-th are taken in
// ascending cluster order.  Thread t owns clusters [t per, (t+1) per), so
// "ascending" is thread order, then position.
__global__ __launch_bounds__(CL_THREADS) void k_cluster_select(const float* part, int nsplit, int N, int N_c, int K_c,
                                                               int32_t* sel)
{
    __shared__ uint32_t s_key[CL_MAX_NC];
    __shared__ int s_hist[256];
    __shared__ int s_tmp[CL_THREADS / WAVE];
    __shared__ uint32_t s_digit;
    __shared__ int s_krem;
    const int n = blockIdx.x, t = threadIdx.x;
    if (t == 0) {
        s_digit = 0;
        s_krem = K_c;
    }
    // the splits' partial products, summed in split order, eight clusters
    // per thread in flight
    for (int cb = t; cb < N_c; cb += 8 * CL_THREADS) {
        float v[8] = {};
        for (int q = 0; q < nsplit; ++q) {
            const float* pq = part + ((size_t)q * N + n) * N_c;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = cb + u * CL_THREADS;
                v[u] += c < N_c ? pq[c] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = cb + u * CL_THREADS;
            if (c < N_c) s_key[c] = order_key(v[u]);
        }
    }
    uint32_t prefix = 0, pmask = 0;
    int krem = K_c;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        s_hist[t] = 0;
        __syncthreads();
        for (int c = t; c < N_c; c += CL_THREADS) {
            const uint32_t key = s_key[c];
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread t holds digit 255 - t: the scan counts keys with a digit >= it
        const int hv = s_hist[255 - t];
        const int ge = block_incl_scan(hv, s_tmp);
        if (hv > 0 && ge >= krem && ge - hv < krem) {
            s_digit = 255u - (uint32_t)t;
            s_krem = krem - (ge - hv);
        }
        __syncthreads();
        prefix |= s_digit << shift;
        pmask |= 255u << shift;
        krem = s_krem;
        __syncthreads();
    }
    // prefix = the K_c-th largest key; krem keys equal to it are taken
    const int per = (N_c + CL_THREADS - 1) / CL_THREADS;
    const int c0 = min(t * per, N_c), c1 = min(c0 + per, N_c);
    int ties = 0;
    for (int c = c0; c < c1; ++c) ties += s_key[c] == prefix;
    int tie_rank = block_incl_scan(ties, s_tmp) - ties;
    int nsel = 0;
    for (int c = c0; c < c1; ++c) {
        const uint32_t key = s_key[c];
        nsel += key > prefix || (key == prefix && tie_rank++ < krem);
    }
    int pos = block_incl_scan(nsel, s_tmp) - nsel;
    tie_rank = block_incl_scan(ties, s_tmp) - ties;
    int32_t* out = sel + (size_t)n * K_c;
    for (int c = c0; c < c1; ++c) {
        const uint32_t key = s_key[c];
        if (key > prefix || (key == prefix && tie_rank++ < krem)) {
            if (pos < K_c) out[pos] = c;  // exactly K_c are taken; the guard keeps writes in the row
            ++pos;
        }
    }
}

// ------------------------------------------------------------------ fine

// Workgroup (cluster c, row block rb): the rows of the block that selected
// c (binary search in each row's ascending list) get z = h . E[v] for the
// cluster's tokens, 128 per pass (32 per wave), written to
// zf[row][j][i] (j = c's place in the row's list, i = place in the
// cluster); slots from the cluster's size to max_cl get -inf.  Tokens
// outside [0, V) read row 0 and raise the flag (the sampler rejects the
// row).  Workgroups of clusters no row of the block selected exit at once.
__global__ __launch_bounds__(CL_THREADS) void k_cluster_fine(const bf16w* H, const bf16w* E, const int32_t* cl_off,
                                                             const int32_t* cl_tok, const int32_t* sel, int N, int K_c,
                                                             int max_cl, int d, int V, float* zf, uint32_t* status)
{
    __shared__ __align__(16) uint16_t sA[128 * TS];
    __shared__ __align__(16) uint16_t sB[32 * TS];
    __shared__ int s_arow[128], s_brow[32];
    __shared__ int s_j[32];
    __shared__ int s_any;
    const int c = blockIdx.x, rb = blockIdx.y;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE, h = lane >> 5;
    if (t < WAVE) {
        const int n = rb * 32 + (lane & 31);
        int j = -1;
        if (lane < 32 && n < N) {
            const int32_t* sr = sel + (size_t)n * K_c;
            int lo = 0, hi = K_c;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sr[mid] < c) lo = mid + 1;
                else hi = mid;
            }
            if (lo < K_c && sr[lo] == c) j = lo;
        }
        if (lane < 32) {
            s_j[lane] = j;
            s_brow[lane] = n < N ? n : -1;
        }
        const bool any = __ballot(j >= 0) != 0;
        if (lane == 0) s_any = any;
    }
    __syncthreads();
    if (!s_any) return;
    const int c0 = cl_off[c];
    int m = cl_off[c + 1] - c0;
    if (c0 < 0 || m < 0 || c0 + m > V) m = 0;  // the sampler flags the row
    if (m > max_cl) m = max_cl;
    const int nl = lane & 31;
    const int row = rb * 32 + nl;
    const int jr = s_j[nl];
    for (int i0 = 0; i0 < m; i0 += 128) {
        if (t < 128) {
            int tok = i0 + t < m ? cl_tok[c0 + i0 + t] : -1;
            if (tok >= V || (tok < 0 && i0 + t < m)) {
                raise_flag(status, DEV_BAD_CLUSTER);
                tok = -1;
            }
            s_arow[t] = tok;
        }
        __syncthreads();
        const f32x16 acc = tile_dot(E, s_arow, H, s_brow, d, 0, d, sA, sB);
        if (jr >= 0) {
            float* out = zf + ((size_t)row * K_c + jr) * max_cl;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int im = i0 + 32 * w + 8 * (jj >> 2) + 4 * h + (jj & 3);
                if (im < m) out[im] = acc[jj];
            }
        }
    }
    // padding of the selecting rows
    const int pad = max_cl - m;
    for (int e = t; e < 32 * pad; e += CL_THREADS) {
        const int rr = e / pad, ii = m + e % pad;
        const int jj = s_j[rr];
        if (jj >= 0) zf[((size_t)(rb * 32 + rr) * K_c + jj) * max_cl + ii] = -INFINITY;
    }
}

// ---------------------------------------------------------------- sample

template <typename T>
__device__ inline T block_reduce(T v, T* s_tmp, T (*op)(T, T), T (*wop)(T))
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    v = wop(v);
    if (lane == 0) s_tmp[w] = v;
    __syncthreads();
    T r = s_tmp[0];
    for (int i = 1; i < CL_THREADS / WAVE; ++i) r = op(r, s_tmp[i]);
    __syncthreads();
    return r;
}
__device__ inline float fmax_op(float a, float b) { return fmaxf(a, b); }
__device__ inline int imin_op(int a, int b) { return min(a, b); }
__device__ inline int imax_op(int a, int b) { return max(a, b); }
__device__ inline float wmax_f(float v) { return wave_max(v); }
__device__ inline int wmin_i(int v) { return wave_min(v); }
__device__ inline int wmax_i(int v) { return wave_max_int(v); }

// Running sum of one value per thread over the workgroup, waves in order:
// [lo, hi) is this thread's share.  Consecutive shares meet exactly (the next
// share's lo is computed by the same additions as this one's hi).
template <typename ACC>
__device__ inline void block_share(ACC v, ACC* s_tmp, ACC& lo, ACC& hi, ACC& total)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const ACC x = wave_incl_scan(v);
    ACC xe = __shfl_up(x, 1, WAVE);
    if (lane == 0) xe = 0;
    if (lane == WAVE - 1) s_tmp[w] = x;
    __syncthreads();
    ACC base = 0, tot = 0;
    for (int i = 0; i < CL_THREADS / WAVE; ++i) {
        if (i == w) base = tot;
        tot += s_tmp[i];
    }
    __syncthreads();
    total = tot;
    lo = lane == 0 ? base : base + xe;
    hi = base + x;
}

struct ClusterSampleArgs {
    const float* zf;
    const int32_t* sel;
    const int32_t* cl_off;
    const int32_t* cl_tok;
    int N, gamma, N_c, K_c, max_cl, V;
    float c;
    uint64_t seed, round;
    int32_t* x;
    float* pd_x;
    float* pd_stats;
    uint32_t* status;
};

// One workgroup per row f = (request, position).  Element e = j max_cl + i
// (cluster j of the row's list, place i in it); slots past a cluster's size
// hold -inf, so they weigh nothing and need no test.  Thread t owns the
// contiguous elements [t per, (t+1) per), so running sums follow the
// expansion order: within a thread in sequence, then threads in order.
// Loads go in batches of SB (one memory latency per batch).
constexpr int SB = 16;

// ACC: the precision of the running sums, float when a thread's share is at
// most 32 elements, double for longer shares (up to 256 of them), whose
// fp32 running sums would drift by more than 1e-6 of the row's mass.
template <bool GREEDY, typename ACC>
__global__ __launch_bounds__(CL_THREADS) void k_cluster_sample(ClusterSampleArgs a)
{
    __shared__ int s_c0[CL_MAX_K], s_m[CL_MAX_K];
    __shared__ float s_ftmp[CL_THREADS / WAVE];
    __shared__ ACC s_atmp[CL_THREADS / WAVE];
    __shared__ int s_itmp[CL_THREADS / WAVE];
    __shared__ int s_pick;
    const int f = blockIdx.x, t = threadIdx.x;
    const int r = f / a.gamma, k = f - r * a.gamma + 1;
    bool bad = false;
    if (t < a.K_c) {
        const int cj = a.sel[(size_t)f * a.K_c + t];
        int c0 = 0, m = 0;
        if (cj < 0 || cj >= a.N_c) {
            bad = true;
        } else {
            c0 = a.cl_off[cj];
            m = a.cl_off[cj + 1] - c0;
            bad = c0 < 0 || m < 0 || c0 + m > a.V || m > a.max_cl;
        }
        s_c0[t] = bad ? 0 : c0;
        s_m[t] = bad ? 0 : m;
    }
    const int n_el = a.K_c * a.max_cl;
    const int per = (n_el + CL_THREADS - 1) / CL_THREADS;
    const int e0 = min(t * per, n_el), e1 = min(e0 + per, n_el);
    const float* z = a.zf + (size_t)f * n_el;
    auto blank = [&]() {
        raise_flag(a.status, DEV_BAD_CLUSTER);
        a.x[f] = -1;
        a.pd_x[f] = NAN;
        a.pd_stats[2 * (size_t)f] = NAN;
        a.pd_stats[2 * (size_t)f + 1] = NAN;
    };
    // token of element e (e must hold a token of the row's clusters)
    auto token = [&](int e) { return a.cl_tok[s_c0[e / a.max_cl] + e % a.max_cl]; };
    float mloc = -INFINITY;
    for (int e = e0; e < e1; e += SB) {
        float zz[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) zz[u] = z[min(e + u, e1 - 1)];
#pragma unroll
        for (int u = 0; u < SB; ++u) mloc = fmaxf(mloc, zz[u]);
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (t == 0) blank();
        return;
    }
    const float M = block_reduce<float>(mloc, s_ftmp, fmax_op, wmax_f);
    if (!(M > -INFINITY)) {  // no token (or NaN logits)
        if (t == 0) blank();
        return;
    }
    ACC tsum = 0;
    for (int e = e0; e < e1; e += SB) {
        float zz[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) zz[u] = z[min(e + u, e1 - 1)];
#pragma unroll
        for (int u = 0; u < SB; ++u)
            if (e + u < e1) tsum += (ACC)softw(zz[u], M, a.c);
    }
    ACC Zd, lo, incl;
    block_share(tsum, s_atmp, lo, incl, Zd);
    const float Z = (float)Zd;
    int pick = -1;
    if (GREEDY) {
        // the largest logit; ties to the smaller token id
        int best = 0x7fffffff;
        for (int e = e0; e < e1; ++e)
            if (z[e] == M) best = min(best, token(e));
        pick = block_reduce<int>(best, s_itmp, imin_op, wmin_i);
        if (t == 0) {
            if (pick < 0 || pick >= a.V) {
                blank();
            } else {
                a.x[f] = pick;
                a.pd_x[f] = 1.0f / Z;
            }
        }
    } else {
        const ACC target = (ACC)u24f(philox((uint32_t)k, (uint32_t)r, a.round, a.seed).w[0]) * Zd;
        int last = -1, lpos = -1;
        ACC run = lo;
        // this thread's share [lo, incl) holds the target: walk it
        const bool mine = tsum > 0 && lo <= target && target < incl;
        for (int e = e0; e < e1; ++e) {
            const float wv = softw(z[e], M, a.c);
            if (wv > 0.0f) {
                if (mine && pick < 0 && run + (ACC)wv > target) pick = e;
                lpos = e;
            }
            run += (ACC)wv;
        }
        last = lpos;
        if (mine && pick < 0) pick = last;  // the share's own sum rounded below the target
        if (pick >= 0) s_pick = pick;
        const int found = block_reduce<int>(pick, s_itmp, imax_op, wmax_i);
        // no share holds the target (the total rounded below it): the last
        // element with weight
        const int lastpos = block_reduce<int>(lpos, s_itmp, imax_op, wmax_i);
        if (t == 0) {
            const int e = found >= 0 ? s_pick : lastpos;
            const int v = e >= 0 ? token(e) : -1;
            if (v < 0 || v >= a.V) {
                blank();
            } else {
                a.x[f] = v;
                a.pd_x[f] = softw(z[e], M, a.c) / Z;
            }
        }
    }
    if (t == 0 && a.x[f] >= 0) {
        a.pd_stats[2 * (size_t)f] = M;
        a.pd_stats[2 * (size_t)f + 1] = Z;
    }
}

// ------------------------------------------------------------- launcher

// Splits of d for the coarse product: enough workgroups to spread the
// centres over the chip, at most 4 partial products to sum per logit.
static int coarse_splits(int N, int N_c, int d)
{
    const int nb = ((N + 31) / 32) * ((N_c + 127) / 128);
    if (nb < 1) return 1;  // no rows
    int q = (256 + nb - 1) / nb;
    return std::max(1, std::min(std::min(q, 4), d / 64));
}

size_t cluster_propose_ws_bytes(int N, int N_c, int d)
{
    return WS_HEADER + align256((size_t)coarse_splits(N, N_c, d) * N * N_c * sizeof(float));
}

hipError_t launch_cluster_propose(const ClusterArgs& a, hipStream_t s)
{
    const int N = a.R * a.gamma;
    const int nsplit = coarse_splits(N, a.N_c, a.d);
    float* part = reinterpret_cast<float*>(static_cast<char*>(a.ws) + WS_HEADER);
    const bf16w* H = static_cast<const bf16w*>(a.H);
    {
        ProfScope ps("cluster_coarse", s);
        hipLaunchKernelGGL(k_cluster_coarse, dim3((a.N_c + 127) / 128, (N + 31) / 32, nsplit), dim3(CL_THREADS), 0,
                           s, H, static_cast<const bf16w*>(a.C), N, a.N_c, a.d, nsplit, part);
    }
    {
        ProfScope ps("cluster_select", s);
        hipLaunchKernelGGL(k_cluster_select, dim3(N), dim3(CL_THREADS), 0, s, (const float*)part, nsplit, N, a.N_c,
                           a.K_c, a.sel);
    }
    {
        ProfScope ps("cluster_fine", s);
        hipLaunchKernelGGL(k_cluster_fine, dim3(a.N_c, (N + 31) / 32), dim3(CL_THREADS), 0, s, H,
                           static_cast<const bf16w*>(a.E), a.cl_off, a.cl_tok, (const int32_t*)a.sel, N, a.K_c,
                           a.max_cl, a.d, a.V, a.zf, a.status);
    }
    ClusterSampleArgs sa{};
    sa.zf = a.zf; sa.sel = a.sel; sa.cl_off = a.cl_off; sa.cl_tok = a.cl_tok;
    sa.N = N; sa.gamma = a.gamma; sa.N_c = a.N_c; sa.K_c = a.K_c; sa.max_cl = a.max_cl; sa.V = a.V;
    sa.c = a.c; sa.seed = a.seed; sa.round = a.round;
    sa.x = a.x; sa.pd_x = a.pd_x; sa.pd_stats = a.pd_stats; sa.status = a.status;
    {
        ProfScope ps("cluster_sample", s);
        const bool wide = (long)a.K_c * a.max_cl > 32L * CL_THREADS;  // more than 32 elements per thread
        if (a.greedy) {
            if (wide) hipLaunchKernelGGL((k_cluster_sample<true, double>), dim3(N), dim3(CL_THREADS), 0, s, sa);
            else hipLaunchKernelGGL((k_cluster_sample<true, float>), dim3(N), dim3(CL_THREADS), 0, s, sa);
        } else {
            if (wide) hipLaunchKernelGGL((k_cluster_sample<false, double>), dim3(N), dim3(CL_THREADS), 0, s, sa);
            else hipLaunchKernelGGL((k_cluster_sample<false, float>), dim3(N), dim3(CL_THREADS), 0, s, sa);
        }
    }
    return hipGetLastError();
}

}  // namespace spec
