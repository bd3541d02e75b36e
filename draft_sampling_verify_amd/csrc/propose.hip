// propose.hip -- Markov-head drafting (DSpark blog page, sections 3-4):
// for k = 1..gamma, z_k = U_k + W1[x_{k-1}] W2^T, x_k ~ softmax(z_k / T).
//
// Per position two kernels run back to back on the caller's stream:
//   k_draft_tile   grid over (granule, chunk of 32-row blocks): the bias of
//                  32 rows at 128 ids per workgroup on MFMA (W2 operand held
//                  in registers across the row blocks of the chunk), plus
//                  U, and per (row, granule) max / sum of 2^((z-max)c) /
//                  argmax -- one streaming pass over U_k and W2.
//   k_propose_pick one workgroup per request: merge the granule partials,
//                  draw the Philox uniform, find the granule where the
//                  running sum crosses u*S, recompute that granule's 128
//                  logits with the same tile code and pick the id.
// x_k stays on the device and feeds the next position's W1 gather.
#include "common.h"
#include "internal.h"

namespace spec {

struct TileArgs {
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* x0;
    const int32_t* x;  // drafts; row (req, kk) reads x[req*gamma + kk - 1] when kk > 0
    int R, gamma, r, V;
    float c;
    int vec4;
    int kfix;      // >= 0: rows are requests at position kfix+1; < 0: rows are all (req, kk)
    int nrows;
    int n_gran;
    int n_chunks;  // chunks of row blocks
    int bpc;       // row blocks per chunk
    float2* gstat; // [nrows, n_gran]
    int32_t* gidx; // [nrows, n_gran]
    uint32_t* status;
};

// Row -> (request, position index kk) and the token whose W1 row biases it.
__device__ inline void draft_row(const TileArgs& p, int row, int& req, int& kk, int& tok)
{
    if (p.kfix >= 0) {
        req = row;
        kk = p.kfix;
    } else {
        req = row / p.gamma;
        kk = row - req * p.gamma;
    }
    tok = kk == 0 ? p.x0[req] : p.x[(size_t)req * p.gamma + kk - 1];
}

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(TILE_THREADS) void k_draft_tile(TileArgs p)
{
    const int nlog = p.n_gran * p.n_chunks;
    const int lid = xcd_logical(blockIdx.x, nlog);
    if (lid >= nlog) return;
    const int g = lid / p.n_chunks, chunk = lid - g * p.n_chunks;
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int h = lane >> 5, n = lane & 31;
    const int col0 = g * GRAN + 32 * w;

    W2Operand<WT, KS> A;
    A.load(reinterpret_cast<const WT*>(p.W2), p.r, p.V, col0 + n, h);

    __shared__ float sm_m[4][32], sm_s[4][32];
    __shared__ int sm_i[4][32];

    for (int b = 0; b < p.bpc; ++b) {
        const int rb = chunk * p.bpc + b;
        if (rb * BLOCK_ROWS >= p.nrows) break;
        const int row = rb * BLOCK_ROWS + n;
        int req = 0, kk = 0, tok = -1;
        bool valid = row < p.nrows;
        if (valid) {
            draft_row(p, row, req, kk, tok);
            if (tok < 0 || tok >= p.V) {
                if (g == 0 && w == 0 && h == 0) raise_flag(p.status, 1u);
                tok = -1;
                valid = false;
            }
        }
        const f32x16 acc = A.mul(reinterpret_cast<const WT*>(p.W1), p.r, tok, h);
        float z[16];
        if (valid) {
            load_row16(p.U + ((size_t)req * p.gamma + kk) * p.V, col0, h, p.V, p.vec4, z);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) z[j] = -INFINITY;
        }
        float m = -INFINITY, bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            z[j] = z[j] + acc[j];
            m = fmaxf(m, z[j]);
            if (GREEDY && z[j] > bv) { bv = z[j]; bi = col0 + acc_col(j, h); }
        }
        m = fmaxf(m, shfl_xor(m, 32));
        const float ms = safe_ref(m);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) s += softw(z[j], ms, p.c);
        s += shfl_xor(s, 32);
        if (GREEDY) argmax_merge(bv, bi, shfl_xor(bv, 32), shfl_xor(bi, 32));
        if (h == 0) {
            sm_m[w][n] = m;
            sm_s[w][n] = s;
            sm_i[w][n] = bi;
        }
        __syncthreads();
        if (threadIdx.x < 32 && valid) {
            float M = sm_m[0][n];
#pragma unroll
            for (int i = 1; i < 4; ++i) M = fmaxf(M, sm_m[i][n]);
            const float Ms = safe_ref(M);
            float S = 0.0f;
            int idx = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S += sm_s[i][n] * softw(sm_m[i][n], Ms, p.c);
                if (GREEDY && idx == 0x7fffffff && sm_m[i][n] == M) idx = sm_i[i][n];
            }
            const size_t o = (size_t)row * p.n_gran + g;
            p.gstat[o] = make_float2(M, S);
            if (GREEDY) p.gidx[o] = idx;
        }
        __syncthreads();
    }
}

struct PickArgs {
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* x0;
    int32_t* x;  // [R, gamma]; position k is written, k-1 is read
    int R, gamma, r, V;
    float c;
    int vec4;
    int k;       // 1-based position
    int n_gran;
    uint64_t seed, round;
    const float2* gstat;
    const int32_t* gidx;
    float* pd_x;
    float* pd_stats;
};

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(TILE_THREADS) void k_propose_pick(PickArgs p)
{
    const int q = blockIdx.x;
    const int t = threadIdx.x;
    const size_t o = (size_t)q * p.gamma + (p.k - 1);
    const int tok = p.k == 1 ? p.x0[q] : p.x[(size_t)q * p.gamma + p.k - 2];
    if (tok < 0 || tok >= p.V) {
        if (t == 0) {
            p.x[o] = -1;
            p.pd_x[o] = NAN;
            p.pd_stats[2 * o] = NAN;
            p.pd_stats[2 * o + 1] = NAN;
        }
        return;
    }
    __shared__ float smf[8];
    __shared__ int smi[8];
    __shared__ float zrow[GRAN];

    // merge the granule partials: M = max, w_g = S_g 2^((M_g - M) c)
    const float2* gs = p.gstat + (size_t)q * p.n_gran;
    const int per = (p.n_gran + TILE_THREADS - 1) / TILE_THREADS;
    const int g0 = min(t * per, p.n_gran), g1 = min(g0 + per, p.n_gran);
    float m = -INFINITY;
    for (int g = g0; g < g1; ++g) m = fmaxf(m, gs[g].x);
    const float M = block_max(m, smf);
    const float c = p.c;
    auto wf = [&](int g) { const float2 v = gs[g]; return v.y * softw(v.x, M, c); };
    float tsum, excl, S;
    granule_scan(wf, g0, g1, smf, tsum, excl, S);

    if (GREEDY) {
        int cand = 0x7fffffff;
        for (int g = g0; g < g1; ++g)
            if (gs[g].x == M) { cand = p.gidx[(size_t)q * p.n_gran + g]; break; }
        const int best = block_min(cand, smi);
        if (t == 0) {
            p.x[o] = best;
            p.pd_x[o] = 1.0f / S;
            p.pd_stats[2 * o] = M;
            p.pd_stats[2 * o + 1] = S;
        }
        return;
    }

    const float u = u24f(philox((uint32_t)p.k, (uint32_t)q, p.round, p.seed).w[0]);
    const float target = u * S;
    float before;
    int gfb;
    int gstar = granule_find(wf, g0, g1, excl, target, smf, smi, before, gfb);
    const bool fallback = gstar < 0;
    if (fallback) gstar = gfb < 0 ? 0 : gfb;

    // Recompute the 128 logits of granule gstar for q's row block with the
    // same tile code as k_draft_tile (bit-identical z).
    const int lane = t & (WAVE - 1), w = t / WAVE, h = lane >> 5, n = lane & 31;
    const int col0 = gstar * GRAN + 32 * w;
    W2Operand<WT, KS> A;
    A.load(reinterpret_cast<const WT*>(p.W2), p.r, p.V, col0 + n, h);
    const int rr = (q / BLOCK_ROWS) * BLOCK_ROWS + n;
    int tk = -1;
    if (rr < p.R) {
        tk = p.k == 1 ? p.x0[rr] : p.x[(size_t)rr * p.gamma + p.k - 2];
        if (tk < 0 || tk >= p.V) tk = -1;
    }
    const f32x16 acc = A.mul(reinterpret_cast<const WT*>(p.W1), p.r, tk, h);
    if (n == (q & (BLOCK_ROWS - 1))) {
        float z[16];
        load_row16(p.U + ((size_t)q * p.gamma + (p.k - 1)) * p.V, col0, h, p.V, p.vec4, z);
#pragma unroll
        for (int j = 0; j < 16; ++j) zrow[32 * w + acc_col(j, h)] = z[j] + acc[j];
    }
    __syncthreads();
    if (w == 0) {
        float e;
        const int col = granule_pick(softw(zrow[2 * lane], M, c), softw(zrow[2 * lane + 1], M, c),
                                     before, target, fallback, e);
        if (lane == 0) {
            p.x[o] = gstar * GRAN + col;
            p.pd_x[o] = e / S;
            p.pd_stats[2 * o] = M;
            p.pd_stats[2 * o + 1] = S;
        }
    }
}

// ------------------------------------------------------------ launchers

static int rows_per_chunk_blocks(int nrows, int n_gran)
{
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    long work = (long)n_rb * n_gran;
    int bpc = (int)(work / 2048);
    if (bpc < 1) bpc = 1;
    if (bpc > 4) bpc = 4;
    if (bpc > n_rb) bpc = n_rb;
    return bpc;
}

template <typename WT, int KS>
static hipError_t propose_impl(const DraftArgs& a, int32_t* x_out, float* pd_x, float* pd_stats,
                               const ProposeWs& ws, hipStream_t s)
{
    const int n_gran = n_granules(a.V);
    const int n_rb = (a.R + BLOCK_ROWS - 1) / BLOCK_ROWS;
    const int bpc = rows_per_chunk_blocks(a.R, n_gran);
    const int n_chunks = (n_rb + bpc - 1) / bpc;
    TileArgs t{};
    t.U = a.U; t.W1 = a.W1; t.W2 = a.W2; t.x0 = a.x0; t.x = x_out;
    t.R = a.R; t.gamma = a.gamma; t.r = a.r; t.V = a.V; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.nrows = a.R; t.n_gran = n_gran; t.n_chunks = n_chunks; t.bpc = bpc;
    t.gstat = ws.gstat; t.gidx = ws.gidx; t.status = a.status;
    PickArgs pk{};
    pk.U = a.U; pk.W1 = a.W1; pk.W2 = a.W2; pk.x0 = a.x0; pk.x = x_out;
    pk.R = a.R; pk.gamma = a.gamma; pk.r = a.r; pk.V = a.V; pk.c = a.c; pk.vec4 = t.vec4;
    pk.n_gran = n_gran; pk.seed = a.seed; pk.round = a.round;
    pk.gstat = ws.gstat; pk.gidx = ws.gidx; pk.pd_x = pd_x; pk.pd_stats = pd_stats;
    const int grid = xcd_grid(n_gran * n_chunks);
    for (int k = 1; k <= a.gamma; ++k) {
        t.kfix = k - 1;
        pk.k = k;
        {
            ProfScope ps("draft_tile", s);
            if (a.greedy)
                hipLaunchKernelGGL((k_draft_tile<WT, KS, true>), dim3(grid), dim3(TILE_THREADS), 0, s, t);
            else
                hipLaunchKernelGGL((k_draft_tile<WT, KS, false>), dim3(grid), dim3(TILE_THREADS), 0, s, t);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        {
            ProfScope ps("propose_pick", s);
            if (a.greedy)
                hipLaunchKernelGGL((k_propose_pick<WT, KS, true>), dim3(a.R), dim3(TILE_THREADS), 0, s, pk);
            else
                hipLaunchKernelGGL((k_propose_pick<WT, KS, false>), dim3(a.R), dim3(TILE_THREADS), 0, s, pk);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Per-(row, granule) draft statistics and per-row (M, S) for every (req, kk)
// row; used by spec_confidence when no propose statistics are supplied.
__global__ __launch_bounds__(TILE_THREADS) void k_merge_rows(const float2* gstat, int nrows, int n_gran,
                                                             float c, float2* rows)
{
    const int row = blockIdx.x * (TILE_THREADS / WAVE) + threadIdx.x / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    if (row >= nrows) return;
    const float2* gs = gstat + (size_t)row * n_gran;
    float m = -INFINITY;
    for (int g = lane; g < n_gran; g += WAVE) m = fmaxf(m, gs[g].x);
    const float M = wave_max(m);
    const float Ms = safe_ref(M);
    float s = 0.0f;
    for (int g = lane; g < n_gran; g += WAVE) s += gs[g].y * softw(gs[g].x, Ms, c);
    const float S = wave_sum(s);
    if (lane == 0) rows[row] = make_float2(M, S);
}

template <typename WT, int KS>
static hipError_t row_stats_impl(const DraftArgs& a, const VerifyWs& ws, hipStream_t s)
{
    const int n_gran = n_granules(a.V);
    const int nrows = a.R * a.gamma;
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    const int bpc = rows_per_chunk_blocks(nrows, n_gran);
    const int n_chunks = (n_rb + bpc - 1) / bpc;
    TileArgs t{};
    t.U = a.U; t.W1 = a.W1; t.W2 = a.W2; t.x0 = a.x0; t.x = a.x;
    t.R = a.R; t.gamma = a.gamma; t.r = a.r; t.V = a.V; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.kfix = -1; t.nrows = nrows; t.n_gran = n_gran; t.n_chunks = n_chunks; t.bpc = bpc;
    t.gstat = ws.dgran; t.gidx = ws.dgidx; t.status = a.status;
    {
        ProfScope ps("draft_tile", s);
        hipLaunchKernelGGL((k_draft_tile<WT, KS, false>), dim3(xcd_grid(n_gran * n_chunks)),
                           dim3(TILE_THREADS), 0, s, t);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope ps("merge_rows", s);
        hipLaunchKernelGGL(k_merge_rows, dim3((nrows + 3) / 4), dim3(TILE_THREADS), 0, s,
                           (const float2*)ws.dgran, nrows, n_gran, a.c, ws.drow);
    }
    return hipGetLastError();
}

// Dispatch on weight dtype and the padded number of k-steps.
template <template <typename, int> class F, typename... Args>
static hipError_t dispatch_ks(int w_dtype, int r, Args&&... args)
{
    if (w_dtype == 1) {
        const int ks = r / 16;
        if (ks <= 4) return F<bf16w, 4>::run(args...);
        if (ks <= 8) return F<bf16w, 8>::run(args...);
        if (ks <= 16) return F<bf16w, 16>::run(args...);
        return F<bf16w, 32>::run(args...);
    }
    const int ks = r / 2;
    if (ks <= 8) return F<float, 8>::run(args...);
    if (ks <= 32) return F<float, 32>::run(args...);
    return F<float, 128>::run(args...);
}

template <typename WT, int KS>
struct ProposeF {
    static hipError_t run(const DraftArgs& a, int32_t* x_out, float* pd_x, float* pd_stats,
                          const ProposeWs& ws, hipStream_t s)
    {
        return propose_impl<WT, KS>(a, x_out, pd_x, pd_stats, ws, s);
    }
};
template <typename WT, int KS>
struct RowStatsF {
    static hipError_t run(const DraftArgs& a, const VerifyWs& ws, hipStream_t s)
    {
        return row_stats_impl<WT, KS>(a, ws, s);
    }
};

hipError_t launch_propose(const DraftArgs& a, int32_t* x_out, float* pd_x, float* pd_stats,
                          const ProposeWs& w, hipStream_t s)
{
    return dispatch_ks<ProposeF>(a.w_dtype, a.r, a, x_out, pd_x, pd_stats, w, s);
}

hipError_t launch_draft_row_stats(const DraftArgs& a, const VerifyWs& w, hipStream_t s)
{
    return dispatch_ks<RowStatsF>(a.w_dtype, a.r, a, w, s);
}

}  // namespace spec
