// verify.hip -- lossless verification and the confidence label.
//
//   accept x_k with probability min(1, p_t(x_k)/p_d(x_k)); at the first
//   rejection draw from normalize(max(0, p_t - p_d)); after a full accept draw
//   the bonus token from the next target row (DSpark blog page, section 1
//   diagram; verify window of gamma+1 target rows, SGLang MTP/NextN page,
//   section 3); c*_k = 1 - 1/2 ||p_d - p_t||_1 (DSpark page, section 5).
//
// Kernels, in launch order:
//   k_plan            (only with scheduled lengths) row maps for the ragged
//                     verified rows: flattened, no padding.
//   k_target_rows     one workgroup per target row: max, sum of 2^((L-max)c)
//                     and argmax per granule, and the row's (M_t, S_t,
//                     argmax) -- first streaming pass over the target rows.
//   k_verify_sweep    per (granule, verified rows): recompute the Markov bias
//                     on MFMA, p_d and p_t, and the granule's TV mass
//                     sum |p_t - p_d| and residual mass sum max(0, p_t - p_d)
//                     -- second pass over the target rows plus U and W2.
//   k_verify_resolve  one workgroup per request: accept tests (fp64 on the
//                     single drafted id), first rejection, c*, residual or
//                     bonus draw by inverse CDF over granules plus one
//                     granule rescan.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace spec {

// Verified row f -> (request, k (1-based), target row index).
__device__ inline int4 vrow_info(const int4* vmap, int f, int gamma, int P)
{
    if (vmap) return vmap[f];
    const int r = f / gamma, kk = f - r * gamma;
    return make_int4(r, kk + 1, r * P + kk, 0);
}
// Target row t -> (request, row within the request's gamma+1 target rows).
__device__ inline int2 trow_info(const int2* tmap, int t, int P)
{
    if (tmap) return tmap[t];
    const int r = t / P;
    return make_int2(r, t - r * P);
}

// ------------------------------------------------------------------ plan

// Scan of the scheduled lengths; writes voff/toff, the row maps and the row
// counts.  Lengths outside [0, gamma] raise SPEC_DEV_BAD_LENGTH and count 0.
__global__ __launch_bounds__(TILE_THREADS) void k_plan(const int32_t* ell, int R, int gamma,
                                                       int32_t* voff, int32_t* toff, int4* vmap,
                                                       int2* tmap, int32_t* counts, uint32_t* status)
{
    __shared__ float smf[8];
    const int t = threadIdx.x;
    const int per = (R + TILE_THREADS - 1) / TILE_THREADS;
    const int r0 = min(t * per, R), r1 = min(r0 + per, R);
    int local = 0;
    for (int r = r0; r < r1; ++r) {
        const int L = ell[r];
        if (L < 0 || L > gamma) raise_flag(status, 2u);
        else local += L;
    }
    // block scan in fp32 is exact here: totals stay below 2^24
    float total_f;
    const float ex_f = block_excl_scan((float)local, smf, total_f);
    int ex = (int)ex_f;
    for (int r = r0; r < r1; ++r) {
        int L = ell[r];
        if (L < 0 || L > gamma) L = 0;
        voff[r] = ex;
        toff[r] = ex + r;
        for (int k = 0; k < L; ++k) vmap[ex + k] = make_int4(r, k + 1, ex + r + k, 0);
        for (int k = 0; k <= L; ++k) tmap[ex + r + k] = make_int2(r, k);
        ex += L;
    }
    if (t == 0) {
        counts[0] = (int)total_f;
        counts[1] = (int)total_f + R;
    }
}

// With scheduled lengths: everything the pipelined sweep needs of verified
// row f in two 16-byte records, so that it reads them with one load each
// (no load whose address comes from another): the tokens (x_{k-1}, x_k),
// the U and target rows, and the draft's and target's (M, S).  Runs after
// the target rows' statistics.
__global__ __launch_bounds__(TILE_THREADS) void k_row_table(const int4* vmap, const int32_t* counts,
                                                            const int32_t* x0, const int32_t* x,
                                                            const float* dstats, const float2* trow, int gamma,
                                                            int max_rows, int4* rtab, float4* rctab)
{
    const int f = blockIdx.x * TILE_THREADS + threadIdx.x;
    if (f >= max_rows || f >= counts[0]) return;
    const int4 vi = vmap[f];  // (request, k, compact target row)
    const int so = vi.x * gamma + vi.y - 1;
    rtab[f] = make_int4(vi.y == 1 ? x0[vi.x] : x[so - 1], x[so], so, vi.x * (gamma + 1) + vi.y - 1);
    const float2 ts = trow[vi.z];
    rctab[f] = make_float4(dstats[2 * (size_t)so], dstats[2 * (size_t)so + 1], ts.x, ts.y);
}

// ---------------------------------------------------------- target stats

struct TargetArgs {
    const float* Lt;
    int R, gamma, V, P;  // P: target rows per request in the implicit map
    float c;
    int vec4;
    int n_gran, max_rows;
    int nsplit;              // workgroups per row (1: the row's statistics are final)
    float4* tpart;           // nsplit > 1: [rows, nsplit] (max, sum, argmax bits, -) per part
    const int2* tmap;        // NULL = implicit
    const int32_t* counts;   // counts[1] = rows when tmap != NULL
    float2* tgran;
    int32_t* tgidx;
    float2* trow;
    int32_t* targ;
};

// One workgroup (512 threads) per target row streams the whole row, 8192
// ids per step (next step's loads issued before this step's arithmetic).
// Each 8-lane group reduces one 128-id granule per step (16 consecutive ids
// per lane, DPP reductions) and writes its (max, sum of 2^((L-max)c),
// argmax); a running (max, sum, argmax) per group then folds into the row's
// (M_t, S_t, argmax) at the end, so no separate merge pass is needed.
constexpr int TROW_THREADS = 1024;
constexpr int TROW_GRANS = TROW_THREADS / 8;  // granules per step
constexpr int TROW_MAX_SPLIT = 16;            // workgroups per row at most
constexpr int TROW_TARGET_WGS = 256;          // rows are split while fewer than this (more is slower)
constexpr int TROW_STAGE_GRANS = 4096;        // granule statistics held in LDS per workgroup (48 KB)

// With few rows a row is split over nsplit workgroups (consecutive runs of
// steps); each writes its part's (max, sum, argmax) and k_target_merge folds
// the parts in order.
__global__ __launch_bounds__(TROW_THREADS) void k_target_rows(TargetArgs p)
{
    const int row = blockIdx.x / p.nsplit, part = blockIdx.x - row * p.nsplit;
    const int nrows = p.tmap ? p.counts[1] : p.max_rows;
    if (row >= nrows) return;
    const int2 ti = trow_info(p.tmap, row, p.P);
    const float* L = p.Lt + ((size_t)ti.x * (p.gamma + 1) + ti.y) * p.V;
    const int t = threadIdx.x, gi = t >> 3, l8 = t & 7;
    const int steps_all = (p.n_gran + TROW_GRANS - 1) / TROW_GRANS;
    const int st0 = part * steps_all / p.nsplit, steps = (part + 1) * steps_all / p.nsplit;
    // this part's granule statistics wait in LDS until the row is read:
    // stores mixed into the streamed reads cost far more than their bytes
    __shared__ float2 s_tg[TROW_STAGE_GRANS];
    __shared__ int s_ti[TROW_STAGE_GRANS];
    const int g_first = st0 * TROW_GRANS;
    float rm = -INFINITY, rs = 0.0f;
    int rbi = 0x7fffffff;
    float cur[16], nxt[16];
    load16(L, (st0 * TROW_GRANS + gi) * GRAN + 16 * l8, p.V, p.vec4, cur);
    for (int st = st0; st < steps; ++st) {
        if (st + 1 < steps) load16(L, ((st + 1) * TROW_GRANS + gi) * GRAN + 16 * l8, p.V, p.vec4, nxt);
        const int g = st * TROW_GRANS + gi;
        const int c0 = g * GRAN + 16 * l8;
        float m = -INFINITY, bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            m = fmaxf(m, cur[j]);
            if (cur[j] > bv) { bv = cur[j]; bi = c0 + j; }
        }
        m = oct_max(m);
        const float ms = safe_ref(m);
        float sm = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sm += softw(cur[j], ms, p.c);
        sm = oct_sum(sm);
        oct_argmax(bv, bi);
        if (g < p.n_gran) {
            if (l8 == 0) {
                const int sg = g - g_first;
                if (sg < TROW_STAGE_GRANS) {
                    s_tg[sg] = make_float2(m, sm);
                    s_ti[sg] = bi;
                } else {
                    const size_t o = (size_t)row * p.n_gran + g;
                    p.tgran[o] = make_float2(m, sm);
                    p.tgidx[o] = bi;
                }
            }
            // fold into the group's running row statistics (granules ascend)
            if (m > rm) {
                rs = rs * softw(rm, m, p.c) + sm;
                rm = m;
                rbi = bi;
            } else {
                rs += sm * softw(m, safe_ref(rm), p.c);
            }
        }
        if (st + 1 < steps) {
#pragma unroll
            for (int j = 0; j < 16; ++j) cur[j] = nxt[j];
        }
    }
    // merge the 64 groups: lanes 0, 8, ..., 56 of each wave, then the waves
    __shared__ float s_m[TROW_THREADS / WAVE], s_s[TROW_THREADS / WAVE];
    __shared__ int s_i[TROW_THREADS / WAVE];
    __syncthreads();
    {
        // the staged granule statistics of this part, in one burst
        const int g_end = min(min(steps * TROW_GRANS, p.n_gran), g_first + TROW_STAGE_GRANS);
        for (int g = g_first + t; g < g_end; g += TROW_THREADS) {
            const size_t o = (size_t)row * p.n_gran + g;
            p.tgran[o] = s_tg[g - g_first];
            p.tgidx[o] = s_ti[g - g_first];
        }
    }
#pragma unroll
    for (int o = 8; o < WAVE; o <<= 1) {
        const float m2 = shfl_xor(rm, o), s2 = shfl_xor(rs, o);
        const int i2 = shfl_xor(rbi, o);
        const float M = fmaxf(rm, m2), Ms = safe_ref(M);
        rs = rs * softw(rm, Ms, p.c) + s2 * softw(m2, Ms, p.c);
        if (m2 > rm || (m2 == rm && i2 < rbi)) rbi = i2;
        rm = M;
    }
    const int w = t / WAVE;
    if ((t & (WAVE - 1)) == 0) {
        s_m[w] = rm;
        s_s[w] = rs;
        s_i[w] = rbi;
    }
    __syncthreads();
    if (t == 0) {
        float M = s_m[0];
        for (int i = 1; i < TROW_THREADS / WAVE; ++i) M = fmaxf(M, s_m[i]);
        const float Ms = safe_ref(M);
        float S = 0.0f;
        int best = 0x7fffffff;
        for (int i = 0; i < TROW_THREADS / WAVE; ++i) {
            S += s_s[i] * softw(s_m[i], Ms, p.c);
            if (s_m[i] == M && s_i[i] < best) best = s_i[i];
        }
        if (p.nsplit == 1) {
            p.trow[row] = make_float2(M, S);
            p.targ[row] = best;
        } else {
            p.tpart[(size_t)row * p.nsplit + part] = make_float4(M, S, __int_as_float(best), 0.0f);
        }
    }
}

// One thread per row: the parts' (max, sum, argmax) folded in part order.
__global__ void k_target_merge(TargetArgs p)
{
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    const int nrows = p.tmap ? p.counts[1] : p.max_rows;
    if (row >= nrows) return;
    const float4* tp = p.tpart + (size_t)row * p.nsplit;
    float M = -INFINITY;
    for (int i = 0; i < p.nsplit; ++i) M = fmaxf(M, tp[i].x);
    const float Ms = safe_ref(M);
    float S = 0.0f;
    int best = 0x7fffffff;
    for (int i = 0; i < p.nsplit; ++i) {
        const float4 v = tp[i];
        S += v.y * softw(v.x, Ms, p.c);
        if (v.x == M && __float_as_int(v.z) < best) best = __float_as_int(v.z);
    }
    p.trow[row] = make_float2(M, S);
    p.targ[row] = best;
}

// ------------------------------------------------------------ TV sweep

struct SweepArgs {
    const float* U;
    const void* W1;
    const void* W2p;
    const int32_t* x0;
    const int32_t* x;
    const float* dstats;  // [R*gamma, 2] draft (M, S) (propose output layout)
    const float* Lt;
    int R, gamma, r, V, P;
    float c;
    int vec4;
    int n_gran, n_chunks, bpc, max_rows;
    const int4* vmap;
    const int32_t* counts;
    const float2* trow;
    float2* vpart;        // [rows, n_gran] (TV mass, residual mass)
    float* vbias;         // [rows] Markov bias at the drafted id x_k
    int staged_only;      // the call asked for the staged sweep (PATH_NO_PIPELINED_SWEEP)
    FastDiv div_rb;       // by the number of 32-row blocks (the pipelined sweep, every row verified)
    FastDiv div_g;        // by gamma
    const int4* rtab;     // scheduled lengths: per verified row (x_{k-1}, x_k, U row, target row)
    const float4* rctab;  // scheduled lengths: per verified row (M_d, S_d, M_t, S_t)
};

// Verified row f: where its data lives and the normalisers of p_d and p_t.
struct RowCtx {
    int req, k, trow, xk;  // req = -1: no such row
    float Md, iSd, Mt, iSt;
};

// Token whose W1 row biases verified row f (x_{k-1}), or -1 when the row does
// not exist or its tokens are out of range.
__device__ inline int row_tok(const SweepArgs& p, int f, int nrows)
{
    if (f >= nrows) return -1;
    const int4 vi = vrow_info(p.vmap, f, p.gamma, p.P);
    const int tok = vi.y == 1 ? p.x0[vi.x] : p.x[(size_t)vi.x * p.gamma + vi.y - 2];
    const int xk = p.x[(size_t)vi.x * p.gamma + vi.y - 1];
    return (tok < 0 || tok >= p.V || xk < 0 || xk >= p.V) ? -1 : tok;
}

// Residual weight max(0, p_t - p_d) of one id; the sweep and the resolve's
// rescan both use this expression.
__device__ inline float resid(float zu, float bias, float zt, const RowCtx& rc, float c, float& d)
{
    const float pd = softw(zu + bias, rc.Md, c) * rc.iSd;
    const float pt = softw(zt, rc.Mt, c) * rc.iSt;
    d = pt - pd;
    return fmaxf(d, 0.0f);
}

// What a verified row's epilogue needs, as loaded (no arithmetic on the
// loaded values, so that the loads can be issued one block ahead without the
// compiler waiting for them at once).  Rows past the end load row 0's data
// and carry ok = false.  MAPS: the row map is in memory (scheduled lengths),
// else implicit.
struct RowRaw {
    int4 vi;
    int xk;
    float md, sd;
    float2 ts;
    bool ok;
};

template <bool MAPS>
__device__ inline int4 vrow_at(const SweepArgs& p, int f)
{
    if constexpr (MAPS) return p.vmap[f];
    const int r = f / p.gamma, kk = f - r * p.gamma;
    return make_int4(r, kk + 1, r * p.P + kk, 0);
}

template <bool MAPS>
__device__ inline RowRaw row_raw(const SweepArgs& p, int f, int nrows)
{
    RowRaw w;
    w.ok = f < nrows;
    w.vi = vrow_at<MAPS>(p, w.ok ? f : 0);
    const size_t so = (size_t)w.vi.x * p.gamma + w.vi.y - 1;
    w.xk = p.x[so];
    w.md = p.dstats[2 * so];
    w.sd = p.dstats[2 * so + 1];
    w.ts = p.trow[w.vi.z];
    return w;
}

// The verified row's context from its loaded values (req = -1 past the end).
__device__ inline RowCtx row_finish(const RowRaw& w)
{
    RowCtx rc;
    rc.req = w.ok ? w.vi.x : -1;
    rc.k = w.vi.y;
    rc.trow = w.vi.z;
    rc.xk = w.xk;
    rc.Md = w.md;
    rc.iSd = 1.0f / w.sd;
    rc.Mt = w.ts.x;
    rc.iSt = 1.0f / w.ts.y;
    return rc;
}

// The two tokens row_tok() checks, as loaded: (x_{k-1}, x_k); (-1, -1) past
// the end.  Both loads are unconditional (x_{k-1} of position 1 is x0).
template <bool MAPS>
__device__ inline int2 tok_raw(const SweepArgs& p, int f, int nrows)
{
    const bool ok = f < nrows;
    const int4 vi = vrow_at<MAPS>(p, ok ? f : 0);
    const size_t so = (size_t)vi.x * p.gamma + vi.y - 1;
    const int* src = vi.y == 1 ? p.x0 + vi.x : p.x + (so - 1);
    // masked with an opaque value rather than a select, so that the compiler
    // does not move the loads under a branch
    const int om = opaque_v(ok ? 0 : -1);
    return make_int2(*src | om, p.x[so] | om);
}

__device__ inline int tok_check(int2 tx, int V)
{
    return (tx.x < 0 || tx.x >= V || tx.y < 0 || tx.y >= V) ? -1 : tx.x;
}

// One workgroup per (granule, chunk of 32-row blocks); W2's 128 x r slice of
// the granule stays in registers (the MFMA A operand) for the whole chunk.
// Per block: W1 rows of the 32 tokens are gathered into LDS, the 32 x 128
// bias tile is computed on MFMA into LDS, and each 8-lane group combines one
// row's bias with its U and target logits.  The loads are ordered so that
// the dependent chain (tokens -> W1 rows -> MFMA) never waits for the
// streamed U and target rows: right after the W1 gather is issued come this
// block's U and target loads and then the next block's tokens and row
// context, so the LDS write of W1 waits for W1 alone and the rest stays in
// flight through the MFMA.  (Loads are counted in issue order, so this needs
// straight-line code: no branch around any of these loads.)
template <typename WT, int KS, bool VEC4, bool MAPS>
__global__ __launch_bounds__(TILE_THREADS, 3) void k_verify_sweep(SweepArgs p)
{
    using Ops = TileOps<WT, KS>;
    const int nlog = p.n_gran * p.n_chunks;
    const int lid = xcd_logical(blockIdx.x, nlog);
    if (lid >= nlog) return;
    const int g = lid / p.n_chunks, chunk = lid - g * p.n_chunks;
    const int nrows = MAPS ? p.counts[0] : p.max_rows;
    const int rb0 = chunk * p.bpc;
    const int nb = min(p.bpc, (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS - rb0);
    if (nb <= 0) return;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int ks = k_steps<WT>(p.r);
    const int nblk = (p.V + 31) / 32;

    Ops A;
    A.load_a(p.W2p, ks, 4 * g + w, 4 * g + w < nblk, lane);

    __shared__ __align__(16) char sB[32 * Ops::RS * Ops::ELEM];
    __shared__ __align__(16) float sZ[32 * ZS];
    __shared__ int s_tok[32];

    const int er = t >> 3, ec = (t & 7) * 16;
    const int cbase = g * GRAN + ec;
    // every lane loads a token pair (lanes 32-63 repeat 0-31): no branch
    int2 tx = tok_raw<MAPS>(p, rb0 * BLOCK_ROWS + (t & 31), nrows);
    RowRaw rw = row_raw<MAPS>(p, rb0 * BLOCK_ROWS + er, nrows);
    for (int b = 0; b < nb; ++b) {
        const int f = (rb0 + b) * BLOCK_ROWS + er;
        if (t < 32) s_tok[t] = tok_check(tx, p.V);
        const RowCtx rc = row_finish(rw);
        const int req = rw.vi.x, kk = rw.vi.y;  // row 0's data when the row is past the end
        // s_tok written; the previous block's epilogue is done with sZ
        __syncthreads();
        const bool valid = rc.req >= 0 && s_tok[er] >= 0;
        W1Gather<WT, Ops::RS, KS> gw;
        gw.issue(reinterpret_cast<const WT*>(p.W1), s_tok, p.r);
        float zu[16], zt[16];
        load16_flat<VEC4>(p.U + ((size_t)req * p.gamma + kk - 1) * p.V, cbase, p.V, zu);
        load16_flat<VEC4>(p.Lt + ((size_t)req * (p.gamma + 1) + kk - 1) * p.V, cbase, p.V, zt);
        tx = tok_raw<MAPS>(p, (rb0 + b + 1) * BLOCK_ROWS + (t & 31), nrows);
        rw = row_raw<MAPS>(p, f + BLOCK_ROWS, nrows);
        gw.commit(sB, p.r);
        __syncthreads();
        store_tile(sZ, A.mfma(sB, ks, lane), w, lane);
        __syncthreads();
        if (valid) {
            const float* zr = sZ + er * ZS + ec;
            // ids 0-7 and 8-15 of the thread's 16 summed apart, then reduced
            // in the pipelined sweep's order (identical records)
            float tv[2] = {0.0f, 0.0f}, res[2] = {0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bq = *reinterpret_cast<const float4*>(zr + 4 * q);
                const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float d;
                    res[q >> 1] += resid(zu[4 * q + e], bb[e], zt[4 * q + e], rc, p.c, d);
                    tv[q >> 1] += fabsf(d);
                }
            }
            const float tvs = pair_oct_sum(tv[0], tv[1]), rs = pair_oct_sum(res[0], res[1]);
            if ((t & 7) == 0) p.vpart[(size_t)f * p.n_gran + g] = make_float2(tvs, rs);
            if (rc.xk >= cbase && rc.xk < cbase + 16) p.vbias[f] = zr[rc.xk - cbase];
        }
    }
}

// The pipelined sweep (every position of every request verified, or the
// scheduled rows through the row tables).  The work is a sequence of units, unit u = (granule
// u / n_rb, 32-row block u % n_rb); each workgroup takes a contiguous run of
// units (runs differ in length by at most one), so the pipeline below fills
// and drains once per workgroup and W2 is reloaded only where the run
// crosses into the next granule.  One workgroup of 12 waves per CU; the
// work of a unit is split between two groups of waves that run one stage
// apart:
//   MFMA waves (0-3)      hold W2's granule slice (the A operand) and, in
//                         stage s, write unit s+1's W1 rows (loaded into
//                         registers last stage) into LDS, issue the loads of
//                         unit s+2's, compute unit s's 32 x 128 bias tile
//                         into LDS and move the per-row values that arrived
//                         (tokens, row context) into LDS;
//   epilogue waves (4-11) hold the U and target rows of three units in
//                         registers (16 lanes per row, 8 ids each): in
//                         stage s they finish unit s-1 (p_d, p_t, the TV
//                         and residual masses, the bias at x_k) while units
//                         s and s+1 are in flight, keep its records in LDS,
//                         then issue unit s+2's loads into the registers
//                         just freed.
// One barrier per stage, and no wave waits at it for memory: every value is
// loaded into registers at least one stage before it is needed (the W1 rows
// one stage ahead, U and target rows two, the token pairs that choose the W1
// rows and the row context three stages before they are used).  The
// (row, granule) records are written out at the end of the run (or of each
// chunk of SWEEP_REC_UNITS units): one 8-byte store per row and unit mixed
// into the streamed reads cost about a fifth of the read rate, the same
// bytes written in one burst almost nothing.  Each group first uses what
// arrived and only then issues new loads, all without a branch, so every
// wait the compiler places is for loads of an earlier stage.

// Units whose (row, granule) records the pipelined sweep holds in LDS before
// writing them out (80 KB; a run of more units writes them in chunks).
constexpr int SWEEP_REC_UNITS = 320;

template <int KS, bool VEC4, bool MAPS>
__global__ __launch_bounds__(3 * TILE_THREADS, 1) void k_verify_sweep_ws(SweepArgs p)
{
    using Ops = TileOps<bf16w, KS>;
    using GW = W1Regs<Ops::RS, KS, 1>;
    // rows: every position of every request, or the scheduled rows (their
    // count is known on the device only)
    const int nrows = MAPS ? p.counts[0] : p.max_rows;
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    if (n_rb <= 0) return;
    const UnitRun run(p.n_gran, n_rb);
    const int nu = run.nu;
    if (nu <= 0) return;
    const FastDiv div_rb = MAPS ? FastDiv::make(n_rb) : p.div_rb;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const bf16w* W1 = reinterpret_cast<const bf16w*>(p.W1);
    // unit j of this run (j may pass the run's end: such units repeat the
    // last one; their values are loaded and never used)
    auto unit = [&](int j) { return run.unit(j); };
    auto ugran = [&](int j) { return div_rb.div(unit(j)); };
    auto urow = [&](int j, int i) {
        const int u = unit(j);
        return (u - div_rb.div(u) * n_rb) * BLOCK_ROWS + i;
    };
    // raw values of verified row q (clamped to row 0 past the end): its
    // tokens (x_{k-1}, x_k), its U row and its target row
    auto raw_row = [&](int q) __attribute__((always_inline)) {
        const int qc = q < nrows ? q : 0;
        if constexpr (MAPS) {
            return p.rtab[qc];
        } else {
            const int r = p.div_g.div(qc), kk = qc - r * p.gamma;
            return make_int4(kk == 0 ? p.x0[r] : p.x[qc - 1], p.x[qc], qc, r * (p.gamma + 1) + kk);
        }
    };

    __shared__ __align__(16) char sB[2][32 * Ops::RS * Ops::ELEM];  // W1 tiles, unit j in j & 1
    __shared__ __align__(16) float sZ[2][32 * ZS];                 // bias tiles, unit j in j & 1
    __shared__ int s_tok[8][32];                                    // checked tokens, unit j in j & 7
    __shared__ int2 s_rows[8][32];                                  // (U row, target row), unit j in j & 7
    __shared__ int s_xk[2][32];                                     // x_k
    __shared__ float s_cf[2][4][32];                                // M_d, S_d, M_t, S_t
    __shared__ float2 s_rec[SWEEP_REC_UNITS * 32];                  // records of unit j in slot j % SWEEP_REC_UNITS

    // units 0, 1 and 2: checked tokens.  Rows past the end load row 0's
    // values and are masked where used.
    if (t < 96) {
        const int j = t >> 5, q = urow(j, t & 31);
        const int4 e = raw_row(q);
        s_tok[j][t & 31] = q < nrows ? tok_check(make_int2(e.x, e.y), p.V) : -1;
        s_rows[j][t & 31] = make_int2(e.z, e.w);
    }
    // stage s computes unit s's tile (s < nu), finishes unit s-1 and stores
    // unit s-2's results: stages 0..nu+1, rounded up to a multiple of three
    // (the epilogue's loop takes stages in threes)
    const int n_stages = (nu + 2 + 2) / 3 * 3;
    __syncthreads();

    if (w < 4) {
        // ------------------------------------------------ MFMA waves
        const int nblk = (p.V + 31) / 32;
        int ga = ugran(0);
        Ops A;
        A.load_a(p.W2p, KS, 4 * ga + w, 4 * ga + w < nblk, lane);
        // raw per-row values of unit j for row lane & 31 (wave 0: tokens,
        // wave 1: row context)
        auto raw_tokens = [&](int j) __attribute__((always_inline)) { return raw_row(urow(j, lane & 31)); };
        struct Ctx {
            int xk;
            float md, sd, mt, st;
        };
        auto raw_ctx = [&](int j) __attribute__((always_inline)) {
            const int q = urow(j, lane & 31), qc = q < nrows ? q : 0;
            Ctx c;
            if constexpr (MAPS) {
                const float4 v = p.rctab[qc];
                c.xk = p.rtab[qc].y;
                c.md = v.x;
                c.sd = v.y;
                c.mt = v.z;
                c.st = v.w;
            } else {
                const int r = p.div_g.div(qc), kk = qc - r * p.gamma;
                // target row (r, kk) of the first pass: P rows per request
                const float* ts = reinterpret_cast<const float*>(p.trow) + 2 * ((size_t)r * p.P + kk);
                c.xk = p.x[qc];
                c.md = p.dstats[2 * (size_t)qc];
                c.sd = p.dstats[2 * (size_t)qc + 1];
                c.mt = ts[0];
                c.st = ts[1];
            }
            return c;
        };
        GW gw;
        gw.issue(W1, s_tok[0], 0, t);
        gw.commit(sB[0], 0, t);
        gw.issue(W1, s_tok[1], 0, t);
        // the per-row values of stages 0, 1 and 2 in three register sets
        // (issued after the W1 rows, as in every stage: the waits placed in
        // the loop hold for its first stage too)
        int4 trn[3] = {};
        Ctx cx[3] = {};
        if (w == 0) {
            trn[0] = raw_tokens(3);
            trn[1] = raw_tokens(4);
            trn[2] = raw_tokens(5);
        }
        if (w == 1) {
            cx[0] = raw_ctx(0);
            cx[1] = raw_ctx(1);
            cx[2] = raw_ctx(2);
        }
        __syncthreads();
        // stage s: its own values are in set s % 3, refilled for stage s+3
        auto stage = [&](int4& tr, Ctx& c, int s) __attribute__((always_inline)) {
            // unit s's tile first: the W1 rows of unit s+1, loaded last stage,
            // have until it is done to arrive
            if (s < nu) {
                store_tile(sZ[s & 1], A.template mfma_acc_la<KS >= 16 ? 3 : 6>(sB[s & 1], lane, f32x16{}), w, lane);
                // the next unit in another granule: its W2 slice
                const int gn = ugran(s + 1);
                if (s + 1 < nu && gn != ga) {
                    ga = gn;
                    A.load_a(p.W2p, KS, 4 * ga + w, 4 * ga + w < nblk, lane);
                }
            }
            gw.commit(sB[(s + 1) & 1], 0, t);
            if (t < 32) {
                // unit s+3's tokens and rows
                const int q = urow(s + 3, t);
                s_tok[(s + 3) & 7][t] = q < nrows ? tok_check(make_int2(tr.x, tr.y), p.V) : -1;
                s_rows[(s + 3) & 7][t] = make_int2(tr.z, tr.w);
            } else if (w == 1 && lane < 32) {
                // unit s's row context, read by the epilogue next stage
                s_xk[s & 1][lane] = c.xk;
                s_cf[s & 1][0][lane] = c.md;
                s_cf[s & 1][1][lane] = c.sd;
                s_cf[s & 1][2][lane] = c.mt;
                s_cf[s & 1][3][lane] = c.st;
            }
            gw.issue(W1, s_tok[(s + 2) & 7], 0, t);
            // (one wave each: every vector memory instruction takes a slot in
            // the CU's queue that the streamed rows also need)
            if (w == 0) tr = raw_tokens(s + 6);
            if (w == 1) c = raw_ctx(s + 3);
            __syncthreads();
        };
        for (int s = 0; s < n_stages; s += 3) {
            stage(trn[0], cx[0], s);
            stage(trn[1], cx[1], s + 1);
            stage(trn[2], cx[2], s + 2);
        }
    } else {
        // ---------------------------------------------- epilogue waves
        // 16 lanes per row (a DPP row), 8 ids each
        const int te = t - TILE_THREADS;
        const int er = te >> 4, ec = (te & 15) * 8;
        // issue unit j's U and target rows (j past the run: its last unit
        // again, so the code stays free of branches around loads)
        auto issue = [&](int j, float (&zu)[8], float (&zt)[8]) __attribute__((always_inline)) {
            const int2 rows = s_rows[j & 7][er];  // (units past the run: its last unit's rows)
            const int cbase = ugran(min(j, nu - 1)) * GRAN + ec;
            load8_raw<VEC4>(p.U + (size_t)rows.x * p.V, cbase, p.V, zu);
            load8_raw<VEC4>(p.Lt + (size_t)rows.y * p.V, cbase, p.V, zt);
        };
        float zuA[8], ztA[8], zuB[8], ztB[8], zuC[8], ztC[8];  // unit j in A, B, C by j % 3
        issue(0, zuA, ztA);
        issue(1, zuB, ztB);
        __syncthreads();
        // The records of units [j0, j1) (their slots in s_rec) into vpart.
        // Each wave writes the four rows whose records it wrote itself, so
        // no barrier is needed; rows past the end are skipped.
        const int ew = te / WAVE, el = te & (WAVE - 1);
        auto flush = [&](int j0, int j1) __attribute__((always_inline)) {
            for (int idx = el; idx < 4 * (j1 - j0); idx += WAVE) {
                const int j = j0 + (idx >> 2), i = 4 * ew + (idx & 3);
                const int f = urow(j, i);
                if (f < nrows) p.vpart[(size_t)f * p.n_gran + ugran(j)] = s_rec[(j % SWEEP_REC_UNITS) * 32 + i];
            }
        };
        // stage s: finish unit s-1 (rows in zu/zt, tile in sZ) into LDS,
        // then refill zu/zt with unit s+2
        auto stage = [&](float (&zu)[8], float (&zt)[8], int s) __attribute__((always_inline)) {
            const int e = s - 1;
            const int ge = ugran(e), cbase = ge * GRAN + ec;
            const int f = urow(e, er);
            const bool ok = f < nrows && s_tok[e & 7][er] >= 0;
            // a row without a valid token keeps a record of zeros (its
            // request's outputs are blanked by the resolve)
            if (s >= 1 && s <= nu && !ok && (te & 15) == 0) s_rec[(e % SWEEP_REC_UNITS) * 32 + er] = make_float2(0.0f, 0.0f);
            if (s >= 1 && s <= nu && ok) {
                RowCtx rc;
                rc.req = 0;
                rc.xk = s_xk[e & 1][er];
                rc.Md = s_cf[e & 1][0][er];
                rc.iSd = 1.0f / s_cf[e & 1][1][er];
                rc.Mt = s_cf[e & 1][2][er];
                rc.iSt = 1.0f / s_cf[e & 1][3][er];
                const float* zr = sZ[e & 1] + er * ZS + ec;
                float tv = 0.0f, res = 0.0f;
                if (ge * GRAN + GRAN <= p.V) {
                    // a whole granule (every one but a ragged last)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float4 bq = *reinterpret_cast<const float4*>(zr + 4 * q);
                        const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            float d;
                            res += resid(zu[4 * q + k], bb[k], zt[4 * q + k], rc, p.c, d);
                            tv += fabsf(d);
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float4 bq = *reinterpret_cast<const float4*>(zr + 4 * q);
                        const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            // ids past V as -inf (weight 0 on both sides)
                            const bool in = cbase + 4 * q + k < p.V;
                            float d;
                            res += resid(in ? zu[4 * q + k] : -INFINITY, bb[k], in ? zt[4 * q + k] : -INFINITY, rc,
                                         p.c, d);
                            tv += fabsf(d);
                        }
                    }
                }
                tv = hex_sum(tv);
                res = hex_sum(res);
                // the records wait in LDS: stores mixed into the streamed
                // reads cost far more than the same bytes written in a burst
                if ((te & 15) == 0) s_rec[(e % SWEEP_REC_UNITS) * 32 + er] = make_float2(tv, res);
                if (rc.xk >= cbase && rc.xk < cbase + 8) p.vbias[f] = zr[rc.xk - cbase];
            }
            issue(s + 2, zu, zt);
            // a full chunk of records, or the run's last unit: write them out
            if (s >= 1 && s <= nu && (e % SWEEP_REC_UNITS == SWEEP_REC_UNITS - 1 || e == nu - 1))
                flush(e - e % SWEEP_REC_UNITS, e + 1);
            __syncthreads();
        };
        for (int s = 0; s < n_stages; s += 3) {
            stage(zuC, ztC, s);
            stage(zuA, ztA, s + 1);
            stage(zuB, ztB, s + 2);
        }
    }
}

// ------------------------------------------------------------- resolve

struct ResolveArgs {
    SweepArgs s;             // inputs shared with the sweep
    const int32_t* ell;      // NULL = gamma
    const int32_t* voff;
    const int32_t* toff;
    const float2* tgran;
    const int32_t* targ;
    uint64_t seed, round;
    int32_t* n_acc;
    int32_t* y;
    float* pt_x;
    float* c_star;
    uint32_t* status;
};

// Lane-strided TV mass of one row's granule records: lane l adds granules
// l, l + 64, l + 128, ... in that order, with the loads of a batch of 16
// issued before any of them is added, so a row costs about one memory
// latency rather than one per granule; then the 64-lane tree.  Rows of at
// most 2048 granules sum in fp32 (at most 32 terms per lane), longer rows
// in fp64 (up to 2048 terms per lane at V = 2^24).  Every kernel that
// reports c* sums in this order and precision, so verify, confidence and
// the loss give the same bits.
template <typename ACC>
__device__ inline ACC lane_tv_mass_t(const float2* vp, int n)
{
    constexpr int NB = 16;
    const int lane = threadIdx.x & (WAVE - 1);
    ACC s = 0;
    for (int g0 = 0; g0 < n; g0 += NB * WAVE) {
        float v[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int g = g0 + lane + WAVE * i;
            v[i] = vp[min(g, n - 1)].x;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (g0 + lane + WAVE * i < n) s += (ACC)v[i];
    }
    return s;
}
__device__ inline float row_tv_mass(const float2* vp, int n)
{
    if (n <= 32 * WAVE) return wave_sum(lane_tv_mass_t<float>(vp, n));
    return (float)wave_sum(lane_tv_mass_t<double>(vp, n));
}

// One wave, over the granule records of one verified row: the total TV mass
// (for c*) and the residual draw with uniform u.  Lane l reads granules
// l + 64 i, all at once; rows of more than 64 NR granules take the looped
// scan instead.
template <int NR>
__device__ inline int resid_pick_cached(const float2* vp, int n, float u, float& Z, float& before, bool& fallback,
                                        float& tv)
{
    const int lane = threadIdx.x & (WAVE - 1);
    float w[NR];
    float tl = 0.0f;  // the order and precision of row_tv_mass for n <= 2048
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int g = lane + WAVE * i;
        const float2 v = g < n ? vp[g] : make_float2(0.0f, 0.0f);
        w[i] = v.y;
        tl += v.x;
    }
    tv = wave_sum(tl);
    return wave_rounds_pick(w, u, Z, before, fallback);
}

__device__ inline int resid_pick(const float2* vp, int n, float u, float& Z, float& before, bool& fallback,
                                 float& tv)
{
    if (n <= 16 * WAVE) return resid_pick_cached<16>(vp, n, u, Z, before, fallback, tv);
    if (n <= 32 * WAVE) return resid_pick_cached<32>(vp, n, u, Z, before, fallback, tv);
    const int lane = threadIdx.x & (WAVE - 1);
    const int per = (n + WAVE - 1) / WAVE;
    const int g0 = min(lane * per, n), g1 = min(g0 + per, n);
    tv = row_tv_mass(vp, n);
    auto wf = [&](int g) { return vp[g].y; };
    double excl, Zd, bd = 0.0;
    wave_granule_scan(wf, g0, g1, excl, Zd);
    Z = (float)Zd;
    before = 0.0f;
    fallback = true;
    if (!(Zd > 0.0)) return 0;
    const int gs = wave_granule_find(wf, g0, g1, excl, (double)u * Zd, bd, fallback);
    before = (float)bd;
    return gs;
}

template <int NR>
__device__ inline int target_pick_cached(const float2* gs, int n, float M, float c, float u, float& S, float& before,
                                         bool& fallback)
{
    const int lane = threadIdx.x & (WAVE - 1);
    float w[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int g = lane + WAVE * i;
        const float2 v = g < n ? gs[g] : make_float2(-INFINITY, 0.0f);
        w[i] = v.y * softw(v.x, M, c);  // past the end: 0 * 0
    }
    return wave_rounds_pick(w, u, S, before, fallback);
}

// Draw from target row `trow` (data row (req, kk) of Lt) by inverse CDF with
// uniform u: granule masses from the first pass, then one granule rescan.
// One wave.
__device__ inline int draw_target_row(const ResolveArgs& a, int trow, int req, int kk, float u)
{
    const SweepArgs& p = a.s;
    const int lane = threadIdx.x & (WAVE - 1);
    const float2* gs = a.tgran + (size_t)trow * p.n_gran;
    const float M = p.trow[trow].x;
    const float c = p.c;
    const int n = p.n_gran;
    float S, before;
    bool fallback;
    int gstar;
    if (n <= 16 * WAVE) {
        gstar = target_pick_cached<16>(gs, n, M, c, u, S, before, fallback);
    } else if (n <= 32 * WAVE) {
        gstar = target_pick_cached<32>(gs, n, M, c, u, S, before, fallback);
    } else {
        const int per = (n + WAVE - 1) / WAVE;
        const int g0 = min(lane * per, n), g1 = min(g0 + per, n);
        auto wf = [&](int g) { const float2 v = gs[g]; return v.y * softw(v.x, M, c); };
        double excl, Sd, bd;
        wave_granule_scan(wf, g0, g1, excl, Sd);
        gstar = wave_granule_find(wf, g0, g1, excl, (double)u * Sd, bd, fallback);
        S = (float)Sd;
        before = (float)bd;
    }
    const float target = u * S;
    const float* L = p.Lt + ((size_t)req * (p.gamma + 1) + kk) * p.V;
    const int ca = gstar * GRAN + 2 * lane, cb = ca + 1;
    const float za = ca < p.V ? L[ca] : -INFINITY, zb = cb < p.V ? L[cb] : -INFINITY;
    float e;
    return gstar * GRAN + granule_pick_dpp(softw(za, M, c), softw(zb, M, c), before, target, fallback, e);
}

// Resolve workgroups of eight waves (the granule rescan needs up to 256
// VGPRs): RES_SEARCH waves for the per-position c* and residual search, the
// last one for the accept tests.
constexpr int RES_WAVES = 8;
constexpr int RES_SEARCH = RES_WAVES - 1;
constexpr int RES_THREADS = RES_WAVES * WAVE;

// The draft side of the resolve, for drafts of the Markov head: p_d(x) from
// U, the bias the sweep recorded at x and propose's (M, S); the residual
// rescan of one granule recomputes its bias on MFMA (waves 0-3) with the
// sweep's own expression.
template <typename WT, int KS>
struct MarkovDraft {
    __device__ inline bool bad_anchor(const ResolveArgs& a, int r) const
    {
        const int x0r = a.s.x0[r];
        return x0r < 0 || x0r >= a.s.V;
    }
    // the token before position 1 (the rescan of a rejection there needs its W1 row)
    __device__ inline int anchor(const ResolveArgs& a, int r) const { return a.s.x0[r]; }
    __device__ inline double pd_at(const ResolveArgs& a, int r, int t, int xk, int voff) const
    {
        const SweepArgs& p = a.s;
        const size_t so = (size_t)r * p.gamma + t;
        const double zd = (double)p.U[so * p.V + xk] + (double)p.vbias[voff + t];
        return exp2((zd - (double)p.dstats[2 * so]) * (double)p.c) / (double)p.dstats[2 * so + 1];
    }
    // zrow[i] = residual weight of id 128 gstar + i at position kstar.
    // xp: the token before position kstar (the anchor for kstar = 1); toff:
    // the request's first target row.  The row's softmax statistics are read
    // at addresses known here (not through the verified-row map), so that the
    // W1 row, U, Lt, statistics and W2 loads all go out before any is waited on.
    __device__ inline void residual_granule(const ResolveArgs& a, int r, int kstar, int gstar, int voff, int toff,
                                            int xp, float* zrow, int w, int lane) const
    {
        const SweepArgs& p = a.s;
        if (w >= 4) return;
        const int G = p.gamma;
        const int f = voff + kstar - 1;
        const int n = lane & 31, h = lane >> 5;
        const int nf = f & (BLOCK_ROWS - 1);
        const int ks = k_steps<WT>(p.r);
        const int b = 4 * gstar + w;
        const int c0 = gstar * GRAN + 32 * w;
        const bool v4 = (p.V % 4) == 0;
        const size_t so = (size_t)r * G + kstar - 1;
        typename TileOps<WT, KS>::BRow brow;
        brow.load(reinterpret_cast<const WT*>(p.W1), p.r, n == nf ? xp : -1, ks, lane);
        float uu[16], ll[16];
        load_acc16(p.U + so * p.V, c0, h, p.V, v4, uu);
        load_acc16(p.Lt + ((size_t)r * (G + 1) + kstar - 1) * p.V, c0, h, p.V, v4, ll);
        const float md = p.dstats[2 * so], sd = p.dstats[2 * so + 1];
        const float2 ts = p.trow[toff + kstar - 1];
        TileOps<WT, KS> A;
        A.load_a(p.W2p, ks, b, b < (p.V + 31) / 32, lane);
        RowCtx rc{};
        rc.Md = md;
        rc.iSd = 1.0f / sd;
        rc.Mt = ts.x;
        rc.iSt = 1.0f / ts.y;
        const f32x16 acc = A.mfma_row(brow, ks);
        if (n == nf) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int col = c0 + 8 * (j >> 2) + 4 * h + (j & 3);
                float d;
                zrow[32 * w + 8 * (j >> 2) + 4 * h + (j & 3)] = col < p.V ? resid(uu[j], acc[j], ll[j], rc, p.c, d) : 0.0f;
            }
        }
    }
};

// Residual weight max(0, p_t - p_d) of one id for a clustered draft (p_d = 0
// outside the row's clusters); the sparse sweep and the resolve's rescan both
// use this expression.
__device__ inline float cl_resid(float lt, float zd, bool in, float Mt, float iSt, float Md, float iSd, float c, float& d)
{
    const float pd = in ? softw(zd, Md, c) * iSd : 0.0f;
    const float pt = softw(lt, Mt, c) * iSt;
    d = pt - pd;
    return fmaxf(d, 0.0f);
}

// The draft side of the resolve for drafts of the clustered head: the fine
// logit of id v is found through its cluster and place (tok_slot) and the
// cluster's place in the row's ascending list (binary search).
struct ClusterDraft {
    const int32_t* tok_slot;
    const int32_t* sel;
    const float* zf;
    int N_c, K_c, max_cl;
    __device__ inline bool bad_anchor(const ResolveArgs&, int) const { return false; }
    __device__ inline int anchor(const ResolveArgs&, int) const { return -1; }  // (no anchor: not read)
    __device__ inline float logit(int f, int v, bool& in) const
    {
        in = false;
        const int32_t slot = tok_slot[v];
        if (slot < 0) return 0.0f;
        const int c = (int)((uint32_t)slot >> 16), i = slot & 0xFFFF;
        const int32_t* sr = sel + (size_t)f * K_c;
        int lo = 0, hi = K_c;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sr[mid] < c) lo = mid + 1;
            else hi = mid;
        }
        if (lo >= K_c || sr[lo] != c || i >= max_cl) return 0.0f;
        in = true;
        return zf[((size_t)f * K_c + lo) * max_cl + i];
    }
    __device__ inline double pd_at(const ResolveArgs& a, int r, int t, int xk, int voff) const
    {
        const SweepArgs& p = a.s;
        const int f = voff + t;
        bool in;
        const float z = logit(f, xk, in);
        if (!in) return 0.0;
        const size_t so = (size_t)r * p.gamma + t;
        return exp2(((double)z - (double)p.dstats[2 * so]) * (double)p.c) / (double)p.dstats[2 * so + 1];
    }
    __device__ inline void residual_granule(const ResolveArgs& a, int r, int kstar, int gstar, int voff, int toff,
                                            int, float* zrow, int w, int lane) const
    {
        const SweepArgs& p = a.s;
        if (w >= 2) return;
        const int f = voff + kstar - 1;
        const float2 ts = p.trow[toff + kstar - 1];
        const size_t so = (size_t)r * p.gamma + kstar - 1;
        const float Md = p.dstats[2 * so], iSd = 1.0f / p.dstats[2 * so + 1];
        const float iSt = 1.0f / ts.y;
        const int i = 64 * w + lane, v = gstar * GRAN + i;
        float res = 0.0f;
        if (v < p.V) {
            bool in;
            const float z = logit(f, v, in);
            const float lt = p.Lt[((size_t)r * (p.gamma + 1) + kstar - 1) * p.V + v];
            float d;
            res = cl_resid(lt, z, in, ts.x, iSt, Md, iSd, p.c, d);
        }
        zrow[i] = res;
    }
};

// One workgroup of eight waves per request.
// Phase 1 does everything that does not depend on which position is rejected
// first, in parallel: the accept test of every verified position (one lane
// each of the last wave, fp64 on the drafted id), c* of every position and
// the residual granule search of every position (position k on wave
// (k - 1) % RES_SEARCH), and the bonus draw (the last wave again).
// Phase 2 rescans one granule of the first rejected position's residual
// (the draft side's waves).
template <class D, bool GREEDY>
__device__ inline void resolve_body(const ResolveArgs& a, const D& dr)
{
    const SweepArgs& p = a.s;
    const int r = blockIdx.x, t = threadIdx.x;
    const int lane = t & (WAVE - 1), w = t / WAVE;
    const int G = p.gamma;
    __shared__ int s_acc[64];
    __shared__ int s_g[65];        // granule of the residual draw at k (index k-1)
    __shared__ float s_before[65];
    __shared__ int s_fb[65];
    __shared__ float s_Z[65];
    __shared__ int s_bonus;
    __shared__ int s_y;
    __shared__ int s_x[65];        // the anchor, then the drafted tokens (read by the accept tests)
    __shared__ float zrow[GRAN];

    const int Lr = a.ell ? a.ell[r] : G;
    const bool bad_len = Lr < 0 || Lr > G;
    const int L = bad_len ? 0 : Lr;
    const int voff = a.voff ? a.voff[r] : r * G;
    const int toff = a.toff ? a.toff[r] : r * p.P;
    bool bad = bad_len || dr.bad_anchor(a, r);

    // ---- phase 1a: accept tests, one lane of wave RES_SEARCH per position
    const int ia = t - RES_SEARCH * WAVE;  // the position (0-based) of this lane
    bool rej = false;                      // this lane's position was rejected
    if (t == 0) s_x[0] = dr.anchor(a, r);
    if (ia >= 0 && ia < L) {
        const int xk = p.x[(size_t)r * G + ia];
        s_x[ia + 1] = xk;  // (the rescan's previous token, without a second load)
        if (xk < 0 || xk >= p.V) {
            bad = true;
        } else {
            const int tr = toff + ia;
            const float2 ts = p.trow[tr];
            const double zt = (double)p.Lt[((size_t)r * (G + 1) + ia) * p.V + xk];
            const double pt = exp2((zt - (double)ts.x) * (double)p.c) / (double)ts.y;
            int acc;
            if (GREEDY) {
                acc = xk == a.targ[tr];
            } else {
                const double pd = dr.pd_at(a, r, ia, xk, voff);
                double ratio;
                if (pd > 0.0) ratio = pt / pd;
                else ratio = pt > 0.0 ? INFINITY : 0.0;
                const double u1 = u24d(philox((uint32_t)(ia + 1), (uint32_t)r, a.round, a.seed).w[1]);
                acc = u1 < ratio;
            }
            s_acc[ia] = acc;
            rej = !acc;
            if (a.pt_x) a.pt_x[(size_t)r * G + ia] = (float)pt;
        }
    } else if (ia >= L && ia < G) {
        if (a.pt_x) a.pt_x[(size_t)r * G + ia] = NAN;
        if (a.c_star) a.c_star[(size_t)r * G + ia] = NAN;
    }
    // ---- phase 1b: per position, one wave: c* and the residual granule search
    for (int k = w + 1; w < RES_SEARCH && k <= L; k += RES_SEARCH) {
        const float2* vp = p.vpart + (size_t)(voff + k - 1) * p.n_gran;
        const float u2 = u24f(philox((uint32_t)k, (uint32_t)r, a.round, a.seed).w[2]);
        float Z, before, tv;
        bool fallback;
        const int gs = resid_pick(vp, p.n_gran, u2, Z, before, fallback, tv);
        if (lane == 0) {
            if (a.c_star) a.c_star[(size_t)r * G + k - 1] = fminf(fmaxf(1.0f - 0.5f * tv, 0.0f), 1.0f);
            s_g[k - 1] = Z > 0.0f ? gs : 0;
            s_before[k - 1] = Z > 0.0f ? before : 0.0f;
            s_fb[k - 1] = Z > 0.0f ? fallback : true;
            s_Z[k - 1] = Z;
        }
    }
    // ---- phase 1c: the bonus draw after a full accept (the last wave, after
    // its accept tests; skipped once one of them has rejected, as the bonus
    // is then not emitted)
    if (w == RES_SEARCH && __ballot(rej) == 0) {
        int yb;
        if (GREEDY) {
            yb = a.targ[toff + L];
        } else {
            const float u2 = u24f(philox((uint32_t)(L + 1), (uint32_t)r, a.round, a.seed).w[2]);
            yb = draw_target_row(a, toff + L, r, L, u2);
        }
        if (lane == 0) s_bonus = yb;
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (t == 0) raise_flag(a.status, bad_len ? 2u : 1u);
        if (t == 0) a.n_acc[r] = -1;
        if (t <= G) a.y[(size_t)r * (G + 1) + t] = -1;
        if (t < G) {
            if (a.pt_x) a.pt_x[(size_t)r * G + t] = NAN;
            if (a.c_star) a.c_star[(size_t)r * G + t] = NAN;
        }
        return;
    }
    int kstar = 0;
    for (int k = 1; k <= L; ++k)
        if (!s_acc[k - 1]) { kstar = k; break; }
    const int nacc = kstar ? kstar - 1 : L;

    // ---- phase 2: the emitted token
    if (!kstar) {
        if (t == 0) s_y = s_bonus;
    } else if (GREEDY) {
        if (t == 0) s_y = a.targ[toff + kstar - 1];
    } else if (s_Z[kstar - 1] > 0.0f) {
        const int gstar = s_g[kstar - 1];
        dr.residual_granule(a, r, kstar, gstar, voff, toff, s_x[kstar - 1], zrow, w, lane);
        __syncthreads();
        if (w == 0) {
            float e;
            const int y = gstar * GRAN + granule_pick_dpp(zrow[2 * lane], zrow[2 * lane + 1], s_before[kstar - 1],
                                                      s_Z[kstar - 1] * u24f(philox((uint32_t)kstar, (uint32_t)r,
                                                                                   a.round, a.seed).w[2]),
                                                      s_fb[kstar - 1], e);
            if (lane == 0) s_y = y;
        }
    } else if (w == 0) {
        // no residual mass (p_t == p_d in fp32): draw from p_t itself
        const float u2 = u24f(philox((uint32_t)kstar, (uint32_t)r, a.round, a.seed).w[2]);
        const int y = draw_target_row(a, toff + kstar - 1, r, kstar - 1, u2);
        if (lane == 0) s_y = y;
    }
    __syncthreads();
    if (t == 0) a.n_acc[r] = nacc;
    if (t <= G) {
        int v = -1;
        if (t < nacc) v = p.x[(size_t)r * G + t];
        else if (t == nacc) v = s_y;
        a.y[(size_t)r * (G + 1) + t] = v;
    }
}

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(RES_THREADS) void k_verify_resolve(ResolveArgs a)
{
    resolve_body<MarkovDraft<WT, KS>, GREEDY>(a, MarkovDraft<WT, KS>{});
}

template <bool GREEDY>
__global__ __launch_bounds__(RES_THREADS) void k_cluster_resolve(ResolveArgs a, ClusterDraft cd)
{
    resolve_body<ClusterDraft, GREEDY>(a, cd);
}

// ------------------------------------------------------ clustered drafts

// The sweep for drafts of the clustered head: one workgroup per (verified
// row f = blockIdx.x, run of gpc granules = blockIdx.y).  An LDS table maps every cluster to its place
// in the row's list (-1: not selected); each wave takes one granule at a
// time (two ids per lane): p_t from the target row, p_d from the fine
// logit of the id's cluster and place (0 outside the row's clusters), and
// the granule's (TV mass, residual mass).  There is no contraction here:
// the kernel streams the target rows and looks up the fine logits.
struct ClusterSweepArgs {
    const float* Lt;
    const int32_t* tok_slot;
    const int32_t* sel;
    const float* zf;
    const float* dstats;
    const float2* trow;
    int gamma, P, N_c, K_c, max_cl, V, n_gran, gpc;
    float c;
    float2* vpart;
};

__global__ __launch_bounds__(TILE_THREADS) void k_cluster_sweep(ClusterSweepArgs a)
{
    __shared__ short s_j[CL_MAX_NC];
    const int f = blockIdx.x, t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int r = f / a.gamma, kk = f - r * a.gamma;
    for (int c = t; c < a.N_c; c += TILE_THREADS) s_j[c] = -1;
    __syncthreads();
    if (t < a.K_c) {
        const int cj = a.sel[(size_t)f * a.K_c + t];
        if (cj >= 0 && cj < a.N_c) s_j[cj] = (short)t;
    }
    __syncthreads();
    const float Md = a.dstats[2 * (size_t)f], iSd = 1.0f / a.dstats[2 * (size_t)f + 1];
    const float2 ts = a.trow[r * a.P + kk];
    const float iSt = 1.0f / ts.y;
    const float* lrow = a.Lt + ((size_t)r * (a.gamma + 1) + kk) * a.V;
    const float* zr = a.zf + (size_t)f * a.K_c * a.max_cl;
    const int g0 = blockIdx.y * a.gpc, g1 = min(g0 + a.gpc, a.n_gran);
    // batches of CSB granules per wave: the target values and slots of the
    // whole batch are loaded first, then the fine logits they name
    constexpr int CSB = 8;
    for (int gb = g0 + w; gb < g1; gb += CSB * (TILE_THREADS / WAVE)) {
        float lt[CSB][2];
        int32_t sl[CSB][2];
#pragma unroll
        for (int u = 0; u < CSB; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int v = min((gb + u * (TILE_THREADS / WAVE)) * GRAN + 2 * lane + e, a.V - 1);
                lt[u][e] = lrow[v];
                sl[u][e] = a.tok_slot[v];
            }
        float zz[CSB][2];
        int jj[CSB][2];
#pragma unroll
        for (int u = 0; u < CSB; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int32_t slot = sl[u][e];
                int j = -1, i = 0;
                if (slot >= 0) {
                    const int c = (int)((uint32_t)slot >> 16);
                    i = slot & 0xFFFF;
                    j = c < a.N_c && i < a.max_cl ? s_j[c] : -1;
                }
                jj[u][e] = j;
                zz[u][e] = j >= 0 ? zr[(size_t)j * a.max_cl + i] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < CSB; ++u) {
            const int g = gb + u * (TILE_THREADS / WAVE);
            float tv = 0.0f, res = 0.0f;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (g * GRAN + 2 * lane + e < a.V) {
                    float d;
                    res += cl_resid(lt[u][e], zz[u][e], jj[u][e] >= 0, ts.x, iSt, Md, iSd, a.c, d);
                    tv += fabsf(d);
                }
            }
            tv = wave_sum(tv);
            res = wave_sum(res);
            if (lane == 0 && g < g1) a.vpart[(size_t)f * a.n_gran + g] = make_float2(tv, res);
        }
    }
}

// --------------------------------------------------------- confidence

// One workgroup per request, one wave per drafted position (positions
// k, k + 4, ... for wave k): c*_k, then the running products a*_k (fp64,
// left to right) by one thread.
__global__ __launch_bounds__(TILE_THREADS) void k_conf_finalize(const float2* vpart, const int32_t* x0,
                                                                const int32_t* x, int R, int gamma, int V,
                                                                int n_gran, float* c_star, double* a_star,
                                                                uint32_t* status)
{
    __shared__ float s_cs[64];
    const int r = blockIdx.x;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    // every wave checks the request's ids, so each takes the same branch
    bool bad = lane == 0 && (x0[r] < 0 || x0[r] >= V);
    for (int k = lane; k < gamma; k += WAVE) bad = bad || x[(size_t)r * gamma + k] < 0 || x[(size_t)r * gamma + k] >= V;
    if (__any(bad)) {
        if (t == 0) raise_flag(status, 1u);
        for (int k = t; k < gamma; k += TILE_THREADS) {
            c_star[(size_t)r * gamma + k] = NAN;
            if (a_star) a_star[(size_t)r * gamma + k] = NAN;
        }
        return;
    }
    for (int k = w; k < gamma; k += TILE_THREADS / WAVE) {
        const float tv = row_tv_mass(vpart + ((size_t)r * gamma + k) * n_gran, n_gran);
        if (lane == 0) s_cs[k] = fminf(fmaxf(1.0f - 0.5f * tv, 0.0f), 1.0f);
    }
    __syncthreads();
    if (t < gamma) c_star[(size_t)r * gamma + t] = s_cs[t];
    if (a_star && t == 0) {
        double run = 1.0;
        for (int k = 0; k < gamma; ++k) {
            run *= (double)s_cs[k];
            a_star[(size_t)r * gamma + k] = run;
        }
    }
}

// ------------------------------------------------------- training loss

// One wave per drafted position f = (r, k): the TV mass over the granule
// records (in the order every c* is summed), the draft
// log-probability of the label from the draft row's (M, S) and the bias the
// sweep recorded at it, the confidence BCE, the position weight
// w_k = exp(-(k-1)/gamma) and d loss / dq.  A position whose label chain
// holds an id outside [0, V) gets NaN terms, no contribution, and the flag.
__global__ __launch_bounds__(TILE_THREADS) void k_loss_terms(const float2* vpart, const float* vbias, const float* U,
                                                             const float* dstats, const float* q, const int32_t* x0,
                                                             const int32_t* y, int R, int gamma, int V, int n_gran,
                                                             float invT, float a_ce, float a_tv, float a_conf,
                                                             double inv_wsum, float* terms, float* dq,
                                                             double* contrib, uint32_t* status)
{
    const int f = blockIdx.x * (TILE_THREADS / WAVE) + threadIdx.x / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    if (f >= R * gamma) return;
    const int r = f / gamma, k = f - r * gamma + 1;
    // the chain of labels up to this position: the anchor and y_1 .. y_k
    bool bad = lane == 0 && (x0[r] < 0 || x0[r] >= V);
    for (int j = lane; j < k; j += WAVE) bad = bad || y[(size_t)r * gamma + j] < 0 || y[(size_t)r * gamma + j] >= V;
    if (__any(bad)) {
        if (lane == 0) {
            raise_flag(status, 1u);
            contrib[f] = 0.0;
            if (terms) terms[3 * (size_t)f] = terms[3 * (size_t)f + 1] = terms[3 * (size_t)f + 2] = NAN;
            if (dq) dq[f] = NAN;
        }
        return;
    }
    const float l1 = row_tv_mass(vpart + (size_t)f * n_gran, n_gran);
    if (lane == 0) {
        const float cs = fminf(fmaxf(1.0f - 0.5f * l1, 0.0f), 1.0f);
        const int yk = y[f];
        const float zy = U[(size_t)f * V + yk] + vbias[f];
        const float ce = logf(dstats[2 * (size_t)f + 1]) - (zy - dstats[2 * (size_t)f]) * invT;
        const float qv = q[f];
        const float bce = fmaxf(qv, 0.0f) - qv * cs + log1pf(expf(-fabsf(qv)));
        const double wk = exp(-(double)(k - 1) / (double)gamma);
        contrib[f] = wk * ((double)a_ce * ce + (double)a_tv * l1 + (double)a_conf * bce);
        if (terms) {
            terms[3 * (size_t)f] = ce;
            terms[3 * (size_t)f + 1] = l1;
            terms[3 * (size_t)f + 2] = bce;
        }
        if (dq) dq[f] = (float)(wk * (double)a_conf * (double)(1.0f / (1.0f + expf(-qv)) - cs) * inv_wsum);
    }
}

// The weighted mean: one workgroup, contributions summed in a fixed order
// (lane-strided, then waves), so the loss is deterministic.
__global__ __launch_bounds__(TILE_THREADS) void k_loss_reduce(const double* contrib, int n, double inv_wsum,
                                                              double* loss)
{
    __shared__ double sw[TILE_THREADS / WAVE];
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    double s = 0.0;
    for (int i = t; i < n; i += TILE_THREADS) s += contrib[i];
    s = wave_sum(s);
    if (lane == 0) sw[w] = s;
    __syncthreads();
    if (t == 0) {
        double tot = 0.0;
        for (int i = 0; i < TILE_THREADS / WAVE; ++i) tot += sw[i];
        *loss = tot * inv_wsum;
    }
}

// ------------------------------------------------------------ launchers

// Workgroups cover one granule and `bpc` consecutive 32-row blocks; the row
// blocks are split into just enough chunks to give about `target`
// workgroups.
static void sweep_grid(int nrows, int n_gran, int& bpc, int& n_chunks, int target = 1024)
{
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    n_chunks = (target + n_gran - 1) / n_gran;
    if (n_chunks > n_rb) n_chunks = n_rb;
    if (n_chunks < 1) n_chunks = 1;
    bpc = (n_rb + n_chunks - 1) / n_chunks;
    n_chunks = (n_rb + bpc - 1) / bpc;
}

static SweepArgs make_sweep(const DraftArgs& a, const float* dstats, const float* Lt, int P,
                            const VerifyWs& w, const int32_t* counts, bool maps)
{
    SweepArgs s{};
    s.U = a.U; s.W1 = a.W1; s.W2p = a.W2; s.x0 = a.x0; s.x = a.x; s.dstats = dstats; s.Lt = Lt;
    s.R = a.R; s.gamma = a.gamma; s.r = a.r; s.V = a.V; s.P = P; s.c = a.c; s.vec4 = (a.V % 4) == 0;
    s.n_gran = n_granules(a.V);
    s.max_rows = a.R * a.gamma;
    sweep_grid(s.max_rows, s.n_gran, s.bpc, s.n_chunks);
    s.div_rb = FastDiv::make((s.max_rows + BLOCK_ROWS - 1) / BLOCK_ROWS);
    s.div_g = FastDiv::make(a.gamma);
    s.rtab = w.rtab;
    s.rctab = w.rctab;
    s.vmap = maps ? w.vmap : nullptr;
    s.counts = counts;
    s.trow = w.trow;
    s.vpart = w.vpart;
    s.vbias = w.vbias;
    s.staged_only = (a.path & PATH_NO_PIPELINED_SWEEP) != 0;
    return s;
}

// Workgroups of k_target_rows the current device holds at once; cached per
// device.
static int trow_slots()
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];  // slots + 1; 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 512;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_target_rows, TROW_THREADS, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        v = per_cu * cus + 1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

static hipError_t target_pass(const DraftArgs& a, const float* Lt, int P, int max_rows,
                              const VerifyWs& w, const int32_t* counts, bool maps, hipStream_t s)
{
    TargetArgs t{};
    t.Lt = Lt; t.R = a.R; t.gamma = a.gamma; t.V = a.V; t.P = P; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.n_gran = n_granules(a.V);
    t.max_rows = max_rows;
    t.tmap = maps ? w.tmap : nullptr;
    t.counts = counts;
    t.tgran = w.tgran; t.tgidx = w.tgidx; t.trow = w.trow; t.targ = w.targ;
    // split rows over several workgroups while there are fewer than about
    // 256 of them; with more rows than the device holds workgroups at once,
    // into as many parts (1, 2 or 4) as make the last round of workgroups
    // least ragged (rounds per part, fewest parts on a tie)
    const int steps = (t.n_gran + TROW_GRANS - 1) / TROW_GRANS;
    t.nsplit = std::max(1, std::min(std::min(TROW_TARGET_WGS / std::max(max_rows, 1), steps), TROW_MAX_SPLIT));
    const int slots = trow_slots();
    if (max_rows > slots) {
        long best_num = -1, best_den = 1;
        for (int n = 1; n <= 4 && n <= steps; n *= 2) {
            const long rounds = ((long)max_rows * n + slots - 1) / slots;
            if (best_num < 0 || rounds * best_den < best_num * n) {
                best_num = rounds;
                best_den = n;
                t.nsplit = n;
            }
        }
    }
    t.tpart = w.tpart;
    {
        ProfScope ps("target_rows", s);
        hipLaunchKernelGGL(k_target_rows, dim3(max_rows * t.nsplit), dim3(TROW_THREADS), 0, s, t);
        if (t.nsplit > 1) hipLaunchKernelGGL(k_target_merge, dim3((max_rows + 255) / 256), dim3(256), 0, s, t);
    }
    return hipGetLastError();
}

// Workgroups of k_verify_sweep_ws<KS, VEC4> the current device holds at once
// (the occupancy API's figure times the CUs), cached per device.
template <int KS, bool VEC4>
static int sweep_ws_slots()
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];  // slots + 1; 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_verify_sweep_ws<KS, VEC4, false>,
                                                         3 * TILE_THREADS, 0) != hipSuccess || per_cu <= 0)
            per_cu = 1;
        v = per_cu * cus + 1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

template <typename WT, int KS>
static void launch_sweep(const SweepArgs& sw, hipStream_t s)
{
    const dim3 grid(xcd_grid(sw.n_gran * sw.n_chunks));
    const dim3 blk(TILE_THREADS);
    // (r = 512 keeps the staged kernel: its W2 slice alone would take 128 of
    // the pipelined kernel's 170 registers per lane)
    if constexpr (std::is_same<WT, bf16w>::value && (KS == 8 || KS == 16)) {
        if (sw.r == 16 * KS && !sw.staged_only) {
            if (sw.vmap) {
                // the scheduled rows' records, after the target rows' statistics
                hipLaunchKernelGGL(k_row_table, dim3((sw.max_rows + TILE_THREADS - 1) / TILE_THREADS),
                                   dim3(TILE_THREADS), 0, s, sw.vmap, sw.counts, sw.x0, sw.x, sw.dstats, sw.trow,
                                   sw.gamma, sw.max_rows, const_cast<int4*>(sw.rtab), const_cast<float4*>(sw.rctab));
            }
            // as many workgroups as fit at once, each with one run of units
            const long units = (long)sw.n_gran * ((sw.max_rows + BLOCK_ROWS - 1) / BLOCK_ROWS);
            const dim3 blk2(3 * TILE_THREADS);
            // (a multiple of the XCD count, rounded down unless that is zero)
            auto grid_of = [&](int slots) {
                const long n = std::min<long>(slots, units);
                return (unsigned)(n >= NUM_XCD ? n / NUM_XCD * NUM_XCD : xcd_grid((int)n));
            };
            const dim3 g2(grid_of(sw.vec4 ? sweep_ws_slots<KS, true>() : sweep_ws_slots<KS, false>()));
            if (sw.vmap) {
                if (sw.vec4) hipLaunchKernelGGL((k_verify_sweep_ws<KS, true, true>), g2, blk2, 0, s, sw);
                else hipLaunchKernelGGL((k_verify_sweep_ws<KS, false, true>), g2, blk2, 0, s, sw);
            } else {
                if (sw.vec4) hipLaunchKernelGGL((k_verify_sweep_ws<KS, true, false>), g2, blk2, 0, s, sw);
                else hipLaunchKernelGGL((k_verify_sweep_ws<KS, false, false>), g2, blk2, 0, s, sw);
            }
            return;
        }
    }
    if (sw.vmap) {
        if (sw.vec4) hipLaunchKernelGGL((k_verify_sweep<WT, KS, true, true>), grid, blk, 0, s, sw);
        else hipLaunchKernelGGL((k_verify_sweep<WT, KS, false, true>), grid, blk, 0, s, sw);
    } else {
        if (sw.vec4) hipLaunchKernelGGL((k_verify_sweep<WT, KS, true, false>), grid, blk, 0, s, sw);
        else hipLaunchKernelGGL((k_verify_sweep<WT, KS, false, false>), grid, blk, 0, s, sw);
    }
}

template <typename WT, int KS>
static hipError_t verify_impl(const DraftArgs& a, const float* pd_stats, const float* Lt,
                              const int32_t* ell, int32_t* n_acc, int32_t* y, float* pt_x,
                              float* c_star, const VerifyWs& w, int32_t* counts, hipStream_t s)
{
    const bool maps = ell != nullptr;
    const int P = a.gamma + 1;
    hipError_t e;
    if (maps) {
        ProfScope ps("plan", s);
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(TILE_THREADS), 0, s, ell, a.R, a.gamma, w.voff, w.toff,
                           w.vmap, w.tmap, counts, a.status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = target_pass(a, Lt, P, a.R * P, w, counts, maps, s);
    if (e != hipSuccess) return e;
    SweepArgs sw = make_sweep(a, pd_stats, Lt, P, w, counts, maps);
    {
        ProfScope ps("verify_sweep", s);
        launch_sweep<WT, KS>(sw, s);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ResolveArgs ra{};
    ra.s = sw;
    ra.ell = ell;
    ra.voff = maps ? w.voff : nullptr;
    ra.toff = maps ? w.toff : nullptr;
    ra.tgran = w.tgran;
    ra.targ = w.targ;
    ra.seed = a.seed; ra.round = a.round;
    ra.n_acc = n_acc; ra.y = y; ra.pt_x = pt_x; ra.c_star = c_star; ra.status = a.status;
    {
        ProfScope ps("verify_resolve", s);
        if (a.greedy)
            hipLaunchKernelGGL((k_verify_resolve<WT, KS, true>), dim3(a.R), dim3(RES_THREADS), 0, s, ra);
        else
            hipLaunchKernelGGL((k_verify_resolve<WT, KS, false>), dim3(a.R), dim3(RES_THREADS), 0, s, ra);
    }
    return hipGetLastError();
}

template <typename WT, int KS>
static hipError_t confidence_impl(const DraftArgs& a, const float* pd_stats, const float* Lt,
                                  float* c_star, double* a_star, const VerifyWs& w, hipStream_t s)
{
    hipError_t e;
    const float* dstats = pd_stats;
    if (!dstats) {
        e = launch_draft_row_stats(a, w, s);
        if (e != hipSuccess) return e;
        dstats = reinterpret_cast<const float*>(w.drow);
    }
    const int P = a.gamma;  // no bonus row
    e = target_pass(a, Lt, P, a.R * P, w, nullptr, false, s);
    if (e != hipSuccess) return e;
    SweepArgs sw = make_sweep(a, dstats, Lt, P, w, nullptr, false);
    {
        ProfScope ps("verify_sweep", s);
        launch_sweep<WT, KS>(sw, s);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope ps("conf_finalize", s);
        hipLaunchKernelGGL(k_conf_finalize, dim3(a.R), dim3(TILE_THREADS), 0, s,
                           (const float2*)w.vpart, a.x0, a.x, a.R, a.gamma, a.V, sw.n_gran, c_star, a_star,
                           a.status);
    }
    return hipGetLastError();
}

// Training loss over the drafted positions, teacher-forced on the labels
// a.x: the draft rows' (M, S) with the labels' biases, the target rows'
// (M, S), the sweep (TV mass and the bias at each label), then the terms
// and their weighted mean.
template <typename WT, int KS>
static hipError_t loss_impl(const DraftArgs& a, const float* Lt, const LossArgs& l, const VerifyWs& w,
                            hipStream_t s)
{
    hipError_t e = launch_draft_row_stats(a, w, s);
    if (e != hipSuccess) return e;
    const float* dstats = reinterpret_cast<const float*>(w.drow);
    const int P = a.gamma;  // no bonus row
    e = target_pass(a, Lt, P, a.R * P, w, nullptr, false, s);
    if (e != hipSuccess) return e;
    SweepArgs sw = make_sweep(a, dstats, Lt, P, w, nullptr, false);
    {
        ProfScope ps("verify_sweep", s);
        launch_sweep<WT, KS>(sw, s);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    double wsum = 0.0;
    for (int k = 1; k <= a.gamma; ++k) wsum += (double)a.R * exp(-(double)(k - 1) / (double)a.gamma);
    const int n = a.R * a.gamma;
    {
        ProfScope ps("loss_terms", s);
        hipLaunchKernelGGL(k_loss_terms, dim3((n + 3) / 4), dim3(TILE_THREADS), 0, s, (const float2*)w.vpart,
                           (const float*)w.vbias, a.U, dstats, l.q, a.x0, a.x, a.R, a.gamma, a.V, sw.n_gran,
                           l.invT, l.a_ce, l.a_tv, l.a_conf, 1.0 / wsum, l.terms, l.dq,
                           w.contrib, a.status);
        hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(TILE_THREADS), 0, s, (const double*)w.contrib, n,
                           1.0 / wsum, l.loss);
    }
    return hipGetLastError();
}

template <typename WT, int KS>
struct VerifyF {
    static hipError_t run(const DraftArgs& a, const float* pd_stats, const float* Lt, const int32_t* ell,
                          int32_t* n_acc, int32_t* y, float* pt_x, float* c_star, const VerifyWs& w,
                          int32_t* counts, hipStream_t s)
    {
        return verify_impl<WT, KS>(a, pd_stats, Lt, ell, n_acc, y, pt_x, c_star, w, counts, s);
    }
};
template <typename WT, int KS>
struct ConfF {
    static hipError_t run(const DraftArgs& a, const float* pd_stats, const float* Lt, float* c_star,
                          double* a_star, const VerifyWs& w, hipStream_t s)
    {
        return confidence_impl<WT, KS>(a, pd_stats, Lt, c_star, a_star, w, s);
    }
};

hipError_t launch_verify(const DraftArgs& a, const float* pd_stats, const float* Lt, const int32_t* ell,
                         int32_t* n_acc, int32_t* y, float* pt_x, float* c_star, const VerifyWs& w,
                         int32_t* counts, hipStream_t s)
{
    return dispatch_ks<VerifyF>(a.w_dtype, a.r, a, pd_stats, Lt, ell, n_acc, y, pt_x, c_star, w, counts, s);
}

hipError_t launch_confidence(const DraftArgs& a, const float* pd_stats, const float* Lt, float* c_star,
                             double* a_star, const VerifyWs& w, hipStream_t s)
{
    return dispatch_ks<ConfF>(a.w_dtype, a.r, a, pd_stats, Lt, c_star, a_star, w, s);
}

template <typename WT, int KS>
struct LossF {
    static hipError_t run(const DraftArgs& a, const float* Lt, const LossArgs& l, const VerifyWs& w, hipStream_t s)
    {
        return loss_impl<WT, KS>(a, Lt, l, w, s);
    }
};

hipError_t launch_draft_loss(const DraftArgs& a, const float* Lt, const LossArgs& l, const VerifyWs& w,
                             hipStream_t s)
{
    return dispatch_ks<LossF>(a.w_dtype, a.r, a, Lt, l, w, s);
}

hipError_t launch_cluster_verify(const ClusterVerifyArgs& cv, const VerifyWs& w, hipStream_t s)
{
    DraftArgs a{};
    a.R = cv.R; a.gamma = cv.gamma; a.V = cv.V; a.c = cv.c; a.x = cv.x; a.status = cv.status;
    const int P = cv.gamma + 1;
    hipError_t e = target_pass(a, cv.Lt, P, cv.R * P, w, nullptr, false, s);
    if (e != hipSuccess) return e;
    const int n_gran = n_granules(cv.V);
    const int N = cv.R * cv.gamma;
    ClusterSweepArgs ca{};
    ca.Lt = cv.Lt; ca.tok_slot = cv.tok_slot; ca.sel = cv.sel; ca.zf = cv.zf; ca.dstats = cv.pd_stats;
    ca.trow = w.trow; ca.gamma = cv.gamma; ca.P = P; ca.N_c = cv.N_c; ca.K_c = cv.K_c; ca.max_cl = cv.max_cl;
    ca.V = cv.V; ca.n_gran = n_gran; ca.c = cv.c; ca.vpart = w.vpart;
    // runs of 32 granules (eight per wave), more rows -> longer runs
    ca.gpc = 32 * std::max(1, N / 256);
    {
        ProfScope ps("cluster_sweep", s);
        hipLaunchKernelGGL(k_cluster_sweep, dim3(N, (n_gran + ca.gpc - 1) / ca.gpc), dim3(TILE_THREADS), 0, s, ca);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ResolveArgs ra{};
    SweepArgs& sw = ra.s;
    sw.x = cv.x; sw.dstats = cv.pd_stats; sw.Lt = cv.Lt; sw.R = cv.R; sw.gamma = cv.gamma; sw.V = cv.V; sw.P = P;
    sw.c = cv.c; sw.vec4 = (cv.V % 4) == 0; sw.n_gran = n_gran; sw.max_rows = N; sw.trow = w.trow;
    sw.vpart = w.vpart;
    ra.ell = cv.ell;
    ra.tgran = w.tgran;
    ra.targ = w.targ;
    ra.seed = cv.seed; ra.round = cv.round;
    ra.n_acc = cv.n_acc; ra.y = cv.y; ra.pt_x = cv.pt_x; ra.c_star = cv.c_star; ra.status = cv.status;
    ClusterDraft cd{cv.tok_slot, cv.sel, cv.zf, cv.N_c, cv.K_c, cv.max_cl};
    {
        ProfScope ps("cluster_resolve", s);
        if (cv.greedy)
            hipLaunchKernelGGL(k_cluster_resolve<true>, dim3(cv.R), dim3(RES_THREADS), 0, s, ra, cd);
        else
            hipLaunchKernelGGL(k_cluster_resolve<false>, dim3(cv.R), dim3(RES_THREADS), 0, s, ra, cd);
    }
    return hipGetLastError();
}

}  // namespace spec
