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
//   k_target_tile     per (target row, granule): max, sum of 2^((L-max)c),
//                     argmax -- first streaming pass over the target rows.
//   k_row_merge       per target row: (M_t, S_t) and argmax.
//   k_verify_sweep    per (verified row, granule): recompute the Markov bias
//                     on MFMA, p_d and p_t, and the granule's TV mass
//                     sum |p_t - p_d| and residual mass sum max(0, p_t - p_d)
//                     -- second pass over the target rows plus U and W2.
//   k_verify_resolve  one workgroup per request: accept tests (fp64 on the
//                     single drafted id), first rejection, c*, residual or
//                     bonus draw by inverse CDF over granules plus one
//                     granule rescan.
#include <math.h>

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

// ---------------------------------------------------------- target stats

struct TargetArgs {
    const float* Lt;
    int R, gamma, V, P;  // P: target rows per request in the implicit map
    float c;
    int vec4;
    int n_gran, n_gchunks, max_rows;
    const int2* tmap;        // NULL = implicit
    const int32_t* counts;   // counts[1] = rows when tmap != NULL
    float2* tgran;
    int32_t* tgidx;
};

// One workgroup: one target row x 32 granules; each 32-lane half handles one
// granule per step with float4 loads.
__global__ __launch_bounds__(TILE_THREADS) void k_target_tile(TargetArgs p)
{
    const int row = blockIdx.x / p.n_gchunks, gc = blockIdx.x - row * p.n_gchunks;
    const int nrows = p.tmap ? p.counts[1] : p.max_rows;
    if (row >= nrows) return;
    const int2 ti = trow_info(p.tmap, row, p.P);
    const float* L = p.Lt + ((size_t)ti.x * (p.gamma + 1) + ti.y) * p.V;
    const int hw = threadIdx.x >> 5, li = threadIdx.x & 31;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int g = gc * 32 + it * 8 + hw;
        if (g >= p.n_gran) break;  // uniform within the half
        const int c0 = g * GRAN + 4 * li;
        float v[4];
        if (p.vec4 && c0 + 3 < p.V) {
            const float4 t4 = *reinterpret_cast<const float4*>(L + c0);
            v[0] = t4.x; v[1] = t4.y; v[2] = t4.z; v[3] = t4.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = c0 + e < p.V ? L[c0 + e] : -INFINITY;
        }
        float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        float bv = v[0];
        int bi = c0;
#pragma unroll
        for (int e = 1; e < 4; ++e)
            if (v[e] > bv) { bv = v[e]; bi = c0 + e; }
        m = half_max(m);
        const float ms = safe_ref(m);
        float s = softw(v[0], ms, p.c) + softw(v[1], ms, p.c) + softw(v[2], ms, p.c) + softw(v[3], ms, p.c);
        s = half_sum(s);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) argmax_merge(bv, bi, shfl_xor(bv, o), shfl_xor(bi, o));
        if (li == 0) {
            const size_t o = (size_t)row * p.n_gran + g;
            p.tgran[o] = make_float2(m, s);
            p.tgidx[o] = bi;
        }
    }
}

// One wave per row: merge granule partials into (M, S) and the argmax.
__global__ __launch_bounds__(TILE_THREADS) void k_row_merge(const float2* gran, const int32_t* gidx,
                                                            int max_rows, const int32_t* count,
                                                            int n_gran, float c, float2* rows,
                                                            int32_t* argm)
{
    const int row = blockIdx.x * (TILE_THREADS / WAVE) + threadIdx.x / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    const int nrows = count ? *count : max_rows;
    if (row >= nrows) return;
    const float2* gs = gran + (size_t)row * n_gran;
    float m = -INFINITY;
    for (int g = lane; g < n_gran; g += WAVE) m = fmaxf(m, gs[g].x);
    const float M = wave_max(m);
    const float Ms = safe_ref(M);
    float s = 0.0f;
    int best = 0x7fffffff;
    for (int g = lane; g < n_gran; g += WAVE) {
        const float2 v = gs[g];
        s += v.y * softw(v.x, Ms, c);
        if (best == 0x7fffffff && v.x == M) best = gidx[(size_t)row * n_gran + g];
    }
    const float S = wave_sum(s);
    best = wave_min(best);
    if (lane == 0) {
        rows[row] = make_float2(M, S);
        if (argm) argm[row] = best;
    }
}

// ------------------------------------------------------------ TV sweep

struct SweepArgs {
    const float* U;
    const void* W1;
    const void* W2;
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
    float2* vpart;
};

// Per-element weights of one verified row at the 16 ids a lane holds:
// p_d from the draft logits z_d = U + bias, p_t from the target logits.
struct RowCtx {
    bool valid;
    int req, k, trow, tok;
    float Md, iSd, Mt, iSt;
};

__device__ inline RowCtx sweep_row(const SweepArgs& p, int f, int nrows)
{
    RowCtx rc{};
    rc.valid = f < nrows;
    rc.tok = -1;
    if (!rc.valid) return rc;
    const int4 vi = vrow_info(p.vmap, f, p.gamma, p.P);
    rc.req = vi.x; rc.k = vi.y; rc.trow = vi.z;
    rc.tok = rc.k == 1 ? p.x0[rc.req] : p.x[(size_t)rc.req * p.gamma + rc.k - 2];
    const int xk = p.x[(size_t)rc.req * p.gamma + rc.k - 1];
    if (rc.tok < 0 || rc.tok >= p.V || xk < 0 || xk >= p.V) {
        rc.valid = false;
        rc.tok = -1;
        return rc;
    }
    const size_t so = (size_t)rc.req * p.gamma + rc.k - 1;
    rc.Md = p.dstats[2 * so];
    rc.iSd = 1.0f / p.dstats[2 * so + 1];
    const float2 ts = p.trow[rc.trow];
    rc.Mt = ts.x;
    rc.iSt = 1.0f / ts.y;
    return rc;
}

// p_d and p_t at the 16 ids (col0 + acc_col(j, h)) for a valid row.
__device__ inline void sweep_probs(const SweepArgs& p, const RowCtx& rc, const f32x16& acc, int col0,
                                   int h, float (&pd)[16], float (&pt)[16])
{
    float zd[16], zt[16];
    load_row16(p.U + ((size_t)rc.req * p.gamma + rc.k - 1) * p.V, col0, h, p.V, p.vec4, zd);
    load_row16(p.Lt + ((size_t)rc.req * (p.gamma + 1) + rc.k - 1) * p.V, col0, h, p.V, p.vec4, zt);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        pd[j] = softw(zd[j] + acc[j], rc.Md, p.c) * rc.iSd;
        pt[j] = softw(zt[j], rc.Mt, p.c) * rc.iSt;
    }
}

template <typename WT, int KS>
__global__ __launch_bounds__(TILE_THREADS) void k_verify_sweep(SweepArgs p)
{
    const int nlog = p.n_gran * p.n_chunks;
    const int lid = xcd_logical(blockIdx.x, nlog);
    if (lid >= nlog) return;
    const int g = lid / p.n_chunks, chunk = lid - g * p.n_chunks;
    const int nrows = p.vmap ? p.counts[0] : p.max_rows;
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int h = lane >> 5, n = lane & 31;
    const int col0 = g * GRAN + 32 * w;

    W2Operand<WT, KS> A;
    A.load(reinterpret_cast<const WT*>(p.W2), p.r, p.V, col0 + n, h);
    __shared__ float sm_tv[4][32], sm_res[4][32];

    for (int b = 0; b < p.bpc; ++b) {
        const int rb = chunk * p.bpc + b;
        if (rb * BLOCK_ROWS >= nrows) break;
        const int f = rb * BLOCK_ROWS + n;
        const RowCtx rc = sweep_row(p, f, nrows);
        const f32x16 acc = A.mul(reinterpret_cast<const WT*>(p.W1), p.r, rc.tok, h);
        float tv = 0.0f, res = 0.0f;
        if (rc.valid) {
            float pd[16], pt[16];
            sweep_probs(p, rc, acc, col0, h, pd, pt);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float d = pt[j] - pd[j];
                tv += fabsf(d);
                res += fmaxf(d, 0.0f);
            }
        }
        tv += shfl_xor(tv, 32);
        res += shfl_xor(res, 32);
        if (h == 0) {
            sm_tv[w][n] = tv;
            sm_res[w][n] = res;
        }
        __syncthreads();
        if (threadIdx.x < 32 && rc.valid) {
            const float T4 = ((sm_tv[0][n] + sm_tv[1][n]) + sm_tv[2][n]) + sm_tv[3][n];
            const float R4 = ((sm_res[0][n] + sm_res[1][n]) + sm_res[2][n]) + sm_res[3][n];
            p.vpart[(size_t)f * p.n_gran + g] = make_float2(T4, R4);
        }
        __syncthreads();
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

__device__ inline double weight_d(const float* W, size_t i) { return (double)W[i]; }
__device__ inline double weight_d(const bf16w* W, size_t i)
{
    return (double)__uint_as_float((uint32_t)W[i].bits << 16);
}

// Draw from target row `trow` (data row (req, kk) of Lt) by inverse CDF with
// uniform u: granule masses from the first pass, then one granule rescan.
__device__ inline int draw_target_row(const ResolveArgs& a, int trow, int req, int kk, float u,
                                      float* smf, int* smi)
{
    const SweepArgs& p = a.s;
    const float2* gs = a.tgran + (size_t)trow * p.n_gran;
    const int t = threadIdx.x;
    const int per = (p.n_gran + TILE_THREADS - 1) / TILE_THREADS;
    const int g0 = min(t * per, p.n_gran), g1 = min(g0 + per, p.n_gran);
    float m = -INFINITY;
    for (int g = g0; g < g1; ++g) m = fmaxf(m, gs[g].x);
    const float M = block_max(m, smf);
    const float c = p.c;
    auto wf = [&](int g) { const float2 v = gs[g]; return v.y * softw(v.x, M, c); };
    float tsum, excl, S;
    granule_scan(wf, g0, g1, smf, tsum, excl, S);
    const float target = u * S;
    float before;
    int gfb;
    int gstar = granule_find(wf, g0, g1, excl, target, smf, smi, before, gfb);
    const bool fallback = gstar < 0;
    if (fallback) gstar = gfb < 0 ? 0 : gfb;
    int pick = 0;
    if (t < WAVE) {
        const float* L = p.Lt + ((size_t)req * (p.gamma + 1) + kk) * p.V;
        const int ca = gstar * GRAN + 2 * t, cb = ca + 1;
        const float za = ca < p.V ? L[ca] : -INFINITY, zb = cb < p.V ? L[cb] : -INFINITY;
        float e;
        pick = gstar * GRAN + granule_pick(softw(za, M, c), softw(zb, M, c), before, target, fallback, e);
        if (t == 0) smi[5] = pick;
    }
    __syncthreads();
    pick = smi[5];
    __syncthreads();
    return pick;
}

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(TILE_THREADS) void k_verify_resolve(ResolveArgs a)
{
    const SweepArgs& p = a.s;
    const int r = blockIdx.x, t = threadIdx.x;
    const int lane = t & (WAVE - 1), w = t / WAVE;
    const int G = p.gamma;
    __shared__ float smf[8];
    __shared__ int smi[8];
    __shared__ float rowbuf[GRAN];

    const int Lr = a.ell ? a.ell[r] : G;
    const bool bad_len = Lr < 0 || Lr > G;
    bool bad_tok = false;
    if (!bad_len) {
        if (t == 0) bad_tok = p.x0[r] < 0 || p.x0[r] >= p.V;
        if (t < Lr) {
            const int xv = p.x[(size_t)r * G + t];
            bad_tok = bad_tok || xv < 0 || xv >= p.V;
        }
    }
    bad_tok = __syncthreads_or(bad_tok);
    if (bad_len || bad_tok) {
        if (t == 0) raise_flag(a.status, bad_len ? 2u : 1u);
        if (t == 0) a.n_acc[r] = -1;
        if (t <= G) a.y[(size_t)r * (G + 1) + t] = -1;
        if (t < G) {
            if (a.pt_x) a.pt_x[(size_t)r * G + t] = NAN;
            if (a.c_star) a.c_star[(size_t)r * G + t] = NAN;
        }
        return;
    }
    const int voff = a.voff ? a.voff[r] : r * G;
    const int toff = a.toff ? a.toff[r] : r * p.P;

    // ---- accept tests, one thread per verified position (fp64 on one id)
    bool acc_k = true;
    if (t < Lr) {
        const int xk = p.x[(size_t)r * G + t];
        const int tr = toff + t;
        const float2 ts = p.trow[tr];
        const double zt = (double)p.Lt[((size_t)r * (G + 1) + t) * p.V + xk];
        const double pt = exp2((zt - (double)ts.x) * (double)p.c) / (double)ts.y;
        if (a.pt_x) a.pt_x[(size_t)r * G + t] = (float)pt;
        if (GREEDY) {
            acc_k = xk == a.targ[tr];
        } else {
            const int xp = t == 0 ? p.x0[r] : p.x[(size_t)r * G + t - 1];
            const WT* W1 = reinterpret_cast<const WT*>(p.W1);
            const WT* W2 = reinterpret_cast<const WT*>(p.W2);
            double b = 0.0;
            for (int i = 0; i < p.r; ++i)
                b += weight_d(W1, (size_t)xp * p.r + i) * weight_d(W2, (size_t)xk * p.r + i);
            const size_t so = (size_t)r * G + t;
            const double zd = (double)p.U[so * p.V + xk] + b;
            const double pd = exp2((zd - (double)p.dstats[2 * so]) * (double)p.c) / (double)p.dstats[2 * so + 1];
            double ratio;
            if (pd > 0.0) ratio = pt / pd;
            else ratio = pt > 0.0 ? INFINITY : 0.0;
            const double u1 = u24d(philox((uint32_t)(t + 1), (uint32_t)r, a.round, a.seed).w[1]);
            acc_k = u1 < ratio;
        }
    } else if (t < G) {
        if (a.pt_x) a.pt_x[(size_t)r * G + t] = NAN;
    }
    const int kstar = block_min((t < Lr && !acc_k) ? t + 1 : 0x7fffffff, smi);
    const int nacc = kstar == 0x7fffffff ? Lr : kstar - 1;

    // ---- c* for every verified position: 1 - 1/2 sum over granules of TV mass
    if (a.c_star) {
        for (int k = w + 1; k <= Lr; k += TILE_THREADS / WAVE) {
            const float2* vp = p.vpart + (size_t)(voff + k - 1) * p.n_gran;
            float s = 0.0f;
            for (int g = lane; g < p.n_gran; g += WAVE) s += vp[g].x;
            s = wave_sum(s);
            if (lane == 0) {
                float cs = 1.0f - 0.5f * s;
                cs = fminf(fmaxf(cs, 0.0f), 1.0f);
                a.c_star[(size_t)r * G + k - 1] = cs;
            }
        }
        if (t >= Lr && t < G) a.c_star[(size_t)r * G + t] = NAN;
    }

    // ---- emitted token
    int ytok;
    if (kstar != 0x7fffffff) {
        const int tr = toff + kstar - 1;
        if (GREEDY) {
            ytok = a.targ[tr];
        } else {
            const float u2 = u24f(philox((uint32_t)kstar, (uint32_t)r, a.round, a.seed).w[2]);
            const int f = voff + kstar - 1;
            const float2* vp = p.vpart + (size_t)f * p.n_gran;
            const int per = (p.n_gran + TILE_THREADS - 1) / TILE_THREADS;
            const int g0 = min(t * per, p.n_gran), g1 = min(g0 + per, p.n_gran);
            auto wf = [&](int g) { return vp[g].y; };
            float tsum, excl, Z;
            granule_scan(wf, g0, g1, smf, tsum, excl, Z);
            if (Z > 0.0f) {
                const float target = u2 * Z;
                float before;
                int gfb;
                int gstar = granule_find(wf, g0, g1, excl, target, smf, smi, before, gfb);
                const bool fallback = gstar < 0;
                if (fallback) gstar = gfb < 0 ? 0 : gfb;
                // recompute the residual weights of row f in granule gstar with
                // the sweep's tile code
                const int h = lane >> 5, n = lane & 31;
                const int col0 = gstar * GRAN + 32 * w;
                W2Operand<WT, KS> A;
                A.load(reinterpret_cast<const WT*>(p.W2), p.r, p.V, col0 + n, h);
                const int nrows = p.vmap ? p.counts[0] : p.max_rows;
                const int fr = (f / BLOCK_ROWS) * BLOCK_ROWS + n;
                const RowCtx rc = sweep_row(p, fr, nrows);
                const f32x16 acc = A.mul(reinterpret_cast<const WT*>(p.W1), p.r, rc.tok, h);
                if (fr == f) {
                    float pd[16], pt[16];
                    sweep_probs(p, rc, acc, col0, h, pd, pt);
#pragma unroll
                    for (int j = 0; j < 16; ++j) rowbuf[32 * w + acc_col(j, h)] = fmaxf(pt[j] - pd[j], 0.0f);
                }
                __syncthreads();
                if (w == 0) {
                    float e;
                    const int col = granule_pick(rowbuf[2 * lane], rowbuf[2 * lane + 1], before, target,
                                                 fallback, e);
                    if (lane == 0) smi[6] = gstar * GRAN + col;
                }
                __syncthreads();
                ytok = smi[6];
            } else {
                ytok = draw_target_row(a, tr, r, kstar - 1, u2, smf, smi);
            }
        }
    } else {
        const int tr = toff + Lr;
        if (GREEDY) {
            ytok = a.targ[tr];
        } else {
            const float u2 = u24f(philox((uint32_t)(Lr + 1), (uint32_t)r, a.round, a.seed).w[2]);
            ytok = draw_target_row(a, tr, r, Lr, u2, smf, smi);
        }
    }
    if (t == 0) a.n_acc[r] = nacc;
    if (t <= G) {
        int v = -1;
        if (t < nacc) v = p.x[(size_t)r * G + t];
        else if (t == nacc) v = ytok;
        a.y[(size_t)r * (G + 1) + t] = v;
    }
}

// --------------------------------------------------------- confidence

// One wave per request: c*_k for every drafted position and the running
// products a*_k (fp64, left to right).
__global__ __launch_bounds__(TILE_THREADS) void k_conf_finalize(const float2* vpart, const int32_t* x0,
                                                                const int32_t* x, int R, int gamma, int V,
                                                                int n_gran, float* c_star, double* a_star,
                                                                uint32_t* status)
{
    const int r = blockIdx.x * (TILE_THREADS / WAVE) + threadIdx.x / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    if (r >= R) return;
    bool bad = lane == 0 && (x0[r] < 0 || x0[r] >= V);
    for (int k = lane; k < gamma; k += WAVE) bad = bad || x[(size_t)r * gamma + k] < 0 || x[(size_t)r * gamma + k] >= V;
    if (__any(bad)) {
        if (lane == 0) raise_flag(status, 1u);
        for (int k = lane; k < gamma; k += WAVE) {
            c_star[(size_t)r * gamma + k] = NAN;
            if (a_star) a_star[(size_t)r * gamma + k] = NAN;
        }
        return;
    }
    double run = 1.0;
    for (int k = 0; k < gamma; ++k) {
        const float2* vp = vpart + ((size_t)r * gamma + k) * n_gran;
        float s = 0.0f;
        for (int g = lane; g < n_gran; g += WAVE) s += vp[g].x;
        s = wave_sum(s);
        float cs = fminf(fmaxf(1.0f - 0.5f * s, 0.0f), 1.0f);
        run *= (double)cs;
        if (lane == 0) {
            c_star[(size_t)r * gamma + k] = cs;
            if (a_star) a_star[(size_t)r * gamma + k] = run;
        }
    }
}

// ------------------------------------------------------------ launchers

static int chunk_blocks(int nrows, int n_gran)
{
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    long work = (long)n_rb * n_gran;
    int bpc = (int)(work / 2048);
    if (bpc < 1) bpc = 1;
    if (bpc > 4) bpc = 4;
    if (bpc > n_rb) bpc = n_rb;
    return bpc;
}

static SweepArgs make_sweep(const DraftArgs& a, const float* dstats, const float* Lt, int P,
                            const VerifyWs& w, const int32_t* counts, bool maps)
{
    SweepArgs s{};
    s.U = a.U; s.W1 = a.W1; s.W2 = a.W2; s.x0 = a.x0; s.x = a.x; s.dstats = dstats; s.Lt = Lt;
    s.R = a.R; s.gamma = a.gamma; s.r = a.r; s.V = a.V; s.P = P; s.c = a.c; s.vec4 = (a.V % 4) == 0;
    s.n_gran = n_granules(a.V);
    s.max_rows = a.R * a.gamma;
    s.bpc = chunk_blocks(s.max_rows, s.n_gran);
    const int n_rb = (s.max_rows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    s.n_chunks = (n_rb + s.bpc - 1) / s.bpc;
    s.vmap = maps ? w.vmap : nullptr;
    s.counts = counts;
    s.trow = w.trow;
    s.vpart = w.vpart;
    return s;
}

static hipError_t target_pass(const DraftArgs& a, const float* Lt, int P, int max_rows,
                              const VerifyWs& w, const int32_t* counts, bool maps, hipStream_t s)
{
    TargetArgs t{};
    t.Lt = Lt; t.R = a.R; t.gamma = a.gamma; t.V = a.V; t.P = P; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.n_gran = n_granules(a.V);
    t.n_gchunks = (t.n_gran + 31) / 32;
    t.max_rows = max_rows;
    t.tmap = maps ? w.tmap : nullptr;
    t.counts = counts;
    t.tgran = w.tgran; t.tgidx = w.tgidx;
    {
        ProfScope ps("target_tile", s);
        hipLaunchKernelGGL(k_target_tile, dim3(max_rows * t.n_gchunks), dim3(TILE_THREADS), 0, s, t);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope ps("row_merge", s);
        hipLaunchKernelGGL(k_row_merge, dim3((max_rows + 3) / 4), dim3(TILE_THREADS), 0, s,
                           (const float2*)w.tgran, (const int32_t*)w.tgidx, max_rows,
                           maps ? counts + 1 : (const int32_t*)nullptr, t.n_gran, a.c, w.trow, w.targ);
    }
    return hipGetLastError();
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
        hipLaunchKernelGGL((k_verify_sweep<WT, KS>), dim3(xcd_grid(sw.n_gran * sw.n_chunks)),
                           dim3(TILE_THREADS), 0, s, sw);
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
            hipLaunchKernelGGL((k_verify_resolve<WT, KS, true>), dim3(a.R), dim3(TILE_THREADS), 0, s, ra);
        else
            hipLaunchKernelGGL((k_verify_resolve<WT, KS, false>), dim3(a.R), dim3(TILE_THREADS), 0, s, ra);
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
        hipLaunchKernelGGL((k_verify_sweep<WT, KS>), dim3(xcd_grid(sw.n_gran * sw.n_chunks)),
                           dim3(TILE_THREADS), 0, s, sw);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope ps("conf_finalize", s);
        hipLaunchKernelGGL(k_conf_finalize, dim3((a.R + 3) / 4), dim3(TILE_THREADS), 0, s,
                           (const float2*)w.vpart, a.x0, a.x, a.R, a.gamma, a.V, sw.n_gran, c_star, a_star,
                           a.status);
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

template <template <typename, int> class F, typename... Args>
static hipError_t dispatch_ks_v(int w_dtype, int r, Args&&... args)
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

hipError_t launch_verify(const DraftArgs& a, const float* pd_stats, const float* Lt, const int32_t* ell,
                         int32_t* n_acc, int32_t* y, float* pt_x, float* c_star, const VerifyWs& w,
                         int32_t* counts, hipStream_t s)
{
    return dispatch_ks_v<VerifyF>(a.w_dtype, a.r, a, pd_stats, Lt, ell, n_acc, y, pt_x, c_star, w, counts, s);
}

hipError_t launch_confidence(const DraftArgs& a, const float* pd_stats, const float* Lt, float* c_star,
                             double* a_star, const VerifyWs& w, hipStream_t s)
{
    return dispatch_ks_v<ConfF>(a.w_dtype, a.r, a, pd_stats, Lt, c_star, a_star, w, s);
}

}  // namespace spec
