// propose.hip -- Markov-head drafting (DSpark blog page, sections 3-4):
// for k = 1..gamma, z_k = U_k + W1[x_{k-1}] W2^T, x_k ~ softmax(z_k / T).
//
// Up to 32 requests whose shapes allow it run in one launch
// (k_propose_fused, below: W2 stays in registers for all positions).
// Otherwise, per position two kernels run back to back on the caller's
// stream:
//   k_draft_tile   one workgroup per (128-id granule, chunk of 32-row
//                  blocks): the bias of 32 rows x 128 ids on MFMA (W2
//                  operand stationary in registers, W1 rows staged in LDS),
//                  transposed through LDS so that every thread owns 16
//                  consecutive ids of one row; adds U_k (coalesced 64-byte
//                  loads) and writes per (row, granule) the max, the sum of
//                  2^((z - max) c) and (greedy) the argmax.
//   k_propose_pick one wave per request: merge the granule partials, draw
//                  the Philox uniform, find the granule where the running
//                  sum crosses u * S, recompute that granule's 128 logits
//                  with the same MFMA operands and pick the id.
// x_k stays on the device and feeds the next position's W1 gather.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace spec {

// ------------------------------------------------------------ W2 packing

// Element (v, i) of W2: stored [V, r] (a linear layer's weight, rv = false)
// or [r, V] (the page's formula as written, rv = true).
template <typename T>
__device__ inline T w2_at(const T* W2, int r, int V, int v, int i, bool rv)
{
    return rv ? W2[(size_t)i * V + v] : W2[(size_t)v * r + i];
}

__global__ void k_pack_w2_bf16(const uint16_t* W2, int r, int V, int ks, bool rv, uint4* out, size_t total)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int l = (int)(idx % WAVE);
    const size_t bs = idx / WAVE;
    const int s = (int)(bs % ks);
    const int b = (int)(bs / ks);
    const int v = 32 * b + (l & 31), h = l >> 5;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (v < V) {
        if (!rv) {
            o = *reinterpret_cast<const uint4*>(W2 + (size_t)v * r + 16 * s + 8 * h);
        } else {
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = w2_at(W2, r, V, v, 16 * s + 8 * h + j, true);
            o = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
        }
    }
    out[idx] = o;
}

__global__ void k_pack_w2_f32(const float* W2, int r, int V, int ks, bool rv, float4* out, size_t total)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int l = (int)(idx % WAVE);
    const size_t bt = idx / WAVE;
    const int tq = (int)(bt % ks);
    const int b = (int)(bt / ks);
    const int v = 32 * b + (l & 31), h = l >> 5;
    float4 o = make_float4(0, 0, 0, 0);
    if (v < V) {
        const int i0 = 8 * tq + h;
        o = make_float4(w2_at(W2, r, V, v, i0, rv), w2_at(W2, r, V, v, i0 + 2, rv), w2_at(W2, r, V, v, i0 + 4, rv),
                        w2_at(W2, r, V, v, i0 + 6, rv));
    }
    out[idx] = o;
}

hipError_t launch_pack_w2(const void* W2, int w_dtype, int r, int V, void* W2p, bool rv, hipStream_t s)
{
    const int nblk = (V + 31) / 32;
    if (w_dtype == 1) {
        const int ks = r / 16;
        const size_t total = (size_t)nblk * ks * WAVE;
        hipLaunchKernelGGL(k_pack_w2_bf16, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           (const uint16_t*)W2, r, V, ks, rv, (uint4*)W2p, total);
    } else {
        const int ks = r / 8;
        const size_t total = (size_t)nblk * ks * WAVE;
        hipLaunchKernelGGL(k_pack_w2_f32, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           (const float*)W2, r, V, ks, rv, (float4*)W2p, total);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------ draft tile

struct TileArgs {
    const float* U;
    const void* W1;
    const void* W2p;
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
    FastDiv div_rb; // by the number of 32-row blocks (the pipelined tile)
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
__global__ __launch_bounds__(TILE_THREADS, 4) void k_draft_tile(TileArgs p)
{
    using Ops = TileOps<WT, KS>;
    const int nlog = p.n_gran * p.n_chunks;
    const int lid = xcd_logical(blockIdx.x, nlog);
    if (lid >= nlog) return;
    const int g = lid / p.n_chunks, chunk = lid - g * p.n_chunks;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int ks = k_steps<WT>(p.r);
    const int nblk = (p.V + 31) / 32;

    Ops A;
    A.load_a(p.W2p, ks, 4 * g + w, 4 * g + w < nblk, lane);

    __shared__ __align__(16) char sB[32 * Ops::RS * Ops::ELEM];
    __shared__ __align__(16) float sZ[32 * ZS];
    __shared__ int s_tok[32];

    const int er = t >> 3, ec = (t & 7) * 16;  // epilogue: row er, ids ec..ec+15 of the granule
    const int cbase = g * GRAN + ec;
    for (int b = 0; b < p.bpc; ++b) {
        const int rb = chunk * p.bpc + b;
        if (rb * BLOCK_ROWS >= p.nrows) break;
        // the epilogue row's U segment does not depend on the tokens: issue it first
        const int erow = rb * BLOCK_ROWS + er;
        float z[16];
        if (erow < p.nrows) {
            const int ereq = p.kfix >= 0 ? erow : erow / p.gamma;
            const int ekk = p.kfix >= 0 ? p.kfix : erow - ereq * p.gamma;
            load16(p.U + ((size_t)ereq * p.gamma + ekk) * p.V, cbase, p.V, p.vec4, z);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) z[j] = -INFINITY;
        }
        if (t < 32) {
            const int row = rb * BLOCK_ROWS + t;
            int req = -1, kk = 0, tok = -1;
            if (row < p.nrows) {
                draft_row(p, row, req, kk, tok);
                if (tok < 0 || tok >= p.V) {
                    if (g == 0) raise_flag(p.status, 1u);
                    tok = -1;
                }
            }
            s_tok[t] = tok;
        }
        __syncthreads();
        // read before the next block may overwrite s_tok (two barriers ahead)
        const bool valid = erow < p.nrows && s_tok[er] >= 0;
        stage_w1<WT, Ops::RS, KS>(sB, reinterpret_cast<const WT*>(p.W1), s_tok, p.r);
        __syncthreads();
        store_tile(sZ, A.mfma(sB, ks, lane), w, lane);
        __syncthreads();

        const float* zr = sZ + er * ZS + ec;
        float m = -INFINITY, bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 bq = *reinterpret_cast<const float4*>(zr + 4 * q);
            z[4 * q + 0] = z[4 * q + 0] + bq.x;
            z[4 * q + 1] = z[4 * q + 1] + bq.y;
            z[4 * q + 2] = z[4 * q + 2] + bq.z;
            z[4 * q + 3] = z[4 * q + 3] + bq.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            m = fmaxf(m, z[j]);
            if (GREEDY && z[j] > bv) { bv = z[j]; bi = cbase + j; }
        }
        m = oct_max(m);
        const float ms = safe_ref(m);
        // ids 0-7 and 8-15 summed apart, then reduced in the pipelined
        // tile's order (identical partials)
        float sl = 0.0f, sh = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sl += softw(z[j], ms, p.c);
#pragma unroll
        for (int j = 8; j < 16; ++j) sh += softw(z[j], ms, p.c);
        const float s = pair_oct_sum(sl, sh);
        if (GREEDY) oct_argmax(bv, bi);
        if ((t & 7) == 0 && valid) {
            const size_t o = (size_t)erow * p.n_gran + g;
            p.gstat[o] = make_float2(m, s);
            if (GREEDY) p.gidx[o] = bi;
        }
    }
}

// ------------------------------------------------ pipelined draft tile
//
// The per-position tile for many requests (bf16 weights, r = 128 or 256),
// organised as the pipelined verify sweep: the work is the sequence of
// (granule, 32-row block) units, unit u = (granule u / n_rb, block u %
// n_rb); each workgroup takes a contiguous run of units, so W2's granule
// slice is loaded once per granule a run touches (W2 crosses HBM about
// once per position instead of once per chunk of row blocks) and the
// pipeline fills once per workgroup.  One workgroup of 12 waves per CU, in
// two groups that run one stage apart:
//   MFMA waves (0-3)      hold the granule's W2 slice (A operand); in stage
//                         s they write rows 0..15 of unit s+1's W1 tile
//                         (loaded into registers two stages before) into
//                         LDS, check and write unit s+4's tokens (loaded
//                         three stages before), compute unit s's 32 x 128
//                         bias tile into LDS, and issue the loads of unit
//                         s+3's W1 rows 0..15 and unit s+7's tokens;
//   epilogue waves (4-11) hold the U rows of three units in registers (16
//                         lanes per row, 8 ids each); in stage s they write
//                         rows 16..31 of unit s+1's W1 tile, reduce unit s-1
//                         (z = U + bias: the granule's max, sum of weights
//                         and greedy argmax per row), keep its partials in
//                         LDS, then issue the loads of unit s+3's W1 rows
//                         16..31 and unit s+2's U; the partials are written
//                         out in bursts (stores mixed into the streamed
//                         reads cost more than the same bytes written
//                         together).  The W1 tile is split between the
//                         groups because the MFMA waves' stage is the
//                         longer one.
// One barrier per stage and no wait at it for memory.
// The staged tile sums its 16 ids per thread as two 8-id partials reduced
// in this kernel's order, so both give identical partials.

// Units whose (row, granule) partials the pipelined tile holds in LDS before
// writing them out (a run of more units writes them in chunks).
constexpr int TILE_REC_UNITS = 160;

template <int KS, bool VEC4, bool GREEDY>
__global__ __launch_bounds__(3 * TILE_THREADS, 1) void k_draft_tile_ws(TileArgs p)
{
    using Ops = TileOps<bf16w, KS>;
    using GW = W1Regs<Ops::RS, KS, 2>;  // MFMA waves: rows 0..15 of a unit's W1 tile (part 0 of 2)
    using GE = W1HalfRegs<Ops::RS, KS>;  // epilogue waves: rows 16..31
    const int nrows = p.nrows;  // rows are the requests at position kfix + 1
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    const UnitRun run(p.n_gran, n_rb);
    const int nu = run.nu;
    if (nu <= 0) return;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const bf16w* W1 = reinterpret_cast<const bf16w*>(p.W1);
    const int kfix = p.kfix;
    auto unit = [&](int j) { return run.unit(j); };
    auto ugran = [&](int j) { return p.div_rb.div(unit(j)); };
    auto urow = [&](int j, int i) {
        const int u = unit(j);
        return (u - p.div_rb.div(u) * n_rb) * BLOCK_ROWS + i;
    };
    // the token whose W1 row biases request q at this position
    auto tok_src = [&](int q) { return kfix == 0 ? p.x0 + q : p.x + (size_t)q * p.gamma + kfix - 1; };

    __shared__ __align__(16) char sB[2][32 * Ops::RS * Ops::ELEM];  // W1 tiles, unit j in j & 1
    __shared__ __align__(16) float sZ[2][32 * ZS];                 // bias tiles, unit j in j & 1
    __shared__ int s_tok[8][32];                                    // checked tokens, unit j in j & 7
    __shared__ float2 s_rec[TILE_REC_UNITS * 32];                   // partials of unit j in slot j % TILE_REC_UNITS
    __shared__ int s_ridx[GREEDY ? TILE_REC_UNITS * 32 : 1];        // greedy: argmax of unit j

    auto checked = [&](int tk, int q, int j) {
        if (q >= nrows) return -1;
        if (tk < 0 || tk >= p.V) {
            if (ugran(j) == 0) raise_flag(p.status, 1u);  // once per row: its granule-0 unit
            return -1;
        }
        return tk;
    };
    if (t < 128) {
        const int j = t >> 5, q = urow(j, t & 31);
        s_tok[j][t & 31] = checked(q < nrows ? *tok_src(q) : -1, q, j);
    }
    // stages 0..nu+1, rounded up to a multiple of three (the loops below
    // take stages in threes)
    const int n_stages = (nu + 2 + 2) / 3 * 3;
    __syncthreads();

    if (w < 4) {
        // ------------------------------------------------ MFMA waves
        const int nblk = (p.V + 31) / 32;
        int ga = ugran(0);
        Ops A;
        A.load_a(p.W2p, KS, 4 * ga + w, 4 * ga + w < nblk, lane);
        // raw token of unit j for row lane & 31
        auto raw_token = [&](int j) __attribute__((always_inline)) {
            const int q = urow(j, lane & 31), qc = q < nrows ? q : 0;
            return *tok_src(qc);
        };
        // unit j's W1 rows 0..15 are loaded into g[j % 3], two stages before
        // they are written to LDS (the epilogue waves move rows 16..31 on the
        // same schedule); the tokens of units 4, 5 and 6 into three
        // registers.  The loads go out in the order of every stage (W1 rows,
        // then a token), so the waits of the first stages are the loop's.
        // Every MFMA wave loads the tokens (wave 0 uses them): the count of
        // loads in flight is then the same in every wave, and a wait for W1
        // rows is never a wait for younger loads.
        GW g0, g1, g2;
        int trn[3];
        trn[0] = raw_token(4);
        g0.issue(W1, s_tok[0], 0, t);
        g0.commit(sB[0], 0, t);
        g1.issue(W1, s_tok[1], 0, t);
        trn[1] = raw_token(5);
        g2.issue(W1, s_tok[2], 0, t);
        trn[2] = raw_token(6);
        __syncthreads();
        // stage s: unit s+4's token is in trn[s % 3], refilled for unit s+7.
        // The next granule's W2 slice is loaded before this stage's W1 rows
        // and token: a wait for the slice (in the next stage, on either
        // path of the granule test) is then never a wait for them.
        auto stage = [&](int& tr, GW& gc, GW& gi, int s) __attribute__((always_inline)) {
            gc.commit(sB[(s + 1) & 1], 0, t);
            if (t < 32) s_tok[(s + 4) & 7][t] = checked(tr, urow(s + 4, t), s + 4);
            if (s < nu) {
                store_tile(sZ[s & 1], A.template mfma_acc_la<6>(sB[s & 1], lane, f32x16{}), w, lane);
                const int gn = ugran(s + 1);
                if (s + 1 < nu && gn != ga) {
                    ga = gn;
                    A.load_a(p.W2p, KS, 4 * ga + w, 4 * ga + w < nblk, lane);
                }
            }
            gi.issue(W1, s_tok[(s + 3) & 7], 0, t);
            tr = raw_token(s + 7);
            __syncthreads();
        };
        for (int s = 0; s < n_stages; s += 3) {
            stage(trn[0], g1, g0, s);
            stage(trn[1], g2, g1, s + 1);
            stage(trn[2], g0, g2, s + 2);
        }
    } else {
        // ---------------------------------------------- epilogue waves
        const int te = t - TILE_THREADS;
        const int er = te >> 4, ec = (te & 15) * 8;
        auto issue = [&](int j, float (&zu)[8]) __attribute__((always_inline)) {
            const int jj = min(j, nu - 1);
            const int f = urow(jj, er), fc = f < nrows ? f : 0;
            load8_raw<VEC4>(p.U + ((size_t)fc * p.gamma + kfix) * p.V, ugran(jj) * GRAN + ec, p.V, zu);
        };
        float zuA[8], zuB[8], zuC[8];  // unit j in A, B, C by j % 3
        // rows 16..31 of unit j's W1 tile in h[j % 3], loaded two stages
        // before they are written to LDS (the MFMA waves move rows 0..15)
        GE h0, h1, h2;
        h0.issue(W1, s_tok[0], te);
        h0.commit(sB[0], te);
        h1.issue(W1, s_tok[1], te);
        issue(0, zuA);
        h2.issue(W1, s_tok[2], te);
        issue(1, zuB);
        __syncthreads();
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        // The partials of units [j0, j1) (their slots in s_rec) into gstat
        // and gidx.  Each wave writes the four rows whose partials it wrote
        // itself, so no barrier is needed; rows past the end are skipped.
        const int ew = te / WAVE, el = te & (WAVE - 1);
        auto flush = [&](int j0, int j1) __attribute__((always_inline)) {
            for (int idx = el; idx < 4 * (j1 - j0); idx += WAVE) {
                const int j = j0 + (idx >> 2), i = 4 * ew + (idx & 3);
                const int f = urow(j, i);
                if (f < nrows) {
                    const int sl = (j % TILE_REC_UNITS) * 32 + i;
                    const size_t o = (size_t)f * p.n_gran + ugran(j);
                    p.gstat[o] = s_rec[sl];
                    if (GREEDY) p.gidx[o] = s_ridx[sl];
                }
            }
        };
        // stage s: commit unit s+1's rows 16..31 (hc), reduce unit s-1, then
        // issue unit s+3's W1 rows (hi) and, after them, unit s+2's U: a wait
        // for W1 rows is then never a wait for the younger U loads
        auto stage = [&](float (&zu)[8], GE& hc, GE& hi, int s) __attribute__((always_inline)) {
            hc.commit(sB[(s + 1) & 1], te);
            const int e = s - 1;
            const int ge = ugran(e), cbase = ge * GRAN + ec;
            const int f = urow(e, er);
            const bool ok = f < nrows && s_tok[e & 7][er] >= 0;
            if (s >= 1 && s <= nu && !ok && (te & 15) == 0) {
                // a row without a valid token: no mass (its request drafts -1)
                s_rec[(e % TILE_REC_UNITS) * 32 + er] = make_float2(-INFINITY, 0.0f);
                if (GREEDY) s_ridx[(e % TILE_REC_UNITS) * 32 + er] = 0x7fffffff;
            }
            if (s >= 1 && s <= nu && ok) {
                const float* zr = sZ[e & 1] + er * ZS + ec;
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(zr), b1 = *reinterpret_cast<const f32x4*>(zr + 4);
                const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                float z[8];
                if ((ge + 1) * GRAN <= p.V) {
                    // a whole granule: no id past V
#pragma unroll
                    for (int k = 0; k < 8; ++k) z[k] = zu[k] + bb[k];
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) z[k] = cbase + k < p.V ? zu[k] + bb[k] : -INFINITY;
                }
                float m = -INFINITY, bv = -INFINITY;
                int bi = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    m = fmaxf(m, z[j]);
                    if (GREEDY && z[j] > bv) { bv = z[j]; bi = cbase + j; }
                }
                m = hex_max(m);
                const float ms = safe_ref(m);
                float sw = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) sw += softw(z[j], ms, p.c);
                sw = hex_sum(sw);
                if (GREEDY) hex_argmax(bv, bi);
                // the partials wait in LDS: stores mixed into the streamed
                // reads cost far more than the same bytes written in a burst
                if ((te & 15) == 0) {
                    const int sl = (e % TILE_REC_UNITS) * 32 + er;
                    s_rec[sl] = make_float2(m, sw);
                    if (GREEDY) s_ridx[sl] = bi;
                }
            }
            hi.issue(W1, s_tok[(s + 3) & 7], te);
            issue(s + 2, zu);
            // a full chunk of partials, or the run's last unit: write them out
            if (s >= 1 && s <= nu && (e % TILE_REC_UNITS == TILE_REC_UNITS - 1 || e == nu - 1))
                flush(e - e % TILE_REC_UNITS, e + 1);
            __syncthreads();
        };
        for (int s = 0; s < n_stages; s += 3) {
            stage(zuC, h1, h0, s);
            stage(zuA, h2, h1, s + 1);
            stage(zuB, h0, h2, s + 2);
        }
    }
}

// ------------------------------------------------------------ pick

struct PickArgs {
    const float* U;
    const void* W1;
    const void* W2p;
    const int32_t* x0;
    int32_t* x;  // [R, gamma]; position k is written, k-1 is read
    int R, gamma, r, V;
    float c;
    int k;       // 1-based position
    int n_gran;
    uint64_t seed, round;
    const float2* gstat;
    const int32_t* gidx;
    float* pd_x;
    float* pd_stats;
};

// One workgroup of four waves per request.  Everything that does not depend
// on the drawn granule is loaded first (the previous token, this request's
// W1 row, its granule partials); every wave then merges the partials and
// locates the granule (identical results), wave w recomputes column block w
// of that granule on MFMA with U added, and wave 0 picks the id.
// Rows of at most 64 NR granules (NR = 16, 32) are read lane-strided (lane l
// holds granules l + 64 i: every load instruction reads 64 consecutive
// records) and merged in fp32 on DPP: per 64-granule round its total, the
// round whose running total passes the target, then a scan inside it
// (vocabulary order throughout).  Longer rows (NR = 0) give each lane a
// contiguous run of granules and sum in fp64 (up to 2048 terms a lane).
constexpr int PICK_CACHE = 32;  // granule partials held in registers per lane (fp64 path)

template <typename WT, int KS, bool GREEDY, int NR>
__device__ inline void pick_body(const PickArgs& p)
{
    const int q = blockIdx.x;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int n = lane & 31, h = lane >> 5;
    const size_t o = (size_t)q * p.gamma + (p.k - 1);
    const int ks = k_steps<WT>(p.r);
    const int nblk = (p.V + 31) / 32;
    __shared__ float zrow[GRAN];

    // independent loads first
    const float2* gs = p.gstat + (size_t)q * p.n_gran;
    constexpr int NC = NR > 0 ? NR : PICK_CACHE;
    const int per = (p.n_gran + WAVE - 1) / WAVE;
    const int g0 = min(lane * per, p.n_gran), g1 = min(g0 + per, p.n_gran);  // (fp64 path)
    float2 gc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        if constexpr (NR > 0) {
            const int g = lane + WAVE * i;
            gc[i] = g < p.n_gran ? gs[g] : make_float2(-INFINITY, 0.0f);
        } else {
            gc[i] = (g0 + i < g1) ? gs[g0 + i] : make_float2(-INFINITY, 0.0f);
        }
    }
    const int tok = p.k == 1 ? p.x0[q] : p.x[(size_t)q * p.gamma + p.k - 2];
    const bool ok = tok >= 0 && tok < p.V;
    // B operand: only this request's W1 row (column n == q's slot); a matrix
    // core output element depends only on its own row and column operands
    const int nq = q & (BLOCK_ROWS - 1);
    TileOps<WT, KS> A;
    typename TileOps<WT, KS>::BRow brow;
    brow.load(reinterpret_cast<const WT*>(p.W1), p.r, (ok && n == nq) ? tok : -1, ks, lane);
    if (!ok) {
        if (t == 0) {
            p.x[o] = -1;
            p.pd_x[o] = NAN;
            p.pd_stats[2 * o] = NAN;
            p.pd_stats[2 * o + 1] = NAN;
        }
        return;
    }
    // merge the granule partials: M = max, w_g = S_g 2^((M_g - M) c)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NC; ++i) m = fmaxf(m, gc[i].x);
    if constexpr (NR == 0)
        for (int g = g0 + PICK_CACHE; g < g1; ++g) m = fmaxf(m, gs[g].x);
    const float M = wave_max(m);
    const float c = p.c;
    float wv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) wv[i] = gc[i].y * softw(gc[i].x, M, c);  // padding: 0 * 0
    float S;
    double Sd = 0.0, excl = 0.0;  // (fp64 path)
    const float u = u24f(philox((uint32_t)p.k, (uint32_t)q, p.round, p.seed).w[0]);
    float target = 0.0f, before = 0.0f;
    bool fallback = true;
    int gstar = 0;
    if constexpr (NR > 0) {
        // the total with the bits of the draw's own (which needs it first)
        if (GREEDY) S = wave_rounds_sum(wv);
        else {
            gstar = wave_rounds_pick(wv, u, S, before, fallback);
            target = u * S;
        }
    } else {
        double tsum = 0.0;
#pragma unroll
        for (int i = 0; i < PICK_CACHE; ++i) tsum += (double)wv[i];
        for (int g = g0 + PICK_CACHE; g < g1; ++g) tsum += (double)(gs[g].y * softw(gs[g].x, M, c));
        const double incl = wave_incl_scan(tsum);
        excl = __shfl_up(incl, 1, WAVE);
        if (lane == 0) excl = 0.0;
        Sd = __shfl(incl, WAVE - 1, WAVE);
        S = (float)Sd;
    }

    if (GREEDY) {
        if (w != 0) return;
        // the smallest argmax among the granules whose maximum is M
        int cand = 0x7fffffff;
        if constexpr (NR > 0) {
            int gfirst = -1;
#pragma unroll
            for (int i = NR - 1; i >= 0; --i)
                if (gc[i].x == M) gfirst = lane + WAVE * i;
            if (gfirst >= 0) cand = p.gidx[(size_t)q * p.n_gran + gfirst];
        } else {
            for (int g = g0; g < g1; ++g)
                if (gs[g].x == M) { cand = p.gidx[(size_t)q * p.n_gran + g]; break; }
        }
        const int best = wave_min(cand);
        if (lane == 0) {
            const bool mass = S > 0.0f && best != 0x7fffffff;  // a row of -inf logits has no argmax
            p.x[o] = mass ? best : -1;
            p.pd_x[o] = mass ? 1.0f / S : NAN;
            p.pd_stats[2 * o] = mass ? M : NAN;
            p.pd_stats[2 * o + 1] = mass ? S : NAN;
        }
        return;
    }
    if (!(S > 0.0f)) {  // no probability mass (every logit -inf, or NaN): no sample
        if (t == 0) {
            p.x[o] = -1;
            p.pd_x[o] = NAN;
            p.pd_stats[2 * o] = NAN;
            p.pd_stats[2 * o + 1] = NAN;
        }
        return;
    }

    if constexpr (NR == 0) {
        const double target_d = (double)u * Sd;
        target = (float)target_d;
        // first granule of positive mass whose running sum exceeds target
        double run = excl, prev = excl;
        int pick = -1, lastpos = -1;
#pragma unroll
        for (int i = 0; i < PICK_CACHE; ++i) {
            if (wv[i] > 0.0f) lastpos = g0 + i;
            if (pick < 0) {
                prev = run;
                run += (double)wv[i];
                if (run > target_d && wv[i] > 0.0f) pick = g0 + i;
            }
        }
        for (int g = g0 + PICK_CACHE; g < g1; ++g) {
            const float wg = gs[g].y * softw(gs[g].x, M, c);
            if (wg > 0.0f) lastpos = g;
            if (pick < 0) {
                prev = run;
                run += (double)wg;
                if (run > target_d && wg > 0.0f) pick = g;
            }
        }
        const unsigned long long hit = __ballot(pick >= 0);
        if (hit) {
            const int L = __ffsll((long long)hit) - 1;
            fallback = false;
            before = (float)__shfl(prev, L, WAVE);
            gstar = __shfl(pick, L, WAVE);
        } else {
            fallback = true;
            before = 0.0f;
            const int lp = -wave_min(-lastpos);
            gstar = lp < 0 ? 0 : lp;
        }
    }

    // column block w of granule gstar for q's row (same operands as the tile)
    const int b = 4 * gstar + w;
    float uv[16];
    load_acc16(p.U + ((size_t)q * p.gamma + (p.k - 1)) * p.V, gstar * GRAN + 32 * w, h, p.V, (p.V % 4) == 0, uv);
    A.load_a(p.W2p, ks, b, b < nblk, lane);
    const f32x16 acc = A.mfma_row(brow, ks);
    if (n == nq) {
#pragma unroll
        for (int j = 0; j < 16; ++j) zrow[32 * w + 8 * (j >> 2) + 4 * h + (j & 3)] = softw(uv[j] + acc[j], M, c);
    }
    __syncthreads();
    if (w != 0) return;
    float e;
    const int col = granule_pick(zrow[2 * lane], zrow[2 * lane + 1], before, target, fallback, e);
    if (lane == 0) {
        p.x[o] = gstar * GRAN + col;
        p.pd_x[o] = e / S;
        p.pd_stats[2 * o] = M;
        p.pd_stats[2 * o + 1] = S;
    }
}

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(TILE_THREADS) void k_propose_pick(PickArgs p)
{
    if (p.n_gran <= 16 * WAVE) pick_body<WT, KS, GREEDY, 16>(p);
    else if (p.n_gran <= 32 * WAVE) pick_body<WT, KS, GREEDY, 32>(p);
    else pick_body<WT, KS, GREEDY, 0>(p);
}

// ------------------------------------------------------------ fused propose
//
// All gamma positions in one launch, for one block of up to 32 requests,
// when one workgroup per granule fits on the chip at once.
// Workgroup g keeps the W2 columns of granule g in registers for the whole
// call (W2 is read from HBM once instead of once per position) and, per
// position k:
//   tile  z = U_k + W1[x_{k-1}] W2^T for its 128 ids and every request on
//         MFMA, then per request the granule's (max, sum of weights) or
//         (max, argmax), stored with a tag naming (call, k);
//   pick  for request q = g (and g + n_gran, ...): poll q's partials of all
//         granules until every tag reads k (the values arrive with the
//         poll), merge, draw, recompute the chosen granule on MFMA with the
//         tile's own operands (bit-identical logits) and pick the id; the
//         token goes out as a tagged word, which the next tile phase polls.
// Hand-over values use agent-scope atomic stores and loads (common.h).
// Tags carry a per-workspace call counter, so nothing needs clearing
// between calls; every wait is bounded.

struct FusedArgs {
    TileArgs t;            // nrows = R <= 32, rows are requests
    uint64_t seed, round;
    int32_t* x;            // [R, gamma]
    float* pd_x;           // [R, gamma]
    float* pd_stats;       // [R, gamma, 2]
    uint64_t* part;        // [FUSED_PART_WORDS][R][n_gran] tagged partials: max, sum, argmax
    uint64_t* words;       // [FUSED_TOKEN_COPIES, 32] tagged token words
    uint64_t* exitw;       // [n_gran] tagged exit word of each workgroup
    uint32_t* epoch;       // calls so far on this workspace
    uint32_t* abort_flag;  // abort_word(epoch) of a call that gave up waiting
};

constexpr int SPIN_LIMIT = 1 << 20;     // polls before a wait is declared failed
constexpr int ABORT_EVERY = 32;         // polls between looks at the (single, shared) abort word
constexpr uint32_t DEV_WAIT_FAILED = 8u;
constexpr int FUSED_PER = 4;            // granules per thread in the merge: n_gran <= 1024

// Tag of (call, position), k = 1..64: the low 25 bits of the call counter
// and k.  The hand-over regions hold nothing but tagged words (the workspace
// is zeroed at initialisation, and 0 is no tag), so a word can only match a
// tag if this call wrote it, or if a call 2^25 calls earlier wrote the same
// word and nothing has overwritten it since.
__device__ inline uint32_t call_tag(uint32_t epoch, int k)
{
    return ((epoch & 0x1FFFFFFu) << 7) | (uint32_t)k;
}
// What a call that gives up leaves in the abort word: never 0 (the value of
// a fresh workspace) and distinct for every epoch below 2^31.
__device__ inline uint32_t abort_word(uint32_t epoch) { return epoch | 0x80000000u; }
__device__ inline uint64_t tagged(uint32_t v, uint32_t tag) { return (uint64_t)v | ((uint64_t)tag << 32); }
__device__ inline uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

// End of one poll of a bounded wait (whole block): true when the wait has
// failed (timeout, or another workgroup of this call gave up), after
// raising the status bit and the abort word.
template <int SLEEP>
__device__ inline bool poll_failed(int spin, bool aborted, uint32_t epoch, uint32_t* abort_flag, uint32_t* status)
{
    if (__syncthreads_or(threadIdx.x == 0 && (aborted || spin >= SPIN_LIMIT))) {
        if (threadIdx.x == 0) {
            st_dev(abort_flag, abort_word(epoch));
            raise_flag(status, DEV_WAIT_FAILED);
        }
        return true;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
    return false;
}
// Whether this poll also reads the abort word (thread 0, every ABORT_EVERY polls).
__device__ inline bool look_abort(int spin) { return threadIdx.x == 0 && spin % ABORT_EVERY == ABORT_EVERY - 1; }

template <typename WT, int KS, bool GREEDY>
__global__ __launch_bounds__(TILE_THREADS, 4) void k_propose_fused(FusedArgs f)
{
    using Ops = TileOps<WT, KS>;
    const TileArgs& p = f.t;
    const int g = blockIdx.x;
    const int NG = p.n_gran;
    const int R = p.nrows;
    constexpr int ks = KS;  // launched only when r fills the k-steps exactly
    const int nblk = (p.V + 31) / 32;
    const uint32_t epoch = ld_dev(f.epoch) & 0x7FFFFFFFu;

    Ops A;
    A.load_a(p.W2p, ks, 4 * g + (int)threadIdx.x / WAVE, 4 * g + (int)threadIdx.x / WAVE < nblk,
             threadIdx.x & (WAVE - 1));

    __shared__ __align__(16) char sB[32 * Ops::RS * Ops::ELEM];
    __shared__ __align__(16) float sZ[32 * ZS];
    __shared__ int s_tok[32];
    __shared__ float2 s_mw[TILE_THREADS / WAVE];       // pick: each wave's (max, mass in its own reference)
    __shared__ int s_lastw[TILE_THREADS / WAVE];       // pick: each wave's last granule of positive mass
    __shared__ int s_candw[TILE_THREADS / WAVE];       // pick (greedy): each wave's smallest argmax at its max
    __shared__ __align__(16) float s_w4[FUSED_PER * TILE_THREADS];  // pick: granule weights, wave references
    __shared__ float zrow[GRAN];
    __shared__ int s_prev[FUSED_MAX_R];  // previous token of each request this workgroup picks

    for (int j = threadIdx.x; g + j * NG < R; j += TILE_THREADS) {
        const int a = p.x0[g + j * NG];
        s_prev[j] = a >= 0 && a < p.V ? a : -1;
    }
    // U is parked in the LDS result tile, in the matrix-core output layout,
    // until the MFMA starts from it; no registers hold it meanwhile
    auto load_u = [&](int k, float (&ua)[16]) {
        const int tt = opaque_v(threadIdx.x);
        const int row = tt & 31;
        if (row < R) {
            load_acc16(p.U + ((size_t)row * p.gamma + (k - 1)) * p.V, g * GRAN + 32 * (tt / WAVE), (tt >> 5) & 1,
                       p.V, p.vec4 != 0, ua);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) ua[j] = -INFINITY;
        }
    };
    auto park_u = [&](const float (&ua)[16]) {
        const int tt = opaque_v(threadIdx.x);
        f32x16 u;
#pragma unroll
        for (int j = 0; j < 16; ++j) u[j] = ua[j];
        store_tile(sZ, u, tt / WAVE, tt & (WAVE - 1));
    };
    // the abort word, loaded with U_1 (no round trip of its own): a call
    // that is already marked failed (by the host, or by a workgroup that
    // gave up waiting) ends at once, in every workgroup
    const uint32_t abort0 = threadIdx.x == 0 ? ld_dev(f.abort_flag) : 0u;
    {
        float ua[16];
        load_u(1, ua);
        park_u(ua);
    }
    // U of position kn + 1 (0-based row kn), parked in the result tile while
    // the other workgroups finish, in four waited chunks: spread out, the
    // 16 MB of all workgroups do not queue ahead of the small hand-over loads
    auto park_next = [&](int kn) {
        const int tt = opaque_v(threadIdx.x);
        const int row = tt & 31, ww = tt / WAVE, hh = (tt >> 5) & 1;
        const float* urow = p.U + ((size_t)(row < R ? row : 0) * p.gamma + kn) * p.V;
        float* dst = sZ + row * ZS + 32 * ww + 4 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = g * GRAN + 32 * ww + 8 * q + 4 * hh;
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (row < R) {
                if (p.vec4 && c + 3 < p.V) {
                    v = *reinterpret_cast<const float4*>(urow + c);
                } else {
                    v.x = c < p.V ? urow[c] : -INFINITY;
                    v.y = c + 1 < p.V ? urow[c + 1] : -INFINITY;
                    v.z = c + 2 < p.V ? urow[c + 2] : -INFINITY;
                    v.w = c + 3 < p.V ? urow[c + 3] : -INFINITY;
                }
            }
            *reinterpret_cast<float4*>(dst + 8 * q) = v;
            stores_done();
        }
    };

    bool failed = false;
    if (__syncthreads_or(threadIdx.x == 0 && abort0 == abort_word(epoch))) {
        if (threadIdx.x == 0) raise_flag(p.status, DEV_WAIT_FAILED);
        failed = true;
    }
    for (int k = 1; k <= p.gamma && !failed; ++k) {
        // thread-derived indices are recomputed per position rather than
        // kept live across the loop (register pressure)
        const int t = opaque_v(threadIdx.x), lane = t & (WAVE - 1), w = t / WAVE;
        const int n = lane & 31, h = lane >> 5;
        const int er = t >> 3, ec = (t & 7) * 16;
        const int cbase = g * GRAN + ec;
        const uint32_t tag = call_tag(epoch, k);

        // ---------------- tile phase
        int tok = -1;
        if (k == 1) {
            if (t < R) tok = p.x0[t];
        } else {
            // the previous position's tokens of all requests
            const uint64_t* wd = opaque(f.words) + (size_t)(g % FUSED_TOKEN_COPIES) * 32;
            const uint32_t want = call_tag(epoch, k - 1);
            for (int spin = 0;; ++spin) {
                bool ok = true;
                if (t < R) {
                    const uint64_t v = ld_dev(wd + t);
                    ok = tag_of(v) == want;
                    tok = (int)(uint32_t)v;
                }
                const bool ab = look_abort(spin) && ld_dev(f.abort_flag) == abort_word(epoch);
                if (__syncthreads_and(ok)) break;
                if (poll_failed<2>(spin, ab, epoch, f.abort_flag, p.status)) {
                    failed = true;
                    break;
                }
            }
            if (failed) break;
        }
        if (t < 32) {
            if (t >= R) {
                tok = -1;
            } else if (tok < 0 || tok >= p.V) {
                if (g == 0) raise_flag(p.status, 1u);
                tok = -1;
            }
            s_tok[t] = tok;
        }
        __syncthreads();
        const bool valid = er < R && s_tok[er] >= 0;
        stage_w1_exact<WT, Ops::RS, KS>(sB, reinterpret_cast<const WT*>(p.W1), s_tok);
        __syncthreads();
        {
            f32x16 acc;
            load_tile_own(sZ, acc, w, lane);
            store_tile(sZ, A.mfma_acc(sB, lane, acc), w, lane);
        }
        __syncthreads();
        {
            const float* zr = sZ + er * ZS + ec;
            float z[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(zr + 4 * q);
                z[4 * q] = v.x; z[4 * q + 1] = v.y; z[4 * q + 2] = v.z; z[4 * q + 3] = v.w;
            }
            float m = -INFINITY, bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                m = fmaxf(m, z[j]);
                if (GREEDY && z[j] > bv) { bv = z[j]; bi = cbase + j; }
            }
            m = oct_max(m);
            const float ms = safe_ref(m);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) s += softw(z[j], ms, p.c);
            s = oct_sum(s);
            if (GREEDY) oct_argmax(bv, bi);
            if ((t & 7) == 0 && valid) {
                // partials as three arrays [R][n_gran] (max, sum, argmax), so
                // that a poll reads them granule-contiguous
                const size_t o = (size_t)er * NG + g, plane = (size_t)R * NG;
                st_dev(f.part + o, tagged(__float_as_uint(m), tag));
                st_dev(f.part + plane + o, tagged(__float_as_uint(s), tag));
                if (GREEDY) st_dev(f.part + 2 * plane + o, tagged((uint32_t)bi, tag));
            }
        }
        __syncthreads();          // the tile's reads are complete
        if (k < p.gamma) park_next(k);

        // ---------------- pick phase (W2 registers are free here: reloaded below)
        if (g < R) {
            int j = 0;
            for (int q = g; q < R; q += NG, ++j) {
                const size_t o = (size_t)q * p.gamma + (k - 1);
                int xk = -1;
                float pdx = NAN, sM = NAN, sS = NAN;
                if (s_prev[j] >= 0) {
                    // q's partials of every granule, polled until all carry
                    // this position; thread t reads granules 4t .. 4t+3 (a
                    // single poll in flight: more polling only adds traffic
                    // where the partials are being written)
                    const size_t plane = (size_t)R * NG;
                    const uint64_t* rm = opaque(f.part) + (size_t)q * NG;
                    constexpr int NW_ = GREEDY ? 3 : 2;  // words per granule
                    uint64_t pa[FUSED_PER * NW_];
                    for (int spin = 0;; ++spin) {
                        bool ok = true;
#pragma unroll
                        for (int i = 0; i < FUSED_PER; ++i) {
                            const int gg = min(FUSED_PER * t + i, NG - 1);  // (past NG: a duplicate, not used)
#pragma unroll
                            for (int c = 0; c < NW_; ++c) {
                                pa[i * NW_ + c] = ld_dev(rm + c * plane + gg);
                                ok &= tag_of(pa[i * NW_ + c]) == tag;
                            }
                        }
                        const bool ab = look_abort(spin) && ld_dev(f.abort_flag) == abort_word(epoch);
                        if (__syncthreads_and(ok)) break;
                        if (poll_failed<1>(spin, ab, epoch, f.abort_flag, p.status)) {
                            failed = true;
                            break;
                        }
                    }
                    if (failed) break;
                    float gm[FUSED_PER], gs[FUSED_PER];
                    int gi[FUSED_PER];
#pragma unroll
                    for (int i = 0; i < FUSED_PER; ++i) {
                        const bool in = FUSED_PER * t + i < NG;
                        const uint64_t* v = pa;
                        gm[i] = in ? __uint_as_float((uint32_t)v[i * NW_]) : -INFINITY;
                        gs[i] = in ? __uint_as_float((uint32_t)v[i * NW_ + 1]) : 0.0f;
                        gi[i] = GREEDY && in ? (int)(uint32_t)v[i * NW_ + (NW_ - 1)] : 0x7fffffff;
                    }
                    // per wave: its maximum m_w, its mass s_w in the 2^(c(z - m_w))
                    // reference, and each thread's four granule weights in that
                    // reference (LDS, for the find below)
                    float mt = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
                    const float mw = wave_max_dpp(mt);
                    const float mwr = safe_ref(mw);
                    float wv[FUSED_PER], tsum = 0.0f;
                    int ilast = -1;
#pragma unroll
                    for (int i = 0; i < FUSED_PER; ++i) {
                        wv[i] = gs[i] * softw(gm[i], mwr, p.c);  // padding: 0 * 0
                        tsum += wv[i];
                        if (wv[i] > 0.0f) ilast = i;
                    }
                    const float sw = lane63(wave_scan_dpp(tsum));
                    const int lastw = wave_max_int_dpp(ilast >= 0 ? FUSED_PER * t + ilast : -1);
                    int candw = 0x7fffffff;
                    if (GREEDY) {
#pragma unroll
                        for (int i = 0; i < FUSED_PER; ++i)
                            if (gm[i] == mw) candw = min(candw, gi[i]);
                        candw = wave_min_int_dpp(candw);
                    } else {
                        *reinterpret_cast<float4*>(s_w4 + FUSED_PER * t) = make_float4(wv[0], wv[1], wv[2], wv[3]);
                    }
                    if (lane == 0) {
                        s_mw[w] = make_float2(mw, sw);
                        s_lastw[w] = lastw;
                        s_candw[w] = candw;
                    }
                    __syncthreads();
                    // every wave: M, S and each wave's range of the running sum
                    // (waves in order, each scaled to the M reference)
                    float M = -INFINITY;
#pragma unroll
                    for (int v = 0; v < TILE_THREADS / WAVE; ++v) M = fmaxf(M, s_mw[v].x);
                    const float Mr = safe_ref(M);
                    float sc[TILE_THREADS / WAVE], P[TILE_THREADS / WAVE + 1];
                    P[0] = 0.0f;
#pragma unroll
                    for (int v = 0; v < TILE_THREADS / WAVE; ++v) {
                        sc[v] = softw(s_mw[v].x, Mr, p.c);
                        P[v + 1] = P[v] + s_mw[v].y * sc[v];
                    }
                    const float S = P[TILE_THREADS / WAVE];
                    sM = M;
                    sS = S;
                    if (!(S > 0.0f)) {
                        // no probability mass (every logit -inf, or NaN): no token
                        xk = -1;
                        sM = NAN;
                        sS = NAN;
                    } else if (GREEDY) {
                        int cand = 0x7fffffff;
#pragma unroll
                        for (int v = 0; v < TILE_THREADS / WAVE; ++v)
                            if (s_mw[v].x == M) cand = min(cand, s_candw[v]);
                        xk = cand;
                        pdx = 1.0f / S;
                    } else {
                        const float target = u24f(philox((uint32_t)k, (uint32_t)q, f.round, f.seed).w[0]) * S;
                        // the wave whose range holds the target; every wave replays
                        // that wave's lane scan from LDS (same inputs, same bits)
                        int ws = -1;
#pragma unroll
                        for (int v = TILE_THREADS / WAVE - 1; v >= 0; --v)
                            if (s_mw[v].y > 0.0f && P[v] <= target && target < P[v + 1]) ws = v;
                        int gstar = -1;
                        float before = 0.0f;
                        if (ws >= 0) {
                            const float4 r4 = *reinterpret_cast<const float4*>(s_w4 + FUSED_PER * (ws * WAVE + lane));
                            const float rv[FUSED_PER] = {r4.x, r4.y, r4.z, r4.w};
                            float rsum = 0.0f;
#pragma unroll
                            for (int i = 0; i < FUSED_PER; ++i) rsum += rv[i];
                            const float incl = wave_scan_dpp(rsum);
                            const float scw = sc[ws];
                            // the lane's share of the running sum in the M reference;
                            // consecutive shares meet exactly
                            const float lo = P[ws] + lane_before(incl) * scw, hi = P[ws] + incl * scw;
                            const bool hit = rsum > 0.0f && lo <= target && target < hi;
                            int ig = -1, il = -1;
                            float c = lo, cbefore = lo;
#pragma unroll
                            for (int i = 0; i < FUSED_PER; ++i) {
                                const float wi = rv[i] * scw;
                                if (rv[i] > 0.0f) {
                                    if (ig < 0 && c + wi > target) {
                                        ig = i;
                                        cbefore = c;
                                    }
                                    il = i;
                                }
                                c += wi;
                            }
                            if (hit && ig < 0) {  // the share's own sum rounded below the target
                                ig = il;
                                float c2 = lo;
#pragma unroll
                                for (int i = 0; i < FUSED_PER; ++i)
                                    if (i < il) c2 += rv[i] * scw;
                                cbefore = c2;
                            }
                            const unsigned long long hits = __ballot(hit);
                            if (hits) {
                                const int L = __ffsll((long long)hits) - 1;
                                gstar = FUSED_PER * (ws * WAVE + L) + __builtin_amdgcn_readlane(ig, L);
                                before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cbefore), L));
                            }
                        }
                        const bool fallback = gstar < 0;
                        if (fallback) gstar = max(max(max(s_lastw[0], s_lastw[1]), max(s_lastw[2], s_lastw[3])), 0);
                        // granule gstar for q with the tile's own operands: W2
                        // block, U_k as the starting accumulator, and sB, which
                        // still holds this position's W1 rows (column q)
                        {
                            Ops A2;
                            A2.load_a(p.W2p, ks, 4 * gstar + w, 4 * gstar + w < nblk, lane);
                            float uq[16];
                            load_acc16(p.U + ((size_t)q * p.gamma + (k - 1)) * p.V, gstar * GRAN + 32 * w, h, p.V,
                                       p.vec4 != 0, uq);
                            f32x16 acc;
#pragma unroll
                            for (int jj = 0; jj < 16; ++jj) acc[jj] = uq[jj];
                            acc = A2.mfma_acc(sB, lane, acc);
                            if (n == (q & 31)) {
#pragma unroll
                                for (int jj = 0; jj < 16; ++jj)
                                    zrow[32 * w + 8 * (jj >> 2) + 4 * h + (jj & 3)] = softw(acc[jj], Mr, p.c);
                            }
                        }
                        __syncthreads();
                        if (w == 0) {
                            float e;
                            const int col = granule_pick_dpp(zrow[2 * lane], zrow[2 * lane + 1], before, target,
                                                             fallback, e);
                            xk = gstar * GRAN + col;
                            pdx = e / S;
                        }
                    }
                }
                // wave 0 publishes the token (one copy per lane) and
                // records the outputs
                if (w == 0) {
                    if (lane < FUSED_TOKEN_COPIES) st_dev(f.words + (size_t)lane * 32 + q, tagged((uint32_t)xk, tag));
                    if (lane == 0) {
                        f.x[o] = xk;
                        f.pd_x[o] = pdx;
                        f.pd_stats[2 * o] = sM;
                        f.pd_stats[2 * o + 1] = sS;
                        s_prev[j] = xk;
                    }
                }
                __syncthreads();
            }
            // unconditional, so that the W2 registers are provably free
            // during the picks (32 workgroups re-read 64 KB each)
            A.load_a(p.W2p, ks, 4 * g + w, 4 * g + w < nblk, lane);
        }
    }
    // The call counter advances once every workgroup has read it.  After a
    // complete call that holds when workgroup 0 ends (its last pick needed
    // the partials of all of them).  After a failed call workgroup 0 may end
    // first, so it waits (boundedly) for every workgroup's exit word of this
    // call: a workgroup that started late then still read this call's
    // counter, and saw its abort word.
    const uint32_t done_tag = call_tag(epoch, 0);  // (positions use k >= 1)
    if (threadIdx.x == 0) st_dev(f.exitw + g, tagged(1u, done_tag));
    if (g == 0) {
        if (failed) {
            for (int spin = 0;; ++spin) {
                bool ok = true;
                for (int i = threadIdx.x; i < NG; i += TILE_THREADS) ok &= tag_of(ld_dev(f.exitw + i)) == done_tag;
                if (__syncthreads_and(ok) || spin >= SPIN_LIMIT) break;
                __builtin_amdgcn_s_sleep(2);
            }
        }
        if (threadIdx.x == 0) st_dev(f.epoch, (epoch + 1) & 0x7FFFFFFFu);
    }
}

// ------------------------------------------------------------ launchers

// Workgroups cover one granule and `bpc` consecutive 32-row blocks; the row
// blocks are split into just enough chunks to give ~1024 workgroups.
static void tile_grid(int nrows, int n_gran, int& bpc, int& n_chunks)
{
    const int n_rb = (nrows + BLOCK_ROWS - 1) / BLOCK_ROWS;
    n_chunks = (1024 + n_gran - 1) / n_gran;
    if (n_chunks > n_rb) n_chunks = n_rb;
    if (n_chunks < 1) n_chunks = 1;
    bpc = (n_rb + n_chunks - 1) / n_chunks;
    n_chunks = (n_rb + bpc - 1) / bpc;
}

// Workgroups of k_propose_fused the current device holds at once; cached
// per device.
template <typename WT, int KS, bool GREEDY>
static int fused_capacity()
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];  // capacity + 1; 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_propose_fused<WT, KS, GREEDY>, TILE_THREADS,
                                                         0) != hipSuccess)
            per_cu = 0;
        v = per_cu * cus + 1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

template <typename WT, int KS, bool GREEDY>
static hipError_t propose_fused(const DraftArgs& a, const TileArgs& t, int32_t* x_out, float* pd_x,
                                float* pd_stats, const ProposeWs& ws, hipStream_t s)
{
    FusedArgs f{};
    f.t = t;
    f.seed = a.seed; f.round = a.round;
    f.x = x_out; f.pd_x = pd_x; f.pd_stats = pd_stats;
    f.part = ws.part;
    f.words = ws.words;
    f.exitw = ws.exitw;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(a.status);
    f.epoch = &hdr->epoch;
    f.abort_flag = &hdr->abort;
    // A plain launch: the grid is no larger than what the device holds at
    // once (fused_capacity), so on an otherwise free device every workgroup
    // becomes resident; waits are bounded in any case.  (A cooperative launch
    // gives the same guarantee formally but costs ~17 us per call here.)
    ProfScope ps("propose_fused", s);
    hipLaunchKernelGGL((k_propose_fused<WT, KS, GREEDY>), dim3(t.n_gran), dim3(TILE_THREADS), 0, s, f);
    return hipGetLastError();
}

// Requests above which the per-position path takes the pipelined tile: from
// two 32-row blocks per granule up it is the faster one (R = 64 over 2048
// granules: 34 against 39 us a position); with one block, every unit would
// start a granule and wait for its W2 slice.
constexpr int PIPED_TILE_MIN_R = 32;

// Workgroups of k_draft_tile_ws the current device holds at once; cached
// per device and variant.
template <int KS, bool GREEDY>
static int tile_ws_slots(bool vec4)
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV][2];  // slots + 1; 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 256;
    int v = cache[dev][vec4].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        const hipError_t e = vec4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                        &per_cu, k_draft_tile_ws<KS, true, GREEDY>, 3 * TILE_THREADS, 0)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                        &per_cu, k_draft_tile_ws<KS, false, GREEDY>, 3 * TILE_THREADS, 0);
        if (e != hipSuccess || per_cu <= 0) per_cu = 1;
        v = per_cu * cus + 1;
        cache[dev][vec4].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

template <int KS>
static void launch_tile_ws(const TileArgs& t, bool greedy, int grid, hipStream_t s)
{
    if constexpr (KS == 8 || KS == 16) {
        const dim3 g(grid), b(3 * TILE_THREADS);
        if (greedy) {
            if (t.vec4) hipLaunchKernelGGL((k_draft_tile_ws<KS, true, true>), g, b, 0, s, t);
            else hipLaunchKernelGGL((k_draft_tile_ws<KS, false, true>), g, b, 0, s, t);
        } else {
            if (t.vec4) hipLaunchKernelGGL((k_draft_tile_ws<KS, true, false>), g, b, 0, s, t);
            else hipLaunchKernelGGL((k_draft_tile_ws<KS, false, false>), g, b, 0, s, t);
        }
    }
}

template <typename WT, int KS>
static hipError_t propose_impl(const DraftArgs& a, int32_t* x_out, float* pd_x, float* pd_stats,
                               const ProposeWs& ws, hipStream_t s)
{
    const int n_gran = n_granules(a.V);
    TileArgs t{};
    t.U = a.U; t.W1 = a.W1; t.W2p = a.W2; t.x0 = a.x0; t.x = x_out;
    t.R = a.R; t.gamma = a.gamma; t.r = a.r; t.V = a.V; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.nrows = a.R; t.n_gran = n_gran;
    tile_grid(a.R, n_gran, t.bpc, t.n_chunks);
    t.gstat = ws.gstat; t.gidx = ws.gidx; t.status = a.status;
    PickArgs pk{};
    pk.U = a.U; pk.W1 = a.W1; pk.W2p = a.W2; pk.x0 = a.x0; pk.x = x_out;
    pk.R = a.R; pk.gamma = a.gamma; pk.r = a.r; pk.V = a.V; pk.c = a.c;
    pk.n_gran = n_gran; pk.seed = a.seed; pk.round = a.round;
    pk.gstat = ws.gstat; pk.gidx = ws.gidx; pk.pd_x = pd_x; pk.pd_stats = pd_stats;
    if (ws.part && !(a.path & PATH_NO_FUSED_PROPOSE) && n_gran <= FUSED_PER * TILE_THREADS && k_steps<WT>(a.r) == KS) {
        const bool fits = a.greedy ? n_gran <= fused_capacity<WT, KS, true>()
                                   : n_gran <= fused_capacity<WT, KS, false>();
        if (fits) {
            t.n_chunks = 1;
            t.bpc = (a.R + BLOCK_ROWS - 1) / BLOCK_ROWS;
            return a.greedy ? propose_fused<WT, KS, true>(a, t, x_out, pd_x, pd_stats, ws, s)
                            : propose_fused<WT, KS, false>(a, t, x_out, pd_x, pd_stats, ws, s);
        }
    }
    const int grid = xcd_grid(n_gran * t.n_chunks);
    // many requests, bf16 weights filling the k-steps: the pipelined tile
    // (r = 512 keeps the staged tile: its W2 slice alone would take 128 of
    // the pipelined tile's 170 registers per lane)
    const bool piped = std::is_same<WT, bf16w>::value && (KS == 8 || KS == 16) && a.r == 16 * KS &&
                       a.R > PIPED_TILE_MIN_R;
    int pgrid = 0;
    if constexpr (KS == 8 || KS == 16) {
        if (piped) {
            t.div_rb = FastDiv::make((a.R + BLOCK_ROWS - 1) / BLOCK_ROWS);
            const long units = (long)n_gran * ((a.R + BLOCK_ROWS - 1) / BLOCK_ROWS);
            const int slots =
                a.greedy ? tile_ws_slots<KS, true>(t.vec4 != 0) : tile_ws_slots<KS, false>(t.vec4 != 0);
            const long n = std::min<long>(slots, units);
            pgrid = (int)(n >= NUM_XCD ? n / NUM_XCD * NUM_XCD : xcd_grid((int)n));
        }
    }
    for (int k = 1; k <= a.gamma; ++k) {
        t.kfix = k - 1;
        pk.k = k;
        {
            ProfScope ps("draft_tile", s);
            if (piped)
                launch_tile_ws<KS>(t, a.greedy, pgrid, s);
            else if (a.greedy)
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

// One wave per row: merge granule partials into the row's (M, S).
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

// Draft (M, S) of every (req, kk) row, for spec_confidence without supplied
// propose statistics.
template <typename WT, int KS>
static hipError_t row_stats_impl(const DraftArgs& a, const VerifyWs& ws, hipStream_t s)
{
    const int n_gran = n_granules(a.V);
    const int nrows = a.R * a.gamma;
    TileArgs t{};
    t.U = a.U; t.W1 = a.W1; t.W2p = a.W2; t.x0 = a.x0; t.x = a.x;
    t.R = a.R; t.gamma = a.gamma; t.r = a.r; t.V = a.V; t.c = a.c; t.vec4 = (a.V % 4) == 0;
    t.kfix = -1; t.nrows = nrows; t.n_gran = n_gran;
    tile_grid(nrows, n_gran, t.bpc, t.n_chunks);
    t.gstat = ws.dgran; t.gidx = ws.dgidx; t.status = a.status;
    {
        ProfScope ps("draft_tile", s);
        hipLaunchKernelGGL((k_draft_tile<WT, KS, false>), dim3(xcd_grid(n_gran * t.n_chunks)),
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
