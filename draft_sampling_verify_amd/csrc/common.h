// common.h -- device helpers shared by the libspec kernels (gfx950, wave64).
//
// Vocabulary tiling used by every kernel: the vocabulary is cut into
// granules of GRAN = 128 consecutive ids.  A workgroup of four waves covers
// one granule, each wave 32 ids.  Per-(row, granule) partial results (max,
// sum of exponentials, argmax, TV and residual mass) are written to the
// workspace and merged per row; sampling rescans exactly one granule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

constexpr int WAVE = 64;
constexpr int GRAN = 128;       // vocabulary ids per granule
constexpr int BLOCK_ROWS = 32;  // rows per MFMA block (one 32x32 output tile)
constexpr int TILE_THREADS = 256;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

struct bf16w { uint16_t bits; };  // tag type: weights stored as bf16 bit patterns

// ----------------------------------------------------------------- status

__device__ inline void raise_flag(uint32_t* status, uint32_t bit)
{
    atomicOr(status, bit);
}

// ----------------------------------------------------------------- Philox

// Philox4x32-10 (Salmon et al., SC'11): per round, multiply counter words 0
// and 2 by the round constants, mix the high halves with words 1, 3 and the
// key, keep the low halves, then advance the key by the Weyl increments.
struct u32x4 { uint32_t w[4]; };

__device__ inline u32x4 philox(uint32_t k, uint32_t req, uint64_t round, uint64_t seed)
{
    uint32_t c0 = k, c1 = req, c2 = (uint32_t)round, c3 = (uint32_t)(round >> 32);
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
    }
    u32x4 o;
    o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
    return o;
}

// 24-bit uniform in [0, 1 - 2^-24]; exact in fp32 and fp64.
__device__ inline float u24f(uint32_t w) { return (float)(w >> 8) * (1.0f / 16777216.0f); }
__device__ inline double u24d(uint32_t w) { return (double)(w >> 8) * (1.0 / 16777216.0); }

// ------------------------------------------------------------- arithmetic

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// e = 2^((z - m) * c): the un-normalised softmax weight of logit z against a
// reference m, with c = log2(e) / T.  Every kernel uses this one expression.
__device__ inline float softw(float z, float m, float c) { return fexp2(__fmul_rn(__fsub_rn(z, m), c)); }

__device__ inline float safe_ref(float m) { return m == -INFINITY ? 0.0f : m; }

// ------------------------------------------------------------- reductions

template <typename T>
__device__ inline T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, WAVE); }

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += shfl_xor(v, o);
    return v;
}
__device__ inline double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += shfl_xor(v, o);
    return v;
}
__device__ inline int wave_min(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, shfl_xor(v, o));
    return v;
}
// reductions inside each 32-lane half of the wave
__device__ inline float half_max(float v)
{
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, shfl_xor(v, o));
    return v;
}
__device__ inline float half_sum(float v)
{
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v += shfl_xor(v, o);
    return v;
}

// (value, index) argmax merge: larger value wins, ties go to the lower index.
__device__ inline void argmax_merge(float& v, int& i, float ov, int oi)
{
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}

// Inclusive prefix sum across the 64 lanes of a wave (fixed order).
__device__ inline float wave_incl_scan(float v)
{
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        float t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
    }
    return v;
}

// ---------------------------------------------------- block-wide scans (256)

// Block of 256 threads: exclusive scan of one float per thread plus total.
// `sm` needs 4 floats of shared memory.
__device__ inline float block_excl_scan(float v, float* sm, float& total)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const float incl = wave_incl_scan(v);
    float ex = __shfl_up(incl, 1, WAVE);
    if (lane == 0) ex = 0.0f;
    if (lane == WAVE - 1) sm[w] = incl;
    __syncthreads();
    float before = 0.0f;
    total = 0.0f;
#pragma unroll
    for (int i = 0; i < TILE_THREADS / WAVE; ++i) {
        if (i < w) before += sm[i];
        total += sm[i];
    }
    __syncthreads();
    return before + ex;
}

__device__ inline float block_max(float v, float* sm)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    v = wave_max(v);
    if (lane == 0) sm[w] = v;
    __syncthreads();
    float m = sm[0];
#pragma unroll
    for (int i = 1; i < TILE_THREADS / WAVE; ++i) m = fmaxf(m, sm[i]);
    __syncthreads();
    return m;
}

__device__ inline int block_min(int v, int* sm)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    v = wave_min(v);
    if (lane == 0) sm[w] = v;
    __syncthreads();
    int m = sm[0];
#pragma unroll
    for (int i = 1; i < TILE_THREADS / WAVE; ++i) m = min(m, sm[i]);
    __syncthreads();
    return m;
}


// ------------------------------------------------ inverse-CDF over granules
//
// Sampling by inverse CDF in vocabulary order, two levels: granule masses
// w_g (from the per-granule partials) locate the granule where the running
// sum first exceeds target = u * total; one wave then rescans that
// granule's 128 weights.  Threads of a 256-wide block own contiguous
// granule ranges [g0, g1).

// Thread-local sum of its granule masses and the block-wide exclusive scan.
template <typename WF>
__device__ inline void granule_scan(WF wf, int g0, int g1, float* smf, float& tsum, float& excl,
                                    float& total)
{
    tsum = 0.0f;
    for (int g = g0; g < g1; ++g) tsum += wf(g);
    excl = block_excl_scan(tsum, smf, total);
}

// First granule whose running sum exceeds target.  Every thread re-runs its
// own running sum from its exclusive prefix and claims if it crosses; the
// lowest claiming thread wins (prefix pieces computed by different threads
// may disagree in the last bit).  Returns the granule (same in every thread)
// and the running sum before it, or -1 if no partial sum exceeds target;
// then the last granule with positive mass is returned in *fallback_g.
template <typename WF>
__device__ inline int granule_find(WF wf, int g0, int g1, float excl, float target, float* smf,
                                   int* smi, float& before, int& fallback_g)
{
    float run = excl, prev = excl;
    int pick = -1, lastpos = -1;
    for (int g = g0; g < g1; ++g) {
        const float wg = wf(g);
        if (wg > 0.0f) lastpos = g;
        if (pick < 0) {
            prev = run;
            run += wg;
            if (run > target) pick = g;
        }
    }
    const int first = block_min(pick >= 0 ? (int)threadIdx.x : 0x7fffffff, smi);
    if ((int)threadIdx.x == first) {
        smi[4] = pick;
        smf[4] = prev;
    }
    fallback_g = -block_min(-lastpos, smi);
    if (first == 0x7fffffff && threadIdx.x == 0) smi[4] = -1;
    __syncthreads();
    const int gstar = smi[4];
    before = smf[4];
    __syncthreads();
    return gstar;
}

// Inside one granule, run by a single full wave: lane l holds the weights of
// ids 2l and 2l+1 of the granule.  Picks the first id whose running sum
// (from `before`) exceeds target; if none (rounding, or `fallback`), the
// last id with positive weight.  Returns the id within the granule and its
// weight, identical in every lane.
__device__ inline int granule_pick(float ea, float eb, float before, float target, bool fallback,
                                   float& e_out)
{
    const int lane = threadIdx.x & (WAVE - 1);
    const float incl = wave_incl_scan(ea + eb);
    float ex = __shfl_up(incl, 1, WAVE);
    if (lane == 0) ex = 0.0f;
    const float ca = (before + ex) + ea;
    const float cb = ca + eb;
    const unsigned long long hit = __ballot(!fallback && (ca > target || cb > target));
    if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        const float la = __shfl(ca, L, WAVE), lea = __shfl(ea, L, WAVE), leb = __shfl(eb, L, WAVE);
        e_out = la > target ? lea : leb;
        return la > target ? 2 * L : 2 * L + 1;
    }
    const unsigned long long nz = __ballot(ea > 0.0f || eb > 0.0f);
    const int L = nz ? 63 - __clzll((long long)nz) : 0;
    const float lea = __shfl(ea, L, WAVE), leb = __shfl(eb, L, WAVE);
    e_out = leb > 0.0f ? leb : lea;
    return leb > 0.0f ? 2 * L + 1 : 2 * L;
}

// ------------------------------------------------------ XCD-aware mapping

// Workgroups are dispatched round-robin over the 8 XCDs.  Remap so that
// consecutive logical ids run on the same XCD (they share W2 columns in its
// L2).  The grid is launched with xcd_grid(n) blocks; ids >= n must exit.
constexpr int NUM_XCD = 8;
__host__ __device__ inline int xcd_grid(int n) { return (n + NUM_XCD - 1) / NUM_XCD * NUM_XCD; }
__device__ inline int xcd_logical(int bid, int n)
{
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    return (bid % NUM_XCD) * per + bid / NUM_XCD;
}

// ------------------------------------------------------- MFMA bias tile
//
// One wave computes D[m][n] = sum_i W2[col0 + m, i] * W1[tok_n, i] for the
// 32 vocabulary ids col0..col0+31 (m) and 32 rows (n), i.e. the Markov bias
// of 32 rows at 32 ids, with v_mfma_f32_32x32x16_bf16 (bf16 weights) or
// v_mfma_f32_32x32x2_f32 (fp32 weights).  Operand lane layout (lane l,
// h = l >> 5): A holds W2 row col0 + (l & 31), k-slice 8h..8h+7 of each
// 16-wide k-step; B holds W1 row tok_{l & 31}, same k-slice.  Result lane l
// holds column n = l & 31 (the row of the block) and 16 ids
// col0 + 8*(j>>2) + 4h + (j&3), j = 0..15.
//
// The W2 operand depends only on the granule and is kept in registers while
// a workgroup walks over several row blocks.

template <typename WT, int KS>
struct W2Operand;

template <int KS>
struct W2Operand<bf16w, KS> {
    uint4 a[KS];  // KS k-steps of 16; 8 bf16 per lane per step
    __device__ inline void load(const bf16w* W2, int r, int V, int col, int h)
    {
        const int ks = r >> 4;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks && col < V)
                a[s] = *reinterpret_cast<const uint4*>(W2 + (size_t)col * r + 16 * s + 8 * h);
            else
                a[s] = make_uint4(0, 0, 0, 0);
        }
    }
    // tok < 0 -> zero row
    __device__ inline f32x16 mul(const bf16w* W1, int r, int tok, int h) const
    {
        const int ks = r >> 4;
        f32x16 acc = {};
        const bf16w* row = W1 + (size_t)(tok < 0 ? 0 : tok) * r + 8 * h;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                uint4 b = tok >= 0 ? *reinterpret_cast<const uint4*>(row + 16 * s) : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
            }
        }
        return acc;
    }
};

template <int KS>
struct W2Operand<float, KS> {
    float a[KS];  // KS k-steps of 2; one fp32 per lane per step
    __device__ inline void load(const float* W2, int r, int V, int col, int h)
    {
        const int ks = r >> 1;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            a[s] = (s < ks && col < V) ? W2[(size_t)col * r + 2 * s + h] : 0.0f;
    }
    __device__ inline f32x16 mul(const float* W1, int r, int tok, int h) const
    {
        const int ks = r >> 1;
        f32x16 acc = {};
        const float* row = W1 + (size_t)(tok < 0 ? 0 : tok) * r + h;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                float b = tok >= 0 ? row[2 * s] : 0.0f;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b, acc, 0, 0, 0);
            }
        }
        return acc;
    }
};

// id of accumulator j held by a lane of half h, relative to the wave's col0
__device__ inline int acc_col(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

// Load 16 fp32 values row[col0 + acc_col(j, h)] (ids >= V -> -inf).
// vec4: the row base is 16-byte aligned and V % 4 == 0.
__device__ inline void load_row16(const float* row, int col0, int h, int V, bool vec4, float (&v)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = col0 + 8 * q + 4 * h;
        if (vec4 && c + 3 < V) {
            float4 t = *reinterpret_cast<const float4*>(row + c);
            v[4 * q + 0] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = (c + e < V) ? row[c + e] : -INFINITY;
        }
    }
}

}  // namespace spec
