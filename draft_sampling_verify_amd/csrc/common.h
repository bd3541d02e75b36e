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
constexpr int ZS_ = GRAN + 4;   // row stride (floats) of the 32 x 128 LDS result tile
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

// ------------------------------------------- exchange between workgroups
//
// Values one workgroup of a running kernel hands to another go through
// agent-scope atomic stores and loads.  On gfx950 these carry the sc1 cache
// policy: stores write through to the device coherence point and loads do
// not hit stale lines in the per-XCD L2, so no L2 writeback or invalidate is
// needed.  A producer issues its data stores, waits until they are
// acknowledged (stores_done), and only then stores the flag the consumer
// polls; the consumer reads the data after it has seen the flag.

__device__ inline void st_dev(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int32_t* p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev2(float* p, float a, float b)  // p 8-byte aligned
{
    const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_dev(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t ld_dev(const uint32_t* p)
{
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t ld_dev(const int32_t* p)
{
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float2 ld_dev2(const float* p)  // p 8-byte aligned
{
    const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
// Hide a uniform value from loop-invariant code motion, so that addresses
// derived from it are recomputed where they are used instead of being kept
// live (or spilled) across a long loop body.
template <typename T>
__device__ inline T* opaque(T* p)
{
    asm volatile("" : "+s"(p));
    return p;
}
__device__ inline int opaque(int v)
{
    asm volatile("" : "+s"(v));
    return v;
}
__device__ inline int opaque_v(int v)  // per-lane value
{
    asm volatile("" : "+v"(v));
    return v;
}
// Wait until every memory operation this wave issued has completed.
__device__ inline void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
__device__ inline int wave_max_int(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, shfl_xor(v, o));
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
__device__ inline double wave_incl_scan(double v)
{
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        double t = __shfl_up(v, o, WAVE);
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
//
// Where a lane owns a contiguous run of granules (rows of more than 2048
// granules: up to 131072 at V = 2^24) the sums across granules run in fp64:
// an fp32 running sum of that length drifts by up to its length in units of
// the last place, enough to move a draw whose u lies within 1e-6 of a
// token boundary.  In fp64 the error left is that of the fp32 granule
// masses themselves (about 1e-7 relative).  The register-cached pick below
// (at most 2048 granules: a 64-lane tree, then at most 32 rounds in
// sequence) stays in fp32.

// One wave; lane l owns the contiguous granule range [g0, g1).  Returns the
// lane's exclusive prefix of the granule masses and the wave total.
template <typename WF>
__device__ inline void wave_granule_scan(WF wf, int g0, int g1, double& excl, double& total)
{
    const int lane = threadIdx.x & (WAVE - 1);
    double tsum = 0.0;
    for (int g = g0; g < g1; ++g) tsum += (double)wf(g);
    const double incl = wave_incl_scan(tsum);
    excl = __shfl_up(incl, 1, WAVE);
    if (lane == 0) excl = 0.0;
    total = __shfl(incl, WAVE - 1, WAVE);
}

// First granule of positive mass whose running sum exceeds target.  Every lane re-runs its
// own running sum from its exclusive prefix and claims if it crosses; the
// lowest claiming lane wins (prefix pieces of different lanes may disagree
// in the last bit).  Returns the granule and the running sum before it,
// identical in every lane; if no partial sum exceeds target (rounding),
// returns the last granule with positive mass and sets fallback.
template <typename WF>
__device__ inline int wave_granule_find(WF wf, int g0, int g1, double excl, double target, double& before,
                                        bool& fallback)
{
    double run = excl, prev = excl;
    int pick = -1, lastpos = -1;
    for (int g = g0; g < g1; ++g) {
        const float wg = wf(g);
        if (wg > 0.0f) lastpos = g;
        if (pick < 0) {
            prev = run;
            run += (double)wg;
            if (run > target && wg > 0.0f) pick = g;
        }
    }
    const unsigned long long hit = __ballot(pick >= 0);
    if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        fallback = false;
        before = __shfl(prev, L, WAVE);
        return __shfl(pick, L, WAVE);
    }
    fallback = true;
    before = 0.0;
    const int lp = -wave_min(-lastpos);
    return lp < 0 ? 0 : lp;
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
    // only an id of positive weight can be the first to pass the target
    // (the running sums of neighbouring lanes are rounded differently)
    const bool ha = ca > target && ea > 0.0f, hb = cb > target && eb > 0.0f;
    const unsigned long long hit = __ballot(!fallback && (ha || hb));
    if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        const bool la = __shfl((int)ha, L, WAVE) != 0;
        const float lea = __shfl(ea, L, WAVE), leb = __shfl(eb, L, WAVE);
        e_out = la ? lea : leb;
        return la ? 2 * L : 2 * L + 1;
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
// Division by a divisor fixed for a launch: n / d for 0 <= n < 2^31 with one
// high multiply, an add and a shift (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> l, where the sum stays below 2^32.
struct FastDiv {
    uint32_t m;
    int l;
    __host__ __device__ static inline FastDiv make(int d)
    {
        FastDiv f;
        f.l = 0;
        while ((1u << f.l) < (uint32_t)d) ++f.l;
        f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << f.l) - (uint64_t)d)) / (uint64_t)d + 1);
        return f;
    }
    __device__ inline int div(int n) const { return (int)((__umulhi((uint32_t)n, m) + (uint32_t)n) >> l); }
};

constexpr int NUM_XCD = 8;
__host__ __device__ inline int xcd_grid(int n) { return (n + NUM_XCD - 1) / NUM_XCD * NUM_XCD; }
__device__ inline int xcd_logical(int bid, int n)
{
    const int per = (n + NUM_XCD - 1) / NUM_XCD;
    return (bid % NUM_XCD) * per + bid / NUM_XCD;
}

// ------------------------------------------------------- MFMA bias tile
//
// The Markov bias of 32 rows at 32 vocabulary ids is one wave's
//   D[m][n] = sum_i W2[32b + m, i] * W1[tok_n, i]
// on v_mfma_f32_32x32x16_bf16 (bf16 weights) or v_mfma_f32_32x32x2_f32
// (fp32 weights): m runs over the ids of column block b, n over the rows.
//
// A operand (W2) comes from the packed layout written by k_pack_w2: for
// column block b and k-step s the 64 lanes' operands are one contiguous
// 1 KB (bf16) chunk, lane l = n + 32h holding W2[32b + n][16s + 8h .. +7],
// so every load instruction is fully coalesced.  For fp32 weights a chunk
// holds four k-steps of 2: lane l holds W2[32b + n][8t + 2q + h], q = 0..3.
// The A operand of a wave stays in registers while its workgroup walks
// over row blocks.
//
// B operand (W1 rows of the 32 row tokens) is staged once per row block in
// LDS (row stride RS elements, padded so the 32 rows fall on distinct
// banks), lane l = n + 32h reading row n, k-slice 8h..8h+7 of each step.
//
// Result lane l = n + 32h holds row n and the 16 ids
// 32b + 8*(j>>2) + 4h + (j&3), j = 0..15.

template <typename WT, int KS>
struct TileOps;

template <int KS>
struct TileOps<bf16w, KS> {
    static constexpr int ELEM = 2;
    static constexpr int RS = 16 * KS + 8;  // LDS row stride (elements) of the staged W1 rows
    uint4 a[KS];
    // ks = r / 16 real k-steps (<= KS); the rest multiply zeros
    __device__ inline void load_a(const void* W2p, int ks, int b, bool valid, int lane)
    {
        const uint4* P = reinterpret_cast<const uint4*>(W2p) + (size_t)b * ks * WAVE + lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = (valid && s < ks) ? P[(size_t)s * WAVE] : make_uint4(0, 0, 0, 0);
    }
    __device__ inline f32x16 mfma(const void* sB, int ks, int lane) const
    {
        const uint16_t* B = reinterpret_cast<const uint16_t*>(sB) + (lane & 31) * RS + 8 * (lane >> 5);
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                const uint4 bv = *reinterpret_cast<const uint4*>(B + 16 * s);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        return acc;
    }
    // the ks real k-steps, accumulating onto acc
    __device__ inline f32x16 mfma_acc_n(const void* sB, int ks, int lane, f32x16 acc) const
    {
        const uint16_t* B = reinterpret_cast<const uint16_t*>(sB) + (lane & 31) * RS + 8 * (lane >> 5);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                const uint4 bv = *reinterpret_cast<const uint4*>(B + 16 * s);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        return acc;
    }
    // B operand from global memory, accumulating onto acc (single-row rescans)
    __device__ inline f32x16 mfma_global_acc(const bf16w* W1, int r, int tok, int ks, int lane, f32x16 acc) const
    {
        const uint4* row = reinterpret_cast<const uint4*>(W1 + (size_t)(tok < 0 ? 0 : tok) * r) + (lane >> 5);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                const uint4 bv = tok >= 0 ? row[2 * s] : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        return acc;
    }
    // mfma_acc reading at most LA B fragments ahead of the products that use
    // them, so that its registers stay bounded (same products, same order)
    template <int LA>
    __device__ inline f32x16 mfma_acc_la(const void* sB, int lane, f32x16 acc) const
    {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const uint16_t* B = reinterpret_cast<const uint16_t*>(sB) + (lane & 31) * RS + 8 * (lane >> 5);
        u32x4 bv[LA + 1];
#pragma unroll
        for (int s = 0; s < LA; ++s) bv[s] = *reinterpret_cast<const u32x4*>(B + 16 * s);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s + LA < KS) bv[(s + LA) % (LA + 1)] = *reinterpret_cast<const u32x4*>(B + 16 * (s + LA));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                          __builtin_bit_cast(bf16x8, bv[s % (LA + 1)]), acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        return acc;
    }
    // all KS k-steps (r == 16 KS), accumulating onto acc
    __device__ inline f32x16 mfma_acc(const void* sB, int lane, f32x16 acc) const
    {
        const uint16_t* B = reinterpret_cast<const uint16_t*>(sB) + (lane & 31) * RS + 8 * (lane >> 5);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 bv = *reinterpret_cast<const uint4*>(B + 16 * s);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        }
        return acc;
    }
    // B operand held in registers: lane l = n + 32h keeps W1[tok, 16s+8h..+7]
    // of its own row token (tok < 0: zeros).  Used by the single-row rescans.
    struct BRow {
        uint4 b[KS];
        __device__ inline void load(const bf16w* W1, int r, int tok, int ks, int lane)
        {
            const uint4* row = reinterpret_cast<const uint4*>(W1 + (size_t)(tok < 0 ? 0 : tok) * r) + (lane >> 5);
#pragma unroll
            for (int s = 0; s < KS; ++s) b[s] = (tok >= 0 && s < ks) ? row[2 * s] : make_uint4(0, 0, 0, 0);
        }
    };
    __device__ inline f32x16 mfma_row(const BRow& br, int ks) const
    {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, br.b[s]), acc, 0, 0, 0);
        }
        return acc;
    }
    __device__ inline f32x16 mfma_row_acc(const BRow& br, int ks, f32x16 acc) const
    {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, br.b[s]), acc, 0, 0, 0);
        }
        return acc;
    }
    // B operand straight from global memory (one row per lane; used by the
    // single-row rescans, which must see the same bits as the staged path)
    __device__ inline f32x16 mfma_global(const bf16w* W1, int r, int tok, int ks, int lane) const
    {
        const uint4* row = reinterpret_cast<const uint4*>(W1 + (size_t)(tok < 0 ? 0 : tok) * r) + (lane >> 5);
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s < ks) {
                const uint4 bv = tok >= 0 ? row[2 * s] : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                              __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        return acc;
    }
};

template <int KS>
struct TileOps<float, KS> {
    static constexpr int ELEM = 4;
    static constexpr int RS = 8 * KS + 4;  // KS groups of four 2-wide k-steps
    float4 a[KS];
    __device__ inline void load_a(const void* W2p, int ks, int b, bool valid, int lane)
    {
        const float4* P = reinterpret_cast<const float4*>(W2p) + (size_t)b * ks * WAVE + lane;
#pragma unroll
        for (int t = 0; t < KS; ++t) a[t] = (valid && t < ks) ? P[(size_t)t * WAVE] : make_float4(0, 0, 0, 0);
    }
    __device__ inline f32x16 mfma(const void* sB, int ks, int lane) const
    {
        const float* B = reinterpret_cast<const float*>(sB) + (lane & 31) * RS + (lane >> 5);
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, B[8 * t + 0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, B[8 * t + 2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, B[8 * t + 4], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, B[8 * t + 6], acc, 0, 0, 0);
            }
        }
        return acc;
    }
    // the ks real groups, accumulating onto acc
    __device__ inline f32x16 mfma_acc_n(const void* sB, int ks, int lane, f32x16 acc) const
    {
        const float* B = reinterpret_cast<const float*>(sB) + (lane & 31) * RS + (lane >> 5);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, B[8 * t + 0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, B[8 * t + 2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, B[8 * t + 4], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, B[8 * t + 6], acc, 0, 0, 0);
            }
        }
        return acc;
    }
    __device__ inline f32x16 mfma_global_acc(const float* W1, int r, int tok, int ks, int lane, f32x16 acc) const
    {
        const float* row = W1 + (size_t)(tok < 0 ? 0 : tok) * r + (lane >> 5);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                const float b0 = tok >= 0 ? row[8 * t + 0] : 0.0f, b1 = tok >= 0 ? row[8 * t + 2] : 0.0f;
                const float b2 = tok >= 0 ? row[8 * t + 4] : 0.0f, b3 = tok >= 0 ? row[8 * t + 6] : 0.0f;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, b1, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, b2, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, b3, acc, 0, 0, 0);
            }
        }
        return acc;
    }
    // all KS groups (r == 8 KS), accumulating onto acc
    __device__ inline f32x16 mfma_acc(const void* sB, int lane, f32x16 acc) const
    {
        const float* B = reinterpret_cast<const float*>(sB) + (lane & 31) * RS + (lane >> 5);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, B[8 * t + 0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, B[8 * t + 2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, B[8 * t + 4], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, B[8 * t + 6], acc, 0, 0, 0);
        }
        return acc;
    }
    struct BRow {
        float4 b[KS];  // W1[tok, 8t + 2q + h], q = 0..3
        __device__ inline void load(const float* W1, int r, int tok, int ks, int lane)
        {
            const float* row = W1 + (size_t)(tok < 0 ? 0 : tok) * r + (lane >> 5);
#pragma unroll
            for (int t = 0; t < KS; ++t)
                b[t] = (tok >= 0 && t < ks) ? make_float4(row[8 * t], row[8 * t + 2], row[8 * t + 4], row[8 * t + 6])
                                            : make_float4(0, 0, 0, 0);
        }
    };
    __device__ inline f32x16 mfma_row(const BRow& br, int ks) const
    {
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, br.b[t].x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, br.b[t].y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, br.b[t].z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, br.b[t].w, acc, 0, 0, 0);
            }
        }
        return acc;
    }
    __device__ inline f32x16 mfma_row_acc(const BRow& br, int ks, f32x16 acc) const
    {
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, br.b[t].x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, br.b[t].y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, br.b[t].z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, br.b[t].w, acc, 0, 0, 0);
            }
        }
        return acc;
    }
    __device__ inline f32x16 mfma_global(const float* W1, int r, int tok, int ks, int lane) const
    {
        const float* row = W1 + (size_t)(tok < 0 ? 0 : tok) * r + (lane >> 5);
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            if (t < ks) {
                const float b0 = tok >= 0 ? row[8 * t + 0] : 0.0f, b1 = tok >= 0 ? row[8 * t + 2] : 0.0f;
                const float b2 = tok >= 0 ? row[8 * t + 4] : 0.0f, b3 = tok >= 0 ? row[8 * t + 6] : 0.0f;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].x, b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].y, b1, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].z, b2, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t].w, b3, acc, 0, 0, 0);
            }
        }
        return acc;
    }
};

// k-steps (bf16) or groups of four k-steps (fp32) for rank r
template <typename WT> __host__ __device__ inline int k_steps(int r);
template <> __host__ __device__ inline int k_steps<bf16w>(int r) { return r / 16; }
template <> __host__ __device__ inline int k_steps<float>(int r) { return r / 8; }

// Stage the W1 rows of the 32 tokens tok[0..31] (LDS; -1 = zero row) into
// sB[32][RS]; all threads of the block take part.  KS bounds the row length
// (r <= 16 KS bf16 or 8 KS fp32 elements, 2 KS uint4); every thread issues
// all of its loads before its first LDS write, so the gather costs one
// memory round trip.
// The gather in two halves, so that a caller can issue other loads between
// them: issue() starts every W1 load of this thread, commit() writes them to
// LDS (and so waits for them, but not for loads issued after issue()).
template <typename WT, int RS, int KS>
struct W1Gather {
    static constexpr int ELEM = (int)sizeof(WT);
    static constexpr int NPT = (32 * 2 * KS + TILE_THREADS - 1) / TILE_THREADS;
    uint4 v[NPT];
    uint32_t keep[NPT];

    __device__ inline void issue(const WT* W1, const int* tok, int r)
    {
        const int per_row = r * ELEM / 16;  // uint4 per row
        const int total = 32 * per_row;
        const int t0 = opaque_v(threadIdx.x);
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = min(t0 + i * TILE_THREADS, total - 1);  // duplicates store the same value
            const int row = idx / per_row, c = idx - row * per_row;
            const int tk = tok[row];
            keep[i] = tk >= 0 ? ~0u : 0u;
            v[i] = reinterpret_cast<const uint4*>(W1 + (size_t)(tk >= 0 ? tk : 0) * r)[c];
        }
    }
    __device__ inline void commit(void* sB, int r) const
    {
        const int per_row = r * ELEM / 16;
        const int total = 32 * per_row;
        const int t0 = opaque_v(threadIdx.x);
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = min(t0 + i * TILE_THREADS, total - 1);
            const int row = idx / per_row, c = idx - row * per_row;
            const uint4 m = make_uint4(v[i].x & keep[i], v[i].y & keep[i], v[i].z & keep[i], v[i].w & keep[i]);
            *reinterpret_cast<uint4*>(reinterpret_cast<char*>(sB) + (size_t)row * RS * ELEM + 16 * c) = m;
        }
    }
};

// The W1 rows of a 32-row tile (bf16, r = 16 KS) through registers, for
// pipelines that load them a stage before they are written to LDS.  The
// tile's uint4 are taken in row-major order (2 KS per row) and split into
// PARTS equal parts; thread t of 256 moves uint4 t, t + 256, ... of its
// part.  A missing token (< 0) loads row 0; the caller ignores that row's
// results.
template <int RS, int KS, int PARTS>
struct W1Regs {
    // a native vector type: its copies are plain loads and stores, so the
    // array stays in registers
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    static constexpr int PER_ROW = 2 * KS;
    static constexpr int PART = 32 * PER_ROW / PARTS;
    static constexpr int NPT = PART / TILE_THREADS;
    static_assert(PART % TILE_THREADS == 0, "whole parts");
    u32x4 v[NPT];
    __device__ inline void issue(const bf16w* W1, const int* tok, int part, int t)
    {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = part * PART + t + i * TILE_THREADS;
            const int tk = tok[idx / PER_ROW];
            v[i] = reinterpret_cast<const u32x4*>(W1 + (size_t)(tk >= 0 ? tk : 0) * (16 * KS))[idx % PER_ROW];
        }
    }
    __device__ inline void commit(void* sB, int part, int t) const
    {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int idx = part * PART + t + i * TILE_THREADS;
            *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sB) + (size_t)(idx / PER_ROW) * RS * 2 +
                                      16 * (idx % PER_ROW)) = v[i];
        }
    }
};

// The second half of a 32-row W1 tile (rows 16..31, bf16, r = 16 KS)
// through the registers of 512 threads, one uint4 each: for KS = 8 the half
// has 256 uint4 and threads past it load and store the half's last one again
// (the same value), so that every thread issues exactly one load.
template <int RS, int KS>
struct W1HalfRegs {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    static constexpr int PER_ROW = 2 * KS;
    static constexpr int HALF = 16 * PER_ROW;
    static_assert(HALF <= 2 * TILE_THREADS, "one uint4 per thread");
    u32x4 v;
    __device__ static inline int index(int te) { return HALF + min(te, HALF - 1); }
    __device__ inline void issue(const bf16w* W1, const int* tok, int te)
    {
        const int idx = index(te);
        const int tk = tok[idx / PER_ROW];
        v = reinterpret_cast<const u32x4*>(W1 + (size_t)(tk >= 0 ? tk : 0) * (16 * KS))[idx % PER_ROW];
    }
    __device__ inline void commit(void* sB, int te) const
    {
        const int idx = index(te);
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sB) + (size_t)(idx / PER_ROW) * RS * 2 +
                                  16 * (idx % PER_ROW)) = v;
    }
};

template <typename WT, int RS, int KS>
__device__ inline void stage_w1(void* sB, const WT* W1, const int* tok, int r)
{
    W1Gather<WT, RS, KS> gw;
    gw.issue(W1, tok, r);
    gw.commit(sB, r);
}

// stage_w1 for r that fills the k-steps exactly (2 KS uint4 per row): every
// thread issues all of its loads before its first LDS write, so the gather
// costs one memory round trip.
template <typename WT, int RS, int KS>
__device__ inline void stage_w1_exact(void* sB, const WT* W1, const int* tok)
{
    constexpr int ELEM = (int)sizeof(WT);
    constexpr int PER_ROW = 2 * KS;                  // uint4 per W1 row
    constexpr int R_ELEMS = PER_ROW * 16 / ELEM;     // r
    constexpr int TOTAL = 32 * PER_ROW;
    constexpr int NPT = (TOTAL + TILE_THREADS - 1) / TILE_THREADS;
    // indices recomputed here from an opaque thread id: nothing of this
    // survives between calls (register pressure in the callers' loops)
    const int t0 = opaque_v(threadIdx.x);
    uint4 v[NPT];
    uint32_t keep[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        int idx = t0 + i * TILE_THREADS;
        if (TOTAL % TILE_THREADS != 0) idx = min(idx, TOTAL - 1);  // duplicates store the same value
        const int tk = tok[idx / PER_ROW];
        keep[i] = tk >= 0 ? ~0u : 0u;
        // unconditional load (row 0 for a missing token), masked to zero below
        v[i] = reinterpret_cast<const uint4*>(W1 + (size_t)(tk >= 0 ? tk : 0) * R_ELEMS)[idx % PER_ROW];
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        int idx = t0 + i * TILE_THREADS;
        if (TOTAL % TILE_THREADS != 0) idx = min(idx, TOTAL - 1);
        const uint4 m = make_uint4(v[i].x & keep[i], v[i].y & keep[i], v[i].z & keep[i], v[i].w & keep[i]);
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(sB) + (size_t)(idx / PER_ROW) * RS * ELEM +
                                  16 * (idx % PER_ROW)) = m;
    }
}

// Read back what store_tile wrote for this lane (its own 16 entries).
__device__ inline void load_tile_own(const float* sZ, f32x16& acc, int w, int lane)
{
    const int n = lane & 31, h = lane >> 5;
    const float* row = sZ + n * ZS_ + 32 * w + 4 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(row + 8 * q);
        acc[4 * q] = v.x; acc[4 * q + 1] = v.y; acc[4 * q + 2] = v.z; acc[4 * q + 3] = v.w;
    }
}

// LDS tile of the block's results: 32 rows x 128 ids (+4 floats padding).
constexpr int ZS = ZS_;

// Wave w stores its 32x32 result into sZ[n][32w + ...].
__device__ inline void store_tile(float* sZ, const f32x16& acc, int w, int lane)
{
    const int n = lane & 31, h = lane >> 5;
    float* row = sZ + n * ZS + 32 * w + 4 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(row + 8 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// Load the 16 values a lane of half h holds in the MFMA result layout,
// row[c0 + 8*(j>>2) + 4h + (j&3)] for j = 0..15 (ids >= V read as -inf).
__device__ inline void load_acc16(const float* row, int c0, int h, int V, bool vec4, float (&v)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c0 + 8 * q + 4 * h;
        if (vec4 && c + 3 < V) {
            const float4 t = *reinterpret_cast<const float4*>(row + c);
            v[4 * q + 0] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = (c + e < V) ? row[c + e] : -INFINITY;
        }
    }
}

// Load 16 consecutive fp32 values row[c0 .. c0+15]; ids >= V read as -inf.
// Fully in-bounds aligned segments take four unconditional 16-byte loads.
__device__ inline void load16(const float* row, int c0, int V, bool vec4, float (&v)[16])
{
    if (vec4 && c0 + 15 < V) {
        const float4* p4 = reinterpret_cast<const float4*>(row + c0);
        const float4 a = p4[0], b = p4[1], c = p4[2], d = p4[3];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        v[8] = c.x; v[9] = c.y; v[10] = c.z; v[11] = c.w;
        v[12] = d.x; v[13] = d.y; v[14] = d.z; v[15] = d.w;
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = (c0 + e < V) ? row[c0 + e] : -INFINITY;
    }
}

// load16 without branches (the compiler then counts this thread's loads
// exactly, so a later wait on an earlier load does not also wait for these):
// indices clamped into the row, ids past V replaced by -inf.  c0 is a
// multiple of 16; VEC4 requires V % 4 == 0.
// The loads of load16_flat without the masking: ids past V hold whatever the
// clamped load returned, and the caller masks them where it uses them (so
// that nothing touches the loaded registers before then).
template <bool VEC4>
__device__ inline void load16_raw(const float* row, int c0, int V, float (&v)[16])
{
    if constexpr (VEC4) {
        const float4* p4 = reinterpret_cast<const float4*>(row);
        const int q0 = c0 >> 2, qmax = (V >> 2) - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = p4[min(q0 + j, qmax)];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = row[min(c0 + e, V - 1)];
    }
}

// load16_raw for 8 consecutive floats.
template <bool VEC4>
__device__ inline void load8_raw(const float* row, int c0, int V, float (&v)[8])
{
    if constexpr (VEC4) {
        const float4* p4 = reinterpret_cast<const float4*>(row);
        const int q0 = c0 >> 2, qmax = (V >> 2) - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float4 a = p4[min(q0 + j, qmax)];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = row[min(c0 + e, V - 1)];
    }
}

template <bool VEC4>
__device__ inline void load16_flat(const float* row, int c0, int V, float (&v)[16])
{
    if constexpr (VEC4) {
        const float4* p4 = reinterpret_cast<const float4*>(row);
        const int q0 = c0 >> 2, qmax = (V >> 2) - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = p4[min(q0 + j, qmax)];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = row[min(c0 + e, V - 1)];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c0 + e < V ? v[e] : -INFINITY;
}

// Reductions across the 8 lanes that share an epilogue row, on DPP (no LDS
// round trip): quad_perm swaps lanes 1<->0, 3<->2 (xor 1) and 2,3<->0,1
// (xor 2); row_half_mirror pairs lane i with 7-i, joining the two quads.
// Every lane of the group ends with the same result.
template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_MIRROR = 0x1B, DPP_ROW_ROR8 = 0x128;

__device__ inline float oct_max(float v)
{
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    return fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
}
__device__ inline float oct_sum(float v)
{
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    return v + dpp_f<DPP_HALF_MIRROR>(v);
}
// The sum of a 16-lane group (a DPP row) whose lane l holds the partial sum
// of ids 8l..8l+7 of a granule: pairs (xor 1), quads (xor 2), halves of 8
// (half mirror), then the two halves (rotate by 8).  pair_oct_sum gives the
// same bits when 8 lanes hold two such partials each (lo: lane 2t, hi: lane
// 2t+1): every level adds the same two operands.
__device__ inline float hex_sum(float v)
{
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    return v + dpp_f<DPP_ROW_ROR8>(v);
}
__device__ inline float hex_max(float v)
{
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    return fmaxf(v, dpp_f<DPP_ROW_ROR8>(v));
}
__device__ inline float pair_oct_sum(float lo, float hi)
{
    float v = lo + hi;
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_QUAD_MIRROR>(v);
    return v + dpp_f<DPP_HALF_MIRROR>(v);
}
__device__ inline void oct_argmax(float& v, int& i)
{
    argmax_merge(v, i, dpp_f<DPP_XOR1>(v), dpp_i<DPP_XOR1>(i));
    argmax_merge(v, i, dpp_f<DPP_XOR2>(v), dpp_i<DPP_XOR2>(i));
    argmax_merge(v, i, dpp_f<DPP_HALF_MIRROR>(v), dpp_i<DPP_HALF_MIRROR>(i));
}
__device__ inline void hex_argmax(float& v, int& i)
{
    oct_argmax(v, i);
    argmax_merge(v, i, dpp_f<DPP_ROW_ROR8>(v), dpp_i<DPP_ROW_ROR8>(i));
}

// Whole-wave scans on DPP moves (no LDS round trip): rows of 16 lanes by
// row_shr 1, 2, 4, 8, then row_bcast15 (rows 1 and 3 add lane 15 of the row
// before) and row_bcast31 (rows 2 and 3 add lane 31).  Disabled rows read 0.
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143, DPP_WAVE_SHR1 = 0x138;
template <int CTRL, int ROWS>
__device__ inline float dpp_z(float v)  // source lane's value, 0 where none
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ inline int dpp_zi(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
// Inclusive prefix sum over the wave's lanes in lane order (a fixed order:
// the same inputs give the same bits in every wave).
__device__ inline float wave_scan_dpp(float v)
{
    const int l = threadIdx.x & 15;
    float t = dpp_z<DPP_ROW_SHR1, 0xF>(v);
    if (l >= 1) v += t;
    t = dpp_z<DPP_ROW_SHR2, 0xF>(v);
    if (l >= 2) v += t;
    t = dpp_z<DPP_ROW_SHR4, 0xF>(v);
    if (l >= 4) v += t;
    t = dpp_z<DPP_ROW_SHR8, 0xF>(v);
    if (l >= 8) v += t;
    v += dpp_z<DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_z<DPP_ROW_BCAST31, 0xC>(v);
    return v;
}
// The previous lane's value (0 in lane 0).
__device__ inline float lane_before(float v) { return dpp_z<DPP_WAVE_SHR1, 0xF>(v); }
__device__ inline float lane63(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }
// Sum over the wave, the same bits in every lane: the 16-lane row sums on
// DPP (hex_sum), then (row 0 + row 1) + (row 2 + row 3) from scalar reads.
__device__ inline float wave_total_dpp(float v)
{
    v = hex_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}
// Maximum over the wave, in every lane.
__device__ inline float wave_max_dpp(float v)
{
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));                  // 8-lane groups
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x118, 0xF, 0xF,
                                                            false)));  // row_shr:8: lanes 8-15 see 0-7
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), DPP_ROW_BCAST15,
                                                            0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), DPP_ROW_BCAST31,
                                                            0xC, 0xF, false)));
    return lane63(v);
}
// Totals of NR rounds of granule masses (lane l holds w[i], the mass of
// granule l + 64 i) by a transposing butterfly: at each exchange a lane
// keeps one half of its values, the half its partner lane gives away, and
// adds the partner's copy of it, so NR values per lane become one after
// log2 NR exchanges of halving size (NR - 1 shuffles in all instead of NR
// separate wave reductions); the lanes that still share a round are then
// summed.  Lane l ends with the total of round l >> (6 - log2 NR), the same
// bits in every lane of that group.
template <int NR>
__device__ inline float wave_round_totals(const float (&w)[NR])
{
    static_assert(NR == 16 || NR == 32, "16 or 32 rounds");
    constexpr int LOG = NR == 16 ? 4 : 5;
    const int lane = threadIdx.x & (WAVE - 1);
    float v[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) v[i] = w[i];
#pragma unroll
    for (int k = 0; k < LOG; ++k) {
        const int d = 32 >> k, half = (NR >> k) >> 1;
        const bool up = (lane & d) != 0;
#pragma unroll
        for (int j = 0; j < half; ++j) {
            const float keep = up ? v[j + half] : v[j];
            const float give = up ? v[j] : v[j + half];
            v[j] = keep + shfl_xor(give, d);
        }
    }
    float t = v[0];
#pragma unroll
    for (int d = 32 >> LOG; d >= 1; d >>= 1) t += shfl_xor(t, d);
    return t;
}

// The running totals of the rounds in order: lane l's inclusive sum over the
// rounds up to its own (only the first lane of each round's group
// contributes), on DPP.
template <int NR>
__device__ inline float wave_rounds_scan(const float (&w)[NR], float& T, bool& lead)
{
    const int lane = threadIdx.x & (WAVE - 1);
    T = wave_round_totals(w);
    lead = lane % (WAVE / NR) == 0;
    return wave_scan_dpp(lead ? T : 0.0f);
}

// The total of all rounds, with the bits wave_rounds_pick reports.
template <int NR>
__device__ inline float wave_rounds_sum(const float (&w)[NR])
{
    float T;
    bool lead;
    return lane63(wave_rounds_scan(w, T, lead));
}

// Register-cached inverse CDF over at most 64 NR granule masses, one wave.
// Lane l holds w[i] = mass of granule l + 64 i (0 past the end): the caller
// loads all of them at once (coalesced, one memory round trip).  Round i
// covers granules 64 i .. 64 i + 63 in lane order, so the rounds in order
// are the granules in vocabulary order.  Returns the first granule of
// positive mass whose running sum exceeds u * total, the running sum before
// it and the total, identical in every lane; if rounding leaves none, the
// last granule with positive mass (fallback set).  The round totals, their
// running sums and the scan inside the chosen round stay in registers (no
// LDS round trips).
template <int NR>
__device__ inline int wave_rounds_pick(const float (&w)[NR], float u, float& total, float& before, bool& fallback)
{
    const int lane = threadIdx.x & (WAVE - 1);
    float T;
    bool lead;
    const float incl = wave_rounds_scan(w, T, lead);
    const float Z = lane63(incl);
    total = Z;
    const float target = u * Z;
    // the first round of positive mass whose running total passes the target
    const unsigned long long hr = __ballot(lead && T > 0.0f && incl > target);
    int rstar = -1;
    float rbase = 0.0f;
    if (hr) {
        const int Lr = __ffsll((long long)hr) - 1;
        rstar = Lr / (WAVE / NR);
        rbase = __shfl(lane_before(incl), Lr, WAVE);  // the rounds before it
    }
    float wr = 0.0f;
    int lastpos = -1;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (i == rstar) wr = w[i];
        if (w[i] > 0.0f) lastpos = lane + WAVE * i;
    }
    const float ex = lane_before(wave_scan_dpp(wr));
    const float run0 = rbase + ex;
    const unsigned long long hit = __ballot(rstar >= 0 && wr > 0.0f && run0 + wr > target);
    if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        fallback = false;
        before = __shfl(run0, L, WAVE);
        return L + WAVE * rstar;
    }
    fallback = true;
    before = 0.0f;
    const int lp = -wave_min(-lastpos);
    return lp < 0 ? 0 : lp;
}

__device__ inline int wave_max_int_dpp(int v)
{
    v = max(v, dpp_i<DPP_XOR1>(v));
    v = max(v, dpp_i<DPP_XOR2>(v));
    v = max(v, dpp_i<DPP_HALF_MIRROR>(v));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, DPP_ROW_BCAST15, 0xA, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(v, v, DPP_ROW_BCAST31, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline int wave_min_int_dpp(int v) { return -wave_max_int_dpp(-v); }

// granule_pick with DPP scans: one full wave, lane l holds the weights of
// ids 2l and 2l+1; the first id whose running sum (from `before`) exceeds
// target, else (rounding, or `fallback`) the last id of positive weight.
__device__ inline int granule_pick_dpp(float ea, float eb, float before, float target, bool fallback, float& e_out)
{
    const float incl = wave_scan_dpp(ea + eb);
    const float ex = lane_before(incl);
    const float ca = (before + ex) + ea;
    const float cb = ca + eb;
    const bool ha = ca > target && ea > 0.0f, hb = cb > target && eb > 0.0f;
    const unsigned long long hit = __ballot(!fallback && (ha || hb));
    if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        const bool la = __builtin_amdgcn_readlane((int)ha, L) != 0;
        const float lea = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ea), L));
        const float leb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eb), L));
        e_out = la ? lea : leb;
        return la ? 2 * L : 2 * L + 1;
    }
    const unsigned long long nz = __ballot(ea > 0.0f || eb > 0.0f);
    const int L = nz ? 63 - __clzll((long long)nz) : 0;
    const float lea = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ea), L));
    const float leb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(eb), L));
    e_out = leb > 0.0f ? leb : lea;
    return leb > 0.0f ? 2 * L + 1 : 2 * L;
}

// The (granule, 32-row block) units a workgroup of a pipelined kernel takes,
// unit u = granule u / n_rb, block u % n_rb: run rho of the unit order (runs
// differ by at most one unit).  Consecutive runs sit on one XCD and
// alternate runs go backward, so the two runs that share a boundary granule
// both take it at their start or both at their end, and its W2 slice comes
// from HBM once for the two (the other load hits the XCD's L2).
struct UnitRun {
    int rho, u0, nu;
    bool fwd;
    __device__ inline UnitRun(int n_gran, int n_rb)
    {
        const long NU = (long)n_gran * n_rb;
        rho = xcd_logical(blockIdx.x, gridDim.x);
        u0 = (int)((long)rho * NU / gridDim.x);
        nu = (int)((long)(rho + 1) * NU / gridDim.x) - u0;
        fwd = (rho & 1) == 0;
    }
    // unit j of this run (j past the end repeats the last unit)
    __device__ inline int unit(int j) const
    {
        const int jj = min(j, nu - 1);
        return fwd ? u0 + jj : u0 + nu - 1 - jj;
    }
};

// Instantiations of the rank-dependent kernels: bf16 weights use r/16 k-steps
// (4, 8, 16 or 32 held; fewer real steps multiply zeros), fp32 weights r/8
// groups of four k-steps (2, 8 or 32 held).
template <template <typename, int> class F, typename... Args>
inline hipError_t dispatch_ks(int w_dtype, int r, Args&&... args)
{
    if (w_dtype == 1) {
        const int ks = r / 16;
        if (ks <= 4) return F<bf16w, 4>::run(args...);
        if (ks <= 8) return F<bf16w, 8>::run(args...);
        if (ks <= 16) return F<bf16w, 16>::run(args...);
        return F<bf16w, 32>::run(args...);
    }
    const int ks = r / 8;
    if (ks <= 2) return F<float, 2>::run(args...);
    if (ks <= 8) return F<float, 8>::run(args...);
    return F<float, 32>::run(args...);
}

}  // namespace spec
