// internal.h -- host-side interfaces between the C-ABI layer (api.cpp) and
// the kernel launchers (propose.hip, verify.hip, schedule.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spec {

constexpr int GRAN_IDS = 128;  // same as GRAN in common.h (host copy)

inline int n_granules(int V) { return (V + GRAN_IDS - 1) / GRAN_IDS; }

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace header: status word and device-side counts.
struct WsHeader {
    uint32_t status;     // SPEC_DEV_* bits (sticky)
    uint32_t epoch;      // fused propose calls made with this workspace
    uint32_t abort;      // epoch of a fused propose that gave up waiting
    uint32_t pad0;
    int32_t counts[4];   // [0] verified rows K, [1] target rows K + R
};
constexpr size_t WS_HEADER = 256;

// Carves a workspace into regions; with base == nullptr it only measures.
struct Carver {
    char* base;
    size_t off;
    explicit Carver(void* b) : base((char*)b), off(WS_HEADER) {}
    template <typename T>
    T* take(size_t count)
    {
        T* p = base ? (T*)(base + off) : nullptr;
        off += align256(count * sizeof(T));
        return p;
    }
};

// Regions used by verify and confidence.
struct VerifyWs {
    float2* tgran;   // [TR, n_gran] per-granule (max, sum) of target rows
    int32_t* tgidx;  // [TR, n_gran] per-granule argmax
    float2* trow;    // [TR] merged (M_t, S_t)
    int32_t* targ;   // [TR] row argmax
    float2* vpart;   // [VR, n_gran] per-granule (TV mass, residual mass)
    float* vbias;    // [VR] Markov bias at the drafted id of each verified row
    int4* vmap;      // [VR] verified row -> (request, k, target row, 0)
    int2* tmap;      // [TR] target row -> (request, row within request)
    int32_t* voff;   // [R] first verified row of each request
    int32_t* toff;   // [R] first target row of each request
    float2* dgran;   // confidence only: [VR, n_gran] draft per-granule stats
    int32_t* dgidx;  // confidence only
    float2* drow;    // confidence only: [VR] draft (M, S)
    double* contrib; // loss only: [VR] weighted loss of each position
    float4* tpart;   // [TR, 16] per-part target row statistics (rows split over workgroups)
    int4* rtab;      // [VR] scheduled lengths: per verified row (x_{k-1}, x_k, U row, target row)
    float4* rctab;   // [VR] scheduled lengths: per verified row (M_d, S_d, M_t, S_t)
};

inline VerifyWs carve_verify(void* ws, int R, int gamma, int V, bool confidence, size_t* bytes,
                             bool loss = false)
{
    const size_t ng = (size_t)n_granules(V);
    const size_t VR = (size_t)R * gamma;
    const size_t TR = confidence ? VR : (size_t)R * (gamma + 1);
    Carver c(ws);
    VerifyWs w{};
    w.tgran = c.take<float2>(TR * ng);
    w.tgidx = c.take<int32_t>(TR * ng);
    w.trow = c.take<float2>(TR);
    w.targ = c.take<int32_t>(TR);
    w.vpart = c.take<float2>(VR * ng);
    w.vbias = c.take<float>(VR);
    w.vmap = c.take<int4>(VR);
    w.tmap = c.take<int2>(TR);
    w.voff = c.take<int32_t>(R);
    w.toff = c.take<int32_t>(R);
    if (confidence) {
        w.dgran = c.take<float2>(VR * ng);
        w.dgidx = c.take<int32_t>(VR * ng);
        w.drow = c.take<float2>(VR);
    }
    if (loss) w.contrib = c.take<double>(VR);
    w.tpart = c.take<float4>(TR * 16);
    w.rtab = c.take<int4>(VR);
    w.rctab = c.take<float4>(VR);
    if (bytes) *bytes = c.off;
    return w;
}

// The fused propose (one cooperative launch for all positions) handles one
// block of up to 32 requests; its hand-over words are kept in this many
// copies (every workgroup polls them).
constexpr int FUSED_MAX_R = 32;
constexpr int FUSED_TOKEN_COPIES = 64;
constexpr int FUSED_PART_WORDS = 3;  // per (request, granule): max, sum, argmax

struct ProposeWs {
    float2* gstat;    // [R, n_gran] per-position kernels
    int32_t* gidx;    // [R, n_gran]
    uint64_t* part;   // [FUSED_PART_WORDS][R][n_gran] fused: tagged partials (R <= FUSED_MAX_R), else null
    uint64_t* words;  // [FUSED_TOKEN_COPIES, 32] fused: tagged token words
    uint64_t* exitw;  // [n_gran] fused: tagged exit word of each workgroup
};

// Propose regions start at `start` bytes (the header by default; after the
// verify regions in spec_decode_rounds, so that the tagged hand-over words
// never share memory with other data).  *bytes = the end offset.
inline ProposeWs carve_propose(void* ws, int R, int V, size_t* bytes, size_t start = WS_HEADER)
{
    const size_t ng = (size_t)n_granules(V);
    Carver c(ws);
    c.off = start;
    ProposeWs w{};
    w.gstat = c.take<float2>((size_t)R * ng);
    w.gidx = c.take<int32_t>((size_t)R * ng);
    if (R <= FUSED_MAX_R) {
        w.part = c.take<uint64_t>((size_t)R * ng * FUSED_PART_WORDS);
        w.words = c.take<uint64_t>((size_t)FUSED_TOKEN_COPIES * 32);
        w.exitw = c.take<uint64_t>(ng);
    }
    if (bytes) *bytes = c.off;
    return w;
}

// Kernel-path choices of one call (the SPEC_PATH_* bits of spec.h).
constexpr int PATH_NO_FUSED_PROPOSE = 1;    // per-position propose kernels even where the fused launch fits
constexpr int PATH_NO_PIPELINED_SWEEP = 2;  // staged verify sweep even where the pipelined one applies

// Arguments common to the draft-side kernels.
struct DraftArgs {
    const float* U;
    const void* W1;
    const void* W2;    // packed layout (spec_pack_w2)
    int w_dtype;       // 0 fp32, 1 bf16
    const int32_t* x0;
    const int32_t* x;  // drafts (propose: output being filled; verify: input)
    int R, gamma, r, V;
    float c;           // log2(e) / T, rounded to fp32
    int greedy;
    uint64_t seed, round;
    uint32_t* status;
    int path;          // PATH_* bits
};

// propose.hip
// rv: W2 given as [r, V] instead of [V, r]
hipError_t launch_pack_w2(const void* W2, int w_dtype, int r, int V, void* W2p, bool rv, hipStream_t s);
inline size_t packed_w2_bytes(int w_dtype, int r, int V)
{
    return (size_t)((V + 31) / 32) * 32 * (size_t)r * (w_dtype == 1 ? 2 : 4);
}
hipError_t launch_propose(const DraftArgs& a, int32_t* x_out, float* pd_x, float* pd_stats,
                          const ProposeWs& w, hipStream_t s);
// Draft (max, sum) per granule and per row for all R*gamma drafted rows
// (confidence without supplied statistics).
hipError_t launch_draft_row_stats(const DraftArgs& a, const VerifyWs& w, hipStream_t s);

// verify.hip
hipError_t launch_verify(const DraftArgs& a, const float* pd_stats, const float* Lt,
                         const int32_t* ell, int32_t* n_acc, int32_t* y, float* pt_x,
                         float* c_star, const VerifyWs& w, int32_t* counts, hipStream_t s);
hipError_t launch_confidence(const DraftArgs& a, const float* pd_stats, const float* Lt,
                             float* c_star, double* a_star, const VerifyWs& w, hipStream_t s);
struct LossArgs {
    const float* q;          // [R,gamma] confidence logits
    float invT;              // 1 / T
    float a_ce, a_tv, a_conf;
    double* loss;            // [1]
    float* terms;            // [R,gamma,3] or NULL
    float* dq;               // [R,gamma] or NULL
};
hipError_t launch_draft_loss(const DraftArgs& a, const float* Lt, const LossArgs& l, const VerifyWs& w,
                             hipStream_t s);

// cluster.hip: the clustered draft head.  Limits of the GPU path.
constexpr int CL_MAX_NC = 8192;     // clusters
constexpr int CL_MAX_K = 256;       // clusters expanded per row
constexpr int CL_MAX_SIZE = 65536;  // tokens per cluster (16-bit place in tok_slot)
struct ClusterArgs {
    const void* H;          // [R*gamma, d] bf16
    const void* C;          // [N_c, d] bf16
    const void* E;          // [V, d] bf16
    const int32_t* cl_off;  // [N_c + 1]
    const int32_t* cl_tok;  // [V]
    int R, gamma, d, N_c, K_c, max_cl, V;
    float c;                // log2(e) / T
    int greedy;
    uint64_t seed, round;
    int32_t* x;             // [R, gamma]
    float* pd_x;            // [R, gamma]
    int32_t* sel;           // [R, gamma, K_c]
    float* zf;              // [R, gamma, K_c, max_cl]
    float* pd_stats;        // [R, gamma, 2]
    void* ws;               // header + coarse partial products
    uint32_t* status;
};
struct ClusterVerifyArgs {
    const int32_t* tok_slot;  // [V] (cluster << 16) | place
    const int32_t* sel;       // [R, gamma, K_c]
    const float* zf;          // [R, gamma, K_c, max_cl]
    const float* pd_stats;    // [R, gamma, 2]
    const int32_t* x;         // [R, gamma]
    const float* Lt;          // [R, gamma + 1, V]
    const int32_t* ell;       // [R] or NULL
    int R, gamma, N_c, K_c, max_cl, V;
    float c;
    int greedy;
    uint64_t seed, round;
    int32_t* n_acc;
    int32_t* y;
    float* pt_x;
    float* c_star;
    uint32_t* status;
};
hipError_t launch_cluster_verify(const ClusterVerifyArgs& cv, const VerifyWs& w, hipStream_t s);
size_t cluster_propose_ws_bytes(int N, int N_c, int d);
hipError_t launch_cluster_index(const int32_t* cl_off, const int32_t* cl_tok, int N_c, int V, int32_t* tok_slot,
                                uint32_t* status, hipStream_t s);
hipError_t launch_cluster_propose(const ClusterArgs& a, hipStream_t s);

// schedule.hip
hipError_t launch_schedule(const float* c, int R, int gamma, const float* sps, int B_max,
                           int32_t* ell, double* a, int32_t* K_star, double* theta_star,
                           int32_t* K_hist, int32_t* K_used, uint32_t* status, hipStream_t s);
constexpr int SCHED_MAX_ENTRIES = 8192;

// Profiling hooks (api.cpp): bracket one kernel launch on stream s.
struct ProfScope {
    ProfScope(const char* name, hipStream_t s);
    ~ProfScope();
    int slot;
    hipStream_t stream;
};

}  // namespace spec
