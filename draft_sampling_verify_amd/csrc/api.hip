// api.hip -- extern "C" entry points of libspec (declared in include/spec.h):
// host-side argument validation, workspace carving and launch sequencing.
// Nothing here allocates device memory; every check happens before the
// first enqueue.
#include <math.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spec.h"
#include "../../include/spec_debug.h"
#include "common.h"
#include "internal.h"

namespace {

using spec::DraftArgs;

constexpr int MAX_R = 65536;
constexpr int MAX_GAMMA = 64;
constexpr int MAX_V = 1 << 24;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_draft(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0, int R,
                int gamma, int r, int V, float T)
{
    if (w_dtype != SPEC_F32 && w_dtype != SPEC_BF16) return SPEC_EDTYPE;
    if (R < 0 || gamma < 1 || V < 1 || r < 16 || (r % 16) != 0) return SPEC_EINVAL;
    if (!(T > 0.0f) || isinf(T)) return SPEC_EINVAL;
    if (R > MAX_R || gamma > MAX_GAMMA || V > MAX_V || r > 512) return SPEC_EUNSUPPORTED;
    if (w_dtype == SPEC_F32 && r > 256) return SPEC_EUNSUPPORTED;
    if ((double)R * (gamma + 1) * (double)V >= 1099511627776.0) return SPEC_EUNSUPPORTED;
    if (R > 0 && (!U || !W1 || !W2 || !x0)) return SPEC_EINVAL;
    if (R > 0 && (!aligned16(U) || !aligned16(W1) || !aligned16(W2))) return SPEC_EINVAL;
    return SPEC_OK;
}

DraftArgs make_args(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                    const int32_t* x, int R, int gamma, int r, int V, float T, int greedy, uint64_t seed,
                    uint64_t round, void* ws, int path = 0)
{
    DraftArgs a{};
    a.U = U; a.W1 = W1; a.W2 = W2; a.w_dtype = w_dtype; a.x0 = x0; a.x = x;
    a.R = R; a.gamma = gamma; a.r = r; a.V = V;
    // c = log2(e) / T rounded once to fp32; every exponential is 2^((z - m) c)
    a.c = (float)(1.4426950408889634 / (double)T);
    a.greedy = greedy != 0;
    a.seed = seed; a.round = round;
    a.status = reinterpret_cast<uint32_t*>(ws);
    a.path = path;
    return a;
}

bool path_ok(int path) { return (path & ~(SPEC_PATH_NO_FUSED_PROPOSE | SPEC_PATH_NO_PIPELINED_SWEEP)) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH; }

// Sizes of the clustered head the GPU path takes (everything but pointers).
int check_cluster(int R, int gamma, int d, int N_c, int K_c, int max_cl, int V, float T)
{
    if (R < 0 || gamma < 1 || V < 1 || d < 16 || (d % 16) != 0 || N_c < 1 || K_c < 1 || K_c > N_c || max_cl < 1)
        return SPEC_EINVAL;
    if (!(T > 0.0f) || isinf(T)) return SPEC_EINVAL;
    if (R > MAX_R || gamma > MAX_GAMMA || V > MAX_V || d > 16384 || N_c > spec::CL_MAX_NC || K_c > spec::CL_MAX_K ||
        max_cl > spec::CL_MAX_SIZE || (long)K_c * max_cl > 65536 || (long)R * gamma > (1L << 20))
        return SPEC_EUNSUPPORTED;
    if ((double)R * (gamma + 1) * (double)V >= 1099511627776.0) return SPEC_EUNSUPPORTED;
    return SPEC_OK;
}

// spec_decode_rounds lays its workspace out as [header | verify regions |
// propose regions | p_d(x) | (M, S)]: the propose's tagged hand-over words
// never share memory with the verify's data.
struct RoundsLayout {
    size_t propose_start, pd_x, pd_stats, end;
};
RoundsLayout rounds_layout(int R, int gamma, int V)
{
    RoundsLayout l{};
    spec::carve_verify(nullptr, R, gamma, V, false, &l.propose_start);
    size_t pe = 0;
    spec::carve_propose(nullptr, R, V, &pe, l.propose_start);
    l.pd_x = spec::align256(pe);
    l.pd_stats = l.pd_x + spec::align256((size_t)R * gamma * 4);
    l.end = l.pd_stats + spec::align256((size_t)R * gamma * 8);
    return l;
}

__global__ void k_copy_words(const int32_t* src, int32_t* dst, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Next anchor of every request: the token it emitted last.
__global__ void k_next_anchor(const int32_t* n_acc, const int32_t* y, int R, int gamma, int32_t* next)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= R) return;
    const int n = n_acc[i];
    next[i] = (n >= 0 && n <= gamma) ? y[(size_t)i * (gamma + 1) + n] : -1;
}

__global__ void k_philox_words(uint64_t seed, uint64_t round, size_t n, uint32_t* out)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const spec::u32x4 w = spec::philox((uint32_t)(i & 0xFFFFu), (uint32_t)(i >> 16), round, seed);
        reinterpret_cast<uint4*>(out)[i] = make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]);
    }
}

__global__ void k_zero_words(uint32_t* p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}


// ---- kernel timing records (spec_debug.h): off unless a benchmark turns
// them on; guarded by one mutex
struct ProfRecord {
    std::string name;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_records;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_event_pool;
size_t g_pool_used = 0;

}  // namespace

namespace spec {

ProfScope::ProfScope(const char* name, hipStream_t s) : slot(-1), stream(s)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    if (g_pool_used == g_event_pool.size()) {
        hipEvent_t a, b;
        // no system-scope fence: the events only timestamp work on this device
        if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
        if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
            hipEventDestroy(a);
            return;
        }
        g_event_pool.emplace_back(a, b);
    }
    auto ev = g_event_pool[g_pool_used++];
    if (hipEventRecord(ev.first, s) != hipSuccess) return;
    g_records.push_back(ProfRecord{name, ev.first, ev.second});
    slot = (int)g_records.size() - 1;
}

ProfScope::~ProfScope()
{
    if (slot < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (slot < (int)g_records.size()) hipEventRecord(g_records[slot].stop, stream);
}

}  // namespace spec

extern "C" {

size_t spec_workspace_bytes(int op, int R, int gamma, int r, int V, int B_max)
{
    size_t bytes = 0;
    switch (op) {
    case SPEC_OP_PROPOSE:
        if (check_draft(nullptr, nullptr, nullptr, SPEC_BF16, nullptr, 0, gamma, r, V, 1.0f) != SPEC_OK || R < 0 ||
            R > MAX_R)
            return 0;
        spec::carve_propose(nullptr, R, V, &bytes);
        return bytes;
    case SPEC_OP_VERIFY:
    case SPEC_OP_CONFIDENCE:
        if (check_draft(nullptr, nullptr, nullptr, SPEC_BF16, nullptr, 0, gamma, r, V, 1.0f) != SPEC_OK || R < 0 ||
            R > MAX_R)
            return 0;
        spec::carve_verify(nullptr, R, gamma, V, op == SPEC_OP_CONFIDENCE, &bytes);
        return bytes;
    case SPEC_OP_ROUNDS:
        if (check_draft(nullptr, nullptr, nullptr, SPEC_BF16, nullptr, 0, gamma, r, V, 1.0f) != SPEC_OK || R < 0 ||
            R > MAX_R)
            return 0;
        return rounds_layout(R, gamma, V).end;
    case SPEC_OP_LOSS:
        if (check_draft(nullptr, nullptr, nullptr, SPEC_BF16, nullptr, 0, gamma, r, V, 1.0f) != SPEC_OK || R < 0 ||
            R > MAX_R)
            return 0;
        spec::carve_verify(nullptr, R, gamma, V, true, &bytes, true);
        return bytes;
    case SPEC_OP_SCHEDULE:
        if (R < 1 || gamma < 1 || (long)R * gamma > spec::SCHED_MAX_ENTRIES || B_max < R) return 0;
        return spec::WS_HEADER;
    default:
        return 0;
    }
}

size_t spec_cluster_workspace_bytes(int R, int gamma, int d, int N_c, int K_c, int max_cl, int V)
{
    if (check_cluster(R, gamma, d, N_c, K_c, max_cl, V, 1.0f) != SPEC_OK) return 0;
    size_t vb = 0;
    spec::carve_verify(nullptr, R, gamma, V, false, &vb);
    const size_t pb = spec::cluster_propose_ws_bytes(R * gamma, N_c, d);
    return pb > vb ? pb : vb;
}

int spec_cluster_index(const int32_t* cl_off, const int32_t* cl_tok, int N_c, int V, int32_t* tok_slot, void* ws,
                       size_t ws_bytes, spec_stream_t stream)
{
    if (N_c < 1 || V < 1 || !cl_off || !cl_tok || !tok_slot) return SPEC_EINVAL;
    if (N_c > spec::CL_MAX_NC || V > MAX_V) return SPEC_EUNSUPPORTED;
    if (!ws || ws_bytes < spec::WS_HEADER) return SPEC_EWORKSPACE;
    return launch_status(spec::launch_cluster_index(cl_off, cl_tok, N_c, V, tok_slot, reinterpret_cast<uint32_t*>(ws),
                                                    (hipStream_t)stream));
}

int spec_cluster_propose(const void* H, const void* C, const void* E, int w_dtype, const int32_t* cl_off,
                         const int32_t* cl_tok, int R, int gamma, int d, int N_c, int K_c, int max_cl, int V, float T,
                         int greedy, uint64_t seed, uint64_t round, int32_t* x, float* pd_x, int32_t* sel, float* zf,
                         float* pd_stats, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    if (w_dtype != SPEC_F32 && w_dtype != SPEC_BF16) return SPEC_EDTYPE;
    int st = check_cluster(R, gamma, d, N_c, K_c, max_cl, V, T);
    if (st != SPEC_OK) return st;
    if (w_dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
    if (R > 0 && (!H || !C || !E || !cl_off || !cl_tok || !x || !pd_x || !sel || !zf || !pd_stats))
        return SPEC_EINVAL;
    if (R > 0 && (!aligned16(H) || !aligned16(C) || !aligned16(E))) return SPEC_EINVAL;
    if (!ws || ws_bytes < spec_cluster_workspace_bytes(R, gamma, d, N_c, K_c, max_cl, V)) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    spec::ClusterArgs a{};
    a.H = H; a.C = C; a.E = E; a.cl_off = cl_off; a.cl_tok = cl_tok;
    a.R = R; a.gamma = gamma; a.d = d; a.N_c = N_c; a.K_c = K_c; a.max_cl = max_cl; a.V = V;
    a.c = (float)(1.4426950408889634 / (double)T);
    a.greedy = greedy != 0; a.seed = seed; a.round = round;
    a.x = x; a.pd_x = pd_x; a.sel = sel; a.zf = zf; a.pd_stats = pd_stats;
    a.ws = ws; a.status = reinterpret_cast<uint32_t*>(ws);
    return launch_status(spec::launch_cluster_propose(a, (hipStream_t)stream));
}

int spec_cluster_verify(const int32_t* tok_slot, const int32_t* sel, const float* zf, const float* pd_stats,
                        const int32_t* x, const float* Lt, const int32_t* ell, int R, int gamma, int N_c, int K_c,
                        int max_cl, int V, float T, int greedy, uint64_t seed, uint64_t round, int32_t* n_acc,
                        int32_t* y, float* pt_x, float* c_star, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    int st = check_cluster(R, gamma, 16, N_c, K_c, max_cl, V, T);
    if (st != SPEC_OK) return st;
    if (R > 0 && (!tok_slot || !sel || !zf || !pd_stats || !x || !Lt || !n_acc || !y)) return SPEC_EINVAL;
    if (R > 0 && !aligned16(Lt)) return SPEC_EINVAL;
    size_t need = 0;
    spec::carve_verify(nullptr, R, gamma, V, false, &need);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    const spec::VerifyWs w = spec::carve_verify(ws, R, gamma, V, false, nullptr);
    spec::ClusterVerifyArgs cv{};
    cv.tok_slot = tok_slot; cv.sel = sel; cv.zf = zf; cv.pd_stats = pd_stats; cv.x = x; cv.Lt = Lt; cv.ell = ell;
    cv.R = R; cv.gamma = gamma; cv.N_c = N_c; cv.K_c = K_c; cv.max_cl = max_cl; cv.V = V;
    cv.c = (float)(1.4426950408889634 / (double)T);
    cv.greedy = greedy != 0; cv.seed = seed; cv.round = round;
    cv.n_acc = n_acc; cv.y = y; cv.pt_x = pt_x; cv.c_star = c_star;
    cv.status = reinterpret_cast<uint32_t*>(ws);
    return launch_status(spec::launch_cluster_verify(cv, w, (hipStream_t)stream));
}

int spec_workspace_init(void* ws, size_t ws_bytes, spec_stream_t stream)
{
    if (!ws || ws_bytes < spec::WS_HEADER) return SPEC_EWORKSPACE;
    // the whole workspace: the status word, the call counter of the fused
    // propose and its hand-over words (0 is never a valid tag)
    const size_t words = ws_bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(k_zero_words, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ws, words);
    return launch_status(hipGetLastError());
}

size_t spec_packed_w2_bytes(int w_dtype, int r, int V)
{
    if (check_draft(nullptr, nullptr, nullptr, w_dtype, nullptr, 0, 1, r, V, 1.0f) != SPEC_OK) return 0;
    return spec::packed_w2_bytes(w_dtype, r, V);
}

int spec_pack_w2(const void* W2, int w_dtype, int r, int V, void* W2p, spec_stream_t stream)
{
    int st = check_draft(nullptr, nullptr, nullptr, w_dtype, nullptr, 0, 1, r, V, 1.0f);
    if (st != SPEC_OK) return st;
    if (!W2 || !W2p || !aligned16(W2) || !aligned16(W2p)) return SPEC_EINVAL;
    return launch_status(spec::launch_pack_w2(W2, w_dtype, r, V, W2p, false, (hipStream_t)stream));
}

int spec_pack_w2_rv(const void* W2_rv, int w_dtype, int r, int V, void* W2p, spec_stream_t stream)
{
    int st = check_draft(nullptr, nullptr, nullptr, w_dtype, nullptr, 0, 1, r, V, 1.0f);
    if (st != SPEC_OK) return st;
    if (!W2_rv || !W2p || !aligned16(W2p)) return SPEC_EINVAL;
    return launch_status(spec::launch_pack_w2(W2_rv, w_dtype, r, V, W2p, true, (hipStream_t)stream));
}

int spec_device_status(void* ws, spec_stream_t stream, int clear, int* flags)
{
    if (!ws || !flags) return SPEC_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, ws, sizeof word, hipMemcpyDeviceToHost, s) != hipSuccess) return SPEC_ELAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return SPEC_ELAUNCH;
    *flags = (int)word;
    if (clear) {
        hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, s, (uint32_t*)ws, (size_t)1);
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    }
    return word ? SPEC_EDEVICE : SPEC_OK;
}

namespace {

// propose with its regions starting at `start` (after the header, or after
// the verify regions in spec_decode_rounds)
int propose_at(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0, int R, int gamma,
               int r, int V, float T, int greedy, uint64_t seed, uint64_t round, int32_t* x, float* pd_x,
               float* pd_stats, int path, void* ws, size_t ws_bytes, size_t start, spec_stream_t stream)
{
    int st = check_draft(U, W1, W2, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (!path_ok(path)) return SPEC_EINVAL;
    if (R > 0 && (!x || !pd_x || !pd_stats)) return SPEC_EINVAL;
    size_t need = 0;
    spec::carve_propose(nullptr, R, V, &need, start);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    const spec::ProposeWs w = spec::carve_propose(ws, R, V, nullptr, start);
    DraftArgs a = make_args(U, W1, W2, w_dtype, x0, x, R, gamma, r, V, T, greedy, seed, round, ws, path);
    return launch_status(spec::launch_propose(a, x, pd_x, pd_stats, w, (hipStream_t)stream));
}

}  // namespace

int spec_markov_propose_ex(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0, int R,
                           int gamma, int r, int V, float T, int greedy, uint64_t seed, uint64_t round, int32_t* x,
                           float* pd_x, float* pd_stats, int path, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    return propose_at(U, W1, W2, w_dtype, x0, R, gamma, r, V, T, greedy, seed, round, x, pd_x, pd_stats, path, ws,
                      ws_bytes, spec::WS_HEADER, stream);
}

// ---- spec_markov_propose_noalloc: the workspace in a static device array
//
// `scratch` is a host-side stand-in in host code: its device address on the
// current GPU comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[SPEC_NOALLOC_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEV = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[NOALLOC_MAX_DEV];    // device address of `scratch` per device (null: not yet set up)
bool g_noalloc_zeroed[NOALLOC_MAX_DEV];  // the zero fill has been enqueued on this device

// The current device's scratch address; on the first call on a device, look
// it up and enqueue the one zero fill of the whole array (the status word,
// the fused propose's call counter and hand-over words start at zero).
int noalloc_scratch(hipStream_t s, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEV) return SPEC_ELAUNCH;
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SPEC_ELAUNCH;
        g_noalloc_ptr[dev] = ptr;
    }
    if (!g_noalloc_zeroed[dev]) {
        const size_t words = SPEC_NOALLOC_BYTES / 4;
        hipLaunchKernelGGL(k_zero_words, dim3(1024), dim3(256), 0, s, (uint32_t*)g_noalloc_ptr[dev], words);
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
        g_noalloc_zeroed[dev] = true;
    }
    *out = g_noalloc_ptr[dev];
    return SPEC_OK;
}
}  // namespace

int spec_markov_propose_noalloc(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                                int R, int gamma, int r, int V, float T, int greedy, uint64_t seed, uint64_t round,
                                int32_t* x, float* pd_x, float* pd_stats, uint32_t* flags, spec_stream_t stream)
{
    int st = check_draft(U, W1, W2, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (R > 0 && (!x || !pd_x || !pd_stats || !flags)) return SPEC_EINVAL;
    const size_t need = spec_workspace_bytes(SPEC_OP_PROPOSE, R, gamma, r, V, 0);
    if (need == 0) return SPEC_EINVAL;
    if (need > SPEC_NOALLOC_BYTES) return SPEC_EUNSUPPORTED;
    if (R == 0) return SPEC_OK;
    hipStream_t s = (hipStream_t)stream;
    void* ptr = nullptr;
    st = noalloc_scratch(s, &ptr);
    if (st != SPEC_OK) return st;
    // this call's status bits start clear (a fill kernel: graph-capturable)
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, s, (uint32_t*)ptr, (size_t)1);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    st = propose_at(U, W1, W2, w_dtype, x0, R, gamma, r, V, T, greedy, seed, round, x, pd_x, pd_stats,
                    SPEC_PATH_AUTO, ptr, SPEC_NOALLOC_BYTES, spec::WS_HEADER, stream);
    if (st != SPEC_OK) return st;
    hipLaunchKernelGGL(k_copy_words, dim3(1), dim3(64), 0, s, (const int32_t*)ptr, (int32_t*)flags, 1);
    return launch_status(hipGetLastError());
}

int spec_markov_propose(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0, int R,
                        int gamma, int r, int V, float T, int greedy, uint64_t seed, uint64_t round, int32_t* x,
                        float* pd_x, float* pd_stats, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    return spec_markov_propose_ex(U, W1, W2, w_dtype, x0, R, gamma, r, V, T, greedy, seed, round, x, pd_x, pd_stats,
                                  SPEC_PATH_AUTO, ws, ws_bytes, stream);
}

int spec_verify(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0, const int32_t* x,
                const float* pd_stats, const float* Lt, const int32_t* ell, int R, int gamma, int r, int V, float T,
                int greedy, uint64_t seed, uint64_t round, int32_t* n_acc, int32_t* y, float* pt_x, float* c_star,
                void* ws, size_t ws_bytes, spec_stream_t stream)
{
    return spec_verify_ex(U, W1, W2, w_dtype, x0, x, pd_stats, Lt, ell, R, gamma, r, V, T, greedy, seed, round,
                          n_acc, y, pt_x, c_star, SPEC_PATH_AUTO, ws, ws_bytes, stream);
}

int spec_verify_ex(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                   const int32_t* x, const float* pd_stats, const float* Lt, const int32_t* ell, int R, int gamma,
                   int r, int V, float T, int greedy, uint64_t seed, uint64_t round, int32_t* n_acc, int32_t* y,
                   float* pt_x, float* c_star, int path, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    int st = check_draft(U, W1, W2, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (!path_ok(path)) return SPEC_EINVAL;
    if (R > 0 && (!x || !pd_stats || !Lt || !n_acc || !y)) return SPEC_EINVAL;
    if (R > 0 && !aligned16(Lt)) return SPEC_EINVAL;
    size_t need = 0;
    spec::carve_verify(nullptr, R, gamma, V, false, &need);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    const spec::VerifyWs w = spec::carve_verify(ws, R, gamma, V, false, nullptr);
    DraftArgs a = make_args(U, W1, W2, w_dtype, x0, x, R, gamma, r, V, T, greedy, seed, round, ws, path);
    int32_t* counts = reinterpret_cast<spec::WsHeader*>(ws)->counts;
    return launch_status(
        spec::launch_verify(a, pd_stats, Lt, ell, n_acc, y, pt_x, c_star, w, counts, (hipStream_t)stream));
}

int spec_confidence(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                    const int32_t* x, const float* pd_stats, const float* Lt, int R, int gamma, int r, int V,
                    float T, float* c_star, double* a_star, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    return spec_confidence_ex(U, W1, W2, w_dtype, x0, x, pd_stats, Lt, R, gamma, r, V, T, c_star, a_star,
                              SPEC_PATH_AUTO, ws, ws_bytes, stream);
}

int spec_confidence_ex(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                       const int32_t* x, const float* pd_stats, const float* Lt, int R, int gamma, int r, int V,
                       float T, float* c_star, double* a_star, int path, void* ws, size_t ws_bytes,
                       spec_stream_t stream)
{
    int st = check_draft(U, W1, W2, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (!path_ok(path)) return SPEC_EINVAL;
    if (R > 0 && (!x || !Lt || !c_star)) return SPEC_EINVAL;
    if (R > 0 && !aligned16(Lt)) return SPEC_EINVAL;
    size_t need = 0;
    spec::carve_verify(nullptr, R, gamma, V, true, &need);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    const spec::VerifyWs w = spec::carve_verify(ws, R, gamma, V, true, nullptr);
    DraftArgs a = make_args(U, W1, W2, w_dtype, x0, x, R, gamma, r, V, T, 0, 0, 0, ws, path);
    return launch_status(
        spec::launch_confidence(a, pd_stats, Lt, c_star, a_star, w, (hipStream_t)stream));
}

int spec_draft_loss(const float* U, const void* W1, const void* W2, int w_dtype, const int32_t* x0,
                    const int32_t* y, const float* Lt, const float* q, int R, int gamma, int r, int V, float T,
                    float a_ce, float a_tv, float a_conf, double* loss, float* terms, float* dq, void* ws,
                    size_t ws_bytes, spec_stream_t stream)
{
    int st = check_draft(U, W1, W2, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (!loss || !std::isfinite(a_ce) || !std::isfinite(a_tv) || !std::isfinite(a_conf)) return SPEC_EINVAL;
    if (R > 0 && (!y || !Lt || !q)) return SPEC_EINVAL;
    if (R > 0 && !aligned16(Lt)) return SPEC_EINVAL;
    const size_t need = spec_workspace_bytes(SPEC_OP_LOSS, R, gamma, r, V, 0);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_EINVAL;  // the mean over no positions is undefined
    const spec::VerifyWs w = spec::carve_verify(ws, R, gamma, V, true, nullptr, true);
    DraftArgs a = make_args(U, W1, W2, w_dtype, x0, y, R, gamma, r, V, T, 0, 0, 0, ws);
    spec::LossArgs l{};
    l.q = q;
    l.invT = (float)(1.0 / (double)T);
    l.a_ce = a_ce; l.a_tv = a_tv; l.a_conf = a_conf;
    l.loss = loss; l.terms = terms; l.dq = dq;
    return launch_status(spec::launch_draft_loss(a, Lt, l, w, (hipStream_t)stream));
}

int spec_decode_rounds(const float* U, const void* W1, const void* W2p, int w_dtype, const int32_t* x0,
                       const float* Lt, int R, int gamma, int r, int V, float T, int greedy, uint64_t seed,
                       uint64_t round0, int n_rounds, int32_t* anchors, int32_t* x, int32_t* n_acc, int32_t* y,
                       float* c_star, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    return spec_decode_rounds_ex(U, W1, W2p, w_dtype, x0, Lt, R, gamma, r, V, T, greedy, seed, round0, n_rounds,
                                 anchors, x, n_acc, y, c_star, SPEC_PATH_AUTO, ws, ws_bytes, stream);
}

int spec_decode_rounds_ex(const float* U, const void* W1, const void* W2p, int w_dtype, const int32_t* x0,
                          const float* Lt, int R, int gamma, int r, int V, float T, int greedy, uint64_t seed,
                          uint64_t round0, int n_rounds, int32_t* anchors, int32_t* x, int32_t* n_acc, int32_t* y,
                          float* c_star, int path, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    int st = check_draft(U, W1, W2p, w_dtype, x0, R, gamma, r, V, T);
    if (st != SPEC_OK) return st;
    if (n_rounds < 1 || !path_ok(path)) return SPEC_EINVAL;
    if (R > 0 && (!Lt || !anchors || !x || !n_acc || !y)) return SPEC_EINVAL;
    if (R > 0 && !aligned16(Lt)) return SPEC_EINVAL;
    const size_t need = spec_workspace_bytes(SPEC_OP_ROUNDS, R, gamma, r, V, 0);
    if (!ws || ws_bytes < need) return SPEC_EWORKSPACE;
    if (R == 0) return SPEC_OK;
    const RoundsLayout lay = rounds_layout(R, gamma, V);
    float* pd_x = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.pd_x);
    float* pd_stats = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.pd_stats);
    hipStream_t s = (hipStream_t)stream;
    const int nb = (R + 255) / 256;
    hipLaunchKernelGGL(k_copy_words, dim3(nb), dim3(256), 0, s, x0, anchors, R);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    for (int i = 0; i < n_rounds; ++i) {
        const int32_t* a_i = anchors + (size_t)i * R;
        int32_t* x_i = x + (size_t)i * R * gamma;
        int32_t* n_i = n_acc + (size_t)i * R;
        int32_t* y_i = y + (size_t)i * R * (gamma + 1);
        float* c_i = c_star ? c_star + (size_t)i * R * gamma : nullptr;
        st = propose_at(U, W1, W2p, w_dtype, a_i, R, gamma, r, V, T, greedy, seed, round0 + i, x_i, pd_x, pd_stats,
                        path, ws, ws_bytes, lay.propose_start, stream);
        if (st != SPEC_OK) return st;
        st = spec_verify_ex(U, W1, W2p, w_dtype, a_i, x_i, pd_stats, Lt, nullptr, R, gamma, r, V, T, greedy, seed,
                            round0 + i, n_i, y_i, nullptr, c_i, path, ws, ws_bytes, stream);
        if (st != SPEC_OK) return st;
        hipLaunchKernelGGL(k_next_anchor, dim3(nb), dim3(256), 0, s, n_i, y_i, R, gamma,
                           anchors + (size_t)(i + 1) * R);
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    }
    return SPEC_OK;
}

int spec_schedule(const float* c, int R, int gamma, const float* sps, int B_max, int32_t* ell, double* a,
                  int32_t* K_star, double* theta_star, void* ws, size_t ws_bytes, spec_stream_t stream)
{
    if (R < 1 || gamma < 1 || B_max < R) return SPEC_EINVAL;
    if ((long)R * gamma > spec::SCHED_MAX_ENTRIES) return SPEC_EUNSUPPORTED;
    if (!c || !sps || !ell || !K_star || !theta_star) return SPEC_EINVAL;
    if (!ws || ws_bytes < spec::WS_HEADER) return SPEC_EWORKSPACE;
    return launch_status(spec::launch_schedule(c, R, gamma, sps, B_max, ell, a, K_star, theta_star, nullptr,
                                               nullptr, reinterpret_cast<uint32_t*>(ws), (hipStream_t)stream));
}

int spec_schedule_async(const float* c, int R, int gamma, const float* sps, int B_max, int32_t* K_hist,
                        int32_t* ell, double* a, int32_t* K_used, int32_t* K_star, double* theta_star, void* ws,
                        size_t ws_bytes, spec_stream_t stream)
{
    if (R < 1 || gamma < 1 || B_max < R) return SPEC_EINVAL;
    if ((long)R * gamma > spec::SCHED_MAX_ENTRIES) return SPEC_EUNSUPPORTED;
    if (!c || !sps || !K_hist || !ell || !K_used || !K_star || !theta_star) return SPEC_EINVAL;
    if (!ws || ws_bytes < spec::WS_HEADER) return SPEC_EWORKSPACE;
    return launch_status(spec::launch_schedule(c, R, gamma, sps, B_max, ell, a, K_star, theta_star, K_hist,
                                               K_used, reinterpret_cast<uint32_t*>(ws), (hipStream_t)stream));
}

const char* spec_status_str(int status)
{
    switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EDTYPE: return "unknown weight dtype";
    case SPEC_EWORKSPACE: return "workspace missing or too small";
    case SPEC_ELAUNCH: return "HIP launch error";
    case SPEC_EDEVICE: return "a kernel saw invalid device data (token, length or confidence)";
    case SPEC_EUNSUPPORTED: return "size outside the supported limits";
    default: return "unknown status";
    }
}

int spec_philox_words(uint64_t seed, uint64_t round, size_t n, uint32_t* out, void* stream)
{
    if (!out || n > ((size_t)1 << 32)) return SPEC_EINVAL;
    if (n == 0) return SPEC_OK;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(k_philox_words, dim3(blocks), dim3(256), 0, (hipStream_t)stream, seed, round, n, out);
    return launch_status(hipGetLastError());
}

int spec_profile_enable(int on)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
    return SPEC_OK;
}

int spec_profile_reset(void)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_records.clear();
    g_pool_used = 0;
    return SPEC_OK;
}

int spec_profile_read(const char* kernel, int* launches, double* total_ms)
{
    if (!kernel || !launches || !total_ms) return SPEC_EINVAL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    int n = 0;
    double tot = 0.0;
    for (const ProfRecord& rec : g_records) {
        if (rec.name != kernel) continue;
        if (hipEventSynchronize(rec.stop) != hipSuccess) return SPEC_ELAUNCH;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, rec.start, rec.stop) != hipSuccess) return SPEC_ELAUNCH;
        tot += ms;
        ++n;
    }
    *launches = n;
    *total_ms = tot;
    return SPEC_OK;
}

int spec_profile_names(char* buf, int buf_len)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::string all;
    for (const ProfRecord& rec : g_records) {
        const std::string key = "," + rec.name + ",";
        if (("," + all + ",").find(key) == std::string::npos) all += (all.empty() ? "" : ",") + rec.name;
    }
    if (buf && buf_len > 0) {
        strncpy(buf, all.c_str(), (size_t)buf_len - 1);
        buf[buf_len - 1] = '\0';
    }
    return (int)all.size() + 1;
}

}  // extern "C"
