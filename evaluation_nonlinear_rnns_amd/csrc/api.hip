// C entry points of libdeer (declared in include/deer.h): argument checks,
// workspace layout, the device-driven Newton loop and error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace deer {

// ------------------------------------------------------------------ errors
namespace {
thread_local std::string g_last_error = "no error";
}

void set_error(const std::string &msg) { g_last_error = msg; }

int fail(int code, const std::string &msg)
{
    set_error(msg);
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    set_error(std::string("HIP error ") + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ") in " + what);
    return DEER_ERR_HIP;
}

// --------------------------------------------------------------- profiling
thread_local ProfLaunch g_prof_launch;

namespace {
constexpr int kProfKinds = 4;
std::atomic<int> g_prof_enabled{0};
std::mutex g_prof_mu;
long long g_prof_launches[kProfKinds] = {0, 0, 0, 0};
double g_prof_ms[kProfKinds] = {0, 0, 0, 0};

// Timing events are reused across calls (one pool per host thread and
// device, since an event belongs to the device that was current when it was
// created): creating and destroying two events per launch cost more host time
// than the launch.
constexpr int kPoolDevices = 64;
thread_local std::vector<hipEvent_t> g_event_pool[kPoolDevices];

std::vector<hipEvent_t> *event_pool()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kPoolDevices) return nullptr;
    return &g_event_pool[dev];
}

bool pool_event(hipEvent_t *e)
{
    std::vector<hipEvent_t> *pool = event_pool();
    if (pool && !pool->empty()) {
        *e = pool->back();
        pool->pop_back();
        return true;
    }
    return hipEventCreate(e) == hipSuccess;
}

void unpool_event(hipEvent_t e)
{
    if (!e) return;
    std::vector<hipEvent_t> *pool = event_pool();
    if (pool) pool->push_back(e);
    else (void)hipEventDestroy(e);
}

// Event pairs recorded around launches of one deer_solve call.
struct ProfScope {
    bool on = false;
    hipStream_t stream = nullptr;
    std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> marks;
    int open_kind = -1;
    hipEvent_t open_start = nullptr;

    explicit ProfScope(hipStream_t s) : on(g_prof_enabled.load() != 0), stream(s) {}
    // The launches between begin and end record the pair themselves (DEER_LAUNCH).
    void begin(int kind)
    {
        if (!on) return;
        hipEvent_t e0, e1;
        if (!pool_event(&e0)) { on = false; return; }
        if (!pool_event(&e1)) { unpool_event(e0); on = false; return; }
        open_kind = kind;
        open_start = e0;
        g_prof_launch = ProfLaunch{e0, e1};
    }
    void end()
    {
        if (!on || open_kind < 0) return;
        marks.push_back({open_kind, {open_start, g_prof_launch.stop}});
        g_prof_launch = ProfLaunch{};
        open_kind = -1;
    }
    // Call after the stream has been synchronised.  Only the first limit[k]
    // launches of each kind did work; launches enqueued after convergence exit
    // at once and are not counted.
    void collect(const long long limit[kProfKinds])
    {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        long long seen[kProfKinds] = {0, 0, 0, 0};
        for (auto &m : marks) {
            if (seen[m.first]++ >= limit[m.first]) continue;
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, m.second.first, m.second.second) == hipSuccess) {
                g_prof_launches[m.first] += 1;
                g_prof_ms[m.first] += ms;
            }
        }
        release();
    }
    // Events go back to the pool only once the stream has passed them: after
    // collect() (stream synchronised) or, on an error path, after a
    // synchronisation here, so a pooled event is never re-recorded while pending.
    void release()
    {
        for (auto &m : marks) {
            unpool_event(m.second.first);
            unpool_event(m.second.second);
        }
        marks.clear();
    }
    ~ProfScope()
    {
        if (!marks.empty() || open_kind >= 0) (void)hipStreamSynchronize(stream);
        if (open_kind >= 0) {                    // a scope left open by an error return
            unpool_event(open_start);
            unpool_event(g_prof_launch.stop);
        }
        g_prof_launch = ProfLaunch{};
        release();
    }
};

// Pinned host words for polling the device's all-done flag, one set per host thread.
struct PollSlots {
    int *host = nullptr;
    PollSlots()
    {
        if (hipHostMalloc(reinterpret_cast<void **>(&host), 64 * sizeof(int), hipHostMallocDefault) != hipSuccess)
            host = nullptr;
    }
};
thread_local PollSlots g_poll;

// Pinned staging for the per-sequence results read back at the end of a solve
// (copies into pageable memory take tens of microseconds each); one buffer
// per host thread, grown on demand, reused only after the stream has been
// synchronised.
struct ResultStage {
    char *host = nullptr;
    size_t cap = 0;
    char *get(size_t bytes)
    {
        if (bytes <= cap) return host;
        if (host) (void)hipHostFree(host);
        host = nullptr;
        cap = 0;
        if (hipHostMalloc(reinterpret_cast<void **>(&host), bytes, hipHostMallocDefault) != hipSuccess) {
            host = nullptr;
            return nullptr;
        }
        cap = bytes;
        return host;
    }
};
thread_local ResultStage g_stage;

// Iteration counts, residuals, statuses and (when abort_dev is set) the
// look-back abort word: enqueued into the pinned stage, one stream
// synchronisation, then copied to the caller's host arrays.
int read_results(const int *iters_dev, const int *status_dev, const float *resid_dev, const unsigned *abort_dev,
                 int B, hipStream_t stream, int *iters_out, float *resid_out, std::vector<int> &status_h,
                 unsigned &abort_flag, const char *who)
{
    const size_t need = (2 * sizeof(int) + sizeof(float)) * static_cast<size_t>(B) + sizeof(unsigned);
    char *st = g_stage.get(need);
    if (!st) {
        (void)hipStreamSynchronize(stream);
        return fail(DEER_ERR_HIP, std::string(who) + ": pinned host memory unavailable");
    }
    int *h_iters = reinterpret_cast<int *>(st);
    int *h_status = h_iters + B;
    float *h_resid = reinterpret_cast<float *>(h_status + B);
    unsigned *h_abort = reinterpret_cast<unsigned *>(h_resid + B);
    *h_abort = 0u;
    int rc = DEER_OK;
    if (hipMemcpyAsync(h_iters, iters_dev, sizeof(int) * B, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(h_status, status_dev, sizeof(int) * B, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        (resid_out && hipMemcpyAsync(h_resid, resid_dev, sizeof(float) * B, hipMemcpyDeviceToHost, stream) != hipSuccess) ||
        (abort_dev && hipMemcpyAsync(h_abort, abort_dev, sizeof(unsigned), hipMemcpyDeviceToHost, stream) != hipSuccess))
        rc = fail(DEER_ERR_HIP, std::string(who) + ": result copy failed");
    const hipError_t se = hipStreamSynchronize(stream);
    if (se != hipSuccess && rc == DEER_OK) rc = hip_fail(se, (std::string("hipStreamSynchronize(") + who + ")").c_str());
    if (rc) return rc;
    std::memcpy(iters_out, h_iters, sizeof(int) * B);
    if (resid_out) std::memcpy(resid_out, h_resid, sizeof(float) * B);
    status_h.assign(h_status, h_status + B);
    abort_flag = *h_abort;
    return DEER_OK;
}

// ------------------------------------------------------ small device kernels
__global__ void init_control_kernel(SolveControl *ctl, int *done, int *iters, int *status, float *resid,
                                    unsigned *res_bits, int B)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) { ctl->iter = 0; ctl->all_done = 0; }
    if (i < B) { done[i] = 0; iters[i] = 0; status[i] = 0; resid[i] = 0.0f; res_bits[i] = 0u; }
}

__global__ void fill_kernel(float *__restrict__ p, size_t n, float v)
{
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__global__ void copy_kernel(float *__restrict__ dst, const float *__restrict__ src, size_t n)
{
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) dst[i] = src[i];
}

__global__ void zero_words_kernel(unsigned *__restrict__ p, size_t nwords)
{
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < nwords; i += stride) p[i] = 0u;
}

// Convergence test of the current iteration (see finalize_iteration).
__global__ void check_kernel(SolveControl *ctl, unsigned *res_bits, const unsigned *res_tile, int tps, int *done,
                             int *iters, int *status, float *resid, int B, float tol, int max_iter)
{
    __shared__ unsigned red[256 / 64];
    if (ctl->all_done) return;
    finalize_iteration(ctl, res_bits, res_tile, tps, done, iters, status, resid, B, tol, max_iter, red);
}

// Sequences whose final iterate sits in the second buffer are copied out.  With
// zero_start, traj was never written for sequences that stopped at iteration
// 0; their iterate is the all-zero start.
__global__ void gather_kernel(float *__restrict__ traj, const float *__restrict__ buf1, const int *__restrict__ iters,
                              size_t per_seq, int B, int zero_start)
{
    const int bseq = blockIdx.y;
    if (bseq >= B) return;
    const int it = iters[bseq];
    const bool copy = (it & 1) != 0, zero = zero_start && it == 0;
    if (!copy && !zero) return;
    const size_t base = static_cast<size_t>(bseq) * per_seq;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < per_seq;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        traj[base + i] = copy ? buf1[base + i] : 0.0f;
}

unsigned grid_for(size_t n, unsigned threads = 256, unsigned cap = 8192)
{
    size_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return static_cast<unsigned>(g);
}

// ------------------------------------------------------ argument checks
int check_cell(const deer_cell_params_t *p, int mode_flags)
{
    const int mode = mode_flags & ~(DEER_SCAN_F64 | DEER_MULTI_LAUNCH);
    if ((mode_flags & DEER_SCAN_F64) && mode != DEER_MODE_DENSE)
        return fail(DEER_ERR_UNSUPPORTED, "DEER_SCAN_F64 applies to dense mode only");
    if (!p) return fail(DEER_ERR_INVALID, "cell parameters: null pointer");
    if (p->cell != DEER_CELL_TANH && p->cell != DEER_CELL_GRU)
        return fail(DEER_ERR_INVALID, "cell parameters: unknown cell " + std::to_string(p->cell));
    if (mode < DEER_MODE_DENSE || mode > DEER_MODE_PICARD)
        return fail(DEER_ERR_INVALID, "unknown mode " + std::to_string(mode));
    if (p->D < 1 || p->D > kMaxD)
        return fail(DEER_ERR_UNSUPPORTED, "state size D=" + std::to_string(p->D) + " outside 1..64");
    if (p->M < 1 || p->M > kMaxM)
        return fail(DEER_ERR_UNSUPPORTED, "input size M=" + std::to_string(p->M) + " outside 1..1024");
    if (p->cell == DEER_CELL_GRU && mode == DEER_MODE_DENSE)
        return fail(DEER_ERR_UNSUPPORTED, "the GRU cell has no dense mode (diag, Jacobi and Picard are supported)");
    if (!p->W || !p->U) return fail(DEER_ERR_INVALID, "cell parameters: W and U are required");
    return DEER_OK;
}

int check_sizes(int B, int T)
{
    if (B < 0 || T < 0) return fail(DEER_ERR_INVALID, "negative batch or length");
    if (static_cast<long long>(B) * T > (1ll << 31))
        return fail(DEER_ERR_UNSUPPORTED, "B*T above 2^31 positions");
    return DEER_OK;
}

// The diagonal-block modes (diag, Jacobi, Picard) solve with the diagonal scan.
bool diag_blocks(int mode) { return mode != DEER_MODE_DENSE; }

// The GRU in a diagonal-block mode at D = 32 / 64 runs one fused evaluation +
// scan launch per iteration; everything else runs evaluation and scan as two
// launches.
bool fused_gru_step(const deer_cell_params_t *p, int mode)
{
    return p->cell == DEER_CELL_GRU && diag_blocks(mode) && gru_fast_path(p->D, p->M);
}

// Layout of the deer_solve workspace.
struct SolveLayout {
    void *scan = nullptr;       // scan state (diag: look-back header + descriptors; dense: chunk aggregates)
    SolveControl *ctl = nullptr;
    unsigned *res_bits = nullptr;
    unsigned *res_tile = nullptr;  // per-tile residual maxima (fused GRU step)
    int tps = 0;                   // tiles per sequence for res_tile
    int *done = nullptr, *iters = nullptr, *status = nullptr;
    float *resid = nullptr;
    float *buf1 = nullptr;      // second trajectory buffer [B,T,D]
    float *lin = nullptr;       // a_t (diag) or d_t (dense, factored leaf) [B,T,D]
    float *bvec = nullptr;      // b_t [B,T,D]
    float *proj = nullptr;      // input projection [B,T,PD]
    size_t bytes = 0;
};

SolveLayout solve_layout(void *ws, const deer_cell_params_t *p, int B, int T, int mode_flags)
{
    const int mode = mode_flags & ~(DEER_SCAN_F64 | DEER_MULTI_LAUNCH);
    const bool f64 = (mode_flags & DEER_SCAN_F64) != 0;
    const size_t BTD = static_cast<size_t>(B) * T * p->D;
    const int PD = (p->cell == DEER_CELL_GRU) ? 3 * p->D : p->D;
    Carve c(ws);
    SolveLayout L;
    // the scan state comes first so that its header keeps a fixed place
    const bool fused = fused_gru_step(p, mode);
    const size_t scan_bytes = fused ? gru_step_state_bytes(B, T, p->D)
                              : diag_blocks(mode) ? diag_scan_state_bytes(B, T, p->D)
                                                         : dense_scan_state_bytes(B, T, p->D, f64);
    L.scan = c.take<char>(scan_bytes);
    L.ctl = c.take<SolveControl>(1);
    L.res_bits = c.take<unsigned>(B);
    if (fused) {
        L.tps = (T + gru_step_tile(p->D) - 1) / gru_step_tile(p->D);
        L.res_tile = c.take<unsigned>(static_cast<size_t>(B) * L.tps);
    }
    L.done = c.take<int>(B);
    L.iters = c.take<int>(B);
    L.status = c.take<int>(B);
    L.resid = c.take<float>(B);
    L.buf1 = c.take<float>(BTD);
    L.lin = c.take<float>(BTD);
    L.bvec = c.take<float>(BTD);
    L.proj = c.take<float>(projection_floats(B, T, PD));
    L.bytes = c.off;
    return L;
}

// The two polling events of a solve; destroyed when the solve returns, after
// its final stream synchronisation.
struct PollEvents {
    hipEvent_t ev[2] = {nullptr, nullptr};
    ~PollEvents()
    {
        for (auto &e : ev)
            if (e) (void)hipEventDestroy(e);
    }
};

// Enqueue batches of iterations (1, 2, 4, 4, ...) and, while the current batch
// runs, wait for the copy of the device's all-done flag enqueued after the
// previous batch; stop enqueueing once it reads set.  Kernels enqueued after
// convergence exit at once.  `total` caps the evaluations enqueued.
template <class Enqueue>
int run_polled(Enqueue &&enqueue_iteration, const int *all_done, long long total, hipStream_t stream,
               PollEvents &pe, const char *who)
{
    int rc = DEER_OK;
    long long launched = 0;
    int batch = 1;
    int slot = 0;
    for (auto &e : pe.ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
            return fail(DEER_ERR_HIP, std::string(who) + ": event creation failed");
    bool pending = false;
    int pending_slot = 0;
    volatile int *h = g_poll.host;
    while (launched < total) {
        const long long n = std::min<long long>(batch, total - launched);
        for (long long k = 0; k < n && rc == DEER_OK; ++k) rc = enqueue_iteration();
        if (rc) break;
        launched += n;
        h[slot] = 0;
        if (hipMemcpyAsync(g_poll.host + slot, all_done, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipEventRecord(pe.ev[slot], stream) != hipSuccess) {
            rc = fail(DEER_ERR_HIP, std::string(who) + ": polling copy failed");
            break;
        }
        if (pending) {
            if (hipEventSynchronize(pe.ev[pending_slot]) != hipSuccess) {
                rc = fail(DEER_ERR_HIP, std::string(who) + ": event wait failed");
                break;
            }
            if (h[pending_slot]) break;
        }
        pending = true;
        pending_slot = slot;
        slot ^= 1;
        if (batch < 4) batch *= 2;
    }
    return rc;
}

// Layout of the deer_solve_broyden workspace and of the standalone DPLR scan's.
struct BroydenLayout {
    SolveControl *ctl = nullptr;
    unsigned *res_bits = nullptr;
    int *done = nullptr, *iters = nullptr, *status = nullptr;
    float *resid = nullptr;
    float *buf1 = nullptr;              // second iterate buffer [B,T,D]
    float *f_even = nullptr, *f_odd = nullptr;   // f^(i) by parity [B,T,D]
    float *proj = nullptr;              // input projection
    float *U = nullptr, *V = nullptr, *F = nullptr;   // [B,T,m,D]
    float *agg = nullptr, *entry = nullptr;   // chunk aggregate records, carried entries
    size_t bytes = 0;
};

void carve_dplr_scan(Carve &c, BroydenLayout &L, int B, int T, int D, int m, int chunk)
{
    const size_t nch = static_cast<size_t>(B) * ((T + chunk - 1) / chunk);
    L.agg = c.take<float>(nch * dplr_record_floats(m, D));
    L.entry = c.take<float>(nch * D);
}

BroydenLayout broyden_layout(void *ws, const deer_cell_params_t *p, int B, int T, const deer_broyden_opts_t *o)
{
    const size_t BTD = static_cast<size_t>(B) * T * p->D;
    const int PD = (p->cell == DEER_CELL_GRU) ? 3 * p->D : p->D;
    Carve c(ws);
    BroydenLayout L;
    L.ctl = c.take<SolveControl>(1);
    L.res_bits = c.take<unsigned>(B);
    L.done = c.take<int>(B);
    L.iters = c.take<int>(B);
    L.status = c.take<int>(B);
    L.resid = c.take<float>(B);
    L.buf1 = c.take<float>(BTD);
    L.f_even = c.take<float>(BTD);
    L.f_odd = c.take<float>(BTD);
    L.proj = c.take<float>(projection_floats(B, T, PD));
    L.U = c.take<float>(BTD * o->rank);
    L.V = c.take<float>(BTD * o->rank);
    if (o->multisecant) L.F = c.take<float>(BTD * o->rank);
    carve_dplr_scan(c, L, B, T, p->D, o->rank, o->chunk);
    L.bytes = c.off;
    return L;
}

int check_broyden_opts(const deer_broyden_opts_t *o, bool need_sketch)
{
    if (!o) return fail(DEER_ERR_INVALID, "Broyden options: null pointer");
    if (o->rank < 0 || o->rank > 8) return fail(DEER_ERR_UNSUPPORTED, "Broyden rank outside 0..8");
    if (o->chunk < 1 || o->chunk > 4096) return fail(DEER_ERR_INVALID, "Broyden chunk outside 1..4096");
    if (!std::isfinite(o->alpha)) return fail(DEER_ERR_INVALID, "Broyden alpha not finite");
    if (!(o->damping >= 0.0f && o->damping <= 1.0f)) return fail(DEER_ERR_INVALID, "Broyden damping outside [0, 1]");
    if (!(o->gram_reg >= 0.0f) || std::isinf(o->gram_reg))
        return fail(DEER_ERR_INVALID, "Broyden gram_reg must be finite and >= 0");
    if (need_sketch && o->rank > 0 && !o->sketch)
        return fail(DEER_ERR_INVALID, "Broyden sketch required for rank > 0");
    return DEER_OK;
}

int check_workspace(void *ws, size_t have, size_t need, const char *who)
{
    if (!ws || have < need)
        return fail(DEER_ERR_WORKSPACE, std::string(who) + ": workspace of " + std::to_string(need) + " bytes required");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
        return fail(DEER_ERR_WORKSPACE, std::string(who) + ": workspace not 256-byte aligned");
    return DEER_OK;
}

}  // namespace
}  // namespace deer

using namespace deer;

extern "C" {

const char *deer_last_error(void) { return g_last_error.c_str(); }

int deer_profile_enable(int enable)
{
    g_prof_enabled.store(enable ? 1 : 0);
    return DEER_OK;
}

int deer_profile_read(int which, long long *launches, double *milliseconds)
{
    if (which < 0 || which >= kProfKinds || !launches || !milliseconds)
        return fail(DEER_ERR_INVALID, "deer_profile_read: bad argument");
    std::lock_guard<std::mutex> lock(g_prof_mu);
    *launches = g_prof_launches[which];
    *milliseconds = g_prof_ms[which];
    g_prof_launches[which] = 0;
    g_prof_ms[which] = 0.0;
    return DEER_OK;
}

int deer_workspace_init(void *workspace, size_t ws_bytes, void *stream)
{
    if (!workspace) return fail(DEER_ERR_WORKSPACE, "workspace: null pointer");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
        return fail(DEER_ERR_WORKSPACE, "workspace: not 256-byte aligned");
    const size_t words = ws_bytes / 4;
    if (words == 0) return DEER_OK;
    DEER_LAUNCH(zero_words_kernel, dim3(grid_for(words)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<unsigned *>(workspace), words);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

int linear_scan_workspace_size(int B, int T, int D, int dense, size_t *bytes_out)
{
    if (!bytes_out) return fail(DEER_ERR_INVALID, "linear_scan_workspace_size: null output");
    int rc = check_sizes(B, T);
    if (rc) return rc;
    if (D < 1) return fail(DEER_ERR_INVALID, "D must be >= 1");
    if (dense && D > kMaxD) return fail(DEER_ERR_UNSUPPORTED, "dense scan: D above 64");
    *bytes_out = dense ? dense_scan_state_bytes(B, T, D) : diag_scan_state_bytes(B, T, D);
    return DEER_OK;
}

int linear_scan_diag(const float *a, const float *b, const float *s0, float *s, int B, int T, int D,
                     void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_sizes(B, T);
    if (rc) return rc;
    if (D < 1) return fail(DEER_ERR_INVALID, "linear_scan_diag: D must be >= 1");
    if (B == 0 || T == 0) return DEER_OK;
    if (!a || !b || !s) return fail(DEER_ERR_INVALID, "linear_scan_diag: null a, b or s");
    if (s == a || s == b) return fail(DEER_ERR_INVALID, "linear_scan_diag: s must not alias a or b");
    if (D % 4 == 0 && ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                        reinterpret_cast<uintptr_t>(s)) % 16 != 0))
        return fail(DEER_ERR_INVALID, "linear_scan_diag: a, b and s must be 16-byte aligned");
    rc = check_workspace(workspace, ws_bytes, diag_scan_state_bytes(B, T, D), "linear_scan_diag");
    if (rc) return rc;
    return launch_diag_scan(a, b, s0, s, s, nullptr, nullptr, nullptr, B, T, D, workspace,
                            static_cast<hipStream_t>(stream));
}

int linear_scan_dense(const float *A, const float *b, const float *s0, float *s, int B, int T, int D,
                      void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_sizes(B, T);
    if (rc) return rc;
    if (D < 1 || D > kMaxD) return fail(DEER_ERR_UNSUPPORTED, "linear_scan_dense: D outside 1..64");
    if (B == 0 || T == 0) return DEER_OK;
    if (!A || !b || !s) return fail(DEER_ERR_INVALID, "linear_scan_dense: null A, b or s");
    if (s == b || s == A) return fail(DEER_ERR_INVALID, "linear_scan_dense: s must not alias A or b");
    rc = check_workspace(workspace, ws_bytes, dense_scan_state_bytes(B, T, D), "linear_scan_dense");
    if (rc) return rc;
    return launch_dense_scan(A, nullptr, nullptr, b, s0, s, s, nullptr, nullptr, nullptr, B, T, D, false, workspace,
                             static_cast<hipStream_t>(stream));
}

int deer_workspace_size(const deer_cell_params_t *p, int B, int T, int mode_flags, size_t *bytes_out)
{
    if (!bytes_out) return fail(DEER_ERR_INVALID, "deer_workspace_size: null output");
    int rc = check_cell(p, mode_flags);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    *bytes_out = solve_layout(nullptr, p, B, T, mode_flags).bytes;
    return DEER_OK;
}

int deer_rollout(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T, float *traj_out,
                 void *stream)
{
    if (!p) return fail(DEER_ERR_INVALID, "cell parameters: null pointer");
    int rc = check_cell(p, p->cell == DEER_CELL_GRU ? DEER_MODE_DIAG : DEER_MODE_DENSE);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    if (B == 0 || T == 0) return DEER_OK;
    if (!x || !traj_out) return fail(DEER_ERR_INVALID, "deer_rollout: null x or traj_out");
    return launch_rollout(p, x, s0, B, T, traj_out, static_cast<hipStream_t>(stream));
}

int deer_lle_workspace_size(const deer_cell_params_t *p, int B, int T, size_t *bytes_out)
{
    if (!bytes_out) return fail(DEER_ERR_INVALID, "bytes_out: null pointer");
    int rc = check_cell(p, p && p->cell == DEER_CELL_GRU ? DEER_MODE_DIAG : DEER_MODE_DENSE);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    *bytes_out = lle_layout(nullptr, p, B, T).bytes;
    return DEER_OK;
}

int deer_lle(const deer_cell_params_t *p, const float *x, const float *s0, const float *traj, const float *v0, int B,
             int T, double *lle_out, void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_cell(p, p && p->cell == DEER_CELL_GRU ? DEER_MODE_DIAG : DEER_MODE_DENSE);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    if (B == 0) return DEER_OK;
    if (T <= 0) return fail(DEER_ERR_INVALID, "deer_lle: T must be positive");
    if (!x || !traj || !v0 || !lle_out) return fail(DEER_ERR_INVALID, "deer_lle: x, traj, v0 and lle_out are required");
    const LleLayout need = lle_layout(nullptr, p, B, T);
    rc = check_workspace(workspace, ws_bytes, need.bytes, "deer_lle");
    if (rc) return rc;
    return launch_lle(p, x, s0, traj, v0, B, T, lle_out, lle_layout(workspace, p, B, T),
                      static_cast<hipStream_t>(stream));
}

int deer_solve(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T, int mode_flags,
               float damping, float tol, int max_iter, const float *init_guess, float *traj_out, int *iters_out,
               float *resid_out, int *status_out, void *workspace, size_t ws_bytes, void *stream_)
{
    int rc = check_cell(p, mode_flags);
    const int mode = mode_flags & ~(DEER_SCAN_F64 | DEER_MULTI_LAUNCH);
    const bool scan_f64 = (mode_flags & DEER_SCAN_F64) != 0;
    const bool multi_launch = (mode_flags & DEER_MULTI_LAUNCH) != 0;
    if (rc) return rc;
    if (!(damping >= 0.0f && damping <= 1.0f)) return fail(DEER_ERR_INVALID, "damping must lie in [0, 1]");
    if (damping != 0.0f && mode != DEER_MODE_DENSE && mode != DEER_MODE_DIAG)
        return fail(DEER_ERR_INVALID, "damping applies to the dense and diag modes only");
    const Linearization lz{mode == DEER_MODE_JACOBI ? kLinZero : mode == DEER_MODE_PICARD ? kLinIdentity : kLinJacobian,
                           1.0f - damping};
    rc = check_sizes(B, T);
    if (rc) return rc;
    if (max_iter < 0) return fail(DEER_ERR_INVALID, "max_iter must be >= 0");
    if (std::isnan(tol)) return fail(DEER_ERR_INVALID, "tol is NaN");
    if (B == 0) return DEER_OK;
    if (!iters_out) return fail(DEER_ERR_INVALID, "iters_out: null pointer");
    if (T == 0) {
        // an empty trajectory has residual 0: it passes iff 0 <= tol, else it stops at the cap
        const bool pass = 0.0f <= tol;
        for (int b = 0; b < B; ++b) {
            iters_out[b] = pass ? 0 : max_iter;
            if (resid_out) resid_out[b] = 0.0f;
            if (status_out) status_out[b] = pass ? DEER_SEQ_CONVERGED : DEER_SEQ_NOT_CONVERGED;
        }
        return pass ? DEER_OK : DEER_NOT_CONVERGED;
    }
    if (!x || !traj_out) return fail(DEER_ERR_INVALID, "x and traj_out are required");
    rc = check_workspace(workspace, ws_bytes, solve_layout(nullptr, p, B, T, mode_flags).bytes, "deer_solve");
    if (rc) return rc;
    if (!g_poll.host) return fail(DEER_ERR_HIP, "deer_solve: pinned host memory unavailable");

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const SolveLayout L = solve_layout(workspace, p, B, T, mode_flags);
    const int D = p->D;
    const size_t BTD = static_cast<size_t>(B) * T * D;
    const bool gru = p->cell == DEER_CELL_GRU;
    const int PD = gru ? 3 * D : D;
    ProfScope prof(stream);

    if (!gru && !scan_f64 && !multi_launch && tiny_solve_fits(D, T)) {
        // small problem: the whole solve, projection included, in one launch that
        // writes the per-sequence results straight into the pinned stage
        char *st = g_stage.get((2 * sizeof(int) + sizeof(float)) * static_cast<size_t>(B));
        if (!st) return fail(DEER_ERR_HIP, "deer_solve: pinned host memory unavailable");
        int *h_iters = reinterpret_cast<int *>(st);
        int *h_status = h_iters + B;
        float *h_resid = reinterpret_cast<float *>(h_status + B);
        prof.begin(0);
        rc = launch_tiny_solve(p->W, p->U, p->b, x, p->M, s0, init_guess, traj_out, B, T, D,
                               mode == DEER_MODE_DENSE, lz, tol, max_iter, h_iters, h_status, h_resid, stream);
        prof.end();
        const hipError_t se = hipStreamSynchronize(stream);
        if (rc) return rc;
        if (se != hipSuccess) return hip_fail(se, "hipStreamSynchronize(deer_solve)");
        const long long limit[kProfKinds] = {1, 0, 0, 0};
        prof.collect(limit);
        bool any_nc = false;
        for (int b = 0; b < B; ++b) {
            iters_out[b] = h_iters[b];
            if (resid_out) resid_out[b] = h_resid[b];
            if (status_out) status_out[b] = h_status[b];
            any_nc |= h_status[b] != DEER_SEQ_CONVERGED;
        }
        return any_nc ? DEER_NOT_CONVERGED : DEER_OK;
    }

    // per-solve control state and the starting iterate s^(0) in traj_out
    DEER_LAUNCH(init_control_kernel, dim3(grid_for(static_cast<size_t>(B) + 1)), dim3(256), 0, stream, L.ctl,
                       L.done, L.iters, L.status, L.resid, L.res_bits, B);
    DEER_HIP(hipGetLastError());
    const bool fused = fused_gru_step(p, mode);
    const bool zero_start = fused && !init_guess;   // the fused step reads no s^(0) when it is all zeros
    if (init_guess) {
        if (init_guess != traj_out)
            DEER_LAUNCH(copy_kernel, dim3(grid_for(BTD)), dim3(256), 0, stream, traj_out, init_guess, BTD);
    } else if (!zero_start) {
        DEER_LAUNCH(fill_kernel, dim3(grid_for(BTD)), dim3(256), 0, stream, traj_out, BTD, 0.0f);
    }
    DEER_HIP(hipGetLastError());

    // iteration-invariant input projection (W_ih x + b_ih for the GRU, U x + b for tanh)
    prof.begin(2);
    rc = launch_projection(x, p->U, p->b, L.proj, B, T, p->M, PD, gru && gru_fast_path(D, p->M), stream);
    prof.end();
    if (rc) return rc;

    const int *sel = &L.ctl->iter;
    const int *all_done = &L.ctl->all_done;
    auto enqueue_iteration = [&]() -> int {
        int r;
        if (fused) {
            prof.begin(0);
            r = launch_gru_quasi_step(p->W, p->b2, L.proj, s0, traj_out, L.buf1, L.ctl, L.done, L.iters, L.status,
                                      L.resid, tol, max_iter, L.res_bits, L.res_tile, B, T, D, zero_start, lz, L.scan,
                                      stream);
            prof.end();
            return r;
        }
        prof.begin(0);
        if (gru)
            r = launch_gru_eval(p->W, p->b2, L.proj, s0, traj_out, L.buf1, sel, L.done, all_done, L.lin, L.bvec,
                                L.res_bits, B, T, D, p->M, lz, stream);
        else
            r = launch_tanh_eval(p->W, L.proj, s0, traj_out, L.buf1, sel, L.done, all_done, L.lin, L.bvec,
                                 L.res_bits, B, T, D, mode == DEER_MODE_DENSE, lz, stream);
        prof.end();
        if (r) return r;
        prof.begin(3);
        DEER_LAUNCH(check_kernel, dim3(1), dim3(256), 0, stream, L.ctl, L.res_bits, nullptr, 0, L.done, L.iters,
                           L.status, L.resid, B, tol, max_iter);
        prof.end();
        DEER_HIP(hipGetLastError());
        prof.begin(1);
        if (diag_blocks(mode))
            r = launch_diag_scan(L.lin, L.bvec, s0, traj_out, L.buf1, sel, L.done, all_done, B, T, D, L.scan, stream);
        else
            r = launch_dense_scan(nullptr, L.lin, p->W, L.bvec, s0, traj_out, L.buf1, sel, L.done, all_done, B, T, D,
                                  scan_f64, L.scan, stream);
        prof.end();
        return r;
    };

    const long long total = static_cast<long long>(max_iter) + 1;   // evaluations needed at most
    PollEvents pe;
    rc = run_polled(enqueue_iteration, all_done, total, stream, pe, "deer_solve");
    if (rc == DEER_OK) {
        const size_t per_seq = static_cast<size_t>(T) * D;
        DEER_LAUNCH(gather_kernel, dim3(grid_for(per_seq, 256, 1024), B), dim3(256), 0, stream, traj_out,
                           L.buf1, L.iters, per_seq, B, zero_start ? 1 : 0);
        if (hipGetLastError() != hipSuccess) rc = fail(DEER_ERR_HIP, "deer_solve: gather launch failed");
    }
    std::vector<int> status_h(B, 0);
    unsigned abort_flag = 0;
    if (rc == DEER_OK) {
        const unsigned *abort_dev =
            (diag_blocks(mode) || fused) ? &static_cast<ScanHeader *>(L.scan)->abort : nullptr;
        rc = read_results(L.iters, L.status, L.resid, abort_dev, B, stream, iters_out, resid_out, status_h,
                          abort_flag, "deer_solve");
    } else {
        (void)hipStreamSynchronize(stream);
    }
    if (rc) return rc;
    {
        int last = 0;
        for (int b = 0; b < B; ++b) last = std::max(last, iters_out[b]);
        const long long limit[kProfKinds] = {last + 1, last, 1, last + 1};
        prof.collect(limit);
    }
    if (abort_flag) return fail(DEER_ERR_DEVICE, "deer_solve: the scan look-back wait hit its bound");
    bool any_nc = false;
    for (int b = 0; b < B; ++b) {
        if (status_out) status_out[b] = status_h[b];
        any_nc |= status_h[b] != DEER_SEQ_CONVERGED;
    }
    return any_nc ? DEER_NOT_CONVERGED : DEER_OK;
}

int deer_broyden_workspace_size(const deer_cell_params_t *p, int B, int T, const deer_broyden_opts_t *opts,
                                size_t *bytes_out)
{
    if (!bytes_out) return fail(DEER_ERR_INVALID, "deer_broyden_workspace_size: null output");
    int rc = check_cell(p, DEER_MODE_DIAG);
    if (rc) return rc;
    rc = check_broyden_opts(opts, false);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    *bytes_out = broyden_layout(nullptr, p, B, T, opts).bytes;
    return DEER_OK;
}

int deer_solve_broyden(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T,
                       const deer_broyden_opts_t *opts, float tol, int max_iter, const float *init_guess,
                       float *traj_out, int *iters_out, float *resid_out, int *status_out, void *workspace,
                       size_t ws_bytes, void *stream_)
{
    int rc = check_cell(p, DEER_MODE_DIAG);
    if (rc) return rc;
    rc = check_broyden_opts(opts, true);
    if (rc) return rc;
    rc = check_sizes(B, T);
    if (rc) return rc;
    if (max_iter < 0) return fail(DEER_ERR_INVALID, "max_iter must be >= 0");
    if (std::isnan(tol)) return fail(DEER_ERR_INVALID, "tol is NaN");
    if (B == 0) return DEER_OK;
    if (!iters_out) return fail(DEER_ERR_INVALID, "iters_out: null pointer");
    if (T == 0) {
        const bool pass = 0.0f <= tol;
        for (int b = 0; b < B; ++b) {
            iters_out[b] = pass ? 0 : max_iter;
            if (resid_out) resid_out[b] = 0.0f;
            if (status_out) status_out[b] = pass ? DEER_SEQ_CONVERGED : DEER_SEQ_NOT_CONVERGED;
        }
        return pass ? DEER_OK : DEER_NOT_CONVERGED;
    }
    if (!x || !traj_out) return fail(DEER_ERR_INVALID, "x and traj_out are required");
    rc = check_workspace(workspace, ws_bytes, broyden_layout(nullptr, p, B, T, opts).bytes, "deer_solve_broyden");
    if (rc) return rc;
    if (!g_poll.host) return fail(DEER_ERR_HIP, "deer_solve_broyden: pinned host memory unavailable");

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const BroydenLayout L = broyden_layout(workspace, p, B, T, opts);
    const int D = p->D;
    const size_t BTD = static_cast<size_t>(B) * T * D;
    const bool gru = p->cell == DEER_CELL_GRU;
    const int PD = gru ? 3 * D : D;
    const bool tiled = gru && gru_fast_path(D, p->M);
    ProfScope prof(stream);

    DEER_LAUNCH(init_control_kernel, dim3(grid_for(static_cast<size_t>(B) + 1)), dim3(256), 0, stream, L.ctl,
                L.done, L.iters, L.status, L.resid, L.res_bits, B);
    if (init_guess) {
        if (init_guess != traj_out)
            DEER_LAUNCH(copy_kernel, dim3(grid_for(BTD)), dim3(256), 0, stream, traj_out, init_guess, BTD);
    } else {
        DEER_LAUNCH(fill_kernel, dim3(grid_for(BTD)), dim3(256), 0, stream, traj_out, BTD, 0.0f);
    }
    DEER_HIP(hipGetLastError());
    prof.begin(2);
    rc = launch_projection(x, p->U, p->b, L.proj, B, T, p->M, PD, tiled, stream);
    prof.end();
    if (rc) return rc;

    DplrArgs a;
    a.B = B; a.T = T; a.D = D; a.m = opts->rank;
    a.chunk = opts->chunk; a.nchunk = (T + opts->chunk - 1) / opts->chunk;
    a.alpha = opts->alpha; a.shrink = 1.0f - opts->damping; a.lambda = opts->gram_reg;
    a.multisecant = opts->multisecant ? 1 : 0;
    a.omega = opts->sketch;
    a.U = L.U; a.V = L.V; a.F = L.F;
    a.s0 = s0; a.s_even = traj_out; a.s_odd = L.buf1; a.f_even = L.f_even; a.f_odd = L.f_odd;
    a.ctl = L.ctl; a.skip = L.done;
    a.agg = L.agg;
    a.entry = L.entry;

    const int *sel = &L.ctl->iter;
    const int *all_done = &L.ctl->all_done;
    const Linearization value{kLinValue, 1.0f};
    auto enqueue_iteration = [&]() -> int {
        int r;
        prof.begin(0);
        if (gru)
            r = launch_gru_eval(p->W, p->b2, L.proj, s0, traj_out, L.buf1, sel, L.done, all_done, L.f_even,
                                L.f_odd, L.res_bits, B, T, D, p->M, value, stream);
        else
            r = launch_tanh_eval(p->W, L.proj, s0, traj_out, L.buf1, sel, L.done, all_done, L.f_even, L.f_odd,
                                 L.res_bits, B, T, D, 0, value, stream);
        prof.end();
        if (r) return r;
        prof.begin(3);
        DEER_LAUNCH(check_kernel, dim3(1), dim3(256), 0, stream, L.ctl, L.res_bits, nullptr, 0, L.done, L.iters,
                    L.status, L.resid, B, tol, max_iter);
        prof.end();
        DEER_HIP(hipGetLastError());
        prof.begin(1);
        r = launch_dplr_step(a, stream);
        prof.end();
        return r;
    };
    const long long total = static_cast<long long>(max_iter) + 1;
    PollEvents pe;
    rc = run_polled(enqueue_iteration, all_done, total, stream, pe, "deer_solve_broyden");
    if (rc == DEER_OK) {
        const size_t per_seq = static_cast<size_t>(T) * D;
        DEER_LAUNCH(gather_kernel, dim3(grid_for(per_seq, 256, 1024), B), dim3(256), 0, stream, traj_out, L.buf1,
                    L.iters, per_seq, B, 0);
        if (hipGetLastError() != hipSuccess) rc = fail(DEER_ERR_HIP, "deer_solve_broyden: gather launch failed");
    }
    std::vector<int> status_h(B, 0);
    unsigned abort_flag = 0;
    if (rc == DEER_OK) {
        rc = read_results(L.iters, L.status, L.resid, nullptr, B, stream, iters_out, resid_out, status_h, abort_flag,
                          "deer_solve_broyden");
    } else {
        (void)hipStreamSynchronize(stream);
    }
    if (rc) return rc;
    {
        int last = 0;
        for (int b = 0; b < B; ++b) last = std::max(last, iters_out[b]);
        const long long limit[kProfKinds] = {last + 1, last, 1, last + 1};
        prof.collect(limit);
    }
    bool any_nc = false;
    for (int b = 0; b < B; ++b) {
        if (status_out) status_out[b] = status_h[b];
        any_nc |= status_h[b] != DEER_SEQ_CONVERGED;
    }
    return any_nc ? DEER_NOT_CONVERGED : DEER_OK;
}

int linear_scan_dplr_workspace_size(int B, int T, int D, int rank, int chunk, size_t *bytes_out)
{
    if (!bytes_out) return fail(DEER_ERR_INVALID, "linear_scan_dplr_workspace_size: null output");
    int rc = check_sizes(B, T);
    if (rc) return rc;
    if (D < 1 || D > kMaxD) return fail(DEER_ERR_UNSUPPORTED, "DPLR scan: D outside 1..64");
    if (rank < 0 || rank > 8) return fail(DEER_ERR_UNSUPPORTED, "DPLR scan: rank outside 0..8");
    if (chunk < 1 || chunk > 4096) return fail(DEER_ERR_INVALID, "DPLR scan: chunk outside 1..4096");
    Carve c(nullptr);
    BroydenLayout L;
    carve_dplr_scan(c, L, B, T, D, rank, chunk);
    *bytes_out = c.off;
    return DEER_OK;
}

int linear_scan_dplr(float alpha, const float *U, const float *V, const float *c, const float *sketch, float *delta,
                     int B, int T, int D, int rank, int chunk, void *workspace, size_t ws_bytes, void *stream)
{
    size_t need = 0;
    int rc = linear_scan_dplr_workspace_size(B, T, D, rank, chunk, &need);
    if (rc) return rc;
    if (!std::isfinite(alpha)) return fail(DEER_ERR_INVALID, "DPLR scan: alpha not finite");
    if (static_cast<long long>(B) * T == 0) return DEER_OK;
    if (!c || !delta || (rank > 0 && (!U || !V || !sketch)))
        return fail(DEER_ERR_INVALID, "DPLR scan: c, delta (and U, V, sketch for rank > 0) are required");
    rc = check_workspace(workspace, ws_bytes, need, "linear_scan_dplr");
    if (rc) return rc;
    Carve cv(workspace);
    BroydenLayout L;
    carve_dplr_scan(cv, L, B, T, D, rank, chunk);
    DplrArgs a;
    a.B = B; a.T = T; a.D = D; a.m = rank; a.n_fixed = rank;
    a.chunk = chunk; a.nchunk = (T + chunk - 1) / chunk;
    a.alpha = alpha;
    a.omega = sketch;
    a.U = const_cast<float *>(U); a.V = const_cast<float *>(V);
    a.c = c; a.out = delta;
    a.agg = L.agg;
    a.entry = L.entry;
    return launch_dplr_step(a, static_cast<hipStream_t>(stream));
}

}  // extern "C"
