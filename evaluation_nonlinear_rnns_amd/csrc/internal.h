// Internal declarations shared by the HIP translation units of libdeer.
// Not part of the public interface (include/deer.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/deer.h"

namespace deer {

// ----------------------------------------------------------------- errors
void set_error(const std::string &msg);
int fail(int code, const std::string &msg);
int hip_fail(hipError_t e, const char *what);

#define DEER_HIP(call)                                       \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return ::deer::hip_fail(e_, #call); \
    } while (0)

// --------------------------------------------------------------- constants
constexpr int kWave = 64;
constexpr int kMaxD = 64;
constexpr int kMaxM = 1024;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// Cursor that hands out 256-byte aligned regions of a workspace.
struct Carve {
    char *base;
    size_t off = 0;
    explicit Carve(void *p) : base(static_cast<char *>(p)) {}
    template <class T>
    T *take(size_t count) {
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += align_up(count * sizeof(T));
        return p;
    }
};

// ------------------------------------------------------------ launches
// Every kernel launch goes through DEER_LAUNCH.  While deer_solve profiles a
// class of launches it leaves the class's event pair here; the launches then go
// out through hipExtLaunchKernelGGL, which timestamps the dispatch itself (no
// separate event packets between kernels).  The first launch of the class takes
// the start event and every launch the stop event, so the last one stands.
struct ProfLaunch {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    hipEvent_t mark = nullptr;   // when set: the next launch records this stop event instead (a sub-timing)
};
extern thread_local ProfLaunch g_prof_launch;
// Times the next launch of the open profiling scope as kernel class `kind`
// too (from the scope's start, so it must be the scope's first launch).
void prof_mark_next(int kind);
constexpr int kProfCompose = 4;   // the dense scan's chunk-compose launch

#define DEER_LAUNCH(kernel, grid, block, shmem, stream, ...)                                                     \
    do {                                                                                                      \
        if (::deer::g_prof_launch.stop) {                                                                     \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ::deer::g_prof_launch.start,            \
                                  ::deer::g_prof_launch.mark ? ::deer::g_prof_launch.mark                     \
                                                             : ::deer::g_prof_launch.stop,                    \
                                  0, __VA_ARGS__);                                                            \
            ::deer::g_prof_launch.start = nullptr;                                                            \
            ::deer::g_prof_launch.mark = nullptr;                                                             \
        } else {                                                                                              \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                              \
        }                                                                                                     \
    } while (0)

// ------------------------------------------------------ row contractions
// DPP rotation by K lanes within each row of 16 lanes.
template <int K>
__device__ __forceinline__ int row_ror(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x120 + K, 0xf, 0xf, true);
}

// The 15 rotated products of a row contraction: a0 (even k) and a1 (odd k)
// accumulate w[k] * (x rotated right by k lanes within each row of 16), each
// as one v_fmac_f32_dpp (the compiler would keep every rotation as a separate
// v_mov_b32_dpp next to the FMA).  The same fused multiply-adds on the same
// operands in the same order, so the same bits.  A DPP source written by the
// VALU just before needs two wait states and the hazard check does not look
// inside asm, so the chain is one asm statement that opens with them: no
// compiler instruction can come between the wait and the DPP reads of x.
struct RowRotations {
    static __device__ __forceinline__ void sources(int m, int (&src)[16])
    {
        src[1] = row_ror<1>(m); src[2] = row_ror<2>(m); src[3] = row_ror<3>(m); src[4] = row_ror<4>(m);
        src[5] = row_ror<5>(m); src[6] = row_ror<6>(m); src[7] = row_ror<7>(m); src[8] = row_ror<8>(m);
        src[9] = row_ror<9>(m); src[10] = row_ror<10>(m); src[11] = row_ror<11>(m); src[12] = row_ror<12>(m);
        src[13] = row_ror<13>(m); src[14] = row_ror<14>(m); src[15] = row_ror<15>(m);
    }
    static __device__ __forceinline__ void contract(float x, const float (&w)[16], float &a0, float &a1)
    {
        asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %2, %3 row_ror:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %4 row_ror:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %5 row_ror:3 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %6 row_ror:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %7 row_ror:5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %8 row_ror:6 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %9 row_ror:7 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %10 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %11 row_ror:9 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %12 row_ror:10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %13 row_ror:11 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %14 row_ror:12 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %15 row_ror:13 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %0, %2, %16 row_ror:14 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %2, %17 row_ror:15 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(a0), "+v"(a1)
            : "v"(x), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(w[8]),
              "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]));
    }
};

// ------------------------------------------------------------ solve control
// Device-side state of one deer_solve call.
struct SolveControl {
    int iter;         // current iteration index i (iterate s^(i) lives in buffer (i ^ flip) % 2)
    int all_done;     // 1 once every sequence has stopped
    int escalate;     // 1 once a stall asked for double accumulation (read by the host's poll)
    int flip;         // buffer parity of this solve (0 unless the path supports it, see init_control_kernel)
    int last_parity;  // parity of the iteration that ended the workspace's last solve (kept across solves)
    int pad[59];
};

// Finite-step check.  After i iterations the first i states are exact in
// exact arithmetic ("Parallel Broyden Methods", Theorem 1), so the front --
// the first position whose residual exceeds tol (or is not finite) -- is never
// below i.  The evaluation kernels take the front's minimum per sequence into
// front[] (atomic min; no violation leaves ~0u); finalize_iteration keeps the
// best front and the iteration it last advanced, and calls a sequence stalled
// when its best front is below i and has not advanced for `window`
// iterations.  A stall then either stops the sequence (DEER_SEQ_STALLED) or,
// with `escalate`, raises ctl->escalate for the host and lets it go on.
struct StallCheck {
    unsigned *front = nullptr;   // [B]; nullptr: no check
    int *best = nullptr;         // [B]
    int *last_adv = nullptr;     // [B]
    int window = 0;
    int escalate = 0;
};
constexpr unsigned kNoFront = 0xFFFFFFFFu;

// Where an evaluation kernel takes the front: front[b] (atomic min), or nowhere.
struct FrontOut {
    unsigned *front = nullptr;
    float tol = 0.0f;
};

// Minimum of a per-lane violating position over the wavefront.
__device__ __forceinline__ unsigned wave_min_u32(unsigned v)
{
    for (int o = 32; o > 0; o >>= 1) v = min(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), o, 64)));
    return v;
}

// Position t counts toward the front when its residual is not <= tol.
__device__ __forceinline__ unsigned front_of(float r_abs, float tol, int t)
{
    return (r_abs <= tol) ? kNoFront : static_cast<unsigned>(t);
}

// One sequence's stall bookkeeping at iteration i (the residual did not pass
// and the cap is not reached).  Returns true when the sequence is to stop as
// stalled.
__device__ inline bool stall_step(const StallCheck &sc, SolveControl *ctl, int b, int i)
{
    if (!sc.front) return false;
    const unsigned fr = sc.front[b];
    sc.front[b] = kNoFront;                     // ready for the next evaluation
    if (sc.window <= 0) return false;
    const int f = fr > 0x7FFFFFFFu ? 0x7FFFFFFF : static_cast<int>(fr);
    if (f > sc.best[b]) {
        sc.best[b] = f;
        sc.last_adv[b] = i;
        return false;
    }
    if (sc.best[b] < i && i - sc.last_adv[b] >= sc.window) {
        if (!sc.escalate) return true;
        ctl->escalate = 1;
        sc.last_adv[b] = i;                     // a fresh window after the switch
    }
    return false;
}

// Convergence test of iteration i = ctl->iter for every sequence, run by one
// whole workgroup (blockDim.x a multiple of 64, at most 1024; `red` is a
// __shared__ array of blockDim.x / 64 words).  A sequence passes when the max
// residual of its iterate is <= tol and is then frozen with iters = i; at the
// cap it stops as not converged, or non-finite for a NaN / Inf residual.  The
// residual is one word per sequence (res_bits, reset here) or per-tile maxima
// (res_tile, tps words per sequence).  Non-negative floats order like their
// bit patterns and NaN patterns sit above +Inf, so maxima are taken on bits.
// poll (pinned host memory, or null) receives all_done and escalate, so the
// host's loop reads them once the launch is done, without a copy.
__device__ inline void publish_poll(const SolveControl *ctl, int *poll)
{
    if (!poll) return;
    const int ad = __hip_atomic_load(&ctl->all_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int es = __hip_atomic_load(&ctl->escalate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(poll, ad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(poll + 1, es, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ inline void finalize_iteration(SolveControl *ctl, unsigned *res_bits, const unsigned *res_tile, int tps,
                                          int *done, int *iters, int *status, float *resid, int B, float tol,
                                          int max_iter, unsigned *red, const StallCheck &sc, int *poll)
{
    const int i = ctl->iter;
    int active = 0;
    if (!res_tile) {
        // one sequence per thread: the per-sequence words are read and written
        // in parallel instead of one dependent round trip per sequence
        for (int b = threadIdx.x; b < B; b += blockDim.x) {
            if (done[b]) continue;
            const unsigned m = res_bits[b];
            const float r = __uint_as_float(m);
            res_bits[b] = 0u;
            if (r <= tol) {
                done[b] = 1;
                iters[b] = i;
                status[b] = DEER_SEQ_CONVERGED;
                resid[b] = r;
            } else if (i >= max_iter) {
                done[b] = 1;
                iters[b] = max_iter;
                status[b] = __builtin_isfinite(r) ? DEER_SEQ_NOT_CONVERGED : DEER_SEQ_NONFINITE;
                resid[b] = r;
            } else if (stall_step(sc, ctl, b, i)) {
                done[b] = 1;
                iters[b] = i;
                status[b] = DEER_SEQ_STALLED;
                resid[b] = r;
            } else {
                active = 1;
            }
        }
        active = __syncthreads_or(active);
        if (threadIdx.x == 0) {
            if (active) ctl->iter = i + 1;
            else { ctl->all_done = 1; ctl->last_parity = i & 1; }
            publish_poll(ctl, poll);
        }
        return;
    }
    for (int b = 0; b < B; ++b) {
        if (done[b]) continue;                    // same for every thread
        unsigned m = 0u;
        if (res_tile) {
            for (int k = threadIdx.x; k < tps; k += blockDim.x) m = max(m, res_tile[static_cast<size_t>(b) * tps + k]);
            for (int o = 32; o > 0; o >>= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), o, 64)));
            if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
            __syncthreads();
            m = red[0];
            for (int w = 1; w < static_cast<int>(blockDim.x / 64); ++w) m = max(m, red[w]);
            __syncthreads();
        } else {
            m = res_bits[b];
        }
        if (threadIdx.x == 0) {
            const float r = __uint_as_float(m);
            if (!res_tile) res_bits[b] = 0u;
            if (r <= tol) {
                done[b] = 1;
                iters[b] = i;
                status[b] = DEER_SEQ_CONVERGED;
                resid[b] = r;
            } else if (i >= max_iter) {
                done[b] = 1;
                iters[b] = max_iter;
                status[b] = __builtin_isfinite(r) ? DEER_SEQ_NOT_CONVERGED : DEER_SEQ_NONFINITE;
                resid[b] = r;
            } else if (stall_step(sc, ctl, b, i)) {
                done[b] = 1;
                iters[b] = i;
                status[b] = DEER_SEQ_STALLED;
                resid[b] = r;
            } else {
                active = 1;
            }
        }
    }
    active = __syncthreads_or(active);
    if (threadIdx.x == 0) {
        if (active) ctl->iter = i + 1;
        else { ctl->all_done = 1; ctl->last_parity = i & 1; }
        publish_poll(ctl, poll);
    }
}

// ------------------------------------------------------ diagonal scan state
// Look-back state kept in a workspace between launches.  Zero-filled once by
// the caller; every launch leaves done = 0 and advances epoch.
constexpr int kTicketGroups = 8;   // one tile counter per group of workgroups (see the scans)
struct ScanHeader {
    unsigned done;     // workgroups finished in the current launch
    unsigned epoch;    // tags descriptors of the current launch
    unsigned abort;    // set if a bounded wait gave up (should never happen)
    unsigned pad0;
    unsigned ticket[kTicketGroups];   // next tile of each group to hand out in the current launch
    unsigned pad[52];
};
static_assert(sizeof(ScanHeader) == 256, "header is one alignment unit");

// Deterministic look-back of the single-pass scans.  A chain of tiles (one
// sequence's tiles of the same channels) publishes, per channel, each tile's
// aggregate pair (A, B) and its inclusive prefix (the state after its last
// step), always computed as the left-to-right chain
//     inc_t = fma(A_t, inc_{t-1}, B_t),   inc_0 = fma(A_0, s_0, B_0).
// A tile walks back, WIN descriptors per round trip, to the nearest earlier
// tile k whose inclusive prefix is published (every tile in between having
// published its aggregate), then applies the aggregates k+1 .. t-1 forward with
// the same fused multiply-adds.  That reproduces the chain's value bit for bit
// whichever k the timing delivered, so a scan of the same input gives the same
// bits every time (an iteration that amplifies perturbations, like Picard's,
// depends on that to keep its exact prefix exact) -- at the cost of the
// forward pass over (t-1-k) aggregates, which are L2-resident.  A tile waits
// only on tiles with smaller indices.  Descriptor words are `value | tag << 32`;
// the wait is bounded by spin_limit, after which the abort flag is raised and
// NaN returned.
__device__ __forceinline__ unsigned long long scan_word_load(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float scan_word_val(unsigned long long w) { return __uint_as_float(static_cast<unsigned>(w)); }

template <int WIN>
__device__ inline float chained_carry(const unsigned long long *chain, size_t words_per_tile, int oa, int ob, int oi,
                                      int t, unsigned tag_agg, unsigned tag_inc, unsigned *abort_flag,
                                      unsigned spin_limit)
{
    // 1. the nearest earlier inclusive prefix, WIN tiles per round trip
    int j = t - 1, k = -1, uk = 0;
    float x = 0.0f;
    unsigned long long wa[WIN], wb[WIN];
    unsigned spins = 0;
    while (true) {
        unsigned long long wi[WIN];
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
            const size_t jj = static_cast<size_t>(max(j - u, 0)) * words_per_tile;
            wi[u] = scan_word_load(chain + jj + oi);
            wa[u] = scan_word_load(chain + jj + oa);
            wb[u] = scan_word_load(chain + jj + ob);
        }
        bool stalled = false;
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
            if (k >= 0 || stalled || j - u < 0) continue;
            if (static_cast<unsigned>(wi[u] >> 32) == tag_inc) {
                k = j - u;
                uk = u;
                x = scan_word_val(wi[u]);
            } else if (static_cast<unsigned>(wa[u] >> 32) != tag_agg || static_cast<unsigned>(wb[u] >> 32) != tag_agg) {
                stalled = true;
                j -= u;                             // resume at the first tile not yet published
            }
        }
        if (k >= 0) break;
        if (!stalled) {
            j -= WIN;
            continue;
        }
        ++spins;
        if (spins > spin_limit ||
            ((spins & 1023u) == 0u && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
            __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return __builtin_nanf("");
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // 2. the chain forward from inc_k: tiles k+1 .. j are still in registers
    //    (window slots uk-1 .. 0), tiles j+1 .. t-1 were passed in earlier rounds
#pragma unroll
    for (int u = WIN - 1; u >= 0; --u)
        if (u < uk) x = __builtin_fmaf(scan_word_val(wa[u]), x, scan_word_val(wb[u]));
    for (int m0 = j + 1; m0 < t; m0 += WIN) {
        float A[WIN], Bv[WIN];
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
            const size_t mm = static_cast<size_t>(min(m0 + u, t - 1)) * words_per_tile;
            A[u] = scan_word_val(scan_word_load(chain + mm + oa));
            Bv[u] = scan_word_val(scan_word_load(chain + mm + ob));
        }
#pragma unroll
        for (int u = 0; u < WIN; ++u)
            if (m0 + u < t) x = __builtin_fmaf(A[u], x, Bv[u]);
    }
    return x;
}

// Geometry of one diagonal-scan launch.
struct DiagScanPlan {
    int B, T, D;
    int vec;        // 4 when D % 4 == 0, else 1
    int ch;         // channels per tile
    int chunk_len;  // time steps per chunk
    int groups;     // channel tiles per sequence
    int chains;     // B * groups
    int nchunk;     // chunks per chain
    size_t desc_words;
};
DiagScanPlan diag_scan_plan(int B, int T, int D);
size_t diag_scan_state_bytes(int B, int T, int D);
// Look-back state of the no-allocation diagonal scan: this device's address of
// the library's static scratch array (DEER_NOALLOC_SCRATCH_BYTES), cleared on
// the first call on a device (on `stream`, synchronised).
int diag_scan_static_state(void **state, hipStream_t stream);

// Enqueue the single-pass diagonal scan.  `out_sel` (device int or null)
// selects out1 when odd, out0 otherwise; `skip` (device int[B] or null)
// skips sequences whose flag is set; `all_done` (device int or null) skips
// the whole launch when set.
int launch_diag_scan(const float *a, const float *b, const float *s0, float *out0, float *out1,
                     const int *out_sel, const int *skip, const int *all_done, int B, int T, int D,
                     void *state, hipStream_t stream);

// ---------------------------------------------------------- dense scan
struct DenseScanPlan {
    int B, T, D;
    int chunk_len;
    int nchunk;     // chunks per sequence
};
DenseScanPlan dense_scan_plan(int B, int T, int D);
size_t dense_scan_state_bytes(int B, int T, int D, bool f64 = false);

// Dense scan s_t = A_t s_{t-1} + b_t.  Either A (materialised [B,T,D,D]) or
// the factored form A_t = diag(d_t) W (d [B,T,D], W [D,D]) is given.  f64:
// products, offsets, carries and replayed states accumulate in double.
//
// `ev` (factored form only; null: none) also evaluates the tanh cell
// f_t = tanh(W s_{t-1} + p_t) on the solved trajectory while the replay
// forms W s_{t-1}: the next iteration's d_t = shrink (1 - f_t^2) and
// b_t = f_t - d_t (W s_{t-1}) overwrite d and b in place, and the residual
// |s_t - f_t| goes to res_bits (per-sequence max on float bits) and, with
// front, the first violating position (atomic min).  dense_scan_evaluates()
// says whether a shape takes that path; otherwise `ev` is ignored and the
// caller runs the evaluation itself.
struct ReplayEval {
    const float *p = nullptr;       // [B,T,D] input projection U x_t + b
    float *lin = nullptr;           // = d
    float *bout = nullptr;          // = b
    unsigned *res_bits = nullptr;   // [B]
    unsigned *front = nullptr;      // [B] or null
    float tol = 0.0f;
    float shrink = 1.0f;
};
bool dense_scan_evaluates(int D, bool f64);
int launch_dense_scan(const float *A, const float *d, const float *W, const float *b,
                      const float *s0, float *out0, float *out1, const int *out_sel,
                      const int *skip, const int *all_done, int B, int T, int D, bool f64, void *state,
                      hipStream_t stream, const ReplayEval *ev = nullptr);

// ---------------------------------------------------------- cell kernels
// p = U x + bias for every position, O outputs.  `tiled` writes the layout
// the matrix-core GRU evaluation reads (see cell_mfma.hip); row-major [B,T,O]
// otherwise.
int launch_projection(const float *x, const float *U, const float *bias, float *p, int B, int T, int M,
                      int O, bool tiled, hipStream_t stream);
size_t projection_floats(int B, int T, int O);

// How an iteration linearises f: the Jacobian (or its diagonal) shrunk by
// `shrink` = 1 - k, the zero block (Jacobi) or the identity (Picard).
// kLinValue: evaluation only -- the cell value f_t goes to the first output
// array when the iteration index (*sel) is even, to the second when it is odd.
enum LinKind : int { kLinJacobian = 0, kLinZero = 1, kLinIdentity = 2, kLinValue = 3 };
struct Linearization {
    int kind;
    float shrink;
};

// The diagonal block entry a mode uses, given the Jacobian's diagonal entry.
__device__ __forceinline__ float lin_diag(Linearization l, float jdiag)
{
    return l.kind == kLinJacobian ? l.shrink * jdiag : (l.kind == kLinZero ? 0.0f : 1.0f);
}

// tanh cell: f_t = tanh(W s_{t-1} + p_t).  Dense mode writes the factored
// leaf d_t = shrink (1 - f_t^2) into `lin` and b_t = f_t - d_t * (W s_{t-1});
// the other modes write a_t = lin_diag(d_t * diag(W)) into `lin` and
// b_t = f_t - a_t * s_{t-1}.
// res_bits[b] receives atomic max of |s_t - f_t| (float bits).
int launch_tanh_eval(const float *W, const float *p, const float *s0, const float *s_even,
                     const float *s_odd, const int *sel, const int *skip, const int *all_done,
                     float *lin, float *bvec, unsigned *res_bits, int B, int T, int D, int dense,
                     Linearization lz, FrontOut fo, hipStream_t stream);

// GRU cell, diagonal blocks: writes a_t = lin_diag(diag(d f / d s)) and
// b_t = f_t - a_t * s_{t-1}.  With gru_fast_path(D, M) the projection is
// tiled and the evaluation runs on the matrix cores.
bool gru_fast_path(int D, int M);
int launch_gru_eval(const float *Whh, const float *bhh, const float *p, const float *s0,
                    const float *s_even, const float *s_odd, const int *sel, const int *skip,
                    const int *all_done, float *a, float *bvec, unsigned *res_bits, int B, int T,
                    int D, int M, Linearization lz, FrontOut fo, hipStream_t stream);

// Matrix-core versions (cell_mfma.hip) for the supported sizes.
bool gru_mfma_supported(int D);
int launch_gru_eval_mfma(const float *Whh, const float *bhh, const float *p, const float *s0,
                         const float *s_even, const float *s_odd, const int *sel, const int *skip,
                         const int *all_done, float *a, float *bvec, unsigned *res_bits, int B, int T,
                         int D, Linearization lz, FrontOut fo, hipStream_t stream);
bool proj_mfma_supported(int M, int O);
size_t proj_tiled_floats(int B, int T, int O);
int launch_projection_mfma(const float *x, const float *U, const float *bias, float *p, int B, int T,
                           int M, int O, bool tiled, hipStream_t stream);

// Fused quasi-DEER iteration for the GRU on the matrix cores: evaluation and
// diagonal scan in one persistent launch, writing s^(i+1) into the buffer
// that does not hold s^(i).  res_tile[tile] receives the residual maximum of
// every TP-position tile (gru_step_tile(D) positions).
int gru_step_tile(int D);
size_t gru_step_state_bytes(int B, int T, int D);
// The workgroup that finishes last also runs finalize_iteration(), so one
// launch is a whole iteration.  Residual maxima go to res_bits (one word per
// sequence, zero on entry) for up to 256 sequences, else to res_tile.  zero_start: the iterate s^(0) is all zeros and
// is not read from memory at iteration 0.  With x non-null (zero_start, s0 null,
// inputs of width M = D, the first iteration only) the launch computes the tiled input
// projection W_ih x + b_ih itself, writes it to `pt`, and evaluates the first
// iterate from it; otherwise `pt` holds the projection already.
int launch_gru_quasi_step(const float *Whh, const float *bhh, float *pt, const float *s0, float *s_even,
                          float *s_odd, SolveControl *ctl, int *done, int *iters, int *status, float *resid,
                          float tol, int max_iter, unsigned *res_bits, unsigned *res_tile, int B, int T, int D,
                          bool zero_start, Linearization lz, const StallCheck &sc, void *state, const float *x,
                          const float *Wih, const float *bih, int M, int *poll, hipStream_t stream);

// Sequential rollout (rollout.hip): the projection into `workspace`
// (rollout_workspace_bytes), then one workgroup per sequence.
size_t rollout_workspace_bytes(const deer_cell_params_t *p, int B, int T);
int launch_rollout(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T,
                   float *traj, void *workspace, hipStream_t stream);

// Whole tanh solves in one launch (tiny.hip): one workgroup per sequence forms
// its input projection and runs every iteration on chip; for D <= 4 and
// T <= 1024.  Writes the trajectory, and the iterations, statuses and
// residuals to `iters`, `status`, `resid` (device-visible host memory is
// allowed: they are written once per sequence and fenced system-wide).
bool tiny_solve_fits(int D, int T);
int launch_tiny_solve(const float *W, const float *U, const float *bias, const float *x, int M, const float *s0,
                      const float *init, float *traj, int B, int T, int D, bool dense, Linearization lz, float tol,
                      int max_iter, int stall_window, int *iters, int *status, float *resid, hipStream_t stream);

// Whole dense tanh solves in one launch (dense_solve.hip): each sequence gets a
// group of workgroups that synchronise among themselves, one group barrier per
// iteration; for D <= 16, T <= 8192 and grids the device holds at once (f64:
// double accumulation).  `proj` is the input projection; `init` is the starting
// iterate (null: zeros; it may alias `traj`), `traj` receives the iterate each
// sequence stopped at.  `state` holds
// dense_persist_state_bytes and is set up by each launch; iters, status and
// resid are device arrays.  With `escalate`, a stalled sequence is handed over
// (an internal status) instead of stopped; a launch with `resume` and f64
// continues exactly those sequences and leaves the others alone.  state_f64:
// the state was sized with f64 (needed by any double-precision launch).
bool dense_persist_fits(int B, int D, int T, bool f64);
size_t dense_persist_state_bytes(int B, int T, bool f64);
int launch_dense_persist(const float *W, const float *proj, const float *s0, const float *init, float *traj, int B,
                         int T, int D, float shrink, float tol, int max_iter, int stall_window, bool f64,
                         bool escalate, bool resume, int *iters, int *status, float *resid, void *state,
                         bool state_f64, hipStream_t stream);
// Set (non-zero) when a bounded wait of the launches since the last
// non-resumed one hit its bound.
unsigned *dense_persist_abort_word(void *state, int B, int T, bool state_f64);
// The diagonal linearisations (quasi-Newton, Jacobi, Picard) of the same
// problems in one launch, with the same groups and the same state
// (dense_persist_state_bytes(B, T, false), abort word included); no hand-over.
bool diag_persist_fits(int B, int D, int T);
int launch_diag_persist(const float *W, const float *proj, const float *s0, const float *init, float *traj, int B,
                        int T, int D, Linearization lz, float tol, int max_iter, int stall_window, int *iters,
                        int *status, float *resid, void *state, hipStream_t stream);

// Parallel Broyden (broyden.hip): the block updates and the chunked compressed
// scan of delta_t = A_t delta_{t-1} + c_t, A_t = alpha I + shrink U_t V_t^T.
// Solver mode (ctl set): iteration i = ctl->iter - 1 (the convergence check
// has run); c_t = f^(i)_t - s^(i)_t; blocks are updated from the secants
// against iteration i - 1 first; s^(i+1) = s^(i) + delta goes to the iterate
// buffer that does not hold s^(i).  Standalone mode (ctl null): c given, the
// first n_fixed columns used as they are, delta written to out.
struct DplrArgs {
    int B = 0, T = 0, D = 0;
    int m = 0;                  // columns per block (ring size)
    int chunk = 32, nchunk = 0;
    float alpha = 0.0f, shrink = 1.0f, lambda = 0.0f;
    int multisecant = 0;
    int n_fixed = 0;
    const float *omega = nullptr;                     // [D, m]
    float *U = nullptr, *V = nullptr, *F = nullptr;   // [B, T, m, D]
    const float *c = nullptr;                         // standalone: [B, T, D]
    float *out = nullptr;                             // standalone: delta [B, T, D]
    const float *s0 = nullptr;
    float *s_even = nullptr, *s_odd = nullptr;        // iterate buffers (solver)
    const float *f_even = nullptr, *f_odd = nullptr;  // cell values by iteration parity (solver)
    const SolveControl *ctl = nullptr;
    const int *skip = nullptr;
    float *agg = nullptr;                             // [B * nchunk] records (dplr_record_floats)
    float *entry = nullptr;                           // [B * nchunk, D]
};
int launch_dplr_step(const DplrArgs &a, hipStream_t stream);

// Chunk aggregate record, contiguous per chunk so a run of consecutive chunks
// is one span: with Dp = D rounded up to a multiple of 4, L_j at j Dp, R_j at
// (m + j) Dp, the offset b at 2m Dp, then p (float) and the column count r
// (int bits) at (2m + 1) Dp and + 1, two words of padding.  Words d in [D, Dp)
// of each vector are never written.
__host__ __device__ inline int dplr_padded_dim(int D) { return (D + 3) & ~3; }
__host__ __device__ inline int dplr_record_floats(int m, int D) { return (2 * m + 1) * dplr_padded_dim(D) + 4; }

// Largest Lyapunov exponent along a trajectory (lle.hip): workspace layout and launch.
struct LleLayout {
    float *proj = nullptr;      // input projection [B,T,PD], row-major
    float *F = nullptr;         // per-step Jacobian factors [B,T,NF,D]
    float *junk = nullptr;      // offsets the tanh evaluation also writes (unused)
    unsigned *res_bits = nullptr;
    size_t bytes = 0;
};
LleLayout lle_layout(void *ws, const deer_cell_params_t *p, int B, int T);
int launch_lle(const deer_cell_params_t *p, const float *x, const float *s0, const float *traj, const float *v0, int B,
               int T, double *out, const LleLayout &L, hipStream_t stream);

}  // namespace deer
