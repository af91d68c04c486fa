// Single-pass scan of the diagonal affine recurrence s_t = a_t * s_{t-1} + b_t.
//
// Diagonal blocks stay diagonal when composed, so every channel (b, d) is an
// independent scalar recurrence ("Parallel Broyden Methods", section 2,
// diagonal quasi-Newton).  Two affine maps merge as
//     (a_j, b_j) o (a_i, b_i) = (a_j a_i, a_j b_i + b_j)   (i before j),
// the later map acting on the left (same page, appendix C.2).
//
// Layout [B, T, D], D fastest.  The grid is persistent: one workgroup per
// compute unit (more if occupancy allows).  The chains (one sequence's CH
// channels) are split into ngrp groups (chain c in group c % ngrp), and so are
// the workgroups (workgroup g in group g % ngrp, which keeps a group on one XCD
// when ngrp divides the XCD count).  A group's chunks are numbered time-major
// over its chains and handed out in index order from the group's counter in
// the header, each workgroup drawing its next chunk while it works on the
// current one.  A chunk is a tile of CH channels x L time steps of one
// sequence:
//   1. every thread loads LT consecutive steps of VEC channels into registers
//      (non-temporal 16-byte loads; a wavefront reads whole contiguous row
//      segments, 1 KB for 256-channel tiles) and folds them into one affine
//      pair per channel;
//   2. the time slots of the workgroup are combined through LDS (exclusive
//      prefix per slot, chunk aggregate per channel);
//   3. the chunk publishes its aggregate, looks back over the earlier chunks
//      of the same channels until it meets an inclusive prefix, applies the
//      aggregates in between forward from it (a decoupled look-back made
//      deterministic: the carry is always the left-to-right chain's value), and
//      publishes its own inclusive prefix (the state at its last step);
//   4. every thread replays its registers from the carried-in state and
//      streams s out (non-temporal stores).
// a and b are read once and s written once: 12 bytes per element.  Holding
// 32 steps per thread keeps about 1 KB of loads in flight per thread, which
// is what it takes to approach the HBM roofline on this part.
//
// Look-back descriptors are 64-bit words holding a float and a 32-bit tag
// (epoch * 4 + kind), written and read with agent-scope atomics, so a word is
// valid on its own and no fences are needed.  Forward progress does not
// depend on how many workgroups are resident: a chunk only waits on earlier
// chunks of its chain (smaller indices of the same group), and a group's
// chunks are handed out in index order, only to workgroups of the group
// already running, which take theirs in increasing order.  So a group's
// smallest unfinished chunk is being processed by its holder and waits on
// finished chunks only.  The wait is bounded all the same; if the bound is
// hit the header's abort flag is set and the chunk's carry becomes NaN.
#include <algorithm>
#include <mutex>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 22;

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned long long pack_word(float v, unsigned tag) {
    return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}
__device__ __forceinline__ unsigned word_tag(unsigned long long w) { return static_cast<unsigned>(w >> 32); }
__device__ __forceinline__ float word_val(unsigned long long w) { return __uint_as_float(static_cast<unsigned>(w)); }

__device__ __forceinline__ unsigned long long load_word(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_word(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int VEC, int CH, int LT>
struct DiagGeom {
    static constexpr int LD = CH / VEC;        // threads across a tile row
    static constexpr int NS = kThreads / LD;   // time slots per workgroup
    static constexpr int L = NS * LT;          // time steps per chunk
};

template <int VEC, int CH, int LT>
__global__ __launch_bounds__(kThreads) void diag_scan_kernel(
    const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ s0,
    float *out0, float *out1, const int *__restrict__ out_sel, const int *__restrict__ skip,
    const int *__restrict__ all_done, int T, int D, int groups, int chains, int nchunk, int ngrp,
    ScanHeader *__restrict__ hdr, unsigned long long *__restrict__ desc)
{
    using G = DiagGeom<VEC, CH, LT>;
    constexpr int LD = G::LD, NS = G::NS, L = G::L;

    if (all_done && *all_done) return;   // same value for every workgroup of the launch

    __shared__ float shA[NS][CH];
    __shared__ float shB[NS][CH];
    __shared__ float shC[CH];
    __shared__ long long sh_ticket;

    const int tid = threadIdx.x;
    const unsigned epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tag_agg = epoch * 4u + 1u, tag_inc = epoch * 4u + 2u;
    float *out = (out_sel && (*out_sel & 1)) ? out1 : out0;
    const int slot = tid / LD;
    const int lc = (tid % LD) * VEC;              // channel offset inside the tile
    const int gid = static_cast<int>(blockIdx.x) % ngrp;
    const long long nc = (chains - gid + ngrp - 1) / ngrp;          // chains of the group
    const long long total = nc * nchunk;                            // chunks of the group
    unsigned *ticket = &hdr->ticket[gid];

    if (tid == 0) sh_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    long long cidx = sh_ticket;
    for (; cidx < total;) {
        // the next chunk is drawn now and read back after the look-back, so the
        // round trip overlaps this chunk's loads
        unsigned next = 0u;
        if (tid == 0) next = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int tchunk = static_cast<int>(cidx / nc);
        const int chain = gid + ngrp * static_cast<int>(cidx % nc);
        const int bseq = chain / groups;
        const int grp = chain % groups;
        if (skip && skip[bseq]) {                 // uniform over the workgroup
            __syncthreads();                      // every thread has read sh_ticket
            if (tid == 0) sh_ticket = next;
            __syncthreads();
            cidx = sh_ticket;
            continue;
        }
        const int c0 = grp * CH + lc;             // first channel of this thread
        const bool cvalid = c0 < D;               // VEC == 4 implies D % 4 == 0
        const int t0 = tchunk * L + slot * LT;
        const size_t seq = static_cast<size_t>(bseq) * T * D;

        float av[LT][VEC], bv[LT][VEC];
#pragma unroll
        for (int j = 0; j < LT; ++j) {
            const int t = t0 + j;
            if (cvalid && t < T) {
                const size_t off = seq + static_cast<size_t>(t) * D + c0;
                if constexpr (VEC == 4) {
                    const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(a + off));
                    const v4f y = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(b + off));
#pragma unroll
                    for (int v = 0; v < 4; ++v) { av[j][v] = x[v]; bv[j][v] = y[v]; }
                } else {
                    av[j][0] = __builtin_nontemporal_load(a + off);
                    bv[j][0] = __builtin_nontemporal_load(b + off);
                }
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) { av[j][v] = 1.0f; bv[j][v] = 0.0f; }
            }
        }

        // fold this thread's LT steps into one affine pair per channel
        float A[VEC], Bq[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { A[v] = 1.0f; Bq[v] = 0.0f; }
#pragma unroll
        for (int j = 0; j < LT; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                Bq[v] = av[j][v] * Bq[v] + bv[j][v];
                A[v] = av[j][v] * A[v];
            }
        __syncthreads();   // the previous chunk is done with the LDS tiles
#pragma unroll
        for (int v = 0; v < VEC; ++v) { shA[slot][lc + v] = A[v]; shB[slot][lc + v] = Bq[v]; }
        __syncthreads();

        // exclusive prefix over the earlier time slots of this chunk
        float PA[VEC], PB[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { PA[v] = 1.0f; PB[v] = 0.0f; }
        for (int k = 0; k < slot; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float ak = shA[k][lc + v];
                PB[v] = ak * PB[v] + shB[k][lc + v];
                PA[v] = ak * PA[v];
            }

        // one channel per thread: publish, look back, publish
        for (int c = tid; c < CH; c += kThreads) {
            const int ch = grp * CH + c;
            float carry = 0.0f;
            if (ch < D) {
                float GA = 1.0f, GB = 0.0f;
                for (int k = 0; k < NS; ++k) {
                    const float ak = shA[k][c];
                    GB = ak * GB + shB[k][c];
                    GA = ak * GA;
                }
                const unsigned long long *base = desc + static_cast<size_t>(chain) * nchunk * 3 * CH;
                unsigned long long *mine = desc + (static_cast<size_t>(chain) * nchunk + tchunk) * 3 * CH;
                if (tchunk == 0) {
                    carry = s0 ? s0[static_cast<size_t>(bseq) * D + ch] : 0.0f;
                } else {
                    store_word(mine + c, pack_word(GA, tag_agg));
                    store_word(mine + CH + c, pack_word(GB, tag_agg));
                    carry = chained_carry<4>(base, 3 * CH, c, CH + c, 2 * CH + c, tchunk, tag_agg, tag_inc, &hdr->abort,
                                             kSpinLimit);
                }
                store_word(mine + 2 * CH + c, pack_word(__builtin_fmaf(GA, carry, GB), tag_inc));
            }
            shC[c] = carry;
        }
        if (tid == 0) sh_ticket = next;           // every thread read the current one before the syncs above
        __syncthreads();
        cidx = sh_ticket;

        float st[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) st[v] = PA[v] * shC[lc + v] + PB[v];
#pragma unroll
        for (int j = 0; j < LT; ++j) {
            const int t = t0 + j;
#pragma unroll
            for (int v = 0; v < VEC; ++v) st[v] = av[j][v] * st[v] + bv[j][v];
            if (cvalid && t < T) {
                const size_t off = seq + static_cast<size_t>(t) * D + c0;
                if constexpr (VEC == 4) {
                    v4f y;
                    y[0] = st[0]; y[1] = st[1]; y[2] = st[2]; y[3] = st[3];
                    __builtin_nontemporal_store(y, reinterpret_cast<v4f *>(out + off));
                } else {
                    __builtin_nontemporal_store(st[0], out + off);
                }
            }
        }
    }

    // Last workgroup out resets the done and ticket counters (every workgroup
    // has drawn its last ticket by then) and advances the epoch.
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {
            __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int g = 0; g < ngrp; ++g)
                __hip_atomic_store(&hdr->ticket[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->epoch, epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Tile shapes: 256-channel tiles (a wavefront reads 1 KB rows) for wide
// states, 64-channel tiles otherwise; scalar lanes when D is not a multiple of 4.
enum DiagKind { kWide = 0, kNarrow = 1, kScalar = 2 };
constexpr int kLT = 32;
using GeomWide = DiagGeom<4, 256, kLT>;
using GeomNarrow = DiagGeom<4, 64, kLT>;
using GeomScalar = DiagGeom<1, 64, kLT>;

DiagKind diag_kind(int D)
{
    if (D % 4 != 0) return kScalar;
    return (D >= 256 || D % 256 == 0) ? kWide : kNarrow;
}

// Resident workgroups per compute unit, times compute units (cached per device).
int persistent_capacity(DiagKind k)
{
    static int cache[64][3] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int &slot = cache[dev][k];
    if (slot == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        hipError_t e = hipSuccess;
        if (k == kWide)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, diag_scan_kernel<4, 256, kLT>, kThreads, 0);
        else if (k == kNarrow)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, diag_scan_kernel<4, 64, kLT>, kThreads, 0);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, diag_scan_kernel<1, 64, kLT>, kThreads, 0);
        if (e != hipSuccess || per_cu < 1) per_cu = 1;
        slot = cus * per_cu;
    }
    return slot;
}

// Look-back state of linear_scan_diag_noalloc: a file-scope device array
// instead of a caller workspace.  Each device that loads the library holds its
// own copy until the process ends.  In host code `scratch` is only a symbol
// handle; its device address comes from hipGetSymbolAddress (per device).
static __device__ __align__(256) unsigned char scratch[DEER_NOALLOC_SCRATCH_BYTES];

__global__ void scratch_zero_kernel(unsigned *__restrict__ p, size_t nwords)
{
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < nwords; i += stride) p[i] = 0u;
}

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

}  // namespace

int diag_scan_static_state(void **state, hipStream_t stream)
{
    int dev = 0;
    DEER_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kScratchDevices)
        return fail(DEER_ERR_UNSUPPORTED, "linear_scan_diag_noalloc: device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // Once per device: take this device's address of the array and clear it
        // (a zero header and zero descriptors: no descriptor carries a valid tag,
        // and every later launch leaves the header ready for the next one).
        void *ptr = nullptr;
        DEER_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return fail(DEER_ERR_HIP, "linear_scan_diag_noalloc: no device address for the scratch array");
        const size_t words = DEER_NOALLOC_SCRATCH_BYTES / 4;
        hipLaunchKernelGGL(scratch_zero_kernel, dim3(1024), dim3(256), 0, stream, static_cast<unsigned *>(ptr), words);
        DEER_HIP(hipGetLastError());
        DEER_HIP(hipStreamSynchronize(stream));
        g_scratch_ptr[dev] = ptr;
    }
    *state = g_scratch_ptr[dev];
    return DEER_OK;
}

DiagScanPlan diag_scan_plan(int B, int T, int D)
{
    DiagScanPlan p{};
    p.B = B;
    p.T = T;
    p.D = D;
    const DiagKind k = diag_kind(D);
    p.vec = (k == kScalar) ? 1 : 4;
    p.ch = (k == kWide) ? 256 : 64;
    p.chunk_len = (k == kWide) ? GeomWide::L : (k == kNarrow) ? GeomNarrow::L : GeomScalar::L;
    p.groups = (D + p.ch - 1) / p.ch;
    p.chains = B * p.groups;
    p.nchunk = (T + p.chunk_len - 1) / p.chunk_len;
    p.desc_words = static_cast<size_t>(p.chains) * p.nchunk * 3 * p.ch;
    return p;
}

size_t diag_scan_state_bytes(int B, int T, int D)
{
    const DiagScanPlan p = diag_scan_plan(B, T, D);
    return sizeof(ScanHeader) + align_up(p.desc_words * sizeof(unsigned long long));
}

int launch_diag_scan(const float *a, const float *b, const float *s0, float *out0, float *out1,
                     const int *out_sel, const int *skip, const int *all_done, int B, int T, int D,
                     void *state, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    const DiagScanPlan p = diag_scan_plan(B, T, D);
    const long long total = static_cast<long long>(p.chains) * p.nchunk;
    const DiagKind k = diag_kind(D);
    const unsigned grid = static_cast<unsigned>(std::min<long long>(total, persistent_capacity(k)));
    if (total + 2LL * grid >= (1LL << 32))       // tickets are 32-bit
        return fail(DEER_ERR_UNSUPPORTED, "diagonal scan: too many chunks (above 2^31)");
    const int ngrp = static_cast<int>(std::min<long long>({kTicketGroups, p.chains, grid}));
    auto *hdr = static_cast<ScanHeader *>(state);
    auto *desc = reinterpret_cast<unsigned long long *>(static_cast<char *>(state) + sizeof(ScanHeader));
    if (k == kWide)
        DEER_LAUNCH((diag_scan_kernel<4, 256, kLT>), dim3(grid), dim3(kThreads), 0, stream, a, b, s0, out0,
                           out1, out_sel, skip, all_done, T, D, p.groups, p.chains, p.nchunk, ngrp, hdr, desc);
    else if (k == kNarrow)
        DEER_LAUNCH((diag_scan_kernel<4, 64, kLT>), dim3(grid), dim3(kThreads), 0, stream, a, b, s0, out0,
                           out1, out_sel, skip, all_done, T, D, p.groups, p.chains, p.nchunk, ngrp, hdr, desc);
    else
        DEER_LAUNCH((diag_scan_kernel<1, 64, kLT>), dim3(grid), dim3(kThreads), 0, stream, a, b, s0, out0,
                           out1, out_sel, skip, all_done, T, D, p.groups, p.chains, p.nchunk, ngrp, hdr, desc);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace deer
