// Whole dense-DEER solves of small tanh problems (D <= 16, T <= 8192) in one
// launch.
//
// The multi-launch loop costs five launches and a host poll per Newton
// iteration (about 0.1 ms), while one iteration of such a problem moves a few
// tens of MB that stay in the device caches.  Here the iterations run inside one
// kernel.  Every sequence is its own problem ("Parallel Broyden Methods",
// section 2: the trajectory of each sequence is the root of its own residual),
// so the kernel gives each sequence a group of G workgroups that synchronise
// only among themselves (a counter per sequence in global memory), and a group
// leaves the loop as soon as its sequence stops.
//
// Workgroup w of a group owns NC = 8 consecutive chunks of L = 64 positions,
// one wavefront per chunk; its states s_{tb-1..te-1} stay in LDS from one
// iteration to the next.  Per iteration i:
//   1. evaluation of its positions, each wavefront its chunk: f_t =
//      tanh(W s_{t-1} + p_t) (W s_{t-1} for 16 positions at a time on the matrix
//      cores), the factored Jacobian d_t = (1 - k)(1 - f_t^2) (A_t =
//      diag(d_t) W), the offset b_t = f_t - d_t (W s_{t-1}), and the residual
//      maximum and finite-step front of the sequence (atomics on per-sequence
//      words).  The state before the range comes from the left neighbour's
//      replay; only wavefront 0 waits for it, after its other positions;
//   2. its chunk aggregates (P_c = A_last ... A_first, B_c), each wavefront
//      its chunk, the products on the matrix cores (v_mfma 16x16x4), then the
//      workgroup aggregate (the chunk aggregates composed in order), published;
//   -- group barrier --
//   3. the stopping decision, identical in every workgroup of the group (the
//      same residual words, the same rule as the multi-launch loop); a stopping
//      sequence writes its iterate out;
//   4. the state entering its range: s0 pushed through the aggregates of the
//      earlier workgroups in order, then through its own chunks;
//   5. replay of its chunks from their entries into the state rows; the last
//      state of the range goes to the right neighbour.
// Affine maps merge with the later one on the left ("Parallel Broyden
// Methods", appendix C.2); the chunked tree with a sequential carry is one of
// the trees its appendix B.4 allows.  ACC is the accumulation type of the
// products, offsets, carries and replayed states (float, or double).
//
// Progress: a workgroup only waits on workgroups of its own group with a lower
// index (the left neighbour) or on all of them (the barrier).  Workgroups are
// dispatched in order, so the lowest unfinished group always has every
// workgroup resident or about to be; all waits are bounded all the same (the
// abort word then reports a device error).
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace deer {
namespace {

constexpr int kNC = 8;          // chunks per workgroup, one wavefront each
constexpr int kThreads = 64 * kNC;
constexpr int kL = 64;          // positions per chunk
constexpr int kSub = 16;        // positions per sub-chunk (one row of 16 lanes each)
constexpr int kNS = kL / kSub;  // sub-chunks per chunk
constexpr int kDP = 16;         // padded state size
constexpr int kMaxGroup = 16;   // workgroups per sequence
constexpr unsigned kBarrierSpin = 1u << 22;   // polls of a barrier wait (seconds)
constexpr int kPendingEscalation = 16;        // status of a sequence handed to the double-precision launch
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

// 16x16x4 MFMA operand and accumulator layouts (measured): accumulator v of
// lane l holds C[row16(v, l / 16)][l % 16], rows 4 (l / 16) + v for float and
// l / 16 + 4 v for double.  A product's accumulators are the next product's B
// operands when instruction u contracts over k = row16(u, l / 16).
template <class ACC>
__device__ __forceinline__ int row16(int v, int g) { return sizeof(ACC) == 8 ? g + 4 * v : 4 * g + v; }

template <class ACC>
__device__ __forceinline__ void mfma16(ACC a, ACC b, ACC (&acc)[4]);
template <>
__device__ __forceinline__ void mfma16<float>(float a, float b, float (&acc)[4])
{
    v4f c = {acc[0], acc[1], acc[2], acc[3]};
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    acc[0] = c[0]; acc[1] = c[1]; acc[2] = c[2]; acc[3] = c[3];
}
template <>
__device__ __forceinline__ void mfma16<double>(double a, double b, double (&acc)[4])
{
    v4d c = {acc[0], acc[1], acc[2], acc[3]};
    c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    acc[0] = c[0]; acc[1] = c[1]; acc[2] = c[2]; acc[3] = c[3];
}

// y_j = sum_k w_j[k] x_k for a 16-vector held once per row of 16 lanes (x_k in
// lane k of the row), with w[k] = row j of the matrix at the column that row
// rotation k brings to lane j (src[k] of RowRotations::sources): the rotated
// fused multiply-adds of RowRotations, even and odd terms in two sums.
template <class ACC>
__device__ __forceinline__ ACC row_dot(ACC x, const ACC (&w)[kDP]);
template <>
__device__ __forceinline__ float row_dot<float>(float x, const float (&w)[kDP])
{
    float a0 = w[0] * x, a1 = 0.0f;
    RowRotations::contract(x, w, a0, a1);
    return a0 + a1;
}
// Sum of a value over the four rows of 16 lanes, in every lane: row pairs are
// added through v_permlane16_swap, then the halves through v_permlane32_swap.
// Whatever rows a swap pairs, each lane adds the same two operands (addition
// commutes), so every row ends with the same bits.
__device__ __forceinline__ float rows_sum(float p)
{
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    const float q = __uint_as_float(t[0]) + __uint_as_float(t[1]);
    const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(q), __float_as_uint(q), false, false);
    return __uint_as_float(u[0]) + __uint_as_float(u[1]);
}
__device__ __forceinline__ double join64(unsigned lo, unsigned hi)
{
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
__device__ __forceinline__ double rows_sum(double p)
{
    const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(p));
    const unsigned lo = static_cast<unsigned>(b), hi = static_cast<unsigned>(b >> 32);
    const auto tl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto th = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const double q = join64(tl[0], th[0]) + join64(tl[1], th[1]);
    const unsigned long long c = static_cast<unsigned long long>(__double_as_longlong(q));
    const unsigned lo2 = static_cast<unsigned>(c), hi2 = static_cast<unsigned>(c >> 32);
    const auto ul = __builtin_amdgcn_permlane32_swap(lo2, lo2, false, false);
    const auto uh = __builtin_amdgcn_permlane32_swap(hi2, hi2, false, false);
    return join64(ul[0], uh[0]) + join64(ul[1], uh[1]);
}

// y_j = sum_k M[j][k] x_k for a 16-vector held once per row of 16 lanes (x_j
// in lane j of every row): the vector goes through a per-wavefront LDS line,
// lane (j, g) multiplies columns 4 g .. 4 g + 3 of row j (wq) with the four
// values it reads back, and the rows' partial sums are added across rows.
// The fences keep the compiler from treating the line as private to the
// writing lanes.
template <class ACC>
__device__ __forceinline__ ACC quad_dot(ACC x, const ACC (&wq)[4], ACC *line, int j, int g)
{
    line[j] = x;                                  // every row of lanes writes the same value
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    ACC p;
    if constexpr (sizeof(ACC) == 4) {
        const v4f v = *reinterpret_cast<const v4f *>(line + 4 * g);
        p = wq[0] * v[0];
        p = __builtin_fmaf(wq[1], v[1], p);
        p = __builtin_fmaf(wq[2], v[2], p);
        p = __builtin_fmaf(wq[3], v[3], p);
    } else {
        typedef double v2d __attribute__((ext_vector_type(2)));
        const v2d v0 = *reinterpret_cast<const v2d *>(line + 4 * g);
        const v2d v1 = *reinterpret_cast<const v2d *>(line + 4 * g + 2);
        p = wq[0] * v0[0];
        p = __builtin_fma(wq[1], v0[1], p);
        p = __builtin_fma(wq[2], v1[0], p);
        p = __builtin_fma(wq[3], v1[1], p);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return rows_sum(p);
}

// The same with the matrix row-major in LDS.
template <class ACC>
__device__ __forceinline__ ACC lds_quad_dot(const ACC *M, ACC x, ACC *line, int j, int g)
{
    ACC wq[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) wq[m] = M[j * kDP + 4 * g + m];
    return quad_dot<ACC>(x, wq, line, j, g);
}

// y_j = sum_k W[j][k] x_k with each row of 16 lanes holding its own 16-vector
// (x_j in lane j of the row) and contracting it alone: float by the DPP row
// rotations (w in rotation order), double through the row's own LDS line
// (w in natural order).
template <class ACC>
__device__ __forceinline__ ACC row_dot16(ACC x, const float (&w)[kDP], ACC *row_line, int j);
template <>
__device__ __forceinline__ float row_dot16<float>(float x, const float (&w)[kDP], float *, int)
{
    return row_dot<float>(x, w);
}
template <>
__device__ __forceinline__ double row_dot16<double>(double x, const float (&w)[kDP], double *rl, int j)
{
    rl[j] = x;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    typedef double v2d __attribute__((ext_vector_type(2)));
    const v2d *p = reinterpret_cast<const v2d *>(rl);
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int k2 = 0; k2 < kDP / 2; ++k2) {
        const v2d v = p[k2];
        a0 = __builtin_fma(static_cast<double>(w[2 * k2]), v[0], a0);
        a1 = __builtin_fma(static_cast<double>(w[2 * k2 + 1]), v[1], a1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return a0 + a1;
}

struct PersistArgs {
    const float *W;        // [D, D]
    const float *proj;     // [B, T, D]: U x_t + b
    const float *s0;       // [B, D] or null
    const float *init;     // [B, T, D]: the starting iterate s^(i0), or null for zeros (may alias traj)
    float *traj;           // [B, T, D]: the iterate a sequence stops at, on exit
    int B, T, D, nchunk, G, max_iter, stall_window;
    float tol, shrink;
    int lin_kind;          // diagonal kernel: the linearisation (LinKind)
    int *iters, *status;   // [B]
    float *resid;          // [B]
    // Exchanged between the workgroups of a group as tagged words (below):
    unsigned long long *slot;   // [2][B][G]: residual maximum, front and tag of each workgroup, by parity
    unsigned long long *agg;    // [2][B][G][AGGW]: workgroup aggregates, by parity (the diagonal
                                //   kernel uses the first 2 x 16 words of each)
    unsigned long long *xch;    // [B][G][16]: last state of each workgroup's range
    int *keep;             // [B][2] best finite-step front and iteration of its last advance, of a
                           // sequence handed over
    unsigned *esc_flag;    // set once a sequence stalled (with `escalate`): every sequence hands over
    unsigned *abort_flag;
    int escalate;          // a stall hands the sequence over instead of stopping it
    int resume;            // continue the handed-over sequences, skip the rest
};

// Tagged words.  Every value one workgroup passes to another travels in a
// 64-bit word that also carries the iteration it belongs to, written and read
// with single 64-bit relaxed atomic accesses at device scope: a reader that
// sees the expected tag has the value of that iteration, so no fence or flag
// has to order the words (each word validates itself).  Float words: value in
// the low half, tag i + 1 in the high half; a double takes two words.  Residual
// slots: maximum |r| bits in the low half, then the front (15 bits, 0x7FFF for
// none; positions are below 8192), a bit that asks for the hand-over to double
// precision, and a 16-bit tag in 1..65535.  The buffers are zeroed at launch,
// and zero is never an expected tag.
__device__ __forceinline__ unsigned tag32(int i) { return static_cast<unsigned>(i) + 1u; }
__device__ __forceinline__ unsigned tag16(int i) { return static_cast<unsigned>(i + 1) % 0xFFFFu + 1u; }
__device__ __forceinline__ void put_word(unsigned long long *p, unsigned bits, unsigned tag)
{
    __hip_atomic_store(p, (static_cast<unsigned long long>(tag) << 32) | bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_word(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long slot_word(unsigned rmax, unsigned front, unsigned esc, int i)
{
    const unsigned f16 = (front == kNoFront ? 0x7FFFu : front) | (esc ? 0x8000u : 0u);
    return (static_cast<unsigned long long>((f16 << 16) | tag16(i)) << 32) | rmax;
}

// ACC values as float words: one word per float, two per double.
template <class ACC> struct Words;
template <> struct Words<float> {
    static constexpr int N = 1;
    static __device__ __forceinline__ void put(unsigned long long *p, float v, unsigned t)
    {
        put_word(p, __float_as_uint(v), t);
    }
    // true when the word carries tag t (then v is its value)
    static __device__ __forceinline__ bool get(const unsigned long long *p, unsigned t, float &v)
    {
        const unsigned long long u = get_word(p);
        v = __uint_as_float(static_cast<unsigned>(u));
        return static_cast<unsigned>(u >> 32) == t;
    }
};
template <> struct Words<double> {
    static constexpr int N = 2;
    static __device__ __forceinline__ void put(unsigned long long *p, double v, unsigned t)
    {
        const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(v));
        put_word(p, static_cast<unsigned>(b), t);
        put_word(p + 1, static_cast<unsigned>(b >> 32), t);
    }
    static __device__ __forceinline__ bool get(const unsigned long long *p, unsigned t, double &v)
    {
        const unsigned long long lo = get_word(p), hi = get_word(p + 1);
        v = __longlong_as_double(static_cast<long long>((hi << 32) | (lo & 0xffffffffull)));
        return static_cast<unsigned>(lo >> 32) == t && static_cast<unsigned>(hi >> 32) == t;
    }
};

// One bounded poll step: returns 1 when the wait is to be abandoned (the bound
// was hit, which sets the abort word, or another workgroup set it).
__device__ __forceinline__ int poll_step(unsigned &spins, unsigned *abort_flag)
{
    ++spins;
    if ((spins & 255u) == 0u && __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return 1;
    if (spins > kBarrierSpin) {
        __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 1;
    }
    __builtin_amdgcn_s_sleep(1);
    return 0;
}

template <class ACC>
struct PersistLds {
    static constexpr int NP = kNC * kL;                 // positions of a workgroup
    __align__(16) float S[(NP + 1) * kDP];              // S[r] = s_{tb - 1 + r} of the current iterate
    __align__(16) float d[(NP + 2) * kDP];              // d_t, b_t at local position r (two rows of
    __align__(16) float b[(NP + 2) * kDP];              // padding for reads one step ahead)
    ACC P[kNC * kDP * kDP];                             // chunk products, row-major
    ACC Bc[kNC * kDP];                                  // chunk offsets
    ACC ent[kNC * kDP];                                 // states entering the chunks
    ACC Wg[(kMaxGroup - 1) * (kDP * kDP + kDP)];        // earlier workgroups' aggregates
    __align__(16) ACC line[kNC][kDP];                   // per-wavefront line of the quarter-row contractions
    __align__(16) ACC line4[kNC][kNS][kDP];             // per-row lines of the double row contractions
    unsigned red[2][kNC];                               // per-wavefront residual maximum and front
    unsigned dec_r, dec_f, dec_esc;                     // the group's residual maximum, front, hand-over
    int abort_now;                                      // a wait gave up (from wavefront 0)
};

template <class ACC>
__global__ __launch_bounds__(kThreads) void dense_persist_kernel(PersistArgs a)
{
    __shared__ PersistLds<ACC> sh;
    constexpr int AGG = kDP * kDP + kDP;
    constexpr int NP = kNC * kL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bseq = blockIdx.x / a.G, w = blockIdx.x % a.G;
    const int c0 = w * kNC;
    const int nch = min(kNC, a.nchunk - c0);             // >= 1
    const int tb = c0 * kL, te = min(a.T, (c0 + nch) * kL), np = te - tb;
    const int D = a.D;
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    constexpr int AGGW = AGG * Words<ACC>::N;             // words of one aggregate
    const size_t aggs = static_cast<size_t>(a.B) * a.G * AGGW;   // one parity of the aggregates
    const size_t slots = static_cast<size_t>(a.B) * a.G;         // one parity of the residual slots
    unsigned long long *agg0 = a.agg + static_cast<size_t>(bseq) * a.G * AGGW;
    unsigned long long *slot0 = a.slot + static_cast<size_t>(bseq) * a.G;
    const unsigned long long *xin = a.xch + (static_cast<size_t>(bseq) * a.G + (w > 0 ? w - 1 : 0)) * kDP;
    unsigned long long *xout = a.xch + (static_cast<size_t>(bseq) * a.G + w) * kDP;

    int i0 = 0, best = -1, last_adv = 0;                 // finite-step check (the same in every workgroup)
    if (a.resume) {                                      // a resumed sequence keeps its best front and
        if (a.status[bseq] != kPendingEscalation) return;   // starts a fresh window where it stopped
        i0 = a.iters[bseq];
        best = a.keep[2 * bseq];
        last_adv = a.keep[2 * bseq + 1];
    }

    // W in the layouts the phases need (zero past D)
    const int j = lane & 15, g = lane >> 4;              // MFMA lane coordinates
    ACC WA[4], Wcol[4];
    float WE[4];                                         // A operand of the float evaluation
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int k = row16<ACC>(u, g);
        WA[u] = static_cast<ACC>((j < D && k < D) ? a.W[j * D + k] : 0.0f);
        Wcol[u] = static_cast<ACC>((k < D && j < D) ? a.W[k * D + j] : 0.0f);
        WE[u] = (j < D && 4 * g + u < D) ? a.W[j * D + 4 * g + u] : 0.0f;
    }
    int src[kDP];                                        // column of W that row rotation k brings to lane j
    src[0] = j;
    RowRotations::sources(j, src);
    float Wrow[kDP];                                     // row j of W in the order row_dot16 reads it
#pragma unroll
    for (int k = 0; k < kDP; ++k) {
        const int c = sizeof(ACC) == 4 ? src[k] : k;
        Wrow[k] = (j < D && c < D) ? a.W[j * D + c] : 0.0f;
    }
    ACC *line = sh.line[wave];                           // per-wavefront line of the quarter-row contractions
    ACC *row_line = sh.line4[wave][g];                   // per-row line of the row contractions
    ACC *scratch = sh.Wg + wave * kDP * kDP;             // per-wavefront 16 x 16 matrix (compose, replay)
    const ACC xs0 = static_cast<ACC>((a.s0 && j < D) ? a.s0[static_cast<size_t>(bseq) * D + j] : 0.0f);

    // the input projection at the lane's evaluation outputs (position r0 + 16 q + j,
    // channels 4 g .. 4 g + 3), held for the whole solve
    const int r0 = wave * kL, n = wave < nch ? min(kL, np - r0) : 0;   // the wavefront's chunk
    float pr[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = min(r0 + 16 * q + j, np - 1);
            const int c = min(4 * g + v, D - 1);
            pr[q][v] = a.proj[(seq + tb + r) * D + c];
        }
    // the iterate s^(i0) with the state before the range (s0 or the left neighbour's last); a
    // range read here is written back only after the group's first barrier, which this
    // workgroup's slot holds up, so `init` may alias `traj`
    for (int e = tid; e < (np + 1) * kDP; e += kThreads) {
        const int r = e / kDP, k = e % kDP;
        const int t = tb - 1 + r;
        const int kc = k < D ? k : D - 1;
        const float *src_p = (t < 0) ? (a.s0 ? a.s0 + static_cast<size_t>(bseq) * D + kc : a.W)
                                     : (a.init ? a.init + (seq + t) * D + kc : a.W);
        const float v = *src_p;
        sh.S[e] = (k < D && (t < 0 ? a.s0 != nullptr : a.init != nullptr)) ? v : 0.0f;
    }
    if (tid == 0) sh.abort_now = 0;
    __syncthreads();

    // Evaluation of 16 positions r = r0 + 16 q + j: W s_{t-1} on the matrix
    // cores (accumulator v of lane (j, g): channel 4 g + v of position j), then
    // the lane's 4 channels.
    auto eval16 = [&](int q, unsigned &rmax, unsigned &fmin) {
        const int p = 16 * q + j, r = r0 + p;
        const bool pv = p < n;
        const int rr = pv ? r : r0;
        const v4f sv = *reinterpret_cast<const v4f *>(&sh.S[rr * kDP + 4 * g]);
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(WE[u], sv[u], acc, 0, 0, 0);
        const v4f nx = *reinterpret_cast<const v4f *>(&sh.S[(rr + 1) * kDP + 4 * g]);
        v4f dv, bv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = 4 * g + v;
            const float ws = acc[v];
            const float f = tanhf(ws + pr[q][v]);
            const float dd = a.shrink * (1.0f - f * f);
            const bool cv = c < D;
            dv[v] = cv ? dd : 0.0f;
            bv[v] = cv ? f - dd * ws : 0.0f;
            if (cv && pv) {
                const float ra = fabsf(nx[v] - f);
                rmax = max(rmax, __float_as_uint(ra));
                fmin = min(fmin, front_of(ra, a.tol, tb + r));
            }
        }
        if (pv) {
            *reinterpret_cast<v4f *>(&sh.d[r * kDP + 4 * g]) = dv;
            *reinterpret_cast<v4f *>(&sh.b[r * kDP + 4 * g]) = bv;
        }
    };

    unsigned target = 0;
    for (int i = i0;; ++i) {
        const int slot = i % 3;
        // whether some sequence has asked for the hand-over (read early, used in the slot)
        unsigned esc_seen = 0u;
        if (a.escalate && tid == 0) esc_seen = __hip_atomic_load(a.esc_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // ---- 1. evaluation of the wavefront's chunk; wavefront 0 takes its first
        // 16 positions last, once the state before the range is in (from the left
        // neighbour's replay; the state rows hold it at the first iteration)
        unsigned rmax = 0u, fmin = kNoFront;
        if (wave < nch) {
            eval16(3, rmax, fmin);
            eval16(2, rmax, fmin);
            eval16(1, rmax, fmin);
            if (wave == 0 && w > 0 && i > i0) {
                // lanes 0..15 wait for the 16 words of the left neighbour's last state
                float v = 0.0f;
                bool ok = lane >= kDP;
                unsigned spins = 0;
                int ab = 0;
                for (;;) {
                    if (!ok) ok = Words<float>::get(xin + lane, tag32(i - 1), v);
                    if (__all(ok)) break;
                    if (poll_step(spins, a.abort_flag)) { ab = 1; break; }
                }
                if (lane < kDP) sh.S[lane] = v;
                if (__builtin_amdgcn_readfirstlane(ab) && lane == 0) sh.abort_now = 1;
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
            }
            eval16(0, rmax, fmin);
        }
        for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(rmax), o, 64)));
        fmin = wave_min_u32(fmin);
        if (lane == 0) { sh.red[0][wave] = rmax; sh.red[1][wave] = fmin; }
        // the chunk's d and b rows were written by other lanes of this wavefront
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // ---- 2. chunk aggregates: wavefront q composes chunk q as four
        // sub-chunks of 16 positions.  Sub-chunk k's product runs as Q_0 = W,
        // Q_s = (W diag(d_{s-1})) Q_{s-1}, P_k = diag(d_last) Q_last: the diagonal
        // scales the A operand, each step's accumulators are the next step's B
        // operands, and the four chains interleave on the matrix cores.  Row k of
        // lanes runs sub-chunk k's offset chain B <- d_s (W B) + b_s.  Then the
        // chunk aggregate is P_3 P_2 P_1 P_0 with B folded the same way; P_0..P_2
        // and B_0..B_2 stay in registers for the replay's sub-chunk entries.
        ACC Pk[kNS - 1][4] = {}, Bk[kNS - 1] = {};
        if (wave < nch) {
            const float *dq = sh.d + r0 * kDP, *bq = sh.b + r0 * kDP;
            int nk[kNS];                                   // positions of sub-chunk k
#pragma unroll
            for (int k = 0; k < kNS; ++k) nk[k] = min(max(n - kSub * k, 0), kSub);
            ACC Q[kNS][4];
#pragma unroll
            for (int k = 0; k < kNS; ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v) Q[k][v] = Wcol[v];
            // step st of every sub-chunk's chain: the four chains' instructions
            // interleave, so no MFMA waits on the one before it.  A chain past its
            // sub-chunk's end keeps its product (uniform selects; full chunks, the
            // common case, take the loop without them).
            auto chain_step = [&](int st, auto full) {
                ACC acc[kNS][4];
#pragma unroll
                for (int k = 0; k < kNS; ++k)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[k][v] = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int k = 0; k < kNS; ++k) {
                        const float dv = dq[(kSub * k + st - 1) * kDP + row16<ACC>(u, g)];
                        mfma16<ACC>(WA[u] * static_cast<ACC>(dv), Q[k][u], acc[k]);
                    }
#pragma unroll
                for (int k = 0; k < kNS; ++k) {
                    const bool live = decltype(full)::value || st < nk[k];
#pragma unroll
                    for (int v = 0; v < 4; ++v) Q[k][v] = live ? acc[k][v] : Q[k][v];
                }
            };
            if (n == kL) {
                for (int st = 1; st < kSub; ++st) chain_step(st, std::true_type{});
            } else {
                for (int st = 1; st < kSub; ++st) chain_step(st, std::false_type{});
            }
            // offset chains, row g of lanes for sub-chunk g
            const int ng = nk[0] * (g == 0) + nk[1] * (g == 1) + nk[2] * (g == 2) + nk[3] * (g == 3);
            const float *dg = dq + kSub * g * kDP, *bg = bq + kSub * g * kDP;
            ACC x = ng > 0 ? static_cast<ACC>(bg[j]) : static_cast<ACC>(0);
            for (int st = 1; st < kSub; ++st) {
                const float dc = dg[st * kDP + j], bc = bg[st * kDP + j];   // padding rows past the chunk
                const ACC y = row_dot16<ACC>(x, Wrow, row_line, j);
                const ACC xn = static_cast<ACC>(dc) * y + static_cast<ACC>(bc);
                x = st < ng ? xn : x;
            }
            // the chunk aggregate: P = P_{K-1} ... P_0, B = P_{K-1}(... (P_1 B_0 + B_1) ...) + B_{K-1}
            ACC *scr = scratch;                               // this wavefront's 16 x 16 matrix
            ACC Pc[4], Bc;
            auto sub_P = [&](int k, ACC (&Pm)[4]) {           // P_k in accumulator layout
                const float *dl = dq + (kSub * k + nk[k] - 1) * kDP;
#pragma unroll
                for (int v = 0; v < 4; ++v) Pm[v] = static_cast<ACC>(dl[row16<ACC>(v, g)]) * Q[k][v];
            };
            auto row_bcast = [&](ACC val, int k) -> ACC {     // row k's value in every row
                if (g == k) line[j] = val;
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
                const ACC r = line[j];
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
                return r;
            };
            sub_P(0, Pc);
            Bc = row_bcast(x, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) Pk[0][v] = Pc[v];
            Bk[0] = Bc;
#pragma unroll
            for (int k = 1; k < kNS; ++k) {
                if (nk[k] > 0) {
                    ACC Pm[4];
                    sub_P(k, Pm);
                    const ACC bk = row_bcast(x, k);
                    if (k < kNS - 1) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) Pk[k][v] = Pm[v];
                        Bk[k] = bk;
                    }
                    // P_k to the scratch row-major, then Pc <- P_k Pc, Bc <- P_k Bc + B_k
#pragma unroll
                    for (int v = 0; v < 4; ++v) scr[row16<ACC>(v, g) * kDP + j] = Pm[v];
                    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    ACC acc[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int u = 0; u < 4; ++u) mfma16<ACC>(scr[j * kDP + row16<ACC>(u, g)], Pc[u], acc);
#pragma unroll
                    for (int v = 0; v < 4; ++v) Pc[v] = acc[v];
                    Bc = lds_quad_dot<ACC>(scr, Bc, line, j, g) + bk;
                    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                }
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sh.P[wave * kDP * kDP + row16<ACC>(v, g) * kDP + j] = Pc[v];
            if (g == 0) sh.Bc[wave * kDP + j] = Bc;
        }
        __syncthreads();
        if (sh.abort_now) break;
        // the workgroup aggregate (chunk aggregates composed in order) for the later workgroups
        unsigned long long *agg = agg0 + (i & 1) * aggs;
        if (wave == 0 && w + 1 < a.G) {
            ACC Pw[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) Pw[v] = sh.P[row16<ACC>(v, g) * kDP + j];
            ACC Bw = sh.Bc[j];
            for (int q = 1; q < nch; ++q) {
                const ACC *Pq = sh.P + q * kDP * kDP;
                ACC acc[4] = {0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < 4; ++u) mfma16<ACC>(Pq[j * kDP + row16<ACC>(u, g)], Pw[u], acc);
#pragma unroll
                for (int v = 0; v < 4; ++v) Pw[v] = acc[v];
                Bw = lds_quad_dot<ACC>(Pq, Bw, line, j, g) + sh.Bc[q * kDP + j];
            }
            unsigned long long *dst = agg + static_cast<size_t>(w) * AGGW;
            const unsigned t = tag32(i);
#pragma unroll
            for (int v = 0; v < 4; ++v) Words<ACC>::put(dst + (row16<ACC>(v, g) * kDP + j) * Words<ACC>::N, Pw[v], t);
            if (g == 0) Words<ACC>::put(dst + (kDP * kDP + j) * Words<ACC>::N, Bw, t);
        }
        // the workgroup's residual maximum and front, after its aggregate
        if (tid == 0) {
            unsigned m = sh.red[0][0], f = sh.red[1][0];
            for (int q = 1; q < kNC; ++q) { m = max(m, sh.red[0][q]); f = min(f, sh.red[1][q]); }
            __hip_atomic_store(slot0 + (i & 1) * slots + w, slot_word(m, f, esc_seen, i), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- wait for every workgroup's residual slot of this iteration (lanes
        // 0..G-1 of wavefront 0), then combine them
        if (wave == 0) {
            unsigned long long v = 0;
            bool ok = lane >= a.G;
            unsigned spins = 0;
            int ab = 0;
            for (;;) {
                if (!ok) {
                    v = get_word(slot0 + (i & 1) * slots + lane);
                    ok = (static_cast<unsigned>(v >> 32) & 0xFFFFu) == tag16(i);
                }
                if (__all(ok)) break;
                if (poll_step(spins, a.abort_flag)) { ab = 1; break; }
            }
            unsigned m = lane < a.G ? static_cast<unsigned>(v) : 0u;
            unsigned f = lane < a.G ? static_cast<unsigned>(v >> 48) & 0x7FFFu : 0x7FFFu;
            const bool esc = lane < a.G && ((v >> 63) & 1ull);
            for (int o = 32; o > 0; o >>= 1) {
                m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), o, 64)));
                f = min(f, static_cast<unsigned>(__shfl_xor(static_cast<int>(f), o, 64)));
            }
            const bool esc_any = __any(esc);
            if (lane == 0) {
                sh.dec_r = m;
                sh.dec_f = f == 0x7FFFu ? kNoFront : f;
                sh.dec_esc = esc_any ? 1u : 0u;
                sh.abort_now = __builtin_amdgcn_readfirstlane(ab);
            }
        }
        __syncthreads();
        if (sh.abort_now) break;

        // ---- 3. the stopping decision (the same words in every workgroup of the group)
        const float r = __uint_as_float(sh.dec_r);
        const unsigned fr = sh.dec_f;
        int stop = -1;
        if (r <= a.tol) {
            stop = DEER_SEQ_CONVERGED;
        } else if (i >= a.max_iter) {
            stop = __builtin_isfinite(r) ? DEER_SEQ_NOT_CONVERGED : DEER_SEQ_NONFINITE;
        } else {
            bool stalled = false;
            if (a.stall_window > 0) {
                const int f = fr > 0x7FFFFFFFu ? 0x7FFFFFFF : static_cast<int>(fr);
                if (f > best) {
                    best = f;
                    last_adv = i;
                } else if (best < i && i - last_adv >= a.stall_window) {
                    stalled = true;
                }
            }
            if (stalled && !a.escalate) {
                stop = DEER_SEQ_STALLED;
            } else if (stalled || (a.escalate && sh.dec_esc)) {
                // handed over to double precision at this iteration; a stalled
                // sequence starts a fresh window there, the others keep theirs
                stop = kPendingEscalation;
                if (stalled) last_adv = i;
            }
        }
        if (stop >= 0) {
            // the iterate s^(i) of the range goes out
            for (int e = tid; e < np * kDP; e += kThreads) {
                const int k = e % kDP;
                if (k < D) a.traj[(seq + tb + e / kDP) * D + k] = sh.S[kDP + e];
            }
            if (w == 0 && tid == 0) {
                a.iters[bseq] = i;
                a.status[bseq] = stop;
                a.resid[bseq] = r;
                if (stop == kPendingEscalation) {
                    a.keep[2 * bseq] = best;
                    a.keep[2 * bseq + 1] = last_adv;
                    __hip_atomic_store(a.esc_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            break;
        }

        // ---- 4. the earlier workgroups' aggregates (every word checked for this
        // iteration's tag, the stale ones read again), then the state entering
        // the workgroup's range and its chunks
        {
            constexpr int NSTAGE = ((kMaxGroup - 1) * AGG + kThreads - 1) / kThreads;
            static_assert(NSTAGE <= 32, "one bit per staged value");
            const unsigned t = tag32(i);
            unsigned need = 0;                           // bit u: value tid + u * kThreads still to fetch
#pragma unroll
            for (int u = 0; u < NSTAGE; ++u)
                if (tid + u * kThreads < w * AGG) need |= 1u << u;
            unsigned spins = 0;
            for (;;) {
#pragma unroll
                for (int u = 0; u < NSTAGE; ++u) {
                    if (need & (1u << u)) {
                        const int e = tid + u * kThreads;
                        ACC v;
                        if (Words<ACC>::get(agg + static_cast<size_t>(e) * Words<ACC>::N, t, v)) {
                            sh.Wg[e] = v;
                            need &= ~(1u << u);
                        }
                    }
                }
                if (!__syncthreads_or(need != 0)) break;
                if (__syncthreads_or(poll_step(spins, a.abort_flag))) {
                    if (tid == 0) sh.abort_now = 1;
                    break;
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            ACC x = xs0;
            for (int v = 0; v < w; ++v) {
                const ACC *Pv = sh.Wg + v * AGG;
                x = lds_quad_dot<ACC>(Pv, x, line, j, g) + Pv[kDP * kDP + j];
            }
            for (int q = 0; q < nch; ++q) {
                if (g == 0) sh.ent[q * kDP + j] = x;
                x = lds_quad_dot<ACC>(sh.P + q * kDP * kDP, x, line, j, g) + sh.Bc[q * kDP + j];
            }
        }
        __syncthreads();
        if (sh.abort_now) break;

        // ---- 5. replay of chunk `wave` from its entry: s_t = d_t (W s_{t-1}) + b_t,
        // row g of lanes for sub-chunk g (entries from the kept sub-chunk
        // aggregates), into the state rows; the range's last state also goes to
        // the right neighbour
        if (wave < nch) {
            const float *dq = sh.d + r0 * kDP, *bq = sh.b + r0 * kDP;
            const int ng = min(max(n - kSub * g, 0), kSub);
            const int K = (n + kSub - 1) / kSub;
            ACC *scr = scratch;
            ACC e = sh.ent[wave * kDP + j];
            ACC x = e;                                        // row 0's entry
#pragma unroll
            for (int k = 0; k + 1 < kNS; ++k) {
                if (k + 1 < K) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) scr[row16<ACC>(v, g) * kDP + j] = Pk[k][v];
                    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    e = lds_quad_dot<ACC>(scr, e, line, j, g) + Bk[k];
                    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    x = g == k + 1 ? e : x;
                }
            }
            const float *dg = dq + kSub * g * kDP, *bg = bq + kSub * g * kDP;
            float *Sg = sh.S + (r0 + kSub * g + 1) * kDP;
            for (int st = 0; st < kSub; ++st) {
                const float dc = dg[st * kDP + j], bc = bg[st * kDP + j];   // padding rows past the chunk
                const ACC y = row_dot16<ACC>(x, Wrow, row_line, j);
                const ACC xn = static_cast<ACC>(dc) * y + static_cast<ACC>(bc);
                if (st < ng) {
                    x = xn;
                    Sg[st * kDP + j] = static_cast<float>(xn);
                }
            }
            if (wave == nch - 1 && w + 1 < a.G && g == K - 1) Words<float>::put(xout + j, static_cast<float>(x), tag32(i));
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The diagonal linearisations in one launch: quasi-Newton (A_t the damped
// diagonal of the Jacobian), Jacobi (A_t = 0) and Picard (A_t = I) ("Parallel
// Broyden Methods", section 2 and its Picard paragraph).  The groups, the
// evaluation, the tagged-word exchange and the stopping rule are those of the
// dense kernel above.  A diagonal block stays diagonal under composition, so
// every fold is element-wise: lane (j, g) of a wavefront folds channel j of
// sub-chunk g, and a workgroup aggregate is 2 x 16 floats (the products and
// the offsets of its channels).  Accumulation in float, as the multi-launch
// diagonal scan.

struct DiagLds {
    static constexpr int NP = kNC * kL;
    __align__(16) float S[(NP + 1) * kDP];     // S[r] = s_{tb - 1 + r} of the current iterate
    __align__(16) float a[NP * kDP];           // a_t, b_t at local position r
    __align__(16) float b[NP * kDP];
    float sub[kNC][2][kNS][kDP];               // per wavefront: sub-chunk products and offsets
    float ch[2][kNC][kDP];                     // chunk products and offsets
    float ent[kNC][kDP];                       // states entering the chunks
    float Wg[(kMaxGroup - 1) * 2 * kDP];       // earlier workgroups' aggregates
    unsigned red[2][kNC];                      // per-wavefront residual maximum and front
    unsigned dec_r, dec_f;                     // the group's residual maximum and front
    int abort_now;                             // a wait gave up
};

__global__ __launch_bounds__(kThreads) void diag_persist_kernel(PersistArgs a)
{
    __shared__ DiagLds sh;
    constexpr int AGG = 2 * kDP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bseq = blockIdx.x / a.G, w = blockIdx.x % a.G;
    const int c0 = w * kNC;
    const int nch = min(kNC, a.nchunk - c0);             // >= 1
    const int tb = c0 * kL, te = min(a.T, (c0 + nch) * kL), np = te - tb;
    const int D = a.D;
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    const size_t aggs = static_cast<size_t>(a.B) * a.G * AGG;
    const size_t slots = static_cast<size_t>(a.B) * a.G;
    unsigned long long *agg0 = a.agg + static_cast<size_t>(bseq) * a.G * AGG;
    unsigned long long *slot0 = a.slot + static_cast<size_t>(bseq) * a.G;
    const unsigned long long *xin = a.xch + (static_cast<size_t>(bseq) * a.G + (w > 0 ? w - 1 : 0)) * kDP;
    unsigned long long *xout = a.xch + (static_cast<size_t>(bseq) * a.G + w) * kDP;
    const Linearization lz{a.lin_kind, a.shrink};
    int best = -1, last_adv = 0;                         // finite-step check (the same in every workgroup)

    const int j = lane & 15, g = lane >> 4;
    float WE[4], wcc[4];                                 // A operand of the evaluation; W_cc of channel 4 g + u
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = 4 * g + u;
        WE[u] = (j < D && c < D) ? a.W[j * D + c] : 0.0f;
        wcc[u] = c < D ? a.W[c * D + c] : 0.0f;
    }
    const float xs0 = (a.s0 && j < D) ? a.s0[static_cast<size_t>(bseq) * D + j] : 0.0f;
    const int r0 = wave * kL, n = wave < nch ? min(kL, np - r0) : 0;
    float pr[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = min(r0 + 16 * q + j, np - 1);
            const int c = min(4 * g + v, D - 1);
            pr[q][v] = a.proj[(seq + tb + r) * D + c];
        }
    for (int e = tid; e < (np + 1) * kDP; e += kThreads) {
        const int r = e / kDP, k = e % kDP;
        const int t = tb - 1 + r;
        const int kc = k < D ? k : D - 1;
        const float *src_p = (t < 0) ? (a.s0 ? a.s0 + static_cast<size_t>(bseq) * D + kc : a.W)
                                     : (a.init ? a.init + (seq + t) * D + kc : a.W);
        const float v = *src_p;
        sh.S[e] = (k < D && (t < 0 ? a.s0 != nullptr : a.init != nullptr)) ? v : 0.0f;
    }
    if (tid == 0) sh.abort_now = 0;
    __syncthreads();

    // evaluation of positions r0 + 16 q + j, channels 4 g .. 4 g + 3 (sv holds
    // s_{t-1} at exactly those channels): a_t = lin(diag of the Jacobian),
    // b_t = f_t - a_t s_{t-1}
    auto eval16 = [&](int q, unsigned &rmax, unsigned &fmin) {
        const int p = 16 * q + j, r = r0 + p;
        const bool pv = p < n;
        const int rr = pv ? r : r0;
        const v4f sv = *reinterpret_cast<const v4f *>(&sh.S[rr * kDP + 4 * g]);
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(WE[u], sv[u], acc, 0, 0, 0);
        const v4f nx = *reinterpret_cast<const v4f *>(&sh.S[(rr + 1) * kDP + 4 * g]);
        v4f av, bv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = 4 * g + v;
            const float f = tanhf(acc[v] + pr[q][v]);
            const float al = lin_diag(lz, (1.0f - f * f) * wcc[v]);
            const bool cv = c < D;
            av[v] = cv ? al : 0.0f;
            bv[v] = cv ? f - al * sv[v] : 0.0f;
            if (cv && pv) {
                const float ra = fabsf(nx[v] - f);
                rmax = max(rmax, __float_as_uint(ra));
                fmin = min(fmin, front_of(ra, a.tol, tb + r));
            }
        }
        if (pv) {
            *reinterpret_cast<v4f *>(&sh.a[r * kDP + 4 * g]) = av;
            *reinterpret_cast<v4f *>(&sh.b[r * kDP + 4 * g]) = bv;
        }
    };

    for (int i = 0;; ++i) {
        // ---- 1. evaluation; wavefront 0 takes its first 16 positions last, once
        // the left neighbour's last state is in
        unsigned rmax = 0u, fmin = kNoFront;
        if (wave < nch) {
            eval16(3, rmax, fmin);
            eval16(2, rmax, fmin);
            eval16(1, rmax, fmin);
            if (wave == 0 && w > 0 && i > 0) {
                float v = 0.0f;
                bool ok = lane >= kDP;
                unsigned spins = 0;
                int ab = 0;
                for (;;) {
                    if (!ok) ok = Words<float>::get(xin + lane, tag32(i - 1), v);
                    if (__all(ok)) break;
                    if (poll_step(spins, a.abort_flag)) { ab = 1; break; }
                }
                if (lane < kDP) sh.S[lane] = v;
                if (__builtin_amdgcn_readfirstlane(ab) && lane == 0) sh.abort_now = 1;
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                __builtin_amdgcn_wave_barrier();
            }
            eval16(0, rmax, fmin);
        }
        for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(rmax), o, 64)));
        fmin = wave_min_u32(fmin);
        if (lane == 0) { sh.red[0][wave] = rmax; sh.red[1][wave] = fmin; }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // ---- 2. sub-chunk aggregates (lane (j, g): channel j of sub-chunk g;
        // positions past the chunk are identities), then the chunk aggregate
        if (wave < nch) {
            const int ng = min(max(n - kSub * g, 0), kSub);
            const float *ag = sh.a + (r0 + kSub * g) * kDP + j, *bg = sh.b + (r0 + kSub * g) * kDP + j;
            float A = 1.0f, Bv = 0.0f;
#pragma unroll
            for (int st = 0; st < kSub; ++st) {
                const float as = ag[st * kDP], bs = bg[st * kDP];   // rows past the chunk stay in the array
                const float Bn = __builtin_fmaf(as, Bv, bs), An = as * A;
                Bv = st < ng ? Bn : Bv;
                A = st < ng ? An : A;
            }
            sh.sub[wave][0][g][j] = A;
            sh.sub[wave][1][g][j] = Bv;
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (g == 0) {
                float Ac = 1.0f, Bc = 0.0f;
#pragma unroll
                for (int k = 0; k < kNS; ++k) {
                    const float Ak = sh.sub[wave][0][k][j], Bk = sh.sub[wave][1][k][j];
                    Bc = __builtin_fmaf(Ak, Bc, Bk);
                    Ac = Ak * Ac;
                }
                sh.ch[0][wave][j] = Ac;
                sh.ch[1][wave][j] = Bc;
            }
        }
        __syncthreads();
        if (sh.abort_now) break;
        // the workgroup aggregate for the later workgroups
        unsigned long long *agg = agg0 + (i & 1) * aggs;
        if (wave == 0 && w + 1 < a.G && lane < kDP) {
            float Aw = sh.ch[0][0][lane], Bw = sh.ch[1][0][lane];
            for (int q = 1; q < nch; ++q) {
                const float Aq = sh.ch[0][q][lane], Bq = sh.ch[1][q][lane];
                Bw = __builtin_fmaf(Aq, Bw, Bq);
                Aw = Aq * Aw;
            }
            unsigned long long *dst = agg + static_cast<size_t>(w) * AGG;
            Words<float>::put(dst + lane, Aw, tag32(i));
            Words<float>::put(dst + kDP + lane, Bw, tag32(i));
        }
        if (tid == 0) {
            unsigned m = sh.red[0][0], f = sh.red[1][0];
            for (int q = 1; q < kNC; ++q) { m = max(m, sh.red[0][q]); f = min(f, sh.red[1][q]); }
            __hip_atomic_store(slot0 + (i & 1) * slots + w, slot_word(m, f, 0u, i), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- group barrier: every workgroup's residual slot of this iteration
        if (wave == 0) {
            unsigned long long v = 0;
            bool ok = lane >= a.G;
            unsigned spins = 0;
            int ab = 0;
            for (;;) {
                if (!ok) {
                    v = get_word(slot0 + (i & 1) * slots + lane);
                    ok = (static_cast<unsigned>(v >> 32) & 0xFFFFu) == tag16(i);
                }
                if (__all(ok)) break;
                if (poll_step(spins, a.abort_flag)) { ab = 1; break; }
            }
            unsigned m = lane < a.G ? static_cast<unsigned>(v) : 0u;
            unsigned f = lane < a.G ? static_cast<unsigned>(v >> 48) & 0x7FFFu : 0x7FFFu;
            for (int o = 32; o > 0; o >>= 1) {
                m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), o, 64)));
                f = min(f, static_cast<unsigned>(__shfl_xor(static_cast<int>(f), o, 64)));
            }
            if (lane == 0) {
                sh.dec_r = m;
                sh.dec_f = f == 0x7FFFu ? kNoFront : f;
                sh.abort_now = __builtin_amdgcn_readfirstlane(ab);
            }
        }
        __syncthreads();
        if (sh.abort_now) break;

        // ---- 3. the stopping decision
        const float r = __uint_as_float(sh.dec_r);
        int stop = -1;
        if (r <= a.tol) {
            stop = DEER_SEQ_CONVERGED;
        } else if (i >= a.max_iter) {
            stop = __builtin_isfinite(r) ? DEER_SEQ_NOT_CONVERGED : DEER_SEQ_NONFINITE;
        } else if (a.stall_window > 0) {
            const unsigned fr = sh.dec_f;
            const int f = fr > 0x7FFFFFFFu ? 0x7FFFFFFF : static_cast<int>(fr);
            if (f > best) {
                best = f;
                last_adv = i;
            } else if (best < i && i - last_adv >= a.stall_window) {
                stop = DEER_SEQ_STALLED;
            }
        }
        if (stop >= 0) {
            for (int e = tid; e < np * kDP; e += kThreads) {
                const int k = e % kDP;
                if (k < D) a.traj[(seq + tb + e / kDP) * D + k] = sh.S[kDP + e];
            }
            if (w == 0 && tid == 0) {
                a.iters[bseq] = i;
                a.status[bseq] = stop;
                a.resid[bseq] = r;
            }
            break;
        }

        // ---- 4. the earlier workgroups' aggregates (one value per thread, the
        // stale ones read again), then the states entering the chunks
        {
            static_assert((kMaxGroup - 1) * AGG <= kThreads, "one staged value per thread");
            const unsigned t = tag32(i);
            bool need = tid < w * AGG;
            unsigned spins = 0;
            for (;;) {
                if (need) {
                    float v;
                    if (Words<float>::get(agg + tid, t, v)) {
                        sh.Wg[tid] = v;
                        need = false;
                    }
                }
                if (!__syncthreads_or(need)) break;
                if (__syncthreads_or(poll_step(spins, a.abort_flag))) {
                    if (tid == 0) sh.abort_now = 1;
                    break;
                }
            }
        }
        __syncthreads();
        if (wave == 0 && lane < kDP) {
            float x = xs0;
            for (int v = 0; v < w; ++v) x = __builtin_fmaf(sh.Wg[v * AGG + lane], x, sh.Wg[v * AGG + kDP + lane]);
            for (int q = 0; q < nch; ++q) {
                sh.ent[q][lane] = x;
                x = __builtin_fmaf(sh.ch[0][q][lane], x, sh.ch[1][q][lane]);
            }
        }
        __syncthreads();
        if (sh.abort_now) break;

        // ---- 5. replay: lane (j, g) runs channel j of sub-chunk g from its entry
        // (the chunk's entry through the earlier sub-chunks) into the state rows;
        // the range's last state also goes to the right neighbour
        if (wave < nch) {
            const int ng = min(max(n - kSub * g, 0), kSub);
            const int K = (n + kSub - 1) / kSub;
            float x = sh.ent[wave][j];
#pragma unroll
            for (int k = 0; k + 1 < kNS; ++k)
                if (k < g) x = __builtin_fmaf(sh.sub[wave][0][k][j], x, sh.sub[wave][1][k][j]);
            const float *ag = sh.a + (r0 + kSub * g) * kDP + j, *bg = sh.b + (r0 + kSub * g) * kDP + j;
            float *Sg = sh.S + (r0 + kSub * g + 1) * kDP + j;
#pragma unroll
            for (int st = 0; st < kSub; ++st) {
                const float xn = __builtin_fmaf(ag[st * kDP], x, bg[st * kDP]);
                if (st < ng) {
                    x = xn;
                    Sg[st * kDP] = xn;
                }
            }
            if (wave == nch - 1 && w + 1 < a.G && g == K - 1) Words<float>::put(xout + j, x, tag32(i));
        }
        __syncthreads();
    }
}

// Zeroes the tagged-word buffers of a launch (zero is never an expected tag)
// and, unless the launch resumes another one, the abort word.
__global__ void persist_init_kernel(unsigned long long *words, size_t n, unsigned *esc_flag, unsigned *abort_flag)
{
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) words[e] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x == 0 && abort_flag) {
        *abort_flag = 0u;
        *esc_flag = 0u;
    }
}

template <class ACC>
int launch_persist(const PersistArgs &a, hipStream_t stream)
{
    DEER_LAUNCH((dense_persist_kernel<ACC>), dim3(static_cast<unsigned>(a.B) * a.G), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

// Workgroups of `kernel` (kThreads threads each) resident at once on the
// current device (compute units times workgroups per unit), cached per device
// in `cache`.
template <class F>
int capacity_of(F kernel, int (&cache)[64])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess) per_cu = 0;
        cache[dev] = cus * per_cu > 0 ? cus * per_cu : -1;
    }
    return cache[dev];
}
template <class ACC>
int persist_capacity()
{
    static int cache[64] = {};
    return capacity_of(dense_persist_kernel<ACC>, cache);
}
int diag_persist_capacity()
{
    static int cache[64] = {};
    return capacity_of(diag_persist_kernel, cache);
}

int groups_of(int T) { return (T + kNC * kL - 1) / (kNC * kL); }

// Whether the grid (B groups of groups_of(T) workgroups) is resident at once.
bool persist_resident(int B, int T, bool f64)
{
    const int cap = f64 ? persist_capacity<double>() : persist_capacity<float>();
    return cap > 0 && static_cast<long long>(B) * groups_of(T) <= cap;
}

bool persist_shape(int B, int D, int T) { return D >= 1 && D <= kDP && T >= 1 && T <= kNC * kL * kMaxGroup && B >= 1; }

// Layout of the state: the tagged words (residual slots, aggregates sized for
// double when a double-precision launch may run, exchange rows) in one block,
// then the kept fronts and the abort word.
struct PersistState {
    size_t slot, agg, xch, words_end, keep, esc_off, abort_off, bytes;
};
PersistState persist_state(int B, int T, bool f64)
{
    const size_t BG = static_cast<size_t>(B) * groups_of(T);
    const size_t aggw = static_cast<size_t>(kDP * kDP + kDP) * (f64 ? 2 : 1);
    PersistState st{};
    st.slot = 0;
    st.agg = st.slot + 2 * BG * sizeof(unsigned long long);
    st.xch = st.agg + 2 * BG * aggw * sizeof(unsigned long long);
    st.words_end = st.xch + BG * kDP * sizeof(unsigned long long);
    st.keep = align_up(st.words_end);
    st.esc_off = st.keep + align_up(2 * static_cast<size_t>(B) * sizeof(int));
    st.abort_off = st.esc_off + align_up(sizeof(unsigned));
    st.bytes = st.abort_off + align_up(sizeof(unsigned));
    return st;
}

}  // namespace

bool dense_persist_fits(int B, int D, int T, bool f64) { return persist_shape(B, D, T) && persist_resident(B, T, f64); }

bool diag_persist_fits(int B, int D, int T)
{
    if (!persist_shape(B, D, T)) return false;
    const int cap = diag_persist_capacity();
    return cap > 0 && static_cast<long long>(B) * groups_of(T) <= cap;
}

size_t dense_persist_state_bytes(int B, int T, bool f64) { return persist_state(B, T, f64).bytes; }

unsigned *dense_persist_abort_word(void *state, int B, int T, bool f64)
{
    return reinterpret_cast<unsigned *>(static_cast<char *>(state) + persist_state(B, T, f64).abort_off);
}

int launch_dense_persist(const float *W, const float *proj, const float *s0, const float *init, float *traj, int B,
                         int T, int D, float shrink, float tol, int max_iter, int stall_window, bool f64,
                         bool escalate, bool resume, int *iters, int *status, float *resid, void *state,
                         bool state_f64, hipStream_t stream)
{
    if (B == 0) return DEER_OK;
    if (f64 && !state_f64) return fail(DEER_ERR_INVALID, "persistent dense solve: state sized for float32");
    if (!dense_persist_fits(B, D, T, f64))
        return fail(DEER_ERR_UNSUPPORTED, "persistent dense solve: problem does not fit the device at once");
    PersistArgs a{};
    a.W = W; a.proj = proj; a.s0 = s0; a.init = init; a.traj = traj;
    a.B = B; a.T = T; a.D = D;
    a.nchunk = (T + kL - 1) / kL;
    a.G = groups_of(T);
    a.max_iter = max_iter; a.stall_window = stall_window; a.tol = tol; a.shrink = shrink;
    a.iters = iters; a.status = status; a.resid = resid;
    const PersistState ps = persist_state(B, T, state_f64);
    char *st = static_cast<char *>(state);
    a.slot = reinterpret_cast<unsigned long long *>(st + ps.slot);
    a.agg = reinterpret_cast<unsigned long long *>(st + ps.agg);
    a.xch = reinterpret_cast<unsigned long long *>(st + ps.xch);
    a.keep = reinterpret_cast<int *>(st + ps.keep);
    a.esc_flag = reinterpret_cast<unsigned *>(st + ps.esc_off);
    a.abort_flag = reinterpret_cast<unsigned *>(st + ps.abort_off);
    a.escalate = escalate ? 1 : 0;
    a.resume = resume ? 1 : 0;
    // every tagged word of the launch's layout starts at zero; a resumed launch
    // keeps the abort and hand-over words and the kept fronts of the launch before it
    const size_t nwords = ps.words_end / sizeof(unsigned long long);
    DEER_LAUNCH(persist_init_kernel, dim3(static_cast<unsigned>(std::min<size_t>((nwords + 255) / 256, 2048))),
                dim3(256), 0, stream, reinterpret_cast<unsigned long long *>(st), nwords, a.esc_flag,
                resume ? nullptr : a.abort_flag);
    DEER_HIP(hipGetLastError());
    return f64 ? launch_persist<double>(a, stream) : launch_persist<float>(a, stream);
}

int launch_diag_persist(const float *W, const float *proj, const float *s0, const float *init, float *traj, int B,
                        int T, int D, Linearization lz, float tol, int max_iter, int stall_window, int *iters,
                        int *status, float *resid, void *state, hipStream_t stream)
{
    if (B == 0) return DEER_OK;
    if (lz.kind != kLinJacobian && lz.kind != kLinZero && lz.kind != kLinIdentity)
        return fail(DEER_ERR_INVALID, "persistent diagonal solve: not a linearisation");
    if (!diag_persist_fits(B, D, T))
        return fail(DEER_ERR_UNSUPPORTED, "persistent diagonal solve: problem does not fit the device at once");
    PersistArgs a{};
    a.W = W; a.proj = proj; a.s0 = s0; a.init = init; a.traj = traj;
    a.B = B; a.T = T; a.D = D;
    a.nchunk = (T + kL - 1) / kL;
    a.G = groups_of(T);
    a.max_iter = max_iter; a.stall_window = stall_window; a.tol = tol; a.shrink = lz.shrink;
    a.lin_kind = lz.kind;
    a.iters = iters; a.status = status; a.resid = resid;
    const PersistState ps = persist_state(B, T, false);
    char *st = static_cast<char *>(state);
    a.slot = reinterpret_cast<unsigned long long *>(st + ps.slot);
    a.agg = reinterpret_cast<unsigned long long *>(st + ps.agg);
    a.xch = reinterpret_cast<unsigned long long *>(st + ps.xch);
    a.keep = reinterpret_cast<int *>(st + ps.keep);
    a.esc_flag = reinterpret_cast<unsigned *>(st + ps.esc_off);
    a.abort_flag = reinterpret_cast<unsigned *>(st + ps.abort_off);
    const size_t nwords = ps.words_end / sizeof(unsigned long long);
    DEER_LAUNCH(persist_init_kernel, dim3(static_cast<unsigned>(std::min<size_t>((nwords + 255) / 256, 2048))),
                dim3(256), 0, stream, reinterpret_cast<unsigned long long *>(st), nwords, a.esc_flag, a.abort_flag);
    DEER_HIP(hipGetLastError());
    DEER_LAUNCH(diag_persist_kernel, dim3(static_cast<unsigned>(B) * a.G), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace deer
