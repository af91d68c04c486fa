// Scan of the dense affine recurrence s_t = A_t s_{t-1} + b_t (D x D blocks).
//
// Two affine maps merge as (A_j, b_j) o (A_i, b_i) = (A_j A_i, A_j b_i + b_j),
// the later map on the left ("Parallel Broyden Methods", appendix C.2).  The
// scan runs in three launches over chunks of L consecutive steps:
//   1. aggregate: every chunk folds its steps into one pair (P_c, B_c),
//      P_c = A_last ... A_first and B_c the state reached from a zero start;
//   2. carry: per sequence, the state entering each chunk, s_in(c+1) =
//      P_c s_in(c) + B_c, walked over the chunks in order;
//   3. replay: every chunk re-runs its steps from its carried-in state and
//      writes the trajectory.
// A_t is either materialised ([B,T,D,D]) or given in the factored form
// A_t = diag(d_t) W of a tanh cell's Jacobian, so W stays on chip.
//
// The products P_c are the one dense contraction of the path (2 D^3 flops per
// step).  For factored leaves with D = 32 (and D = 16) they run on the matrix
// cores: P <- diag(d_t) (W P) is one 32 x 32 x 32 product per step, and with
// the K order permuted to follow the accumulator layout, the accumulators of
// one step are the B operands of the next -- the product never leaves the
// registers of the wavefront that owns the chunk.
//
// ACC is the accumulation type of the products, offsets, carries and replayed
// states (float, or double for unpredictable dynamics where chunk products
// grow large enough that float32 rounding breaks the consistency of the
// solution at chunk boundaries); inputs and outputs are float32.
#include <algorithm>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

// --------------------------------------------------------- generic (VALU)
// One wavefront handles 64 / DP chunks: lane j of a chunk's lane group holds
// column j of the running product and component j of the running offset.
template <int DP, bool FACT, class ACC>
__global__ __launch_bounds__(kThreads) void dense_agg_kernel(
    const float *__restrict__ A, const float *__restrict__ dv, const float *__restrict__ W,
    const float *__restrict__ bv, const int *__restrict__ skip, const int *__restrict__ all_done, int B,
    int T, int D, int L, int nchunk, ACC *__restrict__ Pout, ACC *__restrict__ Bout)
{
    if (all_done && *all_done) return;
    constexpr int G = 64 / DP;
    __shared__ float Wb[FACT ? DP : 1][FACT ? DP : 1];        // broadcast copy
    __shared__ float Wr[FACT ? DP : 1][FACT ? DP + 1 : 1];    // row copy (padded)
    if constexpr (FACT) {
        for (int e = threadIdx.x; e < DP * DP; e += kThreads) {
            const int i = e / DP, k = e % DP;
            const float w = (i < D && k < D) ? W[i * D + k] : 0.0f;
            Wb[i][k] = w;
            Wr[i][k] = w;
        }
        __syncthreads();
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / DP, j = lane % DP, gbase = grp * DP;
    const long long nq = static_cast<long long>(B) * nchunk;
    long long q = (static_cast<long long>(blockIdx.x) * (kThreads / 64) + wave) * G + grp;
    const bool qvalid = q < nq;
    if (!qvalid) q = 0;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    const bool act = qvalid && !(skip && skip[bseq]);
    const int t0 = c * L, t1 = min(T, t0 + L);
    const size_t seq = static_cast<size_t>(bseq) * T;
    const bool jv = j < D;

    auto Aget = [&](int t, int i, int k) -> ACC {
        return (i < D && k < D) ? static_cast<ACC>(A[((seq + t) * D + i) * D + k]) : ACC(0);
    };

    ACC P[DP];
    ACC Bq;
    {
        const int t = t0;
        if constexpr (FACT) {
            const ACC dj = jv ? static_cast<ACC>(dv[(seq + t) * D + j]) : ACC(0);
#pragma unroll
            for (int i = 0; i < DP; ++i) P[i] = __shfl(dj, gbase + i, 64) * static_cast<ACC>(Wr[i][j]);
        } else {
#pragma unroll
            for (int i = 0; i < DP; ++i) P[i] = Aget(t, i, j);
        }
        Bq = jv ? static_cast<ACC>(bv[(seq + t) * D + j]) : ACC(0);
    }
    for (int s = 1; s < L; ++s) {
        const int t = t0 + s;
        const bool live = t < t1;
        const int tt = live ? t : t0;
        const ACC bj = jv ? static_cast<ACC>(bv[(seq + tt) * D + j]) : ACC(0);
        ACC Pn[DP];
        ACC Bn;
        if constexpr (FACT) {
            const ACC dj = jv ? static_cast<ACC>(dv[(seq + tt) * D + j]) : ACC(0);
#pragma unroll
            for (int i = 0; i < DP; ++i) {
                asm volatile("" ::: "memory");   // keep W in LDS rather than in registers
                ACC acc = 0;
#pragma unroll
                for (int k = 0; k < DP; ++k) acc += static_cast<ACC>(Wb[i][k]) * P[k];
                Pn[i] = __shfl(dj, gbase + i, 64) * acc;
            }
            ACC accb = 0;
#pragma unroll
            for (int k = 0; k < DP; ++k) accb += static_cast<ACC>(Wr[j][k]) * __shfl(Bq, gbase + k, 64);
            Bn = dj * accb + bj;
        } else {
#pragma unroll
            for (int i = 0; i < DP; ++i) {
                asm volatile("" ::: "memory");   // bound the loads in flight to one row
                ACC acc = 0;
#pragma unroll
                for (int k = 0; k < DP; ++k) acc += Aget(tt, i, k) * P[k];
                Pn[i] = acc;
            }
            ACC accb = 0;
#pragma unroll
            for (int k = 0; k < DP; ++k) accb += Aget(tt, j, k) * __shfl(Bq, gbase + k, 64);
            Bn = accb + bj;
        }
        if (live) {
#pragma unroll
            for (int i = 0; i < DP; ++i) P[i] = Pn[i];
            Bq = Bn;
        }
    }
    if (act && jv) {
        const size_t qb = static_cast<size_t>(q);
#pragma unroll
        for (int i = 0; i < DP; ++i)
            if (i < D) Pout[(qb * D + i) * D + j] = P[i];
        Bout[qb * D + j] = Bq;
    }
}

// ------------------------------------------------ matrix-core aggregates
// Row of the 32x32 accumulator held in register v by a lane of half hf.
__device__ __forceinline__ int row32(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// Offset chain of a D = 32 chunk on one wavefront: B_s = d_s (W B_{s-1}) + b_s
// from B_0 = b_0, written to out[0..31].  The state is split into two blocks of
// 16; each 16-lane row holds one block K of the input and contracts the 16 x 16
// block (I, K) of W against it with row rotations (DPP), so every term is one
// FMA on registers.  The two rows that share an output block I then add their
// partial sums with one exchange.  Steps alternate between two row layouts --
// A: K = r & 1, I = r >> 1, partner lane ^ 16; B: K = r >> 1, I = r & 1,
// partner lane ^ 32 -- because the output blocks of an A step sit exactly where
// a B step expects its input blocks, and the other way round.
__device__ __forceinline__ void offset_chain32(const float *__restrict__ W, const float *ds, const float *bs, int n,
                                               float *__restrict__ out)
{
    constexpr int D = 32;
    const int lane = threadIdx.x & 63, r = lane >> 4, m = lane & 15;
    // source lane (within the row) that rotation k delivers to this lane, measured
    // by rotating the lane indices themselves
    int src[16];
    src[0] = m;
    RowRotations::sources(m, src);
    const int KA = r & 1, IA = r >> 1, KB = r >> 1, IB = r & 1;
    float wA[16], wB[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        wA[k] = W[(16 * IA + m) * D + 16 * KA + src[k]];
        wB[k] = W[(16 * IB + m) * D + 16 * KB + src[k]];
    }
    auto contract = [&](float x, const float (&w)[16]) -> float {
        float a0 = w[0] * x, a1 = 0.0f;
        RowRotations::contract(x, w, a0, a1);
        return a0 + a1;
    };
    float x = bs[16 * KA + m];                        // B_0 in the A layout
    int s = 1;
    for (; s + 1 < n; s += 2) {
        float y = contract(x, wA);                    // A step: output block IA
        y += __shfl_xor(y, 16, 64);
        x = ds[s * D + 16 * IA + m] * y + bs[s * D + 16 * IA + m];
        y = contract(x, wB);                          // B step: output block IB
        y += __shfl_xor(y, 32, 64);
        x = ds[(s + 1) * D + 16 * IB + m] * y + bs[(s + 1) * D + 16 * IB + m];
    }
    int I = KA;                                       // block held after an even number of steps (A layout)
    if (s < n) {
        float y = contract(x, wA);
        y += __shfl_xor(y, 16, 64);
        x = ds[s * D + 16 * IA + m] * y + bs[s * D + 16 * IA + m];
        I = IA;
    }
    out[16 * I + m] = x;                              // rows holding the same block write the same values
}

// D = 32, factored leaves, float32: one 128-thread workgroup per chunk.  Its
// first wavefront runs the product chain on the matrix cores, the second the
// offset chain on VALU; both read the chunk's d_t and b_t from LDS, so the two
// chains overlap.
//   A operand (W diag(d_{t-1})):  lane l, instruction v holds W[l % 32][k] d_{t-1}[k], k = row32(v, l / 32)
//   B operand (Q_old):            lane l, instruction v holds Q_old[row32(v, l / 32)][l % 32] = accumulator v
constexpr int kAggThreads = 128;
__global__ __launch_bounds__(kAggThreads) void dense_agg_mfma32_kernel(
    const float *__restrict__ dv, const float *__restrict__ W, const float *__restrict__ bv,
    const int *__restrict__ skip, const int *__restrict__ all_done, int T, int L, int nchunk,
    float *__restrict__ Pout, float *__restrict__ Bout)
{
    constexpr int D = 32;
    constexpr int kRows = 64 * D / 4 / kAggThreads;  // float4 rows of d (and of b) per thread, L <= 64
    if (all_done && *all_done) return;
    __shared__ float ds[64 * D], bs[64 * D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hf = lane >> 5;
    const long long q = blockIdx.x;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    if (skip && skip[bseq]) return;
    const int t0 = c * L, n = min(L, T - t0);
    {
        // all of the chunk's loads in flight at once
        const size_t base = (static_cast<size_t>(bseq) * T + t0) * D;
        v4f dreg[kRows], breg[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int e = tid + kAggThreads * i;
            const int ec = e < n * (D / 4) ? e : 0;     // clamped: rows past the chunk are never read
            dreg[i] = *reinterpret_cast<const v4f *>(dv + base + static_cast<size_t>(ec) * 4);
            breg[i] = *reinterpret_cast<const v4f *>(bv + base + static_cast<size_t>(ec) * 4);
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int e = tid + kAggThreads * i;
            *reinterpret_cast<v4f *>(ds + e * 4) = dreg[i];
            *reinterpret_cast<v4f *>(bs + e * 4) = breg[i];
        }
    }
    __syncthreads();

    if (wave == 1) {
        offset_chain32(W, ds, bs, n, Bout + static_cast<size_t>(q) * D);
        return;
    }

    // Q_s = W P_{s-1} runs unscaled: Q_0 = W and Q_s = (W diag(d_{s-1})) Q_{s-1}, so
    // the diagonal lands on the A operand and the accumulator of one step is the
    // B operand of the next (two accumulators alternate); P = diag(d_last) Q_last.
    // The scaled A operands of step s+1 are formed while step s runs.
    float WA[16];
    v16f qa, qb;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        WA[v] = W[j * D + row32(v, hf)];
        qa[v] = W[row32(v, hf) * D + j];
    }
    auto scaled = [&](int s, float (&ws)[16]) {       // W diag(d_{s-1}), this lane's A operands
        const v4f *dprev = reinterpret_cast<const v4f *>(ds + (min(s, n - 1) - 1) * D);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const v4f dq = dprev[2 * qd + hf];
#pragma unroll
            for (int r = 0; r < 4; ++r) ws[4 * qd + r] = WA[4 * qd + r] * dq[r];
        }
    };
    auto step = [&](const v16f &qin, const float (&ws)[16]) -> v16f {
        v16f acc = {};
#pragma unroll
        for (int v = 0; v < 16; ++v) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ws[v], qin[v], acc, 0, 0, 0);
        return acc;
    };
    // (rows past the chunk are clamped: a scaled operand formed for a step that
    // never runs is simply unused, which keeps the loop body free of branches)
    float wa[16], wb[16];
    int s = 1;
    scaled(1, wa);
    if ((n - 1) & 1) {                                // odd step count: peel one so the pairs end in qa
        scaled(2, wb);
        qa = step(qa, wa);
        s = 2;
#pragma unroll
        for (int v = 0; v < 16; ++v) wa[v] = wb[v];
    }
    for (; s + 1 < n; s += 2) {
        scaled(s + 1, wb);
        qb = step(qa, wa);
        scaled(s + 2, wa);
        qa = step(qb, wb);
        // issue order: the pair's LDS reads first, then each MFMA with two VALU ops
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int g = 0; g < 32; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x2, 2, 0);
        }
    }
    float *po = Pout + static_cast<size_t>(q) * D * D;
    const v4f *dl = reinterpret_cast<const v4f *>(ds + (n - 1) * D);
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
        const v4f dq = dl[2 * qd + hf];
#pragma unroll
        for (int r = 0; r < 4; ++r) po[row32(4 * qd + r, hf) * D + j] = dq[r] * qa[4 * qd + r];
    }
}

// D = 16, factored leaves, float32 (16x16x4) or float64 (16x16x4 f64).
// Accumulator v of lane l holds C[row16(v, l / 16)][l % 16]: rows 4 (l / 16) + v
// for the float32 instruction, l / 16 + 4 v for the float64 one (measured lane
// layouts).  The running product is fed back as the B operand of the next step,
// so instruction u contracts over k = row16(u, l / 16):
//   A operand (W):      lane l, instruction u holds W[l % 16][row16(u, l / 16)]
//   B operand (P_old):  lane l, instruction u holds P_old[row16(u, l / 16)][l % 16] = accumulator u
template <class ACC>
__device__ __forceinline__ int row16(int v, int g)
{
    return sizeof(ACC) == 8 ? g + 4 * v : 4 * g + v;
}

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

template <class ACC>
__device__ __forceinline__ ACC lane_bcast(ACC v, int k);

template <>
__device__ __forceinline__ float lane_bcast<float>(float v, int k)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

template <>
__device__ __forceinline__ double lane_bcast<double>(double v, int k)
{
    const long long bits = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(bits & 0xffffffffll), k);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(bits >> 32), k);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

template <class ACC>
__global__ __launch_bounds__(64) void dense_agg_mfma16_kernel(const float *__restrict__ dv, const float *__restrict__ W,
                                                            const float *__restrict__ bv, const int *__restrict__ skip,
                                                            const int *__restrict__ all_done, int T, int L, int nchunk,
                                                            ACC *__restrict__ Pout, ACC *__restrict__ Bout)
{
    constexpr int D = 16;
    if (all_done && *all_done) return;
    __shared__ float ds[64 * D], bs[64 * D];
    const int lane = threadIdx.x, j = lane & 15, g = lane >> 4;
    const long long q = blockIdx.x;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    if (skip && skip[bseq]) return;
    const int t0 = c * L, n = min(L, T - t0);
    const size_t seq = static_cast<size_t>(bseq) * T;
    for (int e = lane; e < n * (D / 4); e += 64) {
        const int r = e / (D / 4), col = (e % (D / 4)) * 4;
        const size_t gi = (seq + t0 + r) * D + col;
        *reinterpret_cast<v4f *>(ds + r * D + col) = *reinterpret_cast<const v4f *>(dv + gi);
        *reinterpret_cast<v4f *>(bs + r * D + col) = *reinterpret_cast<const v4f *>(bv + gi);
    }
    ACC WA[4], Wcol[4], Wrow[D];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        WA[u] = static_cast<ACC>(W[j * D + row16<ACC>(u, g)]);
        Wcol[u] = static_cast<ACC>(W[row16<ACC>(u, g) * D + j]);
    }
#pragma unroll
    for (int k = 0; k < D; ++k) Wrow[k] = static_cast<ACC>(W[j * D + k]);
    __syncthreads();

    ACC P[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) P[v] = static_cast<ACC>(ds[row16<ACC>(v, g)]) * Wcol[v];
    ACC Bq = static_cast<ACC>(bs[j]);
    for (int s = 1; s < n; ++s) {
        ACC acc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) mfma16<ACC>(WA[u], P[u], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) P[v] = static_cast<ACC>(ds[s * D + row16<ACC>(v, g)]) * acc[v];
        ACC sum = 0;
#pragma unroll
        for (int k = 0; k < D; ++k) sum += Wrow[k] * lane_bcast<ACC>(Bq, k);
        Bq = static_cast<ACC>(ds[s * D + j]) * sum + static_cast<ACC>(bs[s * D + j]);
    }
    ACC *po = Pout + static_cast<size_t>(q) * D * D;
#pragma unroll
    for (int v = 0; v < 4; ++v) po[row16<ACC>(v, g) * D + j] = P[v];
    if (g == 0) Bout[static_cast<size_t>(q) * D + j] = Bq;
}

// ------------------------------------------------------------- carry walk
// One wavefront per sequence walks its chunks in order: s_in(c+1) = P_c s_in(c) + B_c.
// The chain through s is the only dependency, so the chunk aggregates are
// fetched PF chunks ahead into a register ring and load latency stays off the
// critical path.  Lane (grp, j) holds row j of P_c restricted to the KG
// columns of its group; s is broadcast with cross-lane shuffles (no LDS and no
// barrier, whose release fence would wait for the prefetches) and the G
// partial sums are reduced across groups.
template <int DP, class ACC>
struct CarryGeom {
    static constexpr int G = (64 / DP < DP) ? 64 / DP : DP;    // lane groups splitting the columns
    static constexpr int KG = DP / G;                           // columns per lane
    static constexpr int W = static_cast<int>(sizeof(ACC) / 4); // 32-bit registers per value
    static constexpr int PFr = 160 / ((KG + 1) * W);            // ring depth within ~160 registers
    static constexpr int PF = PFr > 16 ? 16 : PFr < 1 ? 1 : PFr;
    static constexpr int VEC = 16 / static_cast<int>(sizeof(ACC));   // values per 16-byte load
};

// Row segment of one chunk product: KG columns starting at k0.  Every lane
// loads (indices clamped into the matrix) so the loads carry no branch and the
// compiler can keep several chunks of prefetch in flight; columns outside the
// matrix read as zero.
template <int KG, class ACC, bool VECP>
__device__ __forceinline__ void load_row_segment(const ACC *__restrict__ row, int k0, int D, ACC (&r)[KG])
{
    if constexpr (VECP) {       // D == DP: the segment is whole and 16-byte aligned
        constexpr int VEC = 16 / static_cast<int>(sizeof(ACC));
        typedef ACC vt __attribute__((ext_vector_type(VEC)));
#pragma unroll
        for (int i = 0; i < KG; i += VEC) {
            const vt v = *reinterpret_cast<const vt *>(row + k0 + i);
#pragma unroll
            for (int e = 0; e < VEC; ++e) r[i + e] = v[e];
        }
    } else {
#pragma unroll
        for (int i = 0; i < KG; ++i) {
            const int k = k0 + i;
            const ACC v = row[k < D ? k : D - 1];
            r[i] = k < D ? v : ACC(0);
        }
    }
}

template <int DP, class ACC, bool VECP>
__global__ __launch_bounds__(64) void dense_carry_kernel(
    const ACC *__restrict__ Pagg, const ACC *__restrict__ Bagg, const float *__restrict__ s0,
    const int *__restrict__ skip, const int *__restrict__ all_done, int B, int D, int nchunk,
    ACC *__restrict__ carry)
{
    using Gm = CarryGeom<DP, ACC>;
    constexpr int G = Gm::G, KG = Gm::KG, PF = Gm::PF;
    if (all_done && *all_done) return;
    const int bseq = blockIdx.x;
    if (bseq >= B || (skip && skip[bseq])) return;      // uniform per workgroup
    const int lane = threadIdx.x;
    const int grp = lane / DP, j = lane % DP;
    const bool act = grp < G;
    const bool jv = act && j < D;
    const int jr = j < D ? j : D - 1;                   // clamped row for the loads
    const int k0 = act ? grp * KG : 0;
    const size_t q0 = static_cast<size_t>(bseq) * nchunk;
    const bool writer = grp == 0 && j < D;

    ACC ring[PF][KG], bring[PF];
    auto fetch = [&](int c, ACC (&r)[KG], ACC &bq) {
        const size_t q = q0 + static_cast<size_t>(c < nchunk ? c : nchunk - 1);
        load_row_segment<KG, ACC, VECP>(Pagg + (q * D + jr) * D, k0, D, r);
        bq = Bagg[q * D + jr];
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u, ring[u], bring[u]);

    ACC st = (jv && s0) ? static_cast<ACC>(s0[static_cast<size_t>(bseq) * D + j]) : ACC(0);
    auto advance = [&](int c, const ACC (&r)[KG], ACC bq) {
        if (writer) carry[(q0 + c) * D + j] = st;
        ACC a0 = 0, a1 = 0;
#pragma unroll
        for (int i = 0; i < KG; i += 2) {
            a0 += r[i] * __shfl(st, k0 + i, 64);
            if (i + 1 < KG) a1 += r[i + 1] * __shfl(st, k0 + i + 1, 64);
        }
        ACC acc = a0 + a1;
#pragma unroll
        for (int o = DP; o < G * DP; o <<= 1) acc += __shfl_xor(acc, o, 64);
        st = jv ? acc + bq : ACC(0);
    };
    // whole rounds of PF chunks: straight-line bodies, refills clamped past the end
    const int nfull = nchunk - nchunk % PF;
    for (int c0 = 0; c0 < nfull; c0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            advance(c0 + u, ring[u], bring[u]);
            fetch(c0 + u + PF, ring[u], bring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (nfull + u < nchunk) advance(nfull + u, ring[u], bring[u]);
}

// ------------------------------------------------------- two-level carry walk
// Float D = 32 with many chunks: a sequence's chunks form kTlGroups
// consecutive groups.
//   1. dense_group_tl32_kernel, one wavefront per group: the product P_g of
//      the group's chunk products on the matrix cores (the running product
//      stays in the accumulators, as in the compose kernel: P <- P_c P with P_c
//      as the A operands) and the group offset B_g by the matrix-vector chain
//      B <- P_c B + B_c from the same operands;
//   2. dense_carry_tl32_kernel, eight single-wavefront walkers per sequence:
//      each pushes s0 through the maps of the groups before its own, then walks
//      its two groups' chunks and writes the chunk carries.
// The serial chain shrinks from nchunk steps to at most kTlGroups + 2 nchunk / kTlGroups,
// and the group products (one D^3 product per chunk, 1/64 of the compose
// work) run over the whole device.  Pairs of affine maps merge as in the rest
// of the scan (the later on the left); any grouping gives the same result
// under exact composition ("Parallel Broyden Methods", appendix B.4), so only
// rounding differs from the one-level walk.  A group product out of range
// (non-finite, or above kTlLimit in magnitude: strongly expanding dynamics,
// where P_g x + B_g would cancel huge terms or overflow) makes its sequence
// take the one-level walk instead, on its first walker.
constexpr int kTlGroups = 16;
constexpr int kTlPF = 8;                 // chunks fetched ahead by the group kernel's chains
constexpr float kTlLimit = 1e18f;
constexpr int kTlMinChunks = 32;         // fewer chunks: the one-level walk is short already

__host__ __device__ __forceinline__ int tl_group_size(int nchunk) { return (nchunk + kTlGroups - 1) / kTlGroups; }
bool tl_carry_shape(int D, int nchunk) { return D == 32 && nchunk >= kTlMinChunks; }

struct TlChunk {
    v4f a[4];                            // row i of the matrix, columns 8 u + 4 hf .. + 3 (A operand layout)
    float b;                             // offset entry i
};

// Matrix q of a [.][32][32] array and its offset, clamped to index < qend:
// refills past the end load a valid entry that is never used.
__device__ __forceinline__ void tl_fetch(const float *__restrict__ P, const float *__restrict__ Bv, size_t q,
                                         size_t qend, int i, int hf, TlChunk &k)
{
    const size_t qq = q < qend ? q : qend - 1;
    const float *row = P + (qq * 32 + i) * 32 + 4 * hf;
#pragma unroll
    for (int u = 0; u < 4; ++u) k.a[u] = *reinterpret_cast<const v4f *>(row + 8 * u);
    k.b = Bv[qq * 32 + i];
}

// x <- M x + b for the state held in `line` (LDS, 32 floats); every lane
// returns entry i, and the line holds the new state on return.
__device__ __forceinline__ float tl_advance(const TlChunk &k, float *line, int i, int hf)
{
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const v4f xv = *reinterpret_cast<const v4f *>(line + 8 * u + 4 * hf);
        a0 = __builtin_fmaf(k.a[u][0], xv[0], a0);
        a1 = __builtin_fmaf(k.a[u][1], xv[1], a1);
        a0 = __builtin_fmaf(k.a[u][2], xv[2], a0);
        a1 = __builtin_fmaf(k.a[u][3], xv[3], a1);
    }
    float y = a0 + a1;
    y += __shfl_xor(y, 32, 64);
    const float x = y + k.b;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (hf == 0) line[i] = x;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return x;
}

__device__ __forceinline__ void tl_set_line(float *line, float x, int i, int hf)
{
    if (hf == 0) line[i] = x;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Walk matrices [cb, ce) of (P, Bv) from the state x, calling at(c, x) with
// the state before each; whole rounds of PF run as straight-line bodies (a
// branch inside a round would make the compiler wait for every load in flight).
template <int PF, class At>
__device__ __forceinline__ float tl_walk(const float *__restrict__ P, const float *__restrict__ Bv, size_t cb,
                                         size_t ce, float x, float *line, int i, int hf, At &&at)
{
    if (ce <= cb) return x;                              // nothing to walk (and nothing to fetch)
    tl_set_line(line, x, i, hf);
    TlChunk ring[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) tl_fetch(P, Bv, cb + u, ce, i, hf, ring[u]);
    const size_t n = ce - cb, nfull = cb + n - n % PF;
    for (size_t c0 = cb; c0 < nfull; c0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            at(c0 + u, x);
            x = tl_advance(ring[u], line, i, hf);
            tl_fetch(P, Bv, c0 + u + PF, ce, i, hf, ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        if (nfull + u < ce) {
            at(nfull + u, x);
            x = tl_advance(ring[u], line, i, hf);
        }
    }
    return x;
}

// Group products and offsets: one wavefront per (sequence, group).  Writes
// Pg [B][kTlGroups][32][32] (row-major) and Bg [B][kTlGroups][32]; groups past
// the last chunk are left alone.  Each step issues the product's 16 MFMAs and
// then the offset's matrix-vector step from the same operands, which runs
// while the matrix cores work.
__global__ __launch_bounds__(64) void dense_group_tl32_kernel(
    const float *__restrict__ Pagg, const float *__restrict__ Bagg, const int *__restrict__ skip,
    const int *__restrict__ all_done, int nchunk, float *__restrict__ Pg, float *__restrict__ Bg)
{
    constexpr int D = 32;
    if (all_done && *all_done) return;
    const int bseq = blockIdx.x / kTlGroups, g = blockIdx.x % kTlGroups;
    if (skip && skip[bseq]) return;
    const int GS = tl_group_size(nchunk);
    const int cb = g * GS, ce = min(nchunk, cb + GS);
    if (cb >= ce) return;
    __shared__ __align__(16) float line[D];
    const int lane = threadIdx.x;
    const int i = lane & 31, hf = lane >> 5;
    const size_t q0 = static_cast<size_t>(bseq) * nchunk;
    const size_t qg = static_cast<size_t>(bseq) * kTlGroups + g;
    // the product, accumulators in the B operand layout: register v holds P[row32(v, hf)][i];
    // the offset: the state the group's chunks reach from a zero start
    const float *Pf = Pagg + (q0 + cb) * D * D;
    v16f P;
#pragma unroll
    for (int v = 0; v < 16; ++v) P[v] = Pf[row32(v, hf) * D + i];
    float x = Bagg[(q0 + cb) * D + i];
    tl_set_line(line, x, i, hf);
    TlChunk ring[kTlPF];
#pragma unroll
    for (int u = 0; u < kTlPF; ++u) tl_fetch(Pagg, Bagg, q0 + cb + 1 + u, q0 + ce, i, hf, ring[u]);
    auto step = [&](const TlChunk &k) {
        v16f acc = {};
#pragma unroll
        for (int v = 0; v < 16; ++v) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(k.a[v >> 2][v & 3], P[v], acc, 0, 0, 0);
        x = tl_advance(k, line, i, hf);
        P = acc;
    };
    const int n = ce - cb - 1, nfull = cb + 1 + n - n % kTlPF;
    for (int c0 = cb + 1; c0 < nfull; c0 += kTlPF) {
#pragma unroll
        for (int u = 0; u < kTlPF; ++u) {
            step(ring[u]);
            tl_fetch(Pagg, Bagg, q0 + c0 + u + kTlPF, q0 + ce, i, hf, ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < kTlPF; ++u)
        if (nfull + u < ce) step(ring[u]);
    float *po = Pg + qg * D * D;
#pragma unroll
    for (int v = 0; v < 16; ++v) po[row32(v, hf) * D + i] = P[v];
    if (hf == 0) Bg[qg * D + i] = x;
}

// Carries from the group products: kTlWalkers single-wavefront workgroups per
// sequence, spread over the device (a compute unit keeps only so many cache
// lines in flight, and eight walkers sharing one ran at a third of the speed).
// Walker w pushes s0 through the maps of the groups before its own (at most
// kTlGroups - 2 steps, the same bits in every walker), then walks its
// kTlGroups / kTlWalkers groups' chunks from there, kTlWalkPF chunks of loads
// in flight.
constexpr int kTlWalkers = 8;
constexpr int kTlWalkPF = 10;
__global__ __launch_bounds__(64) void dense_carry_tl32_kernel(
    const float *__restrict__ Pagg, const float *__restrict__ Bagg, const float *__restrict__ Pg,
    const float *__restrict__ Bg, const float *__restrict__ s0, const int *__restrict__ skip,
    const int *__restrict__ all_done, int B, int nchunk, float *__restrict__ carry)
{
    constexpr int D = 32, GPW = kTlGroups / kTlWalkers;
    if (all_done && *all_done) return;
    const int bseq = blockIdx.x / kTlWalkers, w = blockIdx.x % kTlWalkers;
    if (bseq >= B || (skip && skip[bseq])) return;      // uniform per workgroup
    __shared__ __align__(16) float line[D];
    const int lane = threadIdx.x;
    const int i = lane & 31, hf = lane >> 5;
    const int GS = tl_group_size(nchunk);
    const int ngroups = (nchunk + GS - 1) / GS;
    const int cb = w * GPW * GS, ce = min(nchunk, cb + GPW * GS);
    const size_t q0 = static_cast<size_t>(bseq) * nchunk;
    const size_t g0 = static_cast<size_t>(bseq) * kTlGroups;
    const float x0 = s0 ? s0[static_cast<size_t>(bseq) * D + i] : 0.0f;
    auto write_carry = [&](size_t q, float x) {
        if (hf == 0) carry[q * D + i] = x;
    };
    // every group product of the sequence in range? (the same answer in every walker)
    bool out_of_range = false;
    for (int g = 0; g < ngroups; ++g) {
        const float *pg = Pg + (g0 + g) * D * D;
#pragma unroll
        for (int u = 0; u < 16; ++u) out_of_range |= !(__builtin_fabsf(pg[u * 64 + lane]) <= kTlLimit);
    }
    if (__any(out_of_range)) {
        if (w == 0) tl_walk<kTlWalkPF>(Pagg, Bagg, q0, q0 + nchunk, x0, line, i, hf, write_carry);
        return;
    }
    if (cb >= ce) return;
    const float xe = tl_walk<kTlWalkPF>(Pg, Bg, g0, g0 + w * GPW, x0, line, i, hf, [](size_t, float) {});
    tl_walk<kTlWalkPF>(Pagg, Bagg, q0 + cb, q0 + ce, xe, line, i, hf, write_carry);
}

// ----------------------------------------------------------------- replay
// Stage a chunk's d_t and b_t rows ([n][D] each, contiguous at base) into LDS
// with one wavefront, every load of a round in flight at once.
__device__ __forceinline__ void stage_chunk64(const float *__restrict__ dv, const float *__restrict__ bv, size_t base,
                                              int nel, int D, float *dsm, float *bsm)
{
    const int lane = threadIdx.x & 63;
    if ((D & 3) == 0) {
        constexpr int kU = 8;                           // float4 loads per array per lane per round
        for (int e0 = 0; e0 < nel / 4; e0 += 64 * kU) {
            v4f dq[kU], bq[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int e = e0 + lane + 64 * u;
                const int ec = e < nel / 4 ? e : 0;
                dq[u] = *reinterpret_cast<const v4f *>(dv + base + static_cast<size_t>(ec) * 4);
                bq[u] = *reinterpret_cast<const v4f *>(bv + base + static_cast<size_t>(ec) * 4);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int e = e0 + lane + 64 * u;
                if (e < nel / 4) {
                    *reinterpret_cast<v4f *>(dsm + e * 4) = dq[u];
                    *reinterpret_cast<v4f *>(bsm + e * 4) = bq[u];
                }
            }
        }
    } else {
        for (int e = lane; e < nel; e += 64) {
            dsm[e] = dv[base + e];
            bsm[e] = bv[base + e];
        }
    }
}

// D = 32, float32: the replay on the offset chain's row layout (two blocks of
// 16, DPP row rotations, one exchange per step, alternating A / B layouts);
// each step's state is written by both rows that hold a block.
//
// EVAL: each step's y = W s_{t-1} is also the tanh cell's pre-activation less
// the projection, so the next iteration's evaluation rides along: f_t =
// tanh(y + p_t), d_t = shrink (1 - f_t^2) and b_t = f_t - d_t y overwrite the
// chunk's d and b rows (already staged in LDS; no other workgroup reads them),
// and |s_t - f_t| feeds the residual maximum and the front.  Each block of a
// step sits in two rows, so the four (step, block) results of a pair of steps
// are spread over the four rows -- row 1: (A step, block 0), row 2: (A step,
// block 1), row 0: (B step, block 0), row 3: (B step, block 1) -- and every
// lane evaluates once per pair.  The projection of the lane's (step, channel)
// is fetched four pairs ahead into a register ring.
//
// The chunk's d and b rows pass through LDS sixteen steps at a time: the rows
// of the next sixteen steps are requested into registers while the current
// ones replay, then written over them.  Staging the whole chunk at once took
// 16 KB of LDS per wavefront and held a compute unit to ten of these
// latency-bound wavefronts; 4 KB leaves the register file as the limit.
template <bool EVAL>
__global__ __launch_bounds__(64) void dense_replay_dpp32_kernel(
    const float *dv, const float *__restrict__ W, const float *bv, const float *__restrict__ carry,
    const int *__restrict__ skip, const int *__restrict__ all_done, int T, int L, int nchunk, float *out0,
    float *out1, const int *__restrict__ out_sel, ReplayEval ev)
{
    constexpr int D = 32;
    constexpr int RP = 4;                                            // projection ring depth (pairs of steps)
    constexpr int kSt = 16;                                          // steps per LDS stage (a multiple of 2 RP)
    constexpr int kSv = kSt * D / 4 / 64;                            // float4 rows of d (and of b) per lane per stage
    __shared__ float dsm[kSt * D], bsm[kSt * D];
    if (all_done && *all_done) return;
    const long long q = blockIdx.x;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    if (skip && skip[bseq]) return;
    const int t0 = c * L, n = min(L, T - t0);
    const size_t base = (static_cast<size_t>(bseq) * T + t0) * D;
    const int nst = (n + kSt - 1) / kSt;
    v4f dq[kSv], bq[kSv];
    // rows of stage st into registers (clamped: rows past the chunk are never read)
    auto fetch = [&](int st) {
#pragma unroll
        for (int u = 0; u < kSv; ++u) {
            const int e = st * (kSt * D / 4) + static_cast<int>(threadIdx.x) + 64 * u;
            const int ec = e < n * (D / 4) ? e : 0;
            dq[u] = *reinterpret_cast<const v4f *>(dv + base + static_cast<size_t>(ec) * 4);
            bq[u] = *reinterpret_cast<const v4f *>(bv + base + static_cast<size_t>(ec) * 4);
        }
    };
    // stage st into LDS once every lane is done with the previous one, then
    // request the next
    auto stage_in = [&](int st) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kSv; ++u) {
            const int e = static_cast<int>(threadIdx.x) + 64 * u;
            *reinterpret_cast<v4f *>(dsm + e * 4) = dq[u];
            *reinterpret_cast<v4f *>(bsm + e * 4) = bq[u];
        }
        __syncthreads();
        if (st + 1 < nst) fetch(st + 1);
    };
    fetch(0);

    const int lane = threadIdx.x, r = lane >> 4, m = lane & 15;
    const int KA = r & 1, IA = r >> 1, KB = r >> 1, IB = r & 1;
    const bool useB = r == 0 || r == 3;                              // evaluates the B step of each pair
    const int ech = useB ? 16 * IB + m : 16 * IA + m;                // its channel
    const int eofs = useB ? 1 : 0;                                   // its step within the pair
    const float *pc = EVAL ? ev.p + base : nullptr;
    float pr[RP];
    if (EVAL) {
#pragma unroll
        for (int k = 0; k < RP; ++k) pr[k] = pc[min(2 * k + eofs, n - 1) * D + ech];
    }

    int src[16];
    src[0] = m;
    RowRotations::sources(m, src);
    float wA[16], wB[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        wA[k] = W[(16 * IA + m) * D + 16 * KA + src[k]];
        wB[k] = W[(16 * IB + m) * D + 16 * KB + src[k]];
    }
    auto contract = [&](float x, const float (&w)[16]) -> float {
        float a0 = w[0] * x, a1 = 0.0f;
        RowRotations::contract(x, w, a0, a1);
        return a0 + a1;
    };
    float *out = ((out_sel && (*out_sel & 1)) ? out1 : out0) + base;
    float x = carry[static_cast<size_t>(q) * D + 16 * KA + m];      // carried-in state, A layout
    // step s (A layout when even, B when odd): y = W s_{t-1} on the lane's
    // output channel, then s_t into x; returns y
    auto step = [&](int s, bool odd) -> float {
        float y = contract(x, odd ? wB : wA);
        y += __shfl_xor(y, odd ? 32 : 16, 64);
        const int ch = odd ? 16 * IB + m : 16 * IA + m;
        const int ls = (s & (kSt - 1)) * D + ch;
        x = dsm[ls] * y + bsm[ls];
        out[s * D + ch] = x;
        return y;
    };
    int s = 0;
    if (EVAL) {
        float *lout = ev.lin + base, *bout = ev.bout + base;
        unsigned rmax = 0u, fmin = kNoFront;
        auto evaluate = [&](float y, float st, float pv, int se) {
            const float f = tanhf(y + pv);
            const float dd = ev.shrink * (1.0f - f * f);
            lout[se * D + ech] = dd;
            bout[se * D + ech] = f - dd * y;
            const float ra = fabsf(st - f);
            rmax = max(rmax, __float_as_uint(ra));
            fmin = min(fmin, front_of(ra, ev.tol, t0 + se));
        };
        for (; s + 2 * RP <= n; s += 2 * RP) {
            if ((s & (kSt - 1)) == 0) stage_in(s / kSt);
#pragma unroll
            for (int k = 0; k < RP; ++k) {
                const int sa = s + 2 * k;
                const float ya = step(sa, false);
                const float xa = x;
                const float yb = step(sa + 1, true);
                evaluate(useB ? yb : ya, useB ? x : xa, pr[k], sa + eofs);
                // refill the slot with the same pair of the next ring round (clamped in bounds)
                pr[k] = pc[min(sa + 2 * RP + eofs, n - 1) * D + ech];
            }
        }
        if (s < n && (s & (kSt - 1)) == 0) stage_in(s / kSt);    // the tail lies in one stage
#pragma unroll
        for (int k = 0; k < RP; ++k) {
            const int sa = s + 2 * k;
            if (sa + 1 < n) {
                const float ya = step(sa, false);
                const float xa = x;
                const float yb = step(sa + 1, true);
                evaluate(useB ? yb : ya, useB ? x : xa, pr[k], sa + eofs);
            } else if (sa < n) {                                     // a last lone A step
                const float ya = step(sa, false);
                if (!useB) evaluate(ya, x, pr[k], sa);
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            rmax = max(rmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(rmax), o, 64)));
            fmin = min(fmin, static_cast<unsigned>(__shfl_xor(static_cast<int>(fmin), o, 64)));
        }
        if (lane == 0) {
            if (rmax) atomicMax(ev.res_bits + bseq, rmax);
            if (ev.front && fmin != kNoFront) atomicMin(ev.front + bseq, fmin);
        }
    } else {
        for (; s + 1 < n; s += 2) {
            if ((s & (kSt - 1)) == 0) stage_in(s / kSt);
            step(s, false);
            step(s + 1, true);
        }
        if (s < n) {
            if ((s & (kSt - 1)) == 0) stage_in(s / kSt);
            step(s, false);
        }
    }
}

// Factored leaves: one wavefront per chunk re-runs s_t = d_t * (W s_{t-1}) + b_t
// from the chunk's carried-in state.  The chunk's d_t and b_t rows are staged
// in LDS first (every load in flight at once), so the step chain only waits on
// LDS.  Lane (grp, j) owns row j and the KG columns of its group (the carry
// walk's split).  When every lane owns a row (D == DP and the groups fill the
// wavefront) every group writes the (identical) new state, so the step body
// has no branch.
template <int DP, class ACC, bool FULL>
__global__ __launch_bounds__(64) void dense_replay_fact_kernel(
    const float *__restrict__ dv, const float *__restrict__ W, const float *__restrict__ bv,
    const ACC *__restrict__ carry, const int *__restrict__ skip, const int *__restrict__ all_done, int B, int T,
    int D, int L, int nchunk, float *out0, float *out1, const int *__restrict__ out_sel)
{
    using Gm = CarryGeom<DP, ACC>;
    constexpr int G = Gm::G, KG = Gm::KG;
    extern __shared__ float rsm[];                  // d rows [L][D], then b rows [L][D]
    if (all_done && *all_done) return;
    const long long q = blockIdx.x;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    if (skip && skip[bseq]) return;
    const int lane = threadIdx.x;
    const int t0 = c * L, n = min(L, T - t0);
    const size_t base = (static_cast<size_t>(bseq) * T + t0) * D;
    float *dsm = rsm, *bsm = rsm + L * D;
    stage_chunk64(dv, bv, base, n * D, D, dsm, bsm);
    __syncthreads();

    const int grp = lane / DP, j = lane % DP;
    const bool act = grp < G;
    const bool jv = act && j < D;
    const int jr = j < D ? j : D - 1;
    const int k0 = act ? grp * KG : 0;
    float *out = (out_sel && (*out_sel & 1)) ? out1 : out0;
    ACC wseg[KG];
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int k = k0 + i;
        const float w = W[jr * D + (k < D ? k : D - 1)];
        wseg[i] = (jv && k < D) ? static_cast<ACC>(w) : ACC(0);
    }
    ACC st = carry[static_cast<size_t>(q) * D + jr];
    st = jv ? st : ACC(0);
    float *orow = out + base + j;
    for (int s = 0; s < n; ++s) {
        ACC a0 = 0, a1 = 0;
#pragma unroll
        for (int i = 0; i < KG; i += 2) {
            a0 += wseg[i] * __shfl(st, k0 + i, 64);
            if (i + 1 < KG) a1 += wseg[i + 1] * __shfl(st, k0 + i + 1, 64);
        }
        ACC acc = a0 + a1;
#pragma unroll
        for (int o = DP; o < G * DP; o <<= 1) acc += __shfl_xor(acc, o, 64);
        const ACC y = static_cast<ACC>(dsm[s * D + jr]) * acc + static_cast<ACC>(bsm[s * D + jr]);
        st = jv ? y : st;
        if constexpr (FULL) {
            orow[static_cast<size_t>(s) * D] = static_cast<float>(st);
        } else {
            if (grp == 0 && jv) orow[static_cast<size_t>(s) * D] = static_cast<float>(st);
        }
    }
}

template <int DP, bool FACT, class ACC>
__global__ __launch_bounds__(kThreads) void dense_replay_kernel(
    const float *__restrict__ A, const float *__restrict__ dv, const float *__restrict__ W,
    const float *__restrict__ bv, const ACC *__restrict__ carry, const int *__restrict__ skip,
    const int *__restrict__ all_done, int B, int T, int D, int L, int nchunk, float *out0, float *out1,
    const int *__restrict__ out_sel)
{
    if (all_done && *all_done) return;
    constexpr int G = 64 / DP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / DP, j = lane % DP, gbase = grp * DP;
    const long long nq = static_cast<long long>(B) * nchunk;
    long long q = (static_cast<long long>(blockIdx.x) * (kThreads / 64) + wave) * G + grp;
    const bool qvalid = q < nq;
    if (!qvalid) q = 0;
    const int bseq = static_cast<int>(q / nchunk), c = static_cast<int>(q % nchunk);
    const bool act = qvalid && !(skip && skip[bseq]);
    const int t0 = c * L, t1 = min(T, t0 + L);
    const size_t seq = static_cast<size_t>(bseq) * T;
    const bool jv = j < D;
    float *out = (out_sel && (*out_sel & 1)) ? out1 : out0;

    ACC wrow[FACT ? DP : 1];
    if constexpr (FACT) {
#pragma unroll
        for (int k = 0; k < DP; ++k) wrow[k] = (jv && k < D) ? static_cast<ACC>(W[j * D + k]) : ACC(0);
    }
    ACC st = jv ? carry[static_cast<size_t>(q) * D + j] : ACC(0);
    if constexpr (FACT) {
        // d_t and b_t are independent of the chain: fetch them PR steps ahead.
        // The loads are unconditional (row and step clamped into the chunk), so
        // the wait before each use leaves the later prefetches in flight.
        constexpr int PR = 8;                           // chunk lengths are multiples of PR
        const int jr = jv ? j : 0;
        float dr[PR], br[PR];
        auto fetch = [&](int t, float &dd, float &bb) {
            const size_t i = (seq + (t < t1 ? t : t0)) * D + jr;
            dd = dv[i];
            bb = bv[i];
        };
#pragma unroll
        for (int u = 0; u < PR; ++u) fetch(t0 + u, dr[u], br[u]);
        for (int sb = 0; sb < L; sb += PR) {
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                const int t = t0 + sb + u;
                ACC a0 = 0, a1 = 0;
#pragma unroll
                for (int k = 0; k < DP; k += 2) {
                    a0 += wrow[k] * __shfl(st, gbase + k, 64);
                    if (k + 1 < DP) a1 += wrow[k + 1] * __shfl(st, gbase + k + 1, 64);
                }
                const ACC acc = static_cast<ACC>(dr[u]) * (a0 + a1) + static_cast<ACC>(br[u]);
                fetch(t + PR, dr[u], br[u]);
                const bool live = t < t1;
                st = live && jv ? acc : st;
                if (live && act && jv) out[(seq + t) * D + j] = static_cast<float>(st);
            }
        }
    } else {
        for (int s = 0; s < L; ++s) {
            const int t = t0 + s;
            const bool live = t < t1;
            const int tt = live ? t : t0;
            const ACC bj = jv ? static_cast<ACC>(bv[(seq + tt) * D + j]) : ACC(0);
            ACC acc = 0;
#pragma unroll
            for (int k = 0; k < DP; ++k) {
                const ACC akj = (jv && k < D) ? static_cast<ACC>(A[((seq + tt) * D + j) * D + k]) : ACC(0);
                acc += akj * __shfl(st, gbase + k, 64);
            }
            acc = acc + bj;
            if (live) {
                st = acc;
                if (act && jv) out[(seq + t) * D + j] = static_cast<float>(st);
            }
        }
    }
}

int pick_dp(int D) { return D <= 4 ? 4 : D <= 8 ? 8 : D <= 16 ? 16 : D <= 32 ? 32 : 64; }

template <int DP, class ACC>
int launch_dense_dp(const float *A, const float *d, const float *W, const float *b, const float *s0, float *out0,
                    float *out1, const int *out_sel, const int *skip, const int *all_done, const DenseScanPlan &pl,
                    ACC *Pagg, ACC *Bagg, ACC *carry, float *Pgrp, float *Bgrp, hipStream_t stream,
                    const ReplayEval *ev)
{
    constexpr int G = 64 / DP;
    const long long nq = static_cast<long long>(pl.B) * pl.nchunk;
    const long long waves = (nq + G - 1) / G;
    const unsigned blocks = static_cast<unsigned>((waves + 3) / 4);
    const bool f64 = sizeof(ACC) == 8;
    prof_mark_next(kProfCompose);
    if (d && DP == 32 && pl.D == 32 && !f64) {
        DEER_LAUNCH(dense_agg_mfma32_kernel, dim3(static_cast<unsigned>(nq)), dim3(kAggThreads), 0, stream, d, W,
                           b, skip, all_done, pl.T, pl.chunk_len, pl.nchunk, reinterpret_cast<float *>(Pagg),
                           reinterpret_cast<float *>(Bagg));
    } else if (d && DP == 16 && pl.D == 16) {
        DEER_LAUNCH((dense_agg_mfma16_kernel<ACC>), dim3(static_cast<unsigned>(nq)), dim3(64), 0, stream, d, W,
                           b, skip, all_done, pl.T, pl.chunk_len, pl.nchunk, Pagg, Bagg);
    } else if (d) {
        DEER_LAUNCH((dense_agg_kernel<DP, true, ACC>), dim3(blocks), dim3(kThreads), 0, stream, A, d, W, b, skip,
                           all_done, pl.B, pl.T, pl.D, pl.chunk_len, pl.nchunk, Pagg, Bagg);
    } else {
        DEER_LAUNCH((dense_agg_kernel<DP, false, ACC>), dim3(blocks), dim3(kThreads), 0, stream, A, d, W, b,
                           skip, all_done, pl.B, pl.T, pl.D, pl.chunk_len, pl.nchunk, Pagg, Bagg);
    }
    DEER_HIP(hipGetLastError());
    constexpr bool kVecOk = CarryGeom<DP, ACC>::KG % CarryGeom<DP, ACC>::VEC == 0;
    if (DP == 32 && pl.D == 32 && !f64 && pl.nchunk >= kTlMinChunks) {
        const float *Pf = reinterpret_cast<const float *>(Pagg), *Bf = reinterpret_cast<const float *>(Bagg);
        DEER_LAUNCH(dense_group_tl32_kernel, dim3(static_cast<unsigned>(pl.B) * kTlGroups), dim3(64), 0, stream, Pf,
                    Bf, skip, all_done, pl.nchunk, Pgrp, Bgrp);
        DEER_HIP(hipGetLastError());
        DEER_LAUNCH(dense_carry_tl32_kernel, dim3(static_cast<unsigned>(pl.B) * kTlWalkers), dim3(64), 0, stream, Pf,
                    Bf, Pgrp, Bgrp, s0, skip, all_done, pl.B, pl.nchunk, reinterpret_cast<float *>(carry));
    } else if (kVecOk && pl.D == DP)
        DEER_LAUNCH((dense_carry_kernel<DP, ACC, kVecOk>), dim3(static_cast<unsigned>(pl.B)), dim3(64), 0, stream,
                           Pagg, Bagg, s0, skip, all_done, pl.B, pl.D, pl.nchunk, carry);
    else
        DEER_LAUNCH((dense_carry_kernel<DP, ACC, false>), dim3(static_cast<unsigned>(pl.B)), dim3(64), 0, stream,
                           Pagg, Bagg, s0, skip, all_done, pl.B, pl.D, pl.nchunk, carry);
    DEER_HIP(hipGetLastError());
    if (d && DP == 32 && pl.D == 32 && !f64) {
        if (ev)
            DEER_LAUNCH(dense_replay_dpp32_kernel<true>, dim3(static_cast<unsigned>(nq)), dim3(64), 0, stream, d,
                        W, b, reinterpret_cast<const float *>(carry), skip, all_done, pl.T, pl.chunk_len, pl.nchunk,
                        out0, out1, out_sel, *ev);
        else
            DEER_LAUNCH(dense_replay_dpp32_kernel<false>, dim3(static_cast<unsigned>(nq)), dim3(64), 0, stream, d,
                        W, b, reinterpret_cast<const float *>(carry), skip, all_done, pl.T, pl.chunk_len, pl.nchunk,
                        out0, out1, out_sel, ReplayEval{});
    } else if (d) {
        const size_t lds = static_cast<size_t>(pl.chunk_len) * pl.D * 2 * sizeof(float);
        if (pl.D == DP && CarryGeom<DP, ACC>::G * DP == 64)       // every lane owns a row
            DEER_LAUNCH((dense_replay_fact_kernel<DP, ACC, true>), dim3(static_cast<unsigned>(nq)), dim3(64), lds,
                               stream, d, W, b, carry, skip, all_done, pl.B, pl.T, pl.D, pl.chunk_len, pl.nchunk, out0,
                               out1, out_sel);
        else
            DEER_LAUNCH((dense_replay_fact_kernel<DP, ACC, false>), dim3(static_cast<unsigned>(nq)), dim3(64), lds,
                               stream, d, W, b, carry, skip, all_done, pl.B, pl.T, pl.D, pl.chunk_len, pl.nchunk, out0,
                               out1, out_sel);
    } else {
        DEER_LAUNCH((dense_replay_kernel<DP, false, ACC>), dim3(blocks), dim3(kThreads), 0, stream, A, d, W, b,
                           carry, skip, all_done, pl.B, pl.T, pl.D, pl.chunk_len, pl.nchunk, out0, out1, out_sel);
    }
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

template <class ACC>
int launch_dense_acc(const float *A, const float *d, const float *W, const float *b, const float *s0, float *out0,
                     float *out1, const int *out_sel, const int *skip, const int *all_done, const DenseScanPlan &pl,
                     void *state, hipStream_t stream, const ReplayEval *ev)
{
    const size_t nq = static_cast<size_t>(pl.B) * pl.nchunk;
    const int D = pl.D;
    Carve cv(state);
    ACC *Pagg = cv.take<ACC>(nq * D * D);
    ACC *Bagg = cv.take<ACC>(nq * D);
    ACC *carry = cv.take<ACC>(nq * D);
    float *Pgrp = nullptr, *Bgrp = nullptr;             // two-level carry (float, D = 32, many chunks)
    if (tl_carry_shape(D, pl.nchunk)) {
        Pgrp = cv.take<float>(static_cast<size_t>(pl.B) * kTlGroups * D * D);
        Bgrp = cv.take<float>(static_cast<size_t>(pl.B) * kTlGroups * D);
    }
    switch (pick_dp(D)) {
    case 4: return launch_dense_dp<4, ACC>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, Pagg, Bagg, carry, Pgrp, Bgrp, stream, ev);
    case 8: return launch_dense_dp<8, ACC>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, Pagg, Bagg, carry, Pgrp, Bgrp, stream, ev);
    case 16: return launch_dense_dp<16, ACC>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, Pagg, Bagg, carry, Pgrp, Bgrp, stream, ev);
    case 32: return launch_dense_dp<32, ACC>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, Pagg, Bagg, carry, Pgrp, Bgrp, stream, ev);
    default: return launch_dense_dp<64, ACC>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, Pagg, Bagg, carry, Pgrp, Bgrp, stream, ev);
    }
}

}  // namespace

DenseScanPlan dense_scan_plan(int B, int T, int D)
{
    DenseScanPlan p{};
    p.B = B;
    p.T = T;
    p.D = D;
    // Chunks of 64 steps (the longest the compose kernels stage).  Shorter chunks
    // give more parallel composes on small problems, but the carry walk, which
    // is serial per sequence, grows as T / L and dominates there: on B = 32,
    // T = 4096, D = 16 a solve took 0.72 ms with 16-step chunks and 0.58 ms
    // with 64-step ones.
    const int L = 64;
    p.chunk_len = L;
    p.nchunk = (T + L - 1) / L;
    return p;
}

size_t dense_scan_state_bytes(int B, int T, int D, bool f64)
{
    const DenseScanPlan p = dense_scan_plan(B, T, D);
    const size_t nq = static_cast<size_t>(B) * p.nchunk;
    const size_t w = f64 ? sizeof(double) : sizeof(float);
    size_t bytes = align_up(nq * D * D * w) + 2 * align_up(nq * D * w);
    if (tl_carry_shape(D, p.nchunk))
        bytes += align_up(static_cast<size_t>(B) * kTlGroups * D * D * sizeof(float)) +
                 align_up(static_cast<size_t>(B) * kTlGroups * D * sizeof(float));
    return bytes;
}

int launch_dense_scan(const float *A, const float *d, const float *W, const float *b, const float *s0, float *out0,
                      float *out1, const int *out_sel, const int *skip, const int *all_done, int B, int T, int D,
                      bool f64, void *state, hipStream_t stream, const ReplayEval *ev)
{
    if (B == 0 || T == 0) return DEER_OK;
    const DenseScanPlan pl = dense_scan_plan(B, T, D);
    if (!d || !dense_scan_evaluates(D, f64)) ev = nullptr;
    if (f64)
        return launch_dense_acc<double>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, state, stream,
                                        nullptr);
    return launch_dense_acc<float>(A, d, W, b, s0, out0, out1, out_sel, skip, all_done, pl, state, stream, ev);
}

// the replay kernels that evaluate the cell on the fly (factored leaves only)
bool dense_scan_evaluates(int D, bool f64) { return D == 32 && !f64; }

}  // namespace deer
