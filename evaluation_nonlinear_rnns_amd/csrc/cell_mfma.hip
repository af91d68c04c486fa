// Matrix-core (MFMA) kernels for the two dense contractions of the cell
// evaluation:
//   * the GRU's recurrent pre-activations q = W_hh s_{t-1} + b_hh at every
//     position of the trajectory guess, fused with the gates, the Jacobian
//     diagonal, the offsets b_t and the residual (the quasi-DEER evaluation);
//   * the iteration-invariant input projection p = U x_t + b.
// Both are [positions x K] x [K x outputs] products, done 32 x 32 at a time
// with v_mfma_f32_32x32x2f32 (full fp32 operands and accumulation).
//
// Operand layout of v_mfma_f32_32x32x2f32 on a 64-lane wavefront:
//   A (32 x 2):  lane l holds A[l % 32][l / 32]
//   B (2 x 32):  lane l holds B[l / 32][l % 32]
//   C (32 x 32): lane l, register v holds C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
// Here rows are positions and columns are output channels, so a lane owns one
// channel at 16 positions: per-channel loads and stores of a wavefront cover
// two 128-byte row segments, and the three GRU gates of a channel land in the
// same lane and register.
//
// Positions are staged in LDS with a row stride of K + 2 words, which makes the
// A-operand reads (32 rows x 2 columns per instruction) bank-conflict free.
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoid_fast(float u) { return __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
__device__ __forceinline__ float tanh_fast(float u) { return 2.0f * sigmoid_fast(2.0f * u) - 1.0f; }

// row m of the accumulator element held in register v by a lane in half `hf`
__device__ __forceinline__ int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

__device__ __forceinline__ void wave_max_atomic(unsigned v, unsigned *dst)
{
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), o, 64)));
    if ((threadIdx.x & 63) == 0 && v != 0u) atomicMax(dst, v);
}
__device__ __forceinline__ void wave_min_atomic(unsigned v, unsigned *dst)
{
    v = wave_min_u32(v);
    if ((threadIdx.x & 63) == 0 && v != kNoFront) atomicMin(dst, v);
}

// Self-validating look-back descriptor words: float value | 32-bit tag.
constexpr unsigned kDescSpinLimit = 1u << 22;
constexpr int kWin = 4;   // predecessors read per look-back round trip
constexpr int kSeqLds = 256;   // sequences whose residual maxima a workgroup keeps in LDS
__device__ __forceinline__ unsigned long long pack_desc(float v, unsigned tag)
{
    return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}
__device__ __forceinline__ unsigned desc_tag(unsigned long long w) { return static_cast<unsigned>(w >> 32); }
__device__ __forceinline__ float desc_val(unsigned long long w) { return __uint_as_float(static_cast<unsigned>(w)); }
__device__ __forceinline__ unsigned long long load_desc(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_desc(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ GRU evaluation
template <int D>
struct GruGeom {
    static constexpr int NCB = D / 32;       // 32-channel blocks
    static constexpr int KK = D / 2;         // k-steps of the 32x32x2 MFMA
    static constexpr int PSUB = 4 / NCB;     // 32-position sub-tiles per workgroup tile
    static constexpr int TP = 32 * PSUB;     // positions per tile
    static constexpr int LDH = D + 2;        // LDS row stride
};

// Gate order (r, z, n); p = W_ih x + b_ih precomputed in the tiled layout of
// proj_tiled_index().  For a lane's channel c:
//   r = sigma(p_r + q_r), z = sigma(p_z + q_z), n = tanh(p_n + r q_n)
//   f = (1 - z) n + z h
//   a = z + (h - n) z (1 - z) Wz_cc + (1 - z)(1 - n^2)(r Wn_cc + r (1 - r) Wr_cc q_n)
//   b = f - a h,   residual |s_t - f|
//
// Tiles of TP positions are software-pipelined: the state rows of tile i+1
// are fetched into registers and its input pre-activations are requested
// while the matrix cores work on tile i.
template <int D>
struct GruTile {
    static constexpr int NH = ((GruGeom<D>::TP + 1) * (D / 4) + kThreads - 1) / kThreads;   // float4 per thread
};

// Tile coordinates (sequence bseq, first position t0) are passed in: the tile
// loops track them incrementally, which keeps 64-bit divisions out of the loop.
template <int D>
__device__ __forceinline__ void gru_fetch_rows(const float *__restrict__ s, const float *__restrict__ s0, int T,
                                               int bseq, int t0, v4f (&hv)[GruTile<D>::NH])
{
    using G = GruGeom<D>;
    const int tid = threadIdx.x;
    const size_t seq = static_cast<size_t>(bseq) * T;
#pragma unroll
    for (int i = 0; i < GruTile<D>::NH; ++i) {
        const int e = tid + i * kThreads;
        v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e < (G::TP + 1) * (D / 4)) {
            const int r = e / (D / 4), q = (e % (D / 4)) * 4;
            const int t = t0 - 1 + r;
            if (t < 0) {
                if (s0) v = *reinterpret_cast<const v4f *>(s0 + static_cast<size_t>(bseq) * D + q);
            } else if (t < T && s) {
                v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(s + (seq + t) * D + q));
            }
        }
        hv[i] = v;
    }
}

// Rows x_{t0} .. x_{t0+TP-1} of the inputs (M = D columns) into the row
// registers, zero past T: the A operands of the first iteration's projection.
template <int D>
__device__ __forceinline__ void gru_fetch_xrows(const float *__restrict__ x, int T, int bseq, int t0,
                                                v4f (&hv)[GruTile<D>::NH])
{
    using G = GruGeom<D>;
    const int tid = threadIdx.x;
    const size_t seq = static_cast<size_t>(bseq) * T;
#pragma unroll
    for (int i = 0; i < GruTile<D>::NH; ++i) {
        const int e = tid + i * kThreads;
        v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e < G::TP * (D / 4)) {
            const int r = e / (D / 4), q = (e % (D / 4)) * 4;
            const int t = t0 + r;
            if (t < T) v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + (seq + t) * D + q));
        }
        hv[i] = v;
    }
}

// Tiled projection of the lane's 16 positions: 32-position block, gate g,
// quad q, half hf, channel c, 4 positions per 16-byte access (load u = 4 g + q).
template <int D>
__device__ __forceinline__ const v4f *gru_proj_base(const float *__restrict__ pt, int tps32, int bseq, int t0, int ps)
{
    const size_t blk = static_cast<size_t>(bseq) * tps32 + (t0 >> 5) + ps;
    return reinterpret_cast<const v4f *>(pt + blk * (96 * static_cast<size_t>(D)));
}
template <int D>
__device__ __forceinline__ v4f gru_proj_load(const v4f *base, int u, int hf, int c)
{
    return __builtin_nontemporal_load(base + (u * 2 + hf) * D + c);
}

template <int D>
__device__ __forceinline__ void gru_fetch(const float *__restrict__ s, const float *__restrict__ s0,
                                          const float *__restrict__ pt, int T, int tps32, int bseq, int t0,
                                          int ps, int hf, int c, v4f (&hv)[GruTile<D>::NH], v4f (&pv)[3][4])
{
    gru_fetch_rows<D>(s, s0, T, bseq, t0, hv);
    const v4f *base = gru_proj_base<D>(pt, tps32, bseq, t0, ps);
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) pv[g][q] = gru_proj_load<D>(base, 4 * g + q, hf, c);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void gru_eval_mfma_kernel(
    const float *__restrict__ Whh, const float *__restrict__ bhh, const float *__restrict__ pt,
    const float *__restrict__ s0, const float *s_even, const float *s_odd, const int *__restrict__ sel,
    const int *__restrict__ skip, const int *__restrict__ all_done, float *__restrict__ aout,
    float *__restrict__ bout, unsigned *__restrict__ res_bits, int T, int tiles_per_seq, long long ntiles,
    Linearization lz, FrontOut fo)
{
    using G = GruGeom<D>;
    if (all_done && *all_done) return;
    __shared__ float H[(G::TP + 1) * G::LDH];   // H[r] = s_{t0 - 1 + r}
    __shared__ float Ws[3 * D * G::LDH];        // Ws[g D + c][k] = W_hh[g D + c][k]  (B operands)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cb = wave % G::NCB, ps = wave / G::NCB;
    const int r32 = lane & 31, hf = lane >> 5;
    const int c = cb * 32 + r32;                 // this lane's channel
    const int tps32 = (T + 31) / 32;

    for (int e = tid; e < 3 * D * D; e += kThreads) {
        const int o = e / D, k = e % D;
        Ws[o * G::LDH + k] = Whh[e];
    }
    const float br = bhh ? bhh[c] : 0.0f, bz = bhh ? bhh[D + c] : 0.0f, bn = bhh ? bhh[2 * D + c] : 0.0f;
    const float wr = Whh[static_cast<size_t>(c) * D + c];
    const float wz = Whh[static_cast<size_t>(D + c) * D + c];
    const float wn = Whh[static_cast<size_t>(2 * D + c) * D + c];
    const float *s = (sel && (*sel & 1)) ? s_odd : s_even;
    float *fdst = (sel && (*sel & 1)) ? bout : aout;   // kLinValue output

    const long long tb = ntiles * blockIdx.x / gridDim.x, te = ntiles * (blockIdx.x + 1) / gridDim.x;
    if (tb >= te) return;
    unsigned rmax = 0u, fmin = kNoFront;
    int cur = -1;
    v4f hv[GruTile<D>::NH];
    v4f pv[3][4];
    // the workgroup's contiguous range of sequence-major tiles, coordinates stepped per tile
    int bseq = static_cast<int>(tb / tiles_per_seq), tt = static_cast<int>(tb % tiles_per_seq);
    gru_fetch<D>(s, s0, pt, T, tps32, bseq, tt * G::TP, ps, hf, c, hv, pv);
    for (long long tile = tb; tile < te; ++tile) {
        const int t0 = tt * G::TP;
        int nb = bseq, nt = tt + 1;                  // the next tile of the range
        if (nt == tiles_per_seq) { nt = 0; ++nb; }
        if (bseq != cur) {
            if (cur >= 0) {
                wave_max_atomic(rmax, res_bits + cur);
                if (fo.front) wave_min_atomic(fmin, fo.front + cur);
            }
            rmax = 0u;
            fmin = kNoFront;
            cur = bseq;
        }
        const bool live = !(skip && skip[bseq]);  // uniform over the workgroup
        __syncthreads();                          // the previous tile is done with H
#pragma unroll
        for (int i = 0; i < GruTile<D>::NH; ++i) {
            const int e = tid + i * kThreads;
            if (e < (G::TP + 1) * (D / 4)) {
                const int r = e / (D / 4), q = (e % (D / 4)) * 4;
                float *hrow = H + r * G::LDH + q;
                hrow[0] = hv[i][0]; hrow[1] = hv[i][1]; hrow[2] = hv[i][2]; hrow[3] = hv[i][3];
            }
        }
        __syncthreads();
        v4f pc[3][4];
#pragma unroll
        for (int g = 0; g < 3; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) pc[g][q] = pv[g][q];
        if (tile + 1 < te) gru_fetch<D>(s, s0, pt, T, tps32, nb, nt * G::TP, ps, hf, c, hv, pv);
        const int this_seq = bseq;
        bseq = nb;
        tt = nt;
        if (!live) continue;

        v16f accR = {}, accZ = {}, accN = {};
        const float *arow = H + (ps * 32 + r32) * G::LDH + hf;
        const float *wrow = Ws + c * G::LDH + hf;
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
            const float av = arow[2 * kk];
            accR = __builtin_amdgcn_mfma_f32_32x32x2f32(av, wrow[2 * kk], accR, 0, 0, 0);
            accZ = __builtin_amdgcn_mfma_f32_32x32x2f32(av, wrow[D * G::LDH + 2 * kk], accZ, 0, 0, 0);
            accN = __builtin_amdgcn_mfma_f32_32x32x2f32(av, wrow[2 * D * G::LDH + 2 * kk], accN, 0, 0, 0);
        }

        const size_t seq = static_cast<size_t>(this_seq) * T;
        const bool full = t0 + ps * 32 + 32 <= T;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int pos = ps * 32 + acc_row(v, hf);
            const int t = t0 + pos;
            if (!full && t >= T) continue;
            const float qr = accR[v] + br, qz = accZ[v] + bz, qn = accN[v] + bn;
            const float h = H[pos * G::LDH + c];
            const float st = H[(pos + 1) * G::LDH + c];
            const float rg = sigmoid_fast(pc[0][v >> 2][v & 3] + qr);
            const float zg = sigmoid_fast(pc[1][v >> 2][v & 3] + qz);
            const float ng = tanh_fast(pc[2][v >> 2][v & 3] + rg * qn);
            const float f = (1.0f - zg) * ng + zg * h;
            const float a = lin_diag(lz, zg + (h - ng) * zg * (1.0f - zg) * wz +
                                             (1.0f - zg) * (1.0f - ng * ng) * (rg * wn + rg * (1.0f - rg) * wr * qn));
            const size_t o = (seq + t) * D + c;
            if (lz.kind == kLinValue) {
                __builtin_nontemporal_store(f, fdst + o);
            } else {
                __builtin_nontemporal_store(a, aout + o);
                __builtin_nontemporal_store(f - a * h, bout + o);
            }
            const float ra = fabsf(st - f);
            rmax = max(rmax, __float_as_uint(ra));
            fmin = min(fmin, front_of(ra, fo.tol, t));
        }
    }
    if (cur >= 0) {
        wave_max_atomic(rmax, res_bits + cur);
        if (fo.front) wave_min_atomic(fmin, fo.front + cur);
    }
}

// ------------------------------------------------- fused quasi-DEER GRU step
// One launch per Newton iteration: the evaluation above, followed in the same
// workgroup by the diagonal scan of the (a_t, b_t) it just produced, so that
// s^(i+1) is written directly and a, b never reach HBM.  Per position the
// launch reads s^(i) and the projection and writes s^(i+1): (D + 3D + D) words.
//
// The scan composes (a_j, b_j) o (a_i, b_i) = (a_j a_i, a_j b_i + b_j), the
// later map on the left ("Parallel Broyden Methods", appendix C.2), at four
// levels: the 4 consecutive positions a lane holds, the 8 position groups of
// a 32-position sub-tile (exchanged between the lane pair l, l ^ 32), the
// sub-tiles of the workgroup's tile (LDS), and the tiles of a sequence (the
// deterministic decoupled look-back of the standalone diagonal scan, with
// self-validating 64-bit descriptors).  Tiles are taken in the
// strided order blockIdx.x, blockIdx.x + G, ...; with the whole persistent grid
// resident the smallest waiting tile's predecessors are always done or in
// progress.
//
// The residual of the iterate is reduced per tile into res_tile[tile] (plain
// stores; the convergence test takes the max over a sequence's tiles).
//
// FIRST: the first iteration from a zero start and a zero initial state, with
// the input projection computed here instead of by a separate launch (inputs of
// width M = D).  Every state read is zero (s_0 included), so W_hh s vanishes and the matrix cores compute the
// projection W_ih x_t of the tile instead (W_ih as the B operands, the rows of
// x as the A operands); the lane adds b_ih, writes its values to the tiled
// projection that the later iterations read, and evaluates the gates with
// q = b_hh and h = 0.  This reads x (D words per position) and writes the
// projection once, where the separate launch read x and wrote the projection
// and this iteration then read it back.
template <int D, bool FIRST>
__global__ __launch_bounds__(kThreads, 2) void gru_quasi_step_kernel(
    const float *__restrict__ Whh, const float *__restrict__ bhh, const float *__restrict__ pt,
    const float *__restrict__ s0, float *s_even, float *s_odd, SolveControl *ctl, int *done, int *iters,
    int *status, float *resid, float tol, int max_iter, unsigned *res_bits, unsigned *__restrict__ res_tile, int T,
    int tiles_per_seq,
    int nseq, long long ntiles, int zero_start, Linearization lz, StallCheck sc, ScanHeader *__restrict__ hdr,
    unsigned long long *__restrict__ desc, const float *__restrict__ xin, const float *__restrict__ Wih,
    const float *__restrict__ bih, float *pt_out, int *poll)
{
    using G = GruGeom<D>;
    if (ctl->all_done) return;                   // same value for every workgroup of the launch
    const int *sel = &ctl->iter;
    const int *skip = done;
    __shared__ float H[(G::TP + 1) * G::LDH];    // H[r] = s_{t0 - 1 + r}
    __shared__ float Ws[3 * D * G::LDH];         // Ws[g D + c][k] = W_hh[g D + c][k]
    __shared__ float shA[G::PSUB][D], shB[G::PSUB][D], shC[D];
    __shared__ unsigned red[kThreads / 64];
    __shared__ unsigned seqmax[kSeqLds];         // this workgroup's residual maxima per sequence

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cb = wave % G::NCB, ps = wave / G::NCB;
    const int r32 = lane & 31, hf = lane >> 5;
    const int c = cb * 32 + r32;
    const int tps32 = (T + 31) / 32;
    const bool per_seq = nseq <= kSeqLds;        // else per-tile maxima go to res_tile
    for (int b = tid; b < kSeqLds; b += kThreads) seqmax[b] = 0u;

    const float *Wop = FIRST ? Wih : Whh;       // B operands of the matrix-core phase
    for (int e = tid; e < 3 * D * D; e += kThreads) {
        const int o = e / D, k = e % D;
        Ws[o * G::LDH + k] = Wop[e];
    }
    const float br = bhh ? bhh[c] : 0.0f, bz = bhh ? bhh[D + c] : 0.0f, bn = bhh ? bhh[2 * D + c] : 0.0f;
    float pb[3] = {0.0f, 0.0f, 0.0f};           // b_ih of the lane's channel (first iteration)
    if (FIRST && bih) {
        pb[0] = bih[c];
        pb[1] = bih[D + c];
        pb[2] = bih[2 * D + c];
    }
    const float wr = Whh[static_cast<size_t>(c) * D + c];
    const float wz = Whh[static_cast<size_t>(D + c) * D + c];
    const float wn = Whh[static_cast<size_t>(2 * D + c) * D + c];
    const int iter = *sel;
    const bool odd = ((iter ^ ctl->flip) & 1) != 0;   // s^(i) lives in buffer (i ^ flip) % 2
    const float *s = (zero_start && iter == 0) ? nullptr : (odd ? s_odd : s_even);   // the iterate s^(i)
    float *out = odd ? s_even : s_odd;           // s^(i+1)
    const unsigned epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tag_agg = epoch * 4u + 1u, tag_inc = epoch * 4u + 2u;

    v4f hv[GruTile<D>::NH];
    v4f pv[3][4];
    // Tiles are numbered time-major (k -> sequence k % nseq, tile k / nseq) so that
    // the tiles in flight at once spread over the sequences and look-back walks stay
    // short.  Workgroup g takes k = g, g + G, ...; the coordinates step by
    // (G % nseq, G / nseq) with a carry, so the loop does no divisions.
    const int gq = static_cast<int>(gridDim.x) / nseq, gr = static_cast<int>(gridDim.x) % nseq;
    int bseq = static_cast<int>(blockIdx.x) % nseq, tt = static_cast<int>(blockIdx.x) / nseq;
    (void)ntiles;
    if (FIRST) {
#pragma unroll
        for (int g = 0; g < 3; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) pv[g][q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        if (tt < tiles_per_seq) gru_fetch_xrows<D>(xin, T, bseq, tt * G::TP, hv);
    } else if (tt < tiles_per_seq) {
        gru_fetch<D>(s, s0, pt, T, tps32, bseq, tt * G::TP, ps, hf, c, hv, pv);
    }
    for (; tt < tiles_per_seq;) {
        const int t0 = tt * G::TP;
        int nb = bseq + gr, nt = tt + gq;         // the workgroup's next tile
        if (nb >= nseq) { nb -= nseq; ++nt; }
        const bool live = !(skip && skip[bseq]);  // uniform over the workgroup
        __syncthreads();                          // the previous tile is done with H and the exchange arrays
#pragma unroll
        for (int i = 0; i < GruTile<D>::NH; ++i) {
            const int e = tid + i * kThreads;
            if (e < (G::TP + 1) * (D / 4)) {
                const int r = e / (D / 4), q = (e % (D / 4)) * 4;
                float *hrow = H + r * G::LDH + q;
                hrow[0] = hv[i][0]; hrow[1] = hv[i][1]; hrow[2] = hv[i][2]; hrow[3] = hv[i][3];
            }
        }
        __syncthreads();
        v4f pc[3][4];
#pragma unroll
        for (int g = 0; g < 3; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) pc[g][q] = pv[g][q];
        if (nt < tiles_per_seq) {
            if (FIRST)
                gru_fetch_xrows<D>(xin, T, nb, nt * G::TP, hv);
            else
                gru_fetch_rows<D>(s, s0, T, nb, nt * G::TP, hv);
        }
        if (!live) {
            if (!FIRST && nt < tiles_per_seq) {
                const v4f *nbase = gru_proj_base<D>(pt, tps32, nb, nt * G::TP, ps);
#pragma unroll
                for (int u = 0; u < 12; ++u) pv[u / 4][u % 4] = gru_proj_load<D>(nbase, u, hf, c);
            }
            // a skipped tile waits for its loads here, so that the live path never
            // enters with loads pending into registers it reuses (which would put
            // waits for them into its MFMA phase)
#pragma unroll
            for (int g = 0; g < 3; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(pv[g][q]));
#pragma unroll
            for (int i = 0; i < GruTile<D>::NH; ++i) asm volatile("" ::"v"(hv[i]));
            bseq = nb;
            tt = nt;
            continue;
        }

        // W_hh s on the matrix cores, one pair of k-steps (6 MFMAs) per fenced
        // segment, with the pair's LDS operands read one segment ahead and the
        // next tile's 12 projection loads spread over the segments: spreading
        // them lets the memory stream run under the MFMA phase instead of
        // arriving as one burst per tile.  The workgroup's last tile runs the
        // same segments without loads.
        v16f accR = {}, accZ = {}, accN = {};
        const float *arow = H + (ps * 32 + r32) * G::LDH + hf;
        const float *wrow = Ws + c * G::LDH + hf;
        auto mfma_phase = [&](auto prefetch) {
            constexpr int NPAIR = G::KK / 2;
            const v4f *nbase = gru_proj_base<D>(pt, tps32, nb, nt * G::TP, ps);
            float oa[2], orr[2], oz[2], on[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                oa[h] = arow[2 * h];
                orr[h] = wrow[2 * h];
                oz[h] = wrow[D * G::LDH + 2 * h];
                on[h] = wrow[2 * D * G::LDH + 2 * h];
            }
#pragma unroll
            for (int kp = 0; kp < NPAIR; ++kp) {
                float na[2], nr[2], nz[2], nn[2];
                if (kp + 1 < NPAIR) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int k2 = 2 * (2 * (kp + 1) + h);
                        na[h] = arow[k2];
                        nr[h] = wrow[k2];
                        nz[h] = wrow[D * G::LDH + k2];
                        nn[h] = wrow[2 * D * G::LDH + k2];
                    }
                }
                if (decltype(prefetch)::value) {
#pragma unroll
                    for (int u = kp * 12 / NPAIR; u < (kp + 1) * 12 / NPAIR; ++u)
                        pv[u / 4][u % 4] = gru_proj_load<D>(nbase, u, hf, c);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    accR = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[h], orr[h], accR, 0, 0, 0);
                    accZ = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[h], oz[h], accZ, 0, 0, 0);
                    accN = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[h], on[h], accN, 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (kp + 1 < NPAIR) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        oa[h] = na[h];
                        orr[h] = nr[h];
                        oz[h] = nz[h];
                        on[h] = nn[h];
                    }
                }
            }
        };
        if (!FIRST && nt < tiles_per_seq)
            mfma_phase(std::true_type{});
        else
            mfma_phase(std::false_type{});

        if (FIRST) {
            // the accumulators hold W_ih x_t: the projection of this tile, written
            // out for the later iterations (sub-tiles past the sequence's last
            // 32-position block are not its own), and W_hh s = 0 for the gates
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                pc[0][v >> 2][v & 3] = accR[v] + pb[0];
                pc[1][v >> 2][v & 3] = accZ[v] + pb[1];
                pc[2][v >> 2][v & 3] = accN[v] + pb[2];
                accR[v] = 0.0f;
                accZ[v] = 0.0f;
                accN[v] = 0.0f;
            }
            if (t0 + ps * 32 < T) {
                v4f *pbase = const_cast<v4f *>(gru_proj_base<D>(pt_out, tps32, bseq, t0, ps));
#pragma unroll
                for (int u = 0; u < 12; ++u)
                    __builtin_nontemporal_store(pc[u / 4][u % 4], pbase + (u * 2 + hf) * D + c);
            }
        }

        // gates, Jacobian diagonal and offsets at the lane's 16 positions
        const bool full = t0 + ps * 32 + 32 <= T;
        float la[16], lb[16];
        unsigned rmax = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int pos = ps * 32 + acc_row(v, hf);
            const int t = t0 + pos;
            const float qr = accR[v] + br, qz = accZ[v] + bz, qn = accN[v] + bn;
            const float h = FIRST ? 0.0f : H[pos * G::LDH + c];          // the first iterate is zero
            const float st = FIRST ? 0.0f : H[(pos + 1) * G::LDH + c];
            const float rg = sigmoid_fast(pc[0][v >> 2][v & 3] + qr);
            const float zg = sigmoid_fast(pc[1][v >> 2][v & 3] + qz);
            const float ng = tanh_fast(pc[2][v >> 2][v & 3] + rg * qn);
            const float f = (1.0f - zg) * ng + zg * h;
            const float a = lin_diag(lz, zg + (h - ng) * zg * (1.0f - zg) * wz +
                                             (1.0f - zg) * (1.0f - ng * ng) * (rg * wn + rg * (1.0f - rg) * wr * qn));
            const bool in = full || t < T;
            la[v] = in ? a : 1.0f;
            lb[v] = in ? f - a * h : 0.0f;
            if (in) rmax = max(rmax, __float_as_uint(fabsf(st - f)));
        }

        // level 1: the lane's four runs of 4 consecutive positions
        float GA[4], GB[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            GA[q] = 1.0f;
            GB[q] = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                GB[q] = la[4 * q + r] * GB[q] + lb[4 * q + r];
                GA[q] = la[4 * q + r] * GA[q];
            }
        }
        // level 2: runs alternate between the lane pair (l, l ^ 32) in position order
        float EA[4], EB[4];
        float accA = 1.0f, accB = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float oA = __shfl_xor(GA[q], 32, 64), oB = __shfl_xor(GB[q], 32, 64);
            const float fA = hf ? oA : GA[q], fB = hf ? oB : GB[q];   // earlier run of the pair
            const float sA = hf ? GA[q] : oA, sB = hf ? GB[q] : oB;   // later run
            const float midA = fA * accA, midB = fA * accB + fB;
            EA[q] = hf ? midA : accA;
            EB[q] = hf ? midB : accB;
            accB = sA * midB + sB;
            accA = sA * midA;
        }
        for (int o = 32; o > 0; o >>= 1) rmax = max(rmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(rmax), o, 64)));
        if (lane == 0) red[wave] = rmax;
        if (hf == 0) { shA[ps][c] = accA; shB[ps][c] = accB; }
        __syncthreads();

        // level 4: tile aggregate per channel, look-back over the sequence's earlier tiles
        if (tid == 0) {
            unsigned m = red[0];
            for (int w = 1; w < kThreads / 64; ++w) m = max(m, red[w]);
            if (per_seq) seqmax[bseq] = max(seqmax[bseq], m);
            else res_tile[static_cast<size_t>(bseq) * tiles_per_seq + tt] = m;
            // finite-step front at tile granularity: the tile's last position
            // bounds the first violating one from above, so a stall read from it
            // is never a false one (it is seen up to one tile later)
            if (sc.front && !(__uint_as_float(m) <= tol))
                atomicMin(sc.front + bseq, static_cast<unsigned>(min(t0 + G::TP, T) - 1));
        }
        if (tid < D) {
            const int cc = tid;
            float TA = 1.0f, TB = 0.0f;
#pragma unroll
            for (int k = 0; k < G::PSUB; ++k) {
                TB = shA[k][cc] * TB + shB[k][cc];
                TA = shA[k][cc] * TA;
            }
            const unsigned long long *base = desc + static_cast<size_t>(bseq) * tiles_per_seq * 3 * D;
            unsigned long long *mine = desc + (static_cast<size_t>(bseq) * tiles_per_seq + tt) * 3 * D;
            float carry;
            if (tt == 0) {
                carry = s0 ? s0[static_cast<size_t>(bseq) * D + cc] : 0.0f;
            } else {
                store_desc(mine + cc, pack_desc(TA, tag_agg));
                store_desc(mine + D + cc, pack_desc(TB, tag_agg));
                carry = chained_carry<kWin>(base, 3 * D, cc, D + cc, 2 * D + cc, tt, tag_agg, tag_inc, &hdr->abort,
                                            kDescSpinLimit);
            }
            store_desc(mine + 2 * D + cc, pack_desc(__builtin_fmaf(TA, carry, TB), tag_inc));
            shC[cc] = carry;
        }
        __syncthreads();

        // replay: state entering the sub-tile, then the lane's runs
        float PA = 1.0f, PB = 0.0f;
        for (int k = 0; k < ps; ++k) {
            PB = shA[k][c] * PB + shB[k][c];
            PA = shA[k][c] * PA;
        }
        const float x0 = PA * shC[c] + PB;
        const size_t seq = static_cast<size_t>(bseq) * T;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float xs = EA[q] * x0 + EB[q];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = 4 * q + r;
                xs = la[v] * xs + lb[v];
                const int t = t0 + ps * 32 + acc_row(v, hf);
                if (full || t < T) __builtin_nontemporal_store(xs, out + (seq + t) * D + c);
            }
        }
        bseq = nb;
        tt = nt;
    }

    // The last workgroup out resets the done counter, advances the epoch and
    // runs the convergence test of this iteration on the residual maxima.
    __shared__ int sh_last;
    __syncthreads();
    if (per_seq)
        for (int b = tid; b < nseq; b += kThreads)
            if (seqmax[b]) atomicMax(res_bits + b, seqmax[b]);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = (prev == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!sh_last) return;
    __threadfence();
    if (tid == 0) {
        __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->epoch, epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (per_seq)
        finalize_iteration(ctl, res_bits, nullptr, 0, done, iters, status, resid, nseq, tol, max_iter, red, sc, poll);
    else
        finalize_iteration(ctl, nullptr, res_tile, tiles_per_seq, done, iters, status, resid, nseq, tol, max_iter, red,
                           sc, poll);
}

// ------------------------------------------------------------ input projection
// out[n][o] = sum_k U[o][k] x[n][k] + bias[o] for O = 32 NOB outputs, K <= KP.
// Row-major output ([B,T,O]) or, with TILED, the layout the GRU evaluation
// reads: per sequence, blocks of 32 positions; inside a block the entry for
// position 8q + 4h + r and output o = g D + c sits at ((g 4 + q) 2 + h) D + c)
// 4 + r, so one lane of the evaluation loads 4 positions of a channel with one
// 16-byte access.
template <int KP, int NOB>
struct ProjGeom {
    static constexpr int KK = KP / 2;
    static constexpr int PS = (NOB % 4 == 0) ? 1 : (NOB % 2 == 0) ? 2 : 4;   // 32-row sub-tiles per tile
    static constexpr int TP = 32 * PS;
    static constexpr int PAIRS = PS * NOB / 4;                               // (sub-tile, block) pairs per wave
    static constexpr int LDX = KP + 2;
};

template <int KP, int NOB>
struct ProjTile {
    static constexpr int NX = (ProjGeom<KP, NOB>::TP * KP / 4 + kThreads - 1) / kThreads;   // float4 per thread
};

// x rows of one tile (sub-tiles of 32 positions never straddle sequences).
// Rows past the end of a sequence and columns past M read as zero.
template <int KP, int NOB>
__device__ __forceinline__ void proj_fetch(const float *__restrict__ x, int T, int M, int tps32, long long nsub,
                                           long long tile, v4f (&xv)[ProjTile<KP, NOB>::NX])
{
    using G = ProjGeom<KP, NOB>;
#pragma unroll
    for (int i = 0; i < ProjTile<KP, NOB>::NX; ++i) {
        const int e = threadIdx.x + i * kThreads;
        v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (e < G::TP * KP / 4) {
            const int r = e / (KP / 4), k = (e % (KP / 4)) * 4;
            const long long u = tile * G::PS + r / 32;
            if (u < nsub) {
                const long long bseq = u / tps32;
                const int t = static_cast<int>(u - bseq * tps32) * 32 + (r % 32);
                if (t < T) {
                    const float *src = x + (static_cast<size_t>(bseq) * T + t) * M + k;
                    if ((M & 3) == 0 && k + 4 <= M) {
                        v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(src));
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = (k + j < M) ? src[j] : 0.0f;
                    }
                }
            }
        }
        xv[i] = v;
    }
}

template <int KP, int NOB, bool TILED>
__global__ __launch_bounds__(kThreads) void projection_mfma_kernel(const float *__restrict__ x,
                                                                   const float *__restrict__ U,
                                                                   const float *__restrict__ bias,
                                                                   float *__restrict__ out, int T, int M,
                                                                   int tps32, long long nsub)
{
    using G = ProjGeom<KP, NOB>;
    constexpr int O = 32 * NOB;
    constexpr int DG = O / 3;                    // GRU state size when TILED (O = 3 D)
    __shared__ float Ws[O * G::LDX];             // Ws[o][k] = U[o][k]
    __shared__ float Xs[G::TP * G::LDX];         // Xs[r][k]: row r of the tile's sub-tiles
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, hf = lane >> 5;
    for (int e = tid; e < O * KP; e += kThreads) {
        const int o = e / KP, k = e % KP;
        Ws[o * G::LDX + k] = (k < M) ? U[static_cast<size_t>(o) * M + k] : 0.0f;
    }
    const long long ntiles = (nsub + G::PS - 1) / G::PS;
    const long long tb = ntiles * blockIdx.x / gridDim.x, te = ntiles * (blockIdx.x + 1) / gridDim.x;
    if (tb >= te) return;
    // biases of this lane's output column in each (sub-tile, block) pair, read
    // once: a conditional load inside the tile loop would wait for the prefetch
    float bov[G::PAIRS];
#pragma unroll
    for (int pi = 0; pi < G::PAIRS; ++pi) {
        const int ob = (wave * G::PAIRS + pi) % NOB;
        bov[pi] = bias ? bias[ob * 32 + r32] : 0.0f;
    }
    v4f xv[ProjTile<KP, NOB>::NX];
    proj_fetch<KP, NOB>(x, T, M, tps32, nsub, tb, xv);
    for (long long tile = tb; tile < te; ++tile) {
        __syncthreads();                         // the previous tile is done with Xs
#pragma unroll
        for (int i = 0; i < ProjTile<KP, NOB>::NX; ++i) {
            const int e = tid + i * kThreads;
            if (e < G::TP * KP / 4) {
                const int r = e / (KP / 4), k = (e % (KP / 4)) * 4;
                float *dst = Xs + r * G::LDX + k;
                dst[0] = xv[i][0]; dst[1] = xv[i][1]; dst[2] = xv[i][2]; dst[3] = xv[i][3];
            }
        }
        __syncthreads();
        if (tile + 1 < te) proj_fetch<KP, NOB>(x, T, M, tps32, nsub, tile + 1, xv);
#pragma unroll
        for (int pi = 0; pi < G::PAIRS; ++pi) {
            const int pair = wave * G::PAIRS + pi;
            const int sub = pair / NOB, ob = pair % NOB;
            const long long u = tile * G::PS + sub;
            if (u >= nsub) continue;
            v16f acc = {};
            const float *arow = Xs + (sub * 32 + r32) * G::LDX + hf;
            const float *brow = Ws + (ob * 32 + r32) * G::LDX + hf;
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[2 * kk], brow[2 * kk], acc, 0, 0, 0);
            const int o = ob * 32 + r32;
            const float bo = bov[pi];
            if constexpr (TILED) {
                const int g = o / DG, cch = o % DG;
                v4f *dst = reinterpret_cast<v4f *>(out + static_cast<size_t>(u) * (32 * O));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4f w;
                    w[0] = acc[4 * q] + bo; w[1] = acc[4 * q + 1] + bo; w[2] = acc[4 * q + 2] + bo; w[3] = acc[4 * q + 3] + bo;
                    __builtin_nontemporal_store(w, dst + ((g * 4 + q) * 2 + hf) * DG + cch);
                }
            } else {
                const long long bseq = u / tps32;
                const int tb32 = static_cast<int>(u - bseq * tps32) * 32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = tb32 + acc_row(v, hf);
                    if (t < T) out[(static_cast<size_t>(bseq) * T + t) * O + o] = acc[v] + bo;
                }
            }
        }
    }
}

// Resident workgroups of `kernel` on the current device (compute units times
// workgroups per unit), cached per device in `cache`.
constexpr int kCapDevices = 64;
template <class K>
int capacity_of(int (&cache)[kCapDevices], K kernel, size_t lds)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kCapDevices && cache[dev] > 0) return cache[dev];
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    if (dev >= 0 && dev < kCapDevices) cache[dev] = cus * per_cu;
    return cus * per_cu;
}

template <int D>
int launch_gru_mfma(const float *Whh, const float *bhh, const float *p, const float *s0, const float *s_even,
                    const float *s_odd, const int *sel, const int *skip, const int *all_done, float *a, float *bvec,
                    unsigned *res_bits, int B, int T, Linearization lz, FrontOut fo, hipStream_t stream)
{
    using G = GruGeom<D>;
    static int caps[kCapDevices] = {};
    const int cap = capacity_of(caps, gru_eval_mfma_kernel<D>, 0);
    const int tps = (T + G::TP - 1) / G::TP;
    const long long ntiles = static_cast<long long>(B) * tps;
    const unsigned grid = static_cast<unsigned>(std::max<long long>(1, std::min<long long>(ntiles, cap)));
    DEER_LAUNCH((gru_eval_mfma_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, Whh, bhh, p, s0, s_even,
                       s_odd, sel, skip, all_done, a, bvec, res_bits, T, tps, ntiles, lz, fo);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

template <int KP, int NOB, bool TILED>
int launch_proj_mfma(const float *x, const float *U, const float *bias, float *p, int B, int T, int M,
                     hipStream_t stream)
{
    using G = ProjGeom<KP, NOB>;
    static int caps[kCapDevices] = {};
    const int cap = capacity_of(caps, projection_mfma_kernel<KP, NOB, TILED>, 0);
    const int tps32 = (T + 31) / 32;
    const long long nsub = static_cast<long long>(B) * tps32;
    const long long ntiles = (nsub + G::PS - 1) / G::PS;
    const unsigned grid = static_cast<unsigned>(std::max<long long>(1, std::min<long long>(ntiles, cap)));
    DEER_LAUNCH((projection_mfma_kernel<KP, NOB, TILED>), dim3(grid), dim3(kThreads), 0, stream, x, U, bias, p,
                       T, M, tps32, nsub);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

template <int D, bool FIRST>
int launch_gru_step(const float *Whh, const float *bhh, const float *pt, const float *s0, float *s_even, float *s_odd,
                    SolveControl *ctl, int *done, int *iters, int *status, float *resid, float tol, int max_iter,
                    unsigned *res_bits, unsigned *res_tile, int B, int T, bool zero_start, Linearization lz,
                    const StallCheck &sc, void *state, const float *x, const float *Wih, const float *bih,
                    float *pt_out, int *poll, hipStream_t stream)
{
    using G = GruGeom<D>;
    static int caps[kCapDevices] = {};
    const int cap = capacity_of(caps, gru_quasi_step_kernel<D, FIRST>, 0);
    const int tps = (T + G::TP - 1) / G::TP;
    const long long ntiles = static_cast<long long>(B) * tps;
    const unsigned grid = static_cast<unsigned>(std::max<long long>(1, std::min<long long>(ntiles, cap)));
    auto *hdr = static_cast<ScanHeader *>(state);
    auto *desc = reinterpret_cast<unsigned long long *>(static_cast<char *>(state) + sizeof(ScanHeader));
    DEER_LAUNCH((gru_quasi_step_kernel<D, FIRST>), dim3(grid), dim3(kThreads), 0, stream, Whh, bhh, pt, s0, s_even,
                s_odd, ctl, done, iters, status, resid, tol, max_iter, res_bits, res_tile, T, tps, B, ntiles,
                zero_start ? 1 : 0, lz, sc, hdr, desc, x, Wih, bih, pt_out, poll);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace

bool gru_mfma_supported(int D) { return D == 32 || D == 64; }

int launch_gru_eval_mfma(const float *Whh, const float *bhh, const float *p, const float *s0, const float *s_even,
                         const float *s_odd, const int *sel, const int *skip, const int *all_done, float *a,
                         float *bvec, unsigned *res_bits, int B, int T, int D, Linearization lz, FrontOut fo,
                         hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    if (D == 64)
        return launch_gru_mfma<64>(Whh, bhh, p, s0, s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, B, T, lz,
                                   fo, stream);
    if (D == 32)
        return launch_gru_mfma<32>(Whh, bhh, p, s0, s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, B, T, lz,
                                   fo, stream);
    return fail(DEER_ERR_UNSUPPORTED, "GRU matrix-core evaluation needs D = 32 or 64");
}

bool proj_mfma_supported(int M, int O) { return M >= 1 && M <= 64 && (O == 32 || O == 64 || O == 96 || O == 192); }

size_t proj_tiled_floats(int B, int T, int O) { return static_cast<size_t>(B) * ((T + 31) / 32) * 32 * O; }

int launch_projection_mfma(const float *x, const float *U, const float *bias, float *p, int B, int T, int M, int O,
                           bool tiled, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    const bool k32 = M <= 32;
#define DEER_PROJ(NOB)                                                                                         \
    if (tiled)                                                                                                 \
        return k32 ? launch_proj_mfma<32, NOB, true>(x, U, bias, p, B, T, M, stream)                          \
                   : launch_proj_mfma<64, NOB, true>(x, U, bias, p, B, T, M, stream);                         \
    return k32 ? launch_proj_mfma<32, NOB, false>(x, U, bias, p, B, T, M, stream)                             \
               : launch_proj_mfma<64, NOB, false>(x, U, bias, p, B, T, M, stream);
    switch (O) {
    case 32: DEER_PROJ(1)
    case 64: DEER_PROJ(2)
    case 96: DEER_PROJ(3)
    case 192: DEER_PROJ(6)
    default: return fail(DEER_ERR_UNSUPPORTED, "projection: output size not a supported multiple of 32");
    }
#undef DEER_PROJ
}

int gru_step_tile(int D) { return D == 64 ? GruGeom<64>::TP : GruGeom<32>::TP; }

size_t gru_step_state_bytes(int B, int T, int D)
{
    const int tps = (T + gru_step_tile(D) - 1) / gru_step_tile(D);
    return sizeof(ScanHeader) + align_up(static_cast<size_t>(B) * tps * 3 * D * sizeof(unsigned long long));
}

int launch_gru_quasi_step(const float *Whh, const float *bhh, float *pt, const float *s0, float *s_even,
                          float *s_odd, SolveControl *ctl, int *done, int *iters, int *status, float *resid,
                          float tol, int max_iter, unsigned *res_bits, unsigned *res_tile, int B, int T, int D,
                          bool zero_start, Linearization lz, const StallCheck &sc, void *state, const float *x,
                          const float *Wih, const float *bih, int M, int *poll, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    const bool first = x != nullptr;
    if (first && (!zero_start || s0 || M != D || !Wih))
        return fail(DEER_ERR_INVALID,
                    "fused GRU step: the projecting first iteration needs a zero start, no s0 and M = D");
#define DEER_GRU_STEP(DV)                                                                                         \
    if (D == DV)                                                                                                  \
        return first ? launch_gru_step<DV, true>(Whh, bhh, pt, s0, s_even, s_odd, ctl, done, iters, status, resid, \
                                                 tol, max_iter, res_bits, res_tile, B, T, zero_start, lz, sc,       \
                                                 state, x, Wih, bih, pt, poll, stream)                              \
                     : launch_gru_step<DV, false>(Whh, bhh, pt, s0, s_even, s_odd, ctl, done, iters, status,      \
                                                  resid, tol, max_iter, res_bits, res_tile, B, T, zero_start, lz,   \
                                                  sc, state, nullptr, nullptr, nullptr, nullptr, poll, stream);
    DEER_GRU_STEP(64)
    DEER_GRU_STEP(32)
#undef DEER_GRU_STEP
    return fail(DEER_ERR_UNSUPPORTED, "fused GRU step needs D = 32 or 64");
}

}  // namespace deer
