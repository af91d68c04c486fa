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

template <int D>
__device__ __forceinline__ void gru_fetch(const float *__restrict__ s, const float *__restrict__ s0,
                                          const float *__restrict__ pt, int T, int tps, int tps32, long long tile,
                                          int ps, int hf, int c, v4f (&hv)[GruTile<D>::NH], v4f (&pv)[3][4])
{
    using G = GruGeom<D>;
    const int tid = threadIdx.x;
    const int bseq = static_cast<int>(tile / tps);
    const int t0 = static_cast<int>(tile % tps) * G::TP;
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
            } else if (t < T) {
                v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(s + (seq + t) * D + q));
            }
        }
        hv[i] = v;
    }
    // tiled projection: 32-position block, gate g, quad q, half hf, channel c, 4 positions
    const size_t blk = static_cast<size_t>(bseq) * tps32 + (t0 >> 5) + ps;
    const v4f *base = reinterpret_cast<const v4f *>(pt + blk * (96 * static_cast<size_t>(D)));
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) pv[g][q] = __builtin_nontemporal_load(base + ((g * 4 + q) * 2 + hf) * D + c);
}

template <int D>
__global__ __launch_bounds__(kThreads) void gru_eval_mfma_kernel(
    const float *__restrict__ Whh, const float *__restrict__ bhh, const float *__restrict__ pt,
    const float *__restrict__ s0, const float *s_even, const float *s_odd, const int *__restrict__ sel,
    const int *__restrict__ skip, const int *__restrict__ all_done, float *__restrict__ aout,
    float *__restrict__ bout, unsigned *__restrict__ res_bits, int T, int tiles_per_seq, long long ntiles)
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

    const long long tb = ntiles * blockIdx.x / gridDim.x, te = ntiles * (blockIdx.x + 1) / gridDim.x;
    if (tb >= te) return;
    unsigned rmax = 0u;
    int cur = -1;
    v4f hv[GruTile<D>::NH];
    v4f pv[3][4];
    gru_fetch<D>(s, s0, pt, T, tiles_per_seq, tps32, tb, ps, hf, c, hv, pv);
    for (long long tile = tb; tile < te; ++tile) {
        const int bseq = static_cast<int>(tile / tiles_per_seq);
        const int t0 = static_cast<int>(tile % tiles_per_seq) * G::TP;
        if (bseq != cur) {
            if (cur >= 0) wave_max_atomic(rmax, res_bits + cur);
            rmax = 0u;
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
        if (tile + 1 < te) gru_fetch<D>(s, s0, pt, T, tiles_per_seq, tps32, tile + 1, ps, hf, c, hv, pv);
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

        const size_t seq = static_cast<size_t>(bseq) * T;
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
            const float a = zg + (h - ng) * zg * (1.0f - zg) * wz +
                            (1.0f - zg) * (1.0f - ng * ng) * (rg * wn + rg * (1.0f - rg) * wr * qn);
            const size_t o = (seq + t) * D + c;
            __builtin_nontemporal_store(a, aout + o);
            __builtin_nontemporal_store(f - a * h, bout + o);
            rmax = max(rmax, __float_as_uint(fabsf(st - f)));
        }
    }
    if (cur >= 0) wave_max_atomic(rmax, res_bits + cur);
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
    // sub-tiles of 32 positions never straddle sequences: u -> (sequence, block)
    const long long ntiles = (nsub + G::PS - 1) / G::PS;
    const long long tb = ntiles * blockIdx.x / gridDim.x, te = ntiles * (blockIdx.x + 1) / gridDim.x;
    for (long long tile = tb; tile < te; ++tile) {
        __syncthreads();
        for (int e = tid; e < G::TP * KP; e += kThreads) {
            const int r = e / KP, k = e % KP;
            const long long u = tile * G::PS + r / 32;
            float v = 0.0f;
            if (u < nsub && k < M) {
                const long long bseq = u / tps32;
                const int t = static_cast<int>(u % tps32) * 32 + (r % 32);
                if (t < T) v = x[(static_cast<size_t>(bseq) * T + t) * M + k];
            }
            Xs[r * G::LDX + k] = v;
        }
        __syncthreads();
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
            const float bo = bias ? bias[o] : 0.0f;
            const long long bseq = u / tps32;
            const int tb32 = static_cast<int>(u % tps32) * 32;
            if constexpr (TILED) {
                const int g = o / DG, cch = o % DG;
                v4f *dst = reinterpret_cast<v4f *>(out + static_cast<size_t>(u) * (32 * O));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4f w;
                    w[0] = acc[4 * q] + bo; w[1] = acc[4 * q + 1] + bo; w[2] = acc[4 * q + 2] + bo; w[3] = acc[4 * q + 3] + bo;
                    dst[((g * 4 + q) * 2 + hf) * DG + cch] = w;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = tb32 + acc_row(v, hf);
                    if (t < T) out[(static_cast<size_t>(bseq) * T + t) * O + o] = acc[v] + bo;
                }
            }
        }
    }
}

template <class K>
int capacity_of(K kernel, size_t lds)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

template <int D>
int launch_gru_mfma(const float *Whh, const float *bhh, const float *p, const float *s0, const float *s_even,
                    const float *s_odd, const int *sel, const int *skip, const int *all_done, float *a, float *bvec,
                    unsigned *res_bits, int B, int T, hipStream_t stream)
{
    using G = GruGeom<D>;
    static int cap = 0;
    if (cap == 0) cap = capacity_of(gru_eval_mfma_kernel<D>, 0);
    const int tps = (T + G::TP - 1) / G::TP;
    const long long ntiles = static_cast<long long>(B) * tps;
    const unsigned grid = static_cast<unsigned>(std::max<long long>(1, std::min<long long>(ntiles, cap)));
    hipLaunchKernelGGL((gru_eval_mfma_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, Whh, bhh, p, s0, s_even,
                       s_odd, sel, skip, all_done, a, bvec, res_bits, T, tps, ntiles);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

template <int KP, int NOB, bool TILED>
int launch_proj_mfma(const float *x, const float *U, const float *bias, float *p, int B, int T, int M,
                     hipStream_t stream)
{
    using G = ProjGeom<KP, NOB>;
    static int cap = 0;
    if (cap == 0) cap = capacity_of(projection_mfma_kernel<KP, NOB, TILED>, 0);
    const int tps32 = (T + 31) / 32;
    const long long nsub = static_cast<long long>(B) * tps32;
    const long long ntiles = (nsub + G::PS - 1) / G::PS;
    const unsigned grid = static_cast<unsigned>(std::max<long long>(1, std::min<long long>(ntiles, cap)));
    hipLaunchKernelGGL((projection_mfma_kernel<KP, NOB, TILED>), dim3(grid), dim3(kThreads), 0, stream, x, U, bias, p,
                       T, M, tps32, nsub);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace

bool gru_mfma_supported(int D) { return D == 32 || D == 64; }

int launch_gru_eval_mfma(const float *Whh, const float *bhh, const float *p, const float *s0, const float *s_even,
                         const float *s_odd, const int *sel, const int *skip, const int *all_done, float *a,
                         float *bvec, unsigned *res_bits, int B, int T, int D, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    if (D == 64)
        return launch_gru_mfma<64>(Whh, bhh, p, s0, s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, B, T, stream);
    if (D == 32)
        return launch_gru_mfma<32>(Whh, bhh, p, s0, s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, B, T, stream);
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

}  // namespace deer
