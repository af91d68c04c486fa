// Cell kernels: the iteration-invariant input projection, the per-iteration
// evaluation of f and its Jacobian at every (sequence, step) of the current
// trajectory guess, and the plain sequential rollout.
//
// Evaluation at the guess s^(i) ("Parallel Broyden Methods", section 2;
// residual as restated in the "Predictability" rebuttal, its equation 2):
//   f_t = f(s_{t-1}, x_t)   (s_{-1} = s0)
//   r_t = s_t - f_t         -> per-sequence max |r_t| (atomic max on the float bits)
//   A_t = J_t or diag(J_t),  b_t = f_t - A_t s_{t-1}
// so that s^(i+1) solves s_t = A_t s_{t-1} + b_t.
//
// Layout: a workgroup owns TP consecutive steps of one sequence.  The TP+1
// state rows it needs (s_{t0-1} .. s_{t0+TP-1}) and the transposed recurrent
// weights sit in LDS; lane c of a lane group handles channel c, so every global
// access is a contiguous row segment.
#include <algorithm>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
constexpr int kTP = 64;   // steps per workgroup in the evaluation kernels
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoidf_(float u) { return 1.0f / (1.0f + expf(-u)); }

// max over the workgroup of unsigned bit patterns (non-negative floats order as
// integers; NaN patterns sit above +Inf), then one atomic per workgroup
__device__ __forceinline__ void block_max_to(unsigned v, unsigned *dst)
{
    __shared__ unsigned red[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), o, 64)));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned m = red[0];
        for (int w = 1; w < kThreads / 64; ++w) m = max(m, red[w]);
        atomicMax(dst, m);
    }
}

// minimum over the workgroup of violating positions, one atomic per workgroup
__device__ __forceinline__ void block_min_to(unsigned v, unsigned *dst)
{
    __shared__ unsigned red[kThreads / 64];
    v = wave_min_u32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned m = red[0];
        for (int w = 1; w < kThreads / 64; ++w) m = min(m, red[w]);
        if (m != kNoFront) atomicMin(dst, m);
    }
}

// ------------------------------------------------------------- projection
// Narrow projections (O <= 64 outputs, M <= 64 inputs): out[n][o] =
// sum_j U[o][j] x[n][j] + bias[o].  Thread (o, rp) keeps row o of U (padded
// with zeros to MP) in registers and computes output o of rows rp, rp + RPP,
// ... of each 64-row tile, reading the rows of x from LDS as 16-byte
// broadcasts.  A tile's rows are contiguous in x and in out, so both stream
// coalesced.  The grid is a few workgroups per CU striding over the tiles
// (thousands of short workgroups were bound by their dispatch), each fetching
// its next tile into registers while it computes the current one.  The sum
// runs in column order, one FMA per column.
template <int OP, int MP>
__global__ __launch_bounds__(kThreads) void projection_rows_kernel(const float *__restrict__ x,
                                                                   const float *__restrict__ U,
                                                                   const float *__restrict__ bias,
                                                                   float *__restrict__ out, long long N, int M, int O)
{
    constexpr int TR = 64;                   // rows per tile
    constexpr int RPP = kThreads / OP;       // rows per pass
    constexpr int LX = MP + 4;               // LDS row stride (16-byte aligned rows)
    constexpr int NX = TR * MP / kThreads;   // x words per thread per tile
    __shared__ __align__(16) float xs[TR * LX];
    const int tid = threadIdx.x;
    const int o = tid % OP, rp = tid / OP;
    const long long tiles = (N + TR - 1) / TR;
    float u[MP];
    const bool ov = o < O;
#pragma unroll
    for (int k = 0; k < MP; ++k) u[k] = (ov && k < M) ? U[static_cast<size_t>(o) * M + k] : 0.0f;
    const float bo = (bias && ov) ? bias[o] : 0.0f;
    // x words of tile t owned by this thread: e = tid + j kThreads -> row e / MP, column e % MP
    float xv[NX];
    auto fetch = [&](long long t) {
        const long long n0 = t * TR;
#pragma unroll
        for (int j = 0; j < NX; ++j) {
            const int e = tid + j * kThreads, r = e / MP, k = e % MP;
            const long long n = n0 + r;
            const bool ok = t < tiles && n < N && k < M;
            const long long idx = ok ? n * M + k : 0;     // clamped: the load stays unconditional
            const float v = x[idx];
            xv[j] = ok ? v : 0.0f;
        }
    };
    long long t = blockIdx.x;
    fetch(t);
    for (; t < tiles; t += gridDim.x) {
        __syncthreads();                     // the previous tile is done with xs
#pragma unroll
        for (int j = 0; j < NX; ++j) {
            const int e = tid + j * kThreads;
            xs[(e / MP) * LX + e % MP] = xv[j];
        }
        __syncthreads();
        fetch(t + gridDim.x);
        const long long n0 = t * TR;
        const int nr = static_cast<int>(min(static_cast<long long>(TR), N - n0));
#pragma unroll
        for (int jr = 0; jr < TR / RPP; ++jr) {
            const int r = rp + jr * RPP;
            const v4f *xr = reinterpret_cast<const v4f *>(xs + r * LX);
            float acc = 0.0f;
#pragma unroll
            for (int k4 = 0; k4 < MP / 4; ++k4) {
                const v4f q = xr[k4];
                acc = __builtin_fmaf(u[4 * k4], q[0], acc);
                acc = __builtin_fmaf(u[4 * k4 + 1], q[1], acc);
                acc = __builtin_fmaf(u[4 * k4 + 2], q[2], acc);
                acc = __builtin_fmaf(u[4 * k4 + 3], q[3], acc);
            }
            if (ov && r < nr) out[(n0 + r) * O + o] = acc + bo;
        }
    }
}

// out[n][o] = sum_j U[o][j] x[n][j] + bias[o], for OG groups of 64 outputs.
template <int OG>
__global__ __launch_bounds__(kThreads) void projection_kernel(const float *__restrict__ x, const float *__restrict__ U,
                                                              const float *__restrict__ bias, float *__restrict__ out,
                                                              int N, int M, int O, int row_tiles)
{
    constexpr int RT = 32;                   // rows per tile
    __shared__ float Ut[64][64 * OG];        // Ut[k][o] = U[o][k0 + k]
    __shared__ float xs[RT][65];
    const int ol = threadIdx.x & 63, pg = threadIdx.x >> 6;
    const int nkt = (M + 63) / 64;
    float bo[OG];
#pragma unroll
    for (int g = 0; g < OG; ++g) {
        const int o = ol + 64 * g;
        bo[g] = (bias && o < O) ? bias[o] : 0.0f;
    }
    auto load_U = [&](int k0) {
        for (int e = threadIdx.x; e < 64 * 64 * OG; e += kThreads) {
            const int o = e / 64, k = e % 64;
            Ut[k][o] = (o < O && k0 + k < M) ? U[static_cast<size_t>(o) * M + k0 + k] : 0.0f;
        }
    };
    if (nkt == 1) load_U(0);
    for (int rt = 0; rt < row_tiles; ++rt) {
        const long long n0 = (static_cast<long long>(blockIdx.x) * row_tiles + rt) * RT;
        if (n0 >= N) break;
        float acc[RT / 4][OG];
#pragma unroll
        for (int r = 0; r < RT / 4; ++r)
#pragma unroll
            for (int g = 0; g < OG; ++g) acc[r][g] = 0.0f;
        for (int kt = 0; kt < nkt; ++kt) {
            const int k0 = kt * 64;
            __syncthreads();
            if (nkt > 1) load_U(k0);
            for (int e = threadIdx.x; e < RT * 64; e += kThreads) {
                const int r = e / 64, k = e % 64;
                const long long n = n0 + r;
                xs[r][k] = (n < N && k0 + k < M) ? x[static_cast<size_t>(n) * M + k0 + k] : 0.0f;
            }
            __syncthreads();
#pragma unroll 8
            for (int k = 0; k < 64; ++k) {
                float u[OG];
#pragma unroll
                for (int g = 0; g < OG; ++g) u[g] = Ut[k][ol + 64 * g];
#pragma unroll
                for (int r = 0; r < RT / 4; ++r) {
                    const float xv = xs[pg + 4 * r][k];
#pragma unroll
                    for (int g = 0; g < OG; ++g) acc[r][g] += u[g] * xv;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RT / 4; ++r) {
            const long long n = n0 + pg + 4 * r;
            if (n >= N) continue;
#pragma unroll
            for (int g = 0; g < OG; ++g) {
                const int o = ol + 64 * g;
                if (o < O) out[static_cast<size_t>(n) * O + o] = acc[r][g] + bo[g];
            }
        }
    }
}

// ------------------------------------------------------------- tanh cell
// f = tanh(W s + p); dense: lin = d = shrink (1 - f^2), b = f - d * (W s)  (A_t = diag(d) W)
//                    other: lin = a = lin_diag((1 - f^2) W_cc), b = f - a * s_c
//
// One workgroup per tile of kTP positions.  Every global load of the tile is
// issued up front at a clamped, in-bounds address (words outside the problem
// are selected away afterwards), so a workgroup waits for memory once.  Thread
// (c, ps) keeps row c of W in registers and reads the state rows as 16-byte
// LDS broadcasts; W s is accumulated with one FMA per column in column order.
template <int DP>
__global__ __launch_bounds__(kThreads) void tanh_eval_kernel(
    const float *__restrict__ W, const float *__restrict__ p, const float *__restrict__ s0,
    const float *s_even, const float *s_odd, const int *__restrict__ sel, const int *__restrict__ skip,
    const int *__restrict__ all_done, float *__restrict__ lin, float *__restrict__ bout, unsigned *__restrict__ res_bits,
    int T, int D, int tiles, int dense, Linearization lz, FrontOut fo)
{
    if (all_done && *all_done) return;
    const int bseq = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (skip && skip[bseq]) return;
    constexpr int PPP = kThreads / DP;                            // positions per pass
    constexpr int NP = kTP / PPP;                                 // positions per thread
    constexpr int NS = ((kTP + 1) * DP + kThreads - 1) / kThreads;   // state words per thread
    constexpr int NW = (DP * DP + kThreads - 1) / kThreads;         // W words per thread
    constexpr int LW = DP + 4;                                    // W row stride (conflict-free 16-byte reads)
    constexpr int WR = (NW * kThreads / DP > DP) ? NW * kThreads / DP : DP;   // W rows incl. padding
    // Both arrays are padded to whole passes of the workgroup, so the staging
    // stores need no guard (a guarded store lets the compiler sink its load).
    __shared__ __align__(16) float Wl[WR * LW];                   // Wl[c][k] = W[c][k], zero past D
    __shared__ __align__(16) float srow[NS * kThreads];           // srow[r][k] = s_{t0 - 1 + r}[k], rows 0..kTP
    const float *s = (sel && (*sel & 1)) ? s_odd : s_even;
    float *fdst = (sel && (*sel & 1)) ? bout : lin;   // kLinValue output
    const int t0 = tile * kTP;
    const size_t seq = static_cast<size_t>(bseq) * T;
    const int tid = threadIdx.x;
    const int c = tid % DP, ps = tid / DP;
    const bool cv = c < D;
    const int cl = min(c, D - 1);

    // issue order: s_0 row, state rows, W, then the projection (needed only after the barrier)
    const float s0v = (s0 && tid < D) ? s0[static_cast<size_t>(bseq) * D + tid] : 0.0f;
    float sv[NS], wv[NW], pv[NP];
    if (s) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = tid + i * kThreads, r = e / DP, k = e % DP;
            const int t = min(max(t0 - 1 + r, 0), T - 1);
            sv[i] = s[(seq + t) * D + min(k, D - 1)];
        }
    } else {                                                      // the all-zero start, never stored
#pragma unroll
        for (int i = 0; i < NS; ++i) sv[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = min(tid + i * kThreads, DP * DP - 1), r = e / DP, k = e % DP;
        wv[i] = W[min(r, D - 1) * D + min(k, D - 1)];
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int t = min(t0 + ps + j * PPP, T - 1);
        pv[j] = p[(seq + t) * D + cl];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int e = tid + i * kThreads, r = e / DP, k = e % DP;
        const int t = t0 - 1 + r;
        srow[e] = (k < D && t >= 0 && t < T) ? sv[i] : 0.0f;
    }
    if (t0 == 0 && tid < DP) srow[tid] = tid < D ? s0v : 0.0f;   // s_0 enters the first tile
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int e = tid + i * kThreads, r = e / DP, k = e % DP;
        Wl[r * LW + k] = (r < D && k < D) ? wv[i] : 0.0f;
    }
    __syncthreads();

    float wr[DP];
#pragma unroll
    for (int k4 = 0; k4 < DP / 4; ++k4) {
        const v4f w4 = *reinterpret_cast<const v4f *>(&Wl[c * LW + 4 * k4]);
        wr[4 * k4] = w4[0]; wr[4 * k4 + 1] = w4[1]; wr[4 * k4 + 2] = w4[2]; wr[4 * k4 + 3] = w4[3];
    }
    const float wcc = Wl[c * LW + c];
    unsigned rmax = 0u, fmin = kNoFront;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int r = ps + j * PPP;
        const int t = t0 + r;
        if (!cv || t >= T) continue;
        const v4f *sr = reinterpret_cast<const v4f *>(&srow[r * DP]);
        float ws = 0.0f;
#pragma unroll
        for (int k4 = 0; k4 < DP / 4; ++k4) {
            const v4f x = sr[k4];
            ws = __builtin_fmaf(wr[4 * k4], x[0], ws);
            ws = __builtin_fmaf(wr[4 * k4 + 1], x[1], ws);
            ws = __builtin_fmaf(wr[4 * k4 + 2], x[2], ws);
            ws = __builtin_fmaf(wr[4 * k4 + 3], x[3], ws);
        }
        const size_t o = (seq + t) * D + c;
        const float h = ws + pv[j];
        const float f = tanhf(h);
        const float d = 1.0f - f * f;
        if (lz.kind == kLinValue) {
            fdst[o] = f;
        } else if (dense) {
            const float dd = lz.shrink * d;
            lin[o] = dd;
            bout[o] = f - dd * ws;
        } else {
            const float a = lin_diag(lz, d * wcc);
            lin[o] = a;
            bout[o] = f - a * srow[r * DP + c];
        }
        const float ra = fabsf(srow[(r + 1) * DP + c] - f);
        rmax = max(rmax, __float_as_uint(ra));
        fmin = min(fmin, front_of(ra, fo.tol, t));
    }
    block_max_to(rmax, res_bits + bseq);
    if (fo.front) block_min_to(fmin, fo.front + bseq);
}

// -------------------------------------------------------------- GRU cell
// Gate order (r, z, n); p = W_ih x + b_ih precomputed, q = W_hh h + b_hh here.
//   a = d f / d h (diagonal) = z + (h - n) z (1 - z) Wz_cc
//                            + (1 - z)(1 - n^2)(r Wn_cc + r (1 - r) Wr_cc q_n)
//   b = f - a h
template <int DP>
__global__ __launch_bounds__(kThreads) void gru_eval_kernel(
    const float *__restrict__ Whh, const float *__restrict__ bhh, const float *__restrict__ p,
    const float *__restrict__ s0, const float *s_even, const float *s_odd, const int *__restrict__ sel,
    const int *__restrict__ skip, const int *__restrict__ all_done, float *__restrict__ aout,
    float *__restrict__ bout, unsigned *__restrict__ res_bits, int T, int D, int tiles, Linearization lz, FrontOut fo)
{
    if (all_done && *all_done) return;
    const int bseq = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (skip && skip[bseq]) return;
    constexpr int PPP = kThreads / DP;
    __shared__ float Wt[DP][3 * DP];     // Wt[k][g*DP + c] = W_hh[g*D + c][k]
    __shared__ float srow[kTP + 1][DP];
    const float *s = (sel && (*sel & 1)) ? s_odd : s_even;
    float *fdst = (sel && (*sel & 1)) ? bout : aout;  // kLinValue output
    const int t0 = tile * kTP;
    const size_t seq = static_cast<size_t>(bseq) * T;
    for (int e = threadIdx.x; e < 3 * DP * DP; e += kThreads) {
        const int row = e / DP, k = e % DP;     // row = g*DP + c
        const int g = row / DP, c = row % DP;
        Wt[k][row] = (k < D && c < D) ? Whh[static_cast<size_t>(g * D + c) * D + k] : 0.0f;
    }
    for (int e = threadIdx.x; e < (kTP + 1) * DP; e += kThreads) {
        const int r = e / DP, c = e % DP;
        const int t = t0 - 1 + r;
        float v = 0.0f;
        if (c < D && t < T) {
            if (t < 0) v = s0 ? s0[static_cast<size_t>(bseq) * D + c] : 0.0f;
            else v = s[(seq + t) * D + c];
        }
        srow[r][c] = v;
    }
    __syncthreads();
    const int c = threadIdx.x % DP, ps = threadIdx.x / DP;
    const bool cv = c < D;
    const float wr = cv ? Wt[c][c] : 0.0f, wz = cv ? Wt[c][DP + c] : 0.0f, wn = cv ? Wt[c][2 * DP + c] : 0.0f;
    const float br = (cv && bhh) ? bhh[c] : 0.0f;
    const float bz = (cv && bhh) ? bhh[D + c] : 0.0f;
    const float bn = (cv && bhh) ? bhh[2 * D + c] : 0.0f;
    unsigned rmax = 0u, fmin = kNoFront;
    for (int r = ps; r < kTP; r += PPP) {
        const int t = t0 + r;
        if (t >= T) break;
        float qr = br, qz = bz, qn = bn;
#pragma unroll 8
        for (int k = 0; k < DP; ++k) {
            const float hk = srow[r][k];
            qr += Wt[k][c] * hk;
            qz += Wt[k][DP + c] * hk;
            qn += Wt[k][2 * DP + c] * hk;
        }
        if (!cv) continue;
        const size_t pb = (seq + t) * (3 * static_cast<size_t>(D));
        const float rg = sigmoidf_(p[pb + c] + qr);
        const float zg = sigmoidf_(p[pb + D + c] + qz);
        const float ng = tanhf(p[pb + 2 * D + c] + rg * qn);
        const float h = srow[r][c];
        const float f = (1.0f - zg) * ng + zg * h;
        const float a = lin_diag(lz, zg + (h - ng) * zg * (1.0f - zg) * wz +
                                         (1.0f - zg) * (1.0f - ng * ng) * (rg * wn + rg * (1.0f - rg) * wr * qn));
        const size_t o = (seq + t) * D + c;
        if (lz.kind == kLinValue) {
            fdst[o] = f;
        } else {
            aout[o] = a;
            bout[o] = f - a * h;
        }
        const float ra = fabsf(srow[r + 1][c] - f);
        rmax = max(rmax, __float_as_uint(ra));
        fmin = min(fmin, front_of(ra, fo.tol, t));
    }
    block_max_to(rmax, res_bits + bseq);
    if (fo.front) block_min_to(fmin, fo.front + bseq);
}

int pick_dp(int D) { return D <= 4 ? 4 : D <= 8 ? 8 : D <= 16 ? 16 : D <= 32 ? 32 : 64; }

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus()
{
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

unsigned eval_blocks(int B, int T, int &tiles)
{
    tiles = (T + kTP - 1) / kTP;
    return static_cast<unsigned>(static_cast<long long>(B) * tiles);
}

}  // namespace

// The matrix-core evaluation kernels read the tiled projection in whole tiles
// of up to 128 positions (4 blocks of 32 positions x O outputs): the last
// sequence's last tile may reach 3 blocks past its data, so 3 blocks of slack
// follow the array (read, never used).
size_t projection_floats(int B, int T, int O)
{
    return std::max(static_cast<size_t>(B) * T * O, proj_tiled_floats(B, T, O)) + 3 * 32 * static_cast<size_t>(O);
}

bool gru_fast_path(int D, int M) { return gru_mfma_supported(D) && proj_mfma_supported(M, 3 * D); }

int launch_projection(const float *x, const float *U, const float *bias, float *p, int B, int T, int M, int O,
                      bool tiled, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    if (tiled || proj_mfma_supported(M, O)) return launch_projection_mfma(x, U, bias, p, B, T, M, O, tiled, stream);
    if (O > 192) return fail(DEER_ERR_UNSUPPORTED, "projection: more than 192 outputs");
    if (O <= 64 && M <= 64) {
        const long long NN = static_cast<long long>(B) * T;
        const unsigned tiles = static_cast<unsigned>(std::min<long long>((NN + 63) / 64, 4ll * device_cus()));
        const int op = pick_dp(O), mp = M <= 16 ? 16 : M <= 32 ? 32 : 64;
#define DEER_PROJ_ROWS(OPV, MPV)                                                                               \
    if (op == OPV && mp == MPV) {                                                                              \
        DEER_LAUNCH((projection_rows_kernel<OPV, MPV>), dim3(tiles), dim3(kThreads), 0, stream, x, U, bias, p, \
                    NN, M, O);                                                                                 \
        DEER_HIP(hipGetLastError());                                                                           \
        return DEER_OK;                                                                                        \
    }
#define DEER_PROJ_ROWS_M(OPV) DEER_PROJ_ROWS(OPV, 16) DEER_PROJ_ROWS(OPV, 32) DEER_PROJ_ROWS(OPV, 64)
        DEER_PROJ_ROWS_M(4)
        DEER_PROJ_ROWS_M(8)
        DEER_PROJ_ROWS_M(16)
        DEER_PROJ_ROWS_M(32)
        DEER_PROJ_ROWS_M(64)
#undef DEER_PROJ_ROWS_M
#undef DEER_PROJ_ROWS
    }
    const int N = B * T;
    const int row_tiles = 4;
    const long long rows_per_block = 32ll * row_tiles;
    const unsigned blocks = static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block);
    const int og = (O + 63) / 64;
    if (og == 1)
        DEER_LAUNCH((projection_kernel<1>), dim3(blocks), dim3(kThreads), 0, stream, x, U, bias, p, N, M, O, row_tiles);
    else if (og == 2)
        DEER_LAUNCH((projection_kernel<2>), dim3(blocks), dim3(kThreads), 0, stream, x, U, bias, p, N, M, O, row_tiles);
    else
        DEER_LAUNCH((projection_kernel<3>), dim3(blocks), dim3(kThreads), 0, stream, x, U, bias, p, N, M, O, row_tiles);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

#define DEER_TANH_CASE(DPV)                                                                                     \
    case DPV:                                                                                                   \
        DEER_LAUNCH((tanh_eval_kernel<DPV>), dim3(blocks), dim3(kThreads), 0, stream, W, p, s0, s_even,  \
                           s_odd, sel, skip, all_done, lin, bvec, res_bits, T, D, tiles, dense, lz, fo);        \
        break;

int launch_tanh_eval(const float *W, const float *p, const float *s0, const float *s_even, const float *s_odd,
                     const int *sel, const int *skip, const int *all_done, float *lin, float *bvec, unsigned *res_bits,
                     int B, int T, int D, int dense, Linearization lz, FrontOut fo, hipStream_t stream)
{
    int tiles;
    const unsigned blocks = eval_blocks(B, T, tiles);
    if (blocks == 0) return DEER_OK;
    switch (pick_dp(D)) {
        DEER_TANH_CASE(4)
        DEER_TANH_CASE(8)
        DEER_TANH_CASE(16)
        DEER_TANH_CASE(32)
        DEER_TANH_CASE(64)
    }
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

#define DEER_GRU_CASE(DPV)                                                                                      \
    case DPV:                                                                                                   \
        DEER_LAUNCH((gru_eval_kernel<DPV>), dim3(blocks), dim3(kThreads), 0, stream, Whh, bhh, p, s0,    \
                           s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, T, D, tiles, lz, fo);         \
        break;

int launch_gru_eval(const float *Whh, const float *bhh, const float *p, const float *s0, const float *s_even,
                    const float *s_odd, const int *sel, const int *skip, const int *all_done, float *a, float *bvec,
                    unsigned *res_bits, int B, int T, int D, int M, Linearization lz, FrontOut fo, hipStream_t stream)
{
    if (gru_fast_path(D, M))
        return launch_gru_eval_mfma(Whh, bhh, p, s0, s_even, s_odd, sel, skip, all_done, a, bvec, res_bits, B, T, D,
                                    lz, fo, stream);
    int tiles;
    const unsigned blocks = eval_blocks(B, T, tiles);
    if (blocks == 0) return DEER_OK;
    switch (pick_dp(D)) {
        DEER_GRU_CASE(4)
        DEER_GRU_CASE(8)
        DEER_GRU_CASE(16)
        DEER_GRU_CASE(32)
        DEER_GRU_CASE(64)
    }
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace deer
