// Largest Lyapunov exponent along a given trajectory, on the GPU.
//
// The "Predictability Enables Parallelization" page estimates the LLE by
// pushing a unit vector through the Jacobians J_t = d f / d s at
// (s_{t-1}, x_t), renormalising after every step and averaging the log growth
// (rebuttal "LLE computation cost", its appendix's Algorithm 1); a negative LLE
// predicts that parallel Newton converges in few iterations.
//
// Two launches: the per-step Jacobian factors are evaluated in parallel over
// all positions (the trajectory is given), then one workgroup per sequence runs
// the inherently sequential vector chain, which then costs a few matrix-vector
// products per step, split over 2-4 lanes per state channel:
//   tanh:  J_t v = d_t * (W v),                d_t = 1 - f_t^2
//   GRU:   J_t v = z * v + al * (Wz v) + be * (Wn v) + ga * (Wr v)
//          al = (s - n) z (1 - z),  be = (1 - z)(1 - n^2) r,
//          ga = (1 - z)(1 - n^2) r (1 - r) (W_hn s + b_hn)
// (the GRU Jacobian in closed form, gate order r, z, n).
#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kTP = 64;   // positions per workgroup in the factor kernel

__device__ __forceinline__ float sigm(float u) { return 1.0f / (1.0f + expf(-u)); }

// GRU factors [B,T,4,D] = (z, al, be, ga) at s_{t-1} = traj[t-1] (s0 at t = 0).
template <int DP>
__global__ __launch_bounds__(kThreads) void gru_lle_factor_kernel(
    const float *__restrict__ Whh, const float *__restrict__ bhh, const float *__restrict__ p,
    const float *__restrict__ s0, const float *__restrict__ traj, float *__restrict__ F, int T, int D, int tiles)
{
    constexpr int PPP = kThreads / DP;
    __shared__ float Wt[DP][3 * DP];     // Wt[k][g*DP + c] = W_hh[g*D + c][k]
    __shared__ float srow[kTP][DP];      // srow[r] = s_{t0 + r - 1}
    const int bseq = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int t0 = tile * kTP;
    const size_t seq = static_cast<size_t>(bseq) * T;
    for (int e = threadIdx.x; e < 3 * DP * DP; e += kThreads) {
        const int row = e / DP, k = e % DP, g = row / DP, c = row % DP;
        Wt[k][row] = (k < D && c < D) ? Whh[static_cast<size_t>(g * D + c) * D + k] : 0.0f;
    }
    for (int e = threadIdx.x; e < kTP * DP; e += kThreads) {
        const int r = e / DP, c = e % DP;
        const int t = t0 + r - 1;
        float v = 0.0f;
        if (c < D && t < T) {
            if (t < 0) v = s0 ? s0[static_cast<size_t>(bseq) * D + c] : 0.0f;
            else v = traj[(seq + t) * D + c];
        }
        srow[r][c] = v;
    }
    __syncthreads();
    const int c = threadIdx.x % DP, ps = threadIdx.x / DP;
    if (c >= D) return;
    const float br = bhh ? bhh[c] : 0.0f, bz = bhh ? bhh[D + c] : 0.0f, bn = bhh ? bhh[2 * D + c] : 0.0f;
    for (int r = ps; r < kTP; r += PPP) {
        const int t = t0 + r;
        if (t >= T) break;
        float qr = br, qz = bz, qn = bn;
        for (int k = 0; k < DP; ++k) {
            const float hk = srow[r][k];
            qr += Wt[k][c] * hk;
            qz += Wt[k][DP + c] * hk;
            qn += Wt[k][2 * DP + c] * hk;
        }
        const size_t pb = (seq + t) * (3 * static_cast<size_t>(D));
        const float rg = sigm(p[pb + c] + qr);
        const float zg = sigm(p[pb + D + c] + qz);
        const float ng = tanhf(p[pb + 2 * D + c] + rg * qn);
        const float h = srow[r][c];
        const float tail = (1.0f - zg) * (1.0f - ng * ng);
        float *fo = F + (seq + t) * (4 * static_cast<size_t>(D));
        fo[c] = zg;
        fo[D + c] = (h - ng) * zg * (1.0f - zg);
        fo[2 * D + c] = tail * rg;
        fo[3 * D + c] = tail * rg * (1.0f - rg) * qn;
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}

// Sum over the 64 lanes of a wavefront, the same bits in every lane: butterflies
// inside quads and rows (each pair adds the same two values, so all lanes of a
// row agree), then the four row sums in a fixed order.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);          // quad_perm [1, 0, 3, 2]
    v += dpp<0x4E>(v);          // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);         // row_half_mirror
    v += dpp<0x140>(v);         // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Chain geometry: KQ lanes share one channel's dot products (each takes DP / KQ
// of the columns); a wavefront covers 64 / KQ channels and NW wavefronts the
// padded state.
template <int DP> struct ChainGeom;
template <> struct ChainGeom<4>  { static constexpr int KQ = 4; };
template <> struct ChainGeom<8>  { static constexpr int KQ = 4; };
template <> struct ChainGeom<16> { static constexpr int KQ = 4; };
template <> struct ChainGeom<32> { static constexpr int KQ = 2; };
template <> struct ChainGeom<64> { static constexpr int KQ = 4; };

template <int DP>
struct Chain {
    static constexpr int KQ = ChainGeom<DP>::KQ;
    static constexpr int CW = 64 / KQ;                    // channels per wavefront
    static constexpr int NW = DP > CW ? DP / CW : 1;      // wavefronts per sequence
    static constexpr int KS = DP / KQ;                    // columns per lane
};

// One workgroup per sequence runs the chain w_t = J_t v_{t-1}, v_t = w_t / |w_t|,
// lle = mean_t log |w_t|.  NF = 1 (tanh: factor d) or 4 (GRU: z, al, be, ga).
// Lane (channel c, quarter kq) keeps its rows of W for its columns in
// registers; the unnormalised w of the previous step sits in LDS (two buffers
// by step parity) and the 1 / |w| scaling is applied to the dot products.  The
// norm is a deterministic wave sum (plus an LDS exchange between wavefronts
// when NW > 1); one barrier per step orders the exchange of w.  Factors are fetched PF steps ahead with
// clamped loads.
template <int DP, int NF>
__global__ __launch_bounds__(64 * Chain<DP>::NW) void lle_chain_kernel(const float *__restrict__ W,
                                                                       const float *__restrict__ F,
                                                                       const float *__restrict__ v0, int T, int D,
                                                                       double *__restrict__ out)
{
    using C = Chain<DP>;
    constexpr int NG = NF == 1 ? 1 : 3;
    constexpr int PF = 8;
    constexpr int KQ = C::KQ, KS = C::KS, NW = C::NW;
    __shared__ __align__(16) float wbuf[2][DP];
    __shared__ float part[2][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, bseq = blockIdx.x;
    const int c = wave * C::CW + lane / KQ, kq = lane % KQ;
    const bool cv = c < D;
    const int cr = cv ? c : 0;
    float wr[NG][KS];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int k = kq * KS + j;
            wr[g][j] = (cv && k < D) ? W[static_cast<size_t>(g * D + c) * D + k] : 0.0f;
        }
    // step 0 input: w = v0 (unnormalised), scale 1 / |v0|
    const float v0c = cv ? v0[static_cast<size_t>(bseq) * D + c] : 0.0f;
    if (kq == 0 && c < DP) wbuf[0][c] = v0c;
    float inv;
    {
        const float sq = wave_sum(kq == 0 ? v0c * v0c : 0.0f);
        if constexpr (NW > 1) {
            if (lane == 0) part[0][wave] = sq;
        }
        __syncthreads();     // also for one wavefront: lanes read what other lanes wrote
        if constexpr (NW > 1) {
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) tot += part[0][w];
            inv = 1.0f / sqrtf(tot);
        } else {
            inv = 1.0f / sqrtf(sq);
        }
    }

    const size_t fb = static_cast<size_t>(bseq) * T * NF * D;
    float ring[PF][NF];
    auto fetch = [&](int t, float (&f)[NF]) {
        const size_t o = fb + static_cast<size_t>(t < T ? t : T - 1) * NF * D + cr;
#pragma unroll
        for (int q = 0; q < NF; ++q) f[q] = F[o + static_cast<size_t>(q) * D];
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u, ring[u]);
    double sum = 0.0;
    int cur = 0;
    auto advance = [&](const float (&f)[NF]) {
        // dot products of this lane's columns with the previous w
        float xs[KS];
        if constexpr (KS >= 4) {
#pragma unroll
            for (int j4 = 0; j4 < KS / 4; ++j4) {
                const v4f x = *reinterpret_cast<const v4f *>(&wbuf[cur][kq * KS + 4 * j4]);
                xs[4 * j4] = x[0]; xs[4 * j4 + 1] = x[1]; xs[4 * j4 + 2] = x[2]; xs[4 * j4 + 3] = x[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < KS; ++j) xs[j] = wbuf[cur][kq * KS + j];
        }
        float acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < KS; ++j) a = __builtin_fmaf(wr[g][j], xs[j], a);
            if constexpr (KQ >= 2) a += dpp<0xB1>(a);
            if constexpr (KQ >= 4) a += dpp<0x4E>(a);
            acc[g] = a * inv;
        }
        float w;
        if constexpr (NF == 1) {
            w = f[0] * acc[0];
        } else {
            const float vc = wbuf[cur][c < DP ? c : 0] * inv;
            w = f[0] * vc + f[1] * acc[1] + f[2] * acc[2] + f[3] * acc[0];   // rows: r = 0, z = 1, n = 2
        }
        w = cv ? w : 0.0f;
        const int nxt = cur ^ 1;
        if (kq == 0 && c < DP) wbuf[nxt][c] = w;
        float tot = wave_sum(kq == 0 ? w * w : 0.0f);
        if constexpr (NW > 1) {
            if (lane == 0) part[nxt][wave] = tot;
        }
        // The next step's lanes read w written by other lanes: a barrier even
        // for a single wavefront, or the compiler may treat the LDS exchange as
        // private to each lane.
        __syncthreads();
        if constexpr (NW > 1) {
            tot = 0.0f;
#pragma unroll
            for (int q = 0; q < NW; ++q) tot += part[nxt][q];
        }
        // log |w| = log2(|w|^2) ln 2 / 2: the hardware log2 and reciprocal square
        // root (about 1 ulp each) keep the chain's latency down; the log2 sum is
        // accumulated in float64 and scaled once at the end
        sum += static_cast<double>(__builtin_amdgcn_logf(tot));
        inv = __builtin_amdgcn_rsqf(tot);
        cur = nxt;
    };
    const int nfull = T - T % PF;
    for (int t0 = 0; t0 < nfull; t0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            advance(ring[u]);
            fetch(t0 + u + PF, ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (nfull + u < T) advance(ring[u]);
    if (tid == 0) out[bseq] = sum * (0.5 * 0.69314718055994530942) / static_cast<double>(T);
}

template <int DP>
int launch_lle_dp(const deer_cell_params_t *p, const float *s0, const float *traj, const float *v0, int B, int T,
                  double *out, const float *proj, float *F, float *junk, unsigned *res_bits, hipStream_t stream)
{
    const int D = p->D;
    if (p->cell == DEER_CELL_GRU) {
        const int tiles = (T + kTP - 1) / kTP;
        DEER_LAUNCH((gru_lle_factor_kernel<DP>), dim3(static_cast<unsigned>(static_cast<long long>(B) * tiles)),
                           dim3(kThreads), 0, stream, p->W, p->b2, proj, s0, traj, F, T, D, tiles);
        DEER_HIP(hipGetLastError());
        DEER_LAUNCH((lle_chain_kernel<DP, 4>), dim3(static_cast<unsigned>(B)), dim3(64 * Chain<DP>::NW), 0, stream,
                    p->W, F, v0, T, D, out);
    } else {
        // d_t = 1 - f_t^2 is the factored dense leaf the tanh evaluation writes
        const int r = launch_tanh_eval(p->W, proj, s0, traj, traj, nullptr, nullptr, nullptr, F, junk, res_bits, B, T,
                                       D, 1, Linearization{kLinJacobian, 1.0f}, FrontOut{}, stream);
        if (r) return r;
        DEER_LAUNCH((lle_chain_kernel<DP, 1>), dim3(static_cast<unsigned>(B)), dim3(64 * Chain<DP>::NW), 0, stream,
                    p->W, F, v0, T, D, out);
    }
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace

LleLayout lle_layout(void *ws, const deer_cell_params_t *p, int B, int T)
{
    const int PD = (p->cell == DEER_CELL_GRU) ? 3 * p->D : p->D;
    const int NF = (p->cell == DEER_CELL_GRU) ? 4 : 1;
    const size_t BT = static_cast<size_t>(B) * T;
    Carve c(ws);
    LleLayout L;
    L.proj = c.take<float>(projection_floats(B, T, PD));
    L.F = c.take<float>(BT * NF * p->D);
    L.junk = c.take<float>(p->cell == DEER_CELL_GRU ? 0 : BT * p->D);
    L.res_bits = c.take<unsigned>(B);
    L.bytes = c.off;
    return L;
}

int launch_lle(const deer_cell_params_t *p, const float *x, const float *s0, const float *traj, const float *v0, int B,
               int T, double *out, const LleLayout &L, hipStream_t stream)
{
    const int PD = (p->cell == DEER_CELL_GRU) ? 3 * p->D : p->D;
    int r = launch_projection(x, p->U, p->b, L.proj, B, T, p->M, PD, false, stream);
    if (r) return r;
    const int D = p->D;
    if (D <= 4) return launch_lle_dp<4>(p, s0, traj, v0, B, T, out, L.proj, L.F, L.junk, L.res_bits, stream);
    if (D <= 8) return launch_lle_dp<8>(p, s0, traj, v0, B, T, out, L.proj, L.F, L.junk, L.res_bits, stream);
    if (D <= 16) return launch_lle_dp<16>(p, s0, traj, v0, B, T, out, L.proj, L.F, L.junk, L.res_bits, stream);
    if (D <= 32) return launch_lle_dp<32>(p, s0, traj, v0, B, T, out, L.proj, L.F, L.junk, L.res_bits, stream);
    return launch_lle_dp<64>(p, s0, traj, v0, B, T, out, L.proj, L.F, L.junk, L.res_bits, stream);
}

}  // namespace deer
