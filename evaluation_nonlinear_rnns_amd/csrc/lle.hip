// Largest Lyapunov exponent along a given trajectory, on the GPU.
//
// The "Predictability Enables Parallelization" page estimates the LLE by
// pushing a unit vector through the Jacobians J_t = d f / d s at
// (s_{t-1}, x_t), renormalising after every step and averaging the log growth
// (rebuttal "LLE computation cost", its appendix's Algorithm 1); a negative LLE
// predicts that parallel Newton converges in few iterations.
//
// Two launches: the per-step Jacobian factors are evaluated in parallel over
// all positions (the trajectory is given), then one wavefront per sequence runs
// the inherently sequential vector chain, which then costs a few matrix-vector
// products per step:
//   tanh:  J_t v = d_t * (W v),                d_t = 1 - f_t^2
//   GRU:   J_t v = z * v + al * (Wz v) + be * (Wn v) + ga * (Wr v)
//          al = (s - n) z (1 - z),  be = (1 - z)(1 - n^2) r,
//          ga = (1 - z)(1 - n^2) r (1 - r) (W_hn s + b_hn)
// (the GRU Jacobian in closed form, gate order r, z, n).
#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
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

// One wavefront per sequence: v <- J_t v / |J_t v|, lle = mean_t log |J_t v|.
// NF = 1 (tanh: factor d) or 4 (GRU: z, al, be, ga).  The factors are fetched
// PF steps ahead with unconditional (clamped) loads; W sits in LDS and v is
// broadcast with lane reads.
template <int DP, int NF>
__global__ __launch_bounds__(64) void lle_chain_kernel(const float *__restrict__ W, const float *__restrict__ F,
                                                       const float *__restrict__ v0, int T, int D,
                                                       double *__restrict__ out)
{
    constexpr int NG = NF == 1 ? 1 : 3;
    constexpr int PF = 8;
    __shared__ float Wsh[NG][DP][DP];    // Wsh[g][k][c] = W[g*D + c][k]
    const int lane = threadIdx.x, bseq = blockIdx.x;
    for (int e = lane; e < NG * DP * DP; e += 64) {
        const int g = e / (DP * DP), k = (e / DP) % DP, c = e % DP;
        Wsh[g][k][c] = (k < D && c < D) ? W[static_cast<size_t>(g * D + c) * D + k] : 0.0f;
    }
    __syncthreads();
    const bool cv = lane < D;
    const int c = lane < DP ? lane : 0;
    const int cr = cv ? lane : 0;
    float v = cv ? v0[static_cast<size_t>(bseq) * D + lane] : 0.0f;
    {
        float s2 = v * v;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
        v = v / sqrtf(s2);
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
    auto advance = [&](const float (&f)[NF]) {
        float acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = 0.0f;
#pragma unroll
        for (int k = 0; k < DP; ++k) {
            const float vk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] += Wsh[g][k][c] * vk;
        }
        float w;
        if constexpr (NF == 1) w = f[0] * acc[0];
        else w = f[0] * v + f[1] * acc[1] + f[2] * acc[2] + f[3] * acc[0];   // rows: r = 0, z = 1, n = 2
        w = cv ? w : 0.0f;
        float s2 = w * w;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
        const float g = sqrtf(s2);
        sum += static_cast<double>(logf(g));
        v = w / g;
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
    if (lane == 0) out[bseq] = sum / static_cast<double>(T);
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
        DEER_LAUNCH((lle_chain_kernel<DP, 4>), dim3(static_cast<unsigned>(B)), dim3(64), 0, stream, p->W, F, v0,
                           T, D, out);
    } else {
        // d_t = 1 - f_t^2 is the factored dense leaf the tanh evaluation writes
        const int r = launch_tanh_eval(p->W, proj, s0, traj, traj, nullptr, nullptr, nullptr, F, junk, res_bits, B, T,
                                       D, 1, Linearization{kLinJacobian, 1.0f}, stream);
        if (r) return r;
        DEER_LAUNCH((lle_chain_kernel<DP, 1>), dim3(static_cast<unsigned>(B)), dim3(64), 0, stream, p->W, F, v0,
                           T, D, out);
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
