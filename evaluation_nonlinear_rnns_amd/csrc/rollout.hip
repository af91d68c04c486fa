// Sequential rollout s_t = f(s_{t-1}, x_t) on the GPU: the evaluation the
// parallel methods are timed against on the same device ("Predictability
// Enables Parallelization" page, rebuttal, "Comparison with sequential speed").
//
// Two launches.  The input projection p_t = U x_t + b does not depend on the
// state, so it runs first over all positions at once (the kernel deer_solve
// uses, plain [B, T, PD] layout).  Then one workgroup per sequence steps the
// recurrence, the only part that is sequential by definition:
//   tanh:  s_t = tanh(W s_{t-1} + p_t)
//   GRU:   q = W_hh s_{t-1} + b_hh;  r = sigma(p_r + q_r), z = sigma(p_z + q_z),
//          n = tanh(p_n + r q_n),    s_t = (1 - z) n + z s_{t-1}
// KQ lanes share one state channel's dot products, each holding its slice of
// W's rows in registers; DPP adds combine the slices, so every lane of the
// channel ends with the same bits.  The new state goes through LDS (two
// buffers by step parity, one barrier per step), and the projection is
// fetched PF steps ahead into a register ring with clamped, unconditional
// loads, so no global load latency sits on the step-to-step chain.
#include "internal.h"

namespace deer {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// The step-to-step chain runs through these, so they use the hardware exp and
// reciprocal (about 1 ulp each): sigma(u) = 1 / (1 + e^-u), and
// tanh(u) = 1 - 2 / (1 + e^{2u}) (absolute error a few 1e-8 near 0; +-1 at
// the ends, NaN in NaN out).
__device__ __forceinline__ float sigm(float u) { return __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
__device__ __forceinline__ float tanh_fast(float u) { return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * u)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}

// KQ lanes per channel, CW channels per wavefront, NW wavefronts, KS columns per lane.
template <int DP> struct RollKQ;
template <> struct RollKQ<4>  { static constexpr int KQ = 4; };
template <> struct RollKQ<8>  { static constexpr int KQ = 4; };
template <> struct RollKQ<16> { static constexpr int KQ = 4; };
template <> struct RollKQ<32> { static constexpr int KQ = 2; };
template <> struct RollKQ<64> { static constexpr int KQ = 4; };

template <int DP>
struct RollGeom {
    static constexpr int KQ = RollKQ<DP>::KQ;
    static constexpr int CW = 64 / KQ;
    static constexpr int NW = DP > CW ? DP / CW : 1;
    static constexpr int KS = DP / KQ;
};

template <int DP, bool GRU>
__global__ __launch_bounds__(64 * RollGeom<DP>::NW) void rollout_chain_kernel(
    const float *__restrict__ W, const float *__restrict__ bhh, const float *__restrict__ proj,
    const float *__restrict__ s0, float *__restrict__ traj, int T, int D)
{
    using G = RollGeom<DP>;
    constexpr int NG = GRU ? 3 : 1;
    constexpr int PF = 8;
    constexpr int KQ = G::KQ, KS = G::KS;
    __shared__ __align__(16) float sbuf[2][DP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, bseq = blockIdx.x;
    const int c = wave * G::CW + lane / KQ, kq = lane % KQ;
    const bool cv = c < D;
    const int cr = cv ? c : 0;
    const int PD = NG * D;

    float wr[NG][KS];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int k = kq * KS + j;
            wr[g][j] = (cv && k < D) ? W[static_cast<size_t>(g * D + c) * D + k] : 0.0f;
        }
    float bq[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) bq[g] = (GRU && bhh && cv) ? bhh[g * D + c] : 0.0f;

    if (kq == 0 && c < DP) sbuf[0][c] = (cv && s0) ? s0[static_cast<size_t>(bseq) * D + c] : 0.0f;
    __syncthreads();

    const size_t pb = static_cast<size_t>(bseq) * T * PD;
    const size_t ob = static_cast<size_t>(bseq) * T * D;
    float ring[PF][NG];
    auto fetch = [&](int t, float (&v)[NG]) {
        const size_t o = pb + static_cast<size_t>(t < T ? t : T - 1) * PD + cr;
#pragma unroll
        for (int g = 0; g < NG; ++g) v[g] = proj[o + static_cast<size_t>(g) * D];
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u, ring[u]);

    int cur = 0;
    auto step = [&](int t, const float (&p)[NG]) {
        float xs[KS];
        if constexpr (KS >= 4) {
#pragma unroll
            for (int j4 = 0; j4 < KS / 4; ++j4) {
                const v4f v = *reinterpret_cast<const v4f *>(&sbuf[cur][kq * KS + 4 * j4]);
                xs[4 * j4] = v[0]; xs[4 * j4 + 1] = v[1]; xs[4 * j4 + 2] = v[2]; xs[4 * j4 + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < KS; ++j) xs[j] = sbuf[cur][kq * KS + j];
        }
        float acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < KS; ++j) a = __builtin_fmaf(wr[g][j], xs[j], a);
            if constexpr (KQ >= 2) a += dpp<0xB1>(a);     // quad_perm [1, 0, 3, 2]
            if constexpr (KQ >= 4) a += dpp<0x4E>(a);     // quad_perm [2, 3, 0, 1]
            acc[g] = a;
        }
        float f;
        if constexpr (GRU) {
            const float h = sbuf[cur][cr];
            const float rg = sigm(p[0] + (acc[0] + bq[0]));
            const float zg = sigm(p[1] + (acc[1] + bq[1]));
            const float ng = tanh_fast(p[2] + rg * (acc[2] + bq[2]));
            f = (1.0f - zg) * ng + zg * h;
        } else {
            f = tanh_fast(p[0] + acc[0]);
        }
        f = cv ? f : 0.0f;
        const int nxt = cur ^ 1;
        if (kq == 0 && c < DP) sbuf[nxt][c] = f;
        if (kq == 0 && cv) traj[ob + static_cast<size_t>(t) * D + c] = f;
        // the next step's lanes read what other lanes wrote: a barrier even for
        // one wavefront, or the compiler may treat the LDS exchange as private
        __syncthreads();
        cur = nxt;
    };
    const int nfull = T - T % PF;
    for (int t0 = 0; t0 < nfull; t0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            step(t0 + u, ring[u]);
            fetch(t0 + u + PF, ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (nfull + u < T) step(nfull + u, ring[u]);
}

template <int DP>
int launch_chain(const deer_cell_params_t *p, const float *proj, const float *s0, int B, int T, float *traj,
                 hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(B)), block(64 * RollGeom<DP>::NW);
    if (p->cell == DEER_CELL_GRU)
        DEER_LAUNCH((rollout_chain_kernel<DP, true>), grid, block, 0, stream, p->W, p->b2, proj, s0, traj, T, p->D);
    else
        DEER_LAUNCH((rollout_chain_kernel<DP, false>), grid, block, 0, stream, p->W, nullptr, proj, s0, traj, T,
                    p->D);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

int proj_width(const deer_cell_params_t *p) { return p->cell == DEER_CELL_GRU ? 3 * p->D : p->D; }

}  // namespace

size_t rollout_workspace_bytes(const deer_cell_params_t *p, int B, int T)
{
    return align_up(projection_floats(B, T, proj_width(p)) * sizeof(float));
}

int launch_rollout(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T, float *traj,
                   void *workspace, hipStream_t stream)
{
    if (B == 0 || T == 0) return DEER_OK;
    float *proj = static_cast<float *>(workspace);
    int rc = launch_projection(x, p->U, p->b, proj, B, T, p->M, proj_width(p), false, stream);
    if (rc) return rc;
    const int D = p->D;
    if (D <= 4) return launch_chain<4>(p, proj, s0, B, T, traj, stream);
    if (D <= 8) return launch_chain<8>(p, proj, s0, B, T, traj, stream);
    if (D <= 16) return launch_chain<16>(p, proj, s0, B, T, traj, stream);
    if (D <= 32) return launch_chain<32>(p, proj, s0, B, T, traj, stream);
    return launch_chain<64>(p, proj, s0, B, T, traj, stream);
}

}  // namespace deer
