// Parallel Broyden ("Parallel Broyden Methods" page, sections 3.1-3.2 and
// appendix E): diagonal-plus-low-rank (DPLR) block approximations built from
// trajectory secants, and the chunked scan with randomized re-compression.
//
// Blocks.  Position t of a sequence holds J^_t = alpha I + sum_j u_j v_j^T with
// at most m columns (U, V: [B, T, m, D], column j of position t contiguous);
// the solver uses A_t = alpha I + (1 - k) sum_j u_j v_j^T (damping k on the
// low-rank correction only, appendix E.4).  Iteration i >= 1 updates every
// block from the secant pair ds = s^(i)_{t-1} - s^(i-1)_{t-1},
// df = f^(i)_t - f^(i-1)_t into column slot (i - 1) mod m:
//   rank-one: drop the slot's column, then u = (df - J^' ds) / |ds|^2, v = ds
//             (zero column for ds = 0);
//   multisecant: the slot takes (ds, df); U = (F - alpha S)(S^T S + lambda I)^{-1},
//             V = S over the min(i, m) valid secants (F: [B, T, m, D]); a
//             failed Cholesky factorisation leaves U = 0.
//
// Linear step, increment form: delta_t = A_t delta_{t-1} + c_t, delta_0 = 0,
// c_t = f_t - s_t, s^(i+1) = s^(i) + delta.  Chunks of L positions:
//   fold   (one wavefront per chunk): block updates, then the chunk aggregate
//          P = p I + sum_a l_a r_a^T with offset Pb, composed left to right
//          (A_t P = alpha p I + [alpha l_a + sum_j u~_j (v_j.l_a) | p u~_j][r_a | v_j]^T,
//          Pb <- A_t Pb + c_t) and re-compressed to m columns whenever it has
//          more: Y = L (R^T Omega), Q = modified Gram-Schmidt basis of Y's
//          columns (a column left with at most 1e-5 of its norm drops to zero),
//          L <- Q, R <- R (L^T Q);
//   carry  (one wavefront per sequence): entry_{q+1} = P_q entry_q + Pb_q;
//   replay (one wavefront per chunk): the exact recurrence from the chunk's entry.
// Exact zeros stay zero, so a converged prefix (c_t = 0) stays exact through
// compressed carries: finite-step recovery holds.
//
// Lane d of a wavefront holds row d of every D-vector (D <= 64); inner
// products are wavefront sums broadcast from lane 0, so every lane takes the
// same decisions.
#include <algorithm>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr float kQrDrop = 1e-5f;

// DPP move of v; lanes outside ROWMASK (rows of 16 lanes) read 0.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF,
                                                                 false));
}

// Sum over the 64 lanes, the same value on every lane: pairs and quads
// (quad_perm), halves of a row (row_half_mirror), rows (row_mirror), then the
// row totals are chained into row 3 (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3) and lane 63's total is broadcast.  The
// order of the additions is fixed, so every call rounds the same way.
__device__ __forceinline__ float wsum(float v)
{
    v += dpp<0xB1>(v);          // quad_perm [1, 0, 3, 2]
    v += dpp<0x4E>(v);          // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);         // row_half_mirror
    v += dpp<0x140>(v);         // row_mirror
    v += dpp<0x142, 0xA>(v);    // row_bcast:15
    v += dpp<0x143, 0xC>(v);    // row_bcast:31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float ld(const float *p, bool ok) { return ok ? *p : 0.0f; }

// Iteration-dependent view of the buffers (solver) or the fixed inputs (scan).
struct StepView {
    const float *s_cur = nullptr, *s_prev = nullptr, *f_cur = nullptr, *f_prev = nullptr;
    float *s_next = nullptr;
    int i = 0;          // iteration index
    int n = 0;          // valid columns after this iteration's update
    bool update = false;
};

__device__ __forceinline__ bool solver_view(const DplrArgs &a, int bseq, StepView &v)
{
    if (!a.ctl) {                                   // standalone scan
        v.n = a.n_fixed;
        return true;
    }
    if (a.ctl->all_done) return false;
    if (a.skip && a.skip[bseq]) return false;
    v.i = a.ctl->iter - 1;                          // the check of iteration i has set iter = i + 1
    const bool odd = (v.i & 1) != 0;
    v.s_cur = odd ? a.s_odd : a.s_even;
    v.s_prev = odd ? a.s_even : a.s_odd;
    v.s_next = odd ? a.s_even : a.s_odd;
    v.f_cur = odd ? a.f_odd : a.f_even;
    v.f_prev = odd ? a.f_even : a.f_odd;
    v.n = min(v.i, a.m);
    v.update = v.i >= 1 && a.m > 0;
    return true;
}

// Block update of one position (see the file header); lane d holds row d.
template <int MR>
__device__ __forceinline__ void block_update(const DplrArgs &a, int i, float ds, float df, float (&u)[MR],
                                             float (&v)[MR], float (&fs)[MR])
{
    const int m = a.m;
    const int slot = (i - 1) % m;
    if (!a.multisecant) {
        const int nb = min(i - 1, m);
        float jds = a.alpha * ds;
#pragma unroll
        for (int j = 0; j < MR; ++j)
            if (j < nb && j != slot) jds += u[j] * wsum(v[j] * ds);
        const float ss = wsum(ds * ds);
#pragma unroll
        for (int j = 0; j < MR; ++j)
            if (j == slot) {
                u[j] = ss > 0.0f ? (df - jds) / ss : 0.0f;
                v[j] = ss > 0.0f ? ds : 0.0f;
            }
        return;
    }
#pragma unroll
    for (int j = 0; j < MR; ++j)
        if (j == slot) {
            v[j] = ds;
            fs[j] = df;
        }
    const int n = min(i, m);
    float C[MR][MR];
    bool ok = true;
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int c = 0; c <= r; ++c) {
            if (r >= n || !ok) continue;
            float acc = wsum(v[r] * v[c]) + (r == c ? a.lambda : 0.0f);
#pragma unroll
            for (int e = 0; e < c; ++e) acc -= C[r][e] * C[c][e];
            if (r == c) {
                if (!(acc > 0.0f) || __builtin_isinf(acc)) ok = false;
                else C[r][r] = sqrtf(acc);
            } else {
                C[r][c] = acc / C[c][c];
            }
        }
    float y[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        if (r >= n) continue;
        float acc = fs[r] - a.alpha * v[r];
#pragma unroll
        for (int e = 0; e < r; ++e) acc -= C[r][e] * y[e];
        y[r] = ok ? acc / C[r][r] : 0.0f;
    }
#pragma unroll
    for (int r = MR - 1; r >= 0; --r) {
        if (r >= n) continue;
        float acc = y[r];
#pragma unroll
        for (int e = r + 1; e < MR; ++e)
            if (e < n) acc -= C[e][r] * y[e];
        y[r] = ok ? acc / C[r][r] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) u[r] = (ok && r < n) ? y[r] : 0.0f;
}

// y = alpha x + sum_{j<n} u_j (v_j . x) for the lane's row
template <int MR>
__device__ __forceinline__ float dplr_apply(float alpha, const float (&u)[MR], const float (&v)[MR], int n, float x)
{
    float y = alpha * x;
#pragma unroll
    for (int j = 0; j < MR; ++j)
        if (j < n) y += u[j] * wsum(v[j] * x);
    return y;
}

// ------------------------------------------------------------------ fold
template <int MR>
__global__ __launch_bounds__(kThreads) void dplr_fold_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63;
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (w >= static_cast<long long>(a.B) * a.nchunk) return;
    const int bseq = static_cast<int>(w / a.nchunk), q = static_cast<int>(w % a.nchunk);
    StepView sv;
    if (!solver_view(a, bseq, sv)) return;
    const int D = a.D, m = a.m, n = sv.n;
    const bool row = lane < D;
    const int t0 = q * a.chunk, t1 = min(t0 + a.chunk, a.T);
    const bool last = q == a.nchunk - 1;
    if (last && !sv.update) return;                 // nothing to fold and no carry to produce
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    float om[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) om[j] = (row && j < m) ? a.omega[lane * m + j] : 0.0f;

    float p = 1.0f, Pb = 0.0f;
    int r = 0;
    float PL[MR], PR[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) PL[j] = PR[j] = 0.0f;

    // inputs of position t, loaded one position ahead of their use (clamped,
    // always-valid addresses; lanes past D and columns past m read as zero)
    const int l = min(lane, D - 1);
    struct In {
        float u[MR], v[MR], fs[MR];
        float sc, fc, fp, sp;       // s^(i)_t, f^(i)_t, f^(i-1)_t, s^(i-1)_{t-1} (or c_t standalone)
    };
    // Branch-free loads: every source is a valid [B,T,...] buffer (an unused one
    // stands in where a mode reads nothing), so the loads stay in flight.
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_f = a.ctl ? sv.f_cur : a.c;
    const float *src_fp = a.ctl ? sv.f_prev : a.c;
    const float *src_sp = a.ctl ? sv.s_prev : a.c;
    const float *src_u = m > 0 ? a.U : src_s;
    const float *src_v = m > 0 ? a.V : src_s;
    const float *src_F = (m > 0 && a.multisecant) ? a.F : src_v;
    const int mm = max(m, 1);
    auto load_in = [&](int t, In &in) {
        const size_t pos = seq + min(t, a.T - 1);
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const size_t o = m > 0 ? (pos * m + min(j, mm - 1)) * D + l : pos * D + l;
            in.u[j] = src_u[o];
            in.v[j] = src_v[o];
            in.fs[j] = src_F[o];
        }
        in.sc = src_s[pos * D + l];
        in.fc = src_f[pos * D + l];
        in.fp = src_fp[pos * D + l];
        in.sp = src_sp[(pos - (t > 0 ? 1 : 0)) * D + l];
    };
    // Values are masked when a position is consumed, not when it is loaded, so
    // the loads of the next position stay in flight: lanes past D and columns
    // past m become zero.
    auto mask_in = [&](In &in) {
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const bool have = row && j < m;
            in.u[j] = have ? in.u[j] : 0.0f;
            in.v[j] = have ? in.v[j] : 0.0f;
            in.fs[j] = have ? in.fs[j] : 0.0f;
        }
        in.sc = row ? in.sc : 0.0f;
        in.fc = row ? in.fc : 0.0f;
        in.fp = row ? in.fp : 0.0f;
        in.sp = row ? in.sp : 0.0f;
    };
    // s^(i)_{t0-1}: the first ds of the chunk
    float s_before = 0.0f;
    if (a.ctl && sv.update && t0 > 0) {
        const float v0 = sv.s_cur[(seq + t0 - 1) * D + l];
        s_before = row ? v0 : 0.0f;
    }
    In cur;
    load_in(t0, cur);
    for (int t = t0; t < t1; ++t) {
        const size_t pos = seq + t;
        In nxt;
        load_in(t + 1, nxt);                        // clamped past the chunk: harmless extra load
        mask_in(cur);
        float(&u)[MR] = cur.u;
        float(&v)[MR] = cur.v;
        float(&fs)[MR] = cur.fs;
        float c;
        if (a.ctl) {
            c = cur.fc - cur.sc;
            if (sv.update) {
                const float ds = (t > 0) ? s_before - cur.sp : 0.0f;
                const float df = cur.fc - cur.fp;
                block_update<MR>(a, sv.i, ds, df, cur.u, cur.v, cur.fs);
                if (row) {
                    float *Up = a.U + pos * m * D + lane, *Vp = a.V + pos * m * D + lane;
                    if (a.multisecant) {
#pragma unroll
                        for (int j = 0; j < MR; ++j)
                            if (j < m) Up[j * D] = u[j];
                    }
                    const int slot = (sv.i - 1) % m;
#pragma unroll
                    for (int j = 0; j < MR; ++j)
                        if (j == slot) {
                            if (!a.multisecant) Up[j * D] = u[j];
                            Vp[j * D] = v[j];
                            if (a.multisecant) a.F[pos * m * D + lane + j * D] = fs[j];
                        }
                }
            }
            s_before = cur.sc;
        } else {
            c = cur.sc;
        }
        if (last) {                                 // the last chunk only updates its blocks
            cur = nxt;
            continue;
        }
#pragma unroll
        for (int j = 0; j < MR; ++j) u[j] *= a.shrink;

        // A_t P: the K = r + n column pairs
        float Lf[2 * MR], Rf[2 * MR];
#pragma unroll
        for (int e = 0; e < MR; ++e) {
            Lf[e] = (e < r) ? dplr_apply<MR>(a.alpha, u, v, n, PL[e]) : 0.0f;
            Rf[e] = (e < r) ? PR[e] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            Lf[MR + j] = p * u[j];
            Rf[MR + j] = v[j];
        }
        // columns in the order of the definition: the r aggregate columns, then the n block columns
        auto col_ok = [&](int e) { return e < MR ? e < r : (e - MR) < n; };
        const int K = r + n;
        p = a.alpha * p;
        if (K <= m) {
            float NL[MR], NR[MR];
            int k = 0;
#pragma unroll
            for (int e = 0; e < 2 * MR; ++e) {
                if (!col_ok(e)) continue;
#pragma unroll
                for (int j = 0; j < MR; ++j)
                    if (j == k) { NL[j] = Lf[e]; NR[j] = Rf[e]; }
                ++k;
            }
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                PL[j] = j < K ? NL[j] : 0.0f;
                PR[j] = j < K ? NR[j] : 0.0f;
            }
            r = K;
        } else {
            // Y = L (R^T Omega), then modified Gram-Schmidt
            float Q[MR];
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                if (j >= m) { Q[j] = 0.0f; continue; }
                float y = 0.0f;
#pragma unroll
                for (int e = 0; e < 2 * MR; ++e)
                    if (col_ok(e)) y += Lf[e] * wsum(Rf[e] * om[j]);
                const float ny = sqrtf(wsum(y * y));
#pragma unroll
                for (int l = 0; l < MR; ++l)
                    if (l < j) y -= wsum(Q[l] * y) * Q[l];
                const float nq = sqrtf(wsum(y * y));
                Q[j] = (nq > kQrDrop * ny) ? y / nq : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                float rr = 0.0f;
                if (j < m) {
#pragma unroll
                    for (int e = 0; e < 2 * MR; ++e)
                        if (col_ok(e)) rr += Rf[e] * wsum(Lf[e] * Q[j]);
                }
                PL[j] = Q[j];
                PR[j] = rr;
            }
            r = m;
        }
        Pb = dplr_apply<MR>(a.alpha, u, v, n, Pb) + c;
        cur = nxt;
    }
    if (last || !row) return;
    const size_t agg = static_cast<size_t>(bseq) * a.nchunk + q;
    if (lane == 0) {
        a.agg_p[agg] = p;
        a.agg_r[agg] = r;
    }
#pragma unroll
    for (int j = 0; j < MR; ++j)
        if (j < m) {
            a.agg_L[(agg * m + j) * D + lane] = PL[j];
            a.agg_R[(agg * m + j) * D + lane] = PR[j];
        }
    a.agg_b[agg * D + lane] = Pb;
}

// ------------------------------------------------------------------ carry
template <int MR>
__global__ __launch_bounds__(kThreads) void dplr_carry_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63;
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (w >= a.B) return;
    const int bseq = static_cast<int>(w);
    StepView sv;
    if (!solver_view(a, bseq, sv)) return;
    const int D = a.D, m = a.m;
    const bool row = lane < D;
    const size_t base = static_cast<size_t>(bseq) * a.nchunk;
    const int nq = a.nchunk - 1;                 // aggregates in the chain
    // ring of the next kPF aggregates, loaded ahead of the dependent chain
    constexpr int kPF = 8;
    float rl[kPF][MR], rrr[kPF][MR], rb[kPF], rp[kPF];
    int rk[kPF];
    // unconditional loads at clamped, always-valid addresses (a load under a
    // divergent branch would make every later wait drain the whole ring)
    const int l = min(lane, D - 1);
    auto fetch = [&](int q, float (&L)[MR], float (&R)[MR], float &b, float &p, int &r) {
        const int qq = min(q, max(nq - 1, 0));
        const size_t agg = base + qq;
        p = a.agg_p[agg];
        r = a.agg_r[agg];
        b = a.agg_b[agg * D + l];
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const size_t o = m > 0 ? (agg * m + min(j, m - 1)) * D + l : agg * D + l;
            L[j] = (m > 0 ? a.agg_L : a.agg_b)[o];
            R[j] = (m > 0 ? a.agg_R : a.agg_b)[o];
        }
    };
    float e = 0.0f;
    if (nq > 0) {
#pragma unroll
        for (int k = 0; k < kPF; ++k) fetch(k, rl[k], rrr[k], rb[k], rp[k], rk[k]);
    }
    for (int q0 = 0; q0 <= nq; q0 += kPF) {
#pragma unroll
        for (int k = 0; k < kPF; ++k) {
            const int q = q0 + k;
            if (q > nq) break;
            if (row) a.entry[(base + q) * D + lane] = e;
            if (q == nq) break;
            // lanes past D hold copies of lane D - 1; e is zero there, so they add nothing
            // every column is computed and the unused ones are selected away (no
            // branches, so the ring's loads stay in flight across steps)
            float ne = rp[k] * e;
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const bool use = j < rk[k];
                const float w = wsum(use ? rrr[k][j] * e : 0.0f);
                ne += use ? rl[k][j] * w : 0.0f;
            }
            e = row ? ne + rb[k] : 0.0f;
            fetch(q + kPF, rl[k], rrr[k], rb[k], rp[k], rk[k]);
        }
    }
}

// ------------------------------------------------------------------ replay
template <int MR>
__global__ __launch_bounds__(kThreads) void dplr_replay_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63;
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (w >= static_cast<long long>(a.B) * a.nchunk) return;
    const int bseq = static_cast<int>(w / a.nchunk), q = static_cast<int>(w % a.nchunk);
    StepView sv;
    if (!solver_view(a, bseq, sv)) return;
    const int D = a.D, m = a.m, n = sv.n;
    const bool row = lane < D;
    const int t0 = q * a.chunk, t1 = min(t0 + a.chunk, a.T);
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    float dl = ld(a.entry + (static_cast<size_t>(bseq) * a.nchunk + q) * D + lane, row);
    const int l = min(lane, D - 1);
    struct In {
        float u[MR], v[MR];
        float sc, c;
    };
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_c = a.ctl ? sv.f_cur : a.c;
    const float *src_u = n > 0 ? a.U : src_s;
    const float *src_v = n > 0 ? a.V : src_s;
    const int nn = max(n, 1);
    auto load_in = [&](int t, In &in) {
        const size_t pos = seq + min(t, a.T - 1);
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const size_t o = n > 0 ? (pos * m + min(j, nn - 1)) * D + l : pos * D + l;
            in.u[j] = src_u[o];
            in.v[j] = src_v[o];
        }
        in.sc = src_s[pos * D + l];
        in.c = src_c[pos * D + l];            // f in the solver; c = f - s once consumed
    };
    In cur;
    load_in(t0, cur);
    for (int t = t0; t < t1; ++t) {
        const size_t pos = seq + t;
        In nxt;
        load_in(t + 1, nxt);
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const bool have = row && j < n;
            cur.u[j] = have ? cur.u[j] * a.shrink : 0.0f;
            cur.v[j] = have ? cur.v[j] : 0.0f;
        }
        const float c = row ? (a.ctl ? cur.c - cur.sc : cur.c) : 0.0f;
        cur.sc = row ? cur.sc : 0.0f;
        dl = dplr_apply<MR>(a.alpha, cur.u, cur.v, n, dl) + c;
        if (row) {
            if (a.ctl) sv.s_next[pos * D + lane] = cur.sc + dl;
            else a.out[pos * D + lane] = dl;
        }
        cur = nxt;
    }
}

template <int MR>
int launch_dplr_mr(const DplrArgs &a, hipStream_t stream)
{
    const long long chunks = static_cast<long long>(a.B) * a.nchunk;
    const unsigned gc = static_cast<unsigned>((chunks + kWavesPerBlock - 1) / kWavesPerBlock);
    const unsigned gs = static_cast<unsigned>((a.B + kWavesPerBlock - 1) / kWavesPerBlock);
    DEER_LAUNCH((dplr_fold_kernel<MR>), dim3(gc), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    DEER_LAUNCH((dplr_carry_kernel<MR>), dim3(gs), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    DEER_LAUNCH((dplr_replay_kernel<MR>), dim3(gc), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace

int launch_dplr_step(const DplrArgs &a, hipStream_t stream)
{
    if (a.B == 0 || a.T == 0) return DEER_OK;
    if (a.m <= 2) return launch_dplr_mr<2>(a, stream);
    if (a.m <= 4) return launch_dplr_mr<4>(a, stream);
    return launch_dplr_mr<8>(a, stream);
}

}  // namespace deer
