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
//   fold   block updates, then the chunk aggregate P = p I + sum_a l_a r_a^T
//          with offset Pb, composed left to right
//          (A_t P = alpha p I + [alpha l_a + sum_j u~_j (v_j.l_a) | p u~_j][r_a | v_j]^T,
//          Pb <- A_t Pb + c_t) and re-compressed to m columns whenever it has
//          more: Y = L (R^T Omega), Q = modified Gram-Schmidt basis of Y's
//          columns (a column left with at most 1e-5 of its norm drops to zero),
//          L <- Q, R <- R (L^T Q);
//   carry  entry_{q+1} = P_q entry_q + Pb_q along each sequence's chunks;
//   replay the exact recurrence from each chunk's entry.
// Exact zeros stay zero, so a converged prefix (c_t = 0) stays exact through
// compressed carries: finite-step recovery holds.
//
// Work mapping: the fold and the replay run four chunks per wavefront, one per
// 16-lane DPP row.  Lane i of a row holds rows i, i + 16, ... of every
// D-vector (D <= 16 KD), so an inner product is KD local products plus four
// DPP steps within the row, and every lane of the row ends with the same bits
// (the additions pair lanes symmetrically); decisions that depend on an inner
// product (a zero secant, a Cholesky pivot, a dropped Gram-Schmidt column) are
// per-row selects.  The carry runs one sequence per block from LDS (see
// dplr_carry_kernel).
#include <algorithm>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kRows = 4;                   // chunks (or sequences) per wavefront
constexpr float kQrDrop = 1e-5f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}

// Sum over the 16 lanes of the lane's DPP row: neighbours, pairs of
// neighbours (quad_perm), quads (row_half_mirror), halves (row_mirror).  Each
// step adds two values that the partner lane adds in the other order, so all
// 16 lanes hold identical bits.
__device__ __forceinline__ float rsum(float v)
{
    v += dpp<0xB1>(v);          // quad_perm [1, 0, 3, 2]
    v += dpp<0x4E>(v);          // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);         // row_half_mirror
    v += dpp<0x140>(v);         // row_mirror
    return v;
}

template <int KD>
__device__ __forceinline__ float dot(const float (&x)[KD], const float (&y)[KD])
{
    float s = x[0] * y[0];
#pragma unroll
    for (int k = 1; k < KD; ++k) s += x[k] * y[k];
    return rsum(s);
}

// y = alpha x + sum_{j<n} u_j (v_j . x)
template <int MR, int KD>
__device__ __forceinline__ void dplr_apply(float alpha, const float (&u)[MR][KD], const float (&v)[MR][KD], int n,
                                           const float (&x)[KD], float (&y)[KD])
{
    float cf[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) cf[j] = (j < n) ? dot<KD>(v[j], x) : 0.0f;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        float acc = alpha * x[k];
#pragma unroll
        for (int j = 0; j < MR; ++j)
            if (j < n) acc += u[j][k] * cf[j];
        y[k] = acc;
    }
}

// Iteration-dependent view of the buffers (solver) or the fixed inputs (scan);
// wavefront-uniform.
struct StepView {
    const float *s_cur = nullptr, *s_prev = nullptr, *f_cur = nullptr, *f_prev = nullptr;
    float *s_next = nullptr;
    int i = 0;          // iteration index
    int n = 0;          // valid columns after this iteration's update
    bool update = false;
};

__device__ __forceinline__ bool step_view(const DplrArgs &a, StepView &v)
{
    if (!a.ctl) {                                   // standalone scan
        v.n = a.n_fixed;
        return true;
    }
    if (a.ctl->all_done) return false;
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

// Block update of one position (see the file header) for the lane's rows.
template <int MR, int KD, bool MS>
__device__ __forceinline__ void block_update(const DplrArgs &a, int i, const float (&ds)[KD], const float (&df)[KD],
                                             float (&u)[MR][KD], float (&v)[MR][KD], float (&fs)[MR][KD])
{
    const int m = a.m;
    const int slot = (i - 1) % m;
    if (!MS) {
        const int nb = min(i - 1, m);
        float cf[MR];
#pragma unroll
        for (int j = 0; j < MR; ++j) cf[j] = (j < nb && j != slot) ? dot<KD>(v[j], ds) : 0.0f;
        const float ss = dot<KD>(ds, ds);
        const bool ok = ss > 0.0f;
        const float inv = ok ? 1.0f / ss : 0.0f;
        // every element is written through a select: a store at the runtime slot
        // would turn the register arrays into an indexed stack array
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            float jds = a.alpha * ds[k];
#pragma unroll
            for (int j = 0; j < MR; ++j)
                if (j < nb && j != slot) jds += u[j][k] * cf[j];
            const float nu = (df[k] - jds) * inv, nv = ok ? ds[k] : 0.0f;
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                u[j][k] = (j == slot) ? nu : u[j][k];
                v[j][k] = (j == slot) ? nv : v[j][k];
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < MR; ++j)
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            v[j][k] = (j == slot) ? ds[k] : v[j][k];
            fs[j][k] = (j == slot) ? df[k] : fs[j][k];
        }
    const int n = min(i, m);
    float C[MR][MR];
    bool ok = true;
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int c = 0; c <= r; ++c) {
            C[r][c] = 1.0f;
            if (r >= n) continue;
            float acc = dot<KD>(v[r], v[c]) + (r == c ? a.lambda : 0.0f);
#pragma unroll
            for (int e = 0; e < c; ++e) acc -= C[r][e] * C[c][e];
            if (r == c) {
                const bool good = acc > 0.0f && !__builtin_isinf(acc);
                ok = ok && good;
                C[r][r] = good ? sqrtf(acc) : 1.0f;
            } else {
                C[r][c] = acc / C[c][c];
            }
        }
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        float y[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            y[r] = 0.0f;
            if (r >= n) continue;
            float acc = fs[r][k] - a.alpha * v[r][k];
#pragma unroll
            for (int e = 0; e < r; ++e) acc -= C[r][e] * y[e];
            y[r] = acc / C[r][r];
        }
#pragma unroll
        for (int r = MR - 1; r >= 0; --r) {
            if (r >= n) continue;
            float acc = y[r];
#pragma unroll
            for (int e = r + 1; e < MR; ++e)
                if (e < n) acc -= C[e][r] * y[e];
            y[r] = acc / C[r][r];
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) u[r][k] = (ok && r < n) ? y[r] : 0.0f;
    }
}

// ------------------------------------------------------------------ fold
template <int MR, int KD, bool MS>
__global__ __launch_bounds__(kThreads) void dplr_fold_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63, row4 = lane >> 4, li = lane & 15;
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const long long nch = static_cast<long long>(a.B) * a.nchunk;
    if (w * kRows >= nch) return;
    StepView sv;
    if (!step_view(a, sv)) return;
    const long long cid0 = w * kRows + row4;
    const bool rvalid = cid0 < nch;
    const long long cid = rvalid ? cid0 : nch - 1;  // rows past the end repeat the last chunk, store nothing
    const int bseq = static_cast<int>(cid / a.nchunk), q = static_cast<int>(cid % a.nchunk);
    const bool rlive = rvalid && !(a.ctl && a.skip && a.skip[bseq]);
    const int D = a.D, m = a.m, n = sv.n;
    const int t0 = q * a.chunk, t1 = min(t0 + a.chunk, a.T);
    const bool last = q == a.nchunk - 1;
    // does any row of the wavefront produce an aggregate (every chunk but a sequence's last)?
    bool wave_agg = false;
    for (int rr = 0; rr < kRows; ++rr) {
        const long long c2 = w * kRows + rr;
        wave_agg = wave_agg || (c2 < nch && c2 % a.nchunk != a.nchunk - 1);
    }
    if (!wave_agg && !sv.update) return;            // nothing to fold and no carry to produce
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    bool rowok[KD];
    int dd[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = li + 16 * k;
        rowok[k] = d < D;
        dd[k] = min(d, D - 1);
    }
    float om[MR][KD];
#pragma unroll
    for (int j = 0; j < MR; ++j)
#pragma unroll
        for (int k = 0; k < KD; ++k) om[j][k] = (rowok[k] && j < m) ? a.omega[dd[k] * m + j] : 0.0f;

    // branch-free loads from always-valid sources (an unused buffer stands in)
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_f = a.ctl ? sv.f_cur : a.c;
    const float *src_fp = a.ctl ? sv.f_prev : a.c;
    const float *src_sp = a.ctl ? sv.s_prev : a.c;
    const float *src_u = m > 0 ? a.U : src_s;
    const float *src_v = m > 0 ? a.V : src_s;
    const float *src_F = (m > 0 && MS) ? a.F : src_v;
    const int mm = max(m, 1);

    float p = 1.0f;
    int r = 0;
    float Pb[KD], PL[MR][KD], PR[MR][KD], s_before[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        Pb[k] = 0.0f;
        s_before[k] = 0.0f;
#pragma unroll
        for (int j = 0; j < MR; ++j) PL[j][k] = PR[j][k] = 0.0f;
    }
    if (a.ctl && sv.update && t0 > 0) {
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            const float v0 = src_s[(seq + t0 - 1) * D + dd[k]];
            s_before[k] = rowok[k] ? v0 : 0.0f;
        }
    }

    const int len = min(a.chunk, a.T);             // only a sequence's last chunk can be shorter
    for (int s = 0; s < len; ++s) {
        const int t = t0 + s;
        const bool ract = rlive && t < t1;
        const size_t pos = seq + min(t, a.T - 1);
        float u[MR][KD], v[MR][KD], fs[MR][KD], c[KD], sc[KD], ds[KD], df[KD];
#pragma unroll
        for (int k = 0; k < KD; ++k) {
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const size_t o = m > 0 ? (pos * m + min(j, mm - 1)) * D + dd[k] : pos * D + dd[k];
                const bool have = rowok[k] && j < m;
                const float uu = src_u[o], vv = src_v[o], ff = src_F[o];
                u[j][k] = have ? uu : 0.0f;
                v[j][k] = have ? vv : 0.0f;
                fs[j][k] = have ? ff : 0.0f;
            }
            const float s_ = src_s[pos * D + dd[k]], f_ = src_f[pos * D + dd[k]];
            const float fp_ = src_fp[pos * D + dd[k]];
            const float sp_ = src_sp[(pos - (t > 0 ? 1 : 0)) * D + dd[k]];
            sc[k] = rowok[k] ? s_ : 0.0f;
            c[k] = rowok[k] ? (a.ctl ? f_ - s_ : s_) : 0.0f;   // standalone: src_s is c
            ds[k] = (rowok[k] && t > 0) ? s_before[k] - sp_ : 0.0f;
            df[k] = rowok[k] ? f_ - fp_ : 0.0f;
        }
        if (a.ctl && sv.update) {
            block_update<MR, KD, MS>(a, sv.i, ds, df, u, v, fs);
            if (ract) {
                // the slot's column is picked by selects (a runtime index into the
                // register arrays would move them to the stack)
                const int slot = (sv.i - 1) % m;
                const size_t so = (pos * m + slot) * D + li;
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    if (!rowok[k]) continue;
                    float su = 0.0f, sv_ = 0.0f, sf = 0.0f;
#pragma unroll
                    for (int j = 0; j < MR; ++j) {
                        su = (j == slot) ? u[j][k] : su;
                        sv_ = (j == slot) ? v[j][k] : sv_;
                        sf = (j == slot) ? fs[j][k] : sf;
                    }
                    a.V[so + 16 * k] = sv_;
                    if (MS) {
                        a.F[so + 16 * k] = sf;
#pragma unroll
                        for (int j = 0; j < MR; ++j)
                            if (j < m) a.U[(pos * m + j) * D + li + 16 * k] = u[j][k];
                    } else {
                        a.U[so + 16 * k] = su;
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KD; ++k) s_before[k] = sc[k];
        }
        if (!wave_agg) continue;                    // the rows' last chunks only update their blocks
#pragma unroll
        for (int j = 0; j < MR; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) u[j][k] *= a.shrink;

        // A_t P: the r aggregate columns, then the n block columns
        float Lf[2 * MR][KD], Rf[2 * MR][KD];
#pragma unroll
        for (int e = 0; e < MR; ++e) {
            float y[KD];
            dplr_apply<MR, KD>(a.alpha, u, v, n, PL[e], y);
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                Lf[e][k] = (e < r) ? y[k] : 0.0f;
                Rf[e][k] = (e < r) ? PR[e][k] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < MR; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                Lf[MR + j][k] = p * u[j][k];
                Rf[MR + j][k] = v[j][k];
            }
        auto col_ok = [&](int e) { return e < MR ? e < r : (e - MR) < n; };
        const int K = r + n;
        p = a.alpha * p;
        if (K <= m) {
            // column j of the result: aggregate column j for j < r, else block column j - r
            // (selects on uniform conditions; no runtime array index)
#pragma unroll
            for (int j = 0; j < MR; ++j)
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    float nl = (j < r) ? Lf[j][k] : 0.0f, nr = (j < r) ? Rf[j][k] : 0.0f;
#pragma unroll
                    for (int jj = 0; jj <= j; ++jj) {
                        const bool pick = j - r == jj && jj < n;
                        nl = pick ? Lf[MR + jj][k] : nl;
                        nr = pick ? Rf[MR + jj][k] : nr;
                    }
                    PL[j][k] = nl;
                    PR[j][k] = nr;
                }
            r = K;
        } else {
            // Y = L (R^T Omega), then modified Gram-Schmidt
            float Q[MR][KD];
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                if (j >= m) {
#pragma unroll
                    for (int k = 0; k < KD; ++k) Q[j][k] = 0.0f;
                    continue;
                }
                float y[KD];
#pragma unroll
                for (int k = 0; k < KD; ++k) y[k] = 0.0f;
                float rto[2 * MR];
#pragma unroll
                for (int e = 0; e < 2 * MR; ++e) rto[e] = col_ok(e) ? dot<KD>(Rf[e], om[j]) : 0.0f;
#pragma unroll
                for (int e = 0; e < 2 * MR; ++e)
                    if (col_ok(e))
#pragma unroll
                        for (int k = 0; k < KD; ++k) y[k] += Lf[e][k] * rto[e];
                const float ny2 = dot<KD>(y, y);
#pragma unroll
                for (int l = 0; l < MR; ++l)
                    if (l < j) {
                        const float cf = dot<KD>(Q[l], y);
#pragma unroll
                        for (int k = 0; k < KD; ++k) y[k] -= cf * Q[l][k];
                    }
                // kept iff |y| > kQrDrop |y before orthogonalisation| (compared as squares)
                const float nq2 = dot<KD>(y, y);
                const bool keep = nq2 > (kQrDrop * kQrDrop) * ny2;
                const float inq = 1.0f / sqrtf(nq2);
#pragma unroll
                for (int k = 0; k < KD; ++k) Q[j][k] = keep ? y[k] * inq : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                float lq[2 * MR];
#pragma unroll
                for (int e = 0; e < 2 * MR; ++e) lq[e] = (j < m && col_ok(e)) ? dot<KD>(Lf[e], Q[j]) : 0.0f;
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    float rr = 0.0f;
#pragma unroll
                    for (int e = 0; e < 2 * MR; ++e)
                        if (j < m && col_ok(e)) rr += Rf[e][k] * lq[e];
                    PL[j][k] = Q[j][k];
                    PR[j][k] = rr;
                }
            }
            r = m;
        }
        float nb[KD];
        dplr_apply<MR, KD>(a.alpha, u, v, n, Pb, nb);
#pragma unroll
        for (int k = 0; k < KD; ++k) Pb[k] = nb[k] + c[k];
    }
    if (last || !rlive) return;
    const int Dp = dplr_padded_dim(D);
    float *rec = a.agg + static_cast<size_t>(cid) * dplr_record_floats(m, D);
    if (li == 0) {
        rec[(2 * m + 1) * Dp] = p;
        reinterpret_cast<int *>(rec)[(2 * m + 1) * Dp + 1] = r;
    }
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        if (!rowok[k]) continue;
        const int d = li + 16 * k;
#pragma unroll
        for (int j = 0; j < MR; ++j)
            if (j < m) {
                rec[j * Dp + d] = PL[j][k];
                rec[(m + j) * Dp + d] = PR[j][k];
            }
        rec[2 * m * Dp + d] = Pb[k];
    }
}

// ------------------------------------------------------------------ carry
constexpr int kCarryLdsBytes = 64 * 1024;          // both batch buffers
inline int carry_batch(int m, int D, int nchunk)
{
    const int fit = kCarryLdsBytes / (2 * 4 * dplr_record_floats(m, D));
    return std::max(1, std::min(std::max(nchunk - 1, 1), fit));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// KD consecutive floats from LDS (one ds_read of 4, 8 or 16 bytes; p is KD-aligned)
template <int KD>
__device__ __forceinline__ void lds_vec(const float *p, float (&o)[KD])
{
    if constexpr (KD == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (KD == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
        o[0] = *p;
    }
}

// One chunk record of the chain, as wavefront 0 reads it from LDS.
template <int MR, int KD>
struct CarryRec {
    float L[MR][KD], R[MR][KD], b[KD];
    float p;
    int r;
};

// One block per sequence.  The chain over the chunk aggregates is serial, so
// wavefront 0 runs it from LDS while wavefronts 1-3 copy the next batch of
// records (one contiguous span, all loads of a thread in flight together)
// into the other buffer.  In wavefront 0 lane i of a DPP row holds rows
// KD i .. KD i + KD - 1 (one vector LDS read per vector and record); all four
// rows run the same chain and row 0 stores the entries.  Records are read one
// step ahead of their use.
template <int MR, int KD>
__global__ __launch_bounds__(kThreads) void dplr_carry_kernel(DplrArgs a, int nb)
{
    extern __shared__ float carry_lds[];
    const int bseq = blockIdx.x;
    StepView sv;
    if (!step_view(a, sv)) return;
    if (a.ctl && a.skip && a.skip[bseq]) return;
    const int D = a.D, m = a.m, Dp = dplr_padded_dim(D);
    const int RS = dplr_record_floats(m, D);          // a multiple of 4
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, row4 = lane >> 4, li = lane & 15;
    const size_t base = static_cast<size_t>(bseq) * a.nchunk;
    const int nq = a.nchunk - 1;                      // aggregates in the chain
    const int nbatch = (nq + nb - 1) / nb;
    const int stride = nb * RS;
    auto stage = [&](int kb, int tid, int nthr) {
        const int q0 = kb * nb, n4 = min(nb, nq - q0) * RS / 4;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(a.agg + (base + q0) * RS);
        f32x4 *dst = reinterpret_cast<f32x4 *>(carry_lds + (kb & 1) * stride);
        for (int i0 = tid; i0 < n4; i0 += 16 * nthr) {
            f32x4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = src[min(i0 + u * nthr, n4 - 1)];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (i0 + u * nthr < n4) dst[i0 + u * nthr] = v[u];
        }
    };
    if (nbatch > 0) stage(0, threadIdx.x, kThreads);
    __syncthreads();

    // lane rows: d = KD li + k; lanes past the padded width read the last vector slot
    const int d0 = KD * li;
    const int ro = min(d0, Dp - KD);
    bool rowok[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) rowok[k] = d0 + k < D;
    const int mm1 = max(m - 1, 0);
    auto read_rec = [&](const float *rec, CarryRec<MR, KD> &c) {
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const int jj = min(j, mm1);
            lds_vec<KD>(rec + jj * Dp + ro, c.L[j]);
            lds_vec<KD>(rec + (m + jj) * Dp + ro, c.R[j]);
        }
        lds_vec<KD>(rec + 2 * m * Dp + ro, c.b);
        c.p = rec[(2 * m + 1) * Dp];
        c.r = reinterpret_cast<const int *>(rec)[(2 * m + 1) * Dp + 1];
    };
    const bool storer = wave == 0 && row4 == 0;
    float e[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) e[k] = 0.0f;
    for (int kb = 0; kb < nbatch; ++kb) {
        if (wave != 0) {
            if (kb + 1 < nbatch) stage(kb + 1, threadIdx.x - 64, kThreads - 64);
        } else {
            const float *buf = carry_lds + (kb & 1) * stride;
            const int q0 = kb * nb, cnt = min(nb, nq - q0);
            CarryRec<MR, KD> cur;
            read_rec(buf, cur);
            for (int qi = 0; qi < cnt; ++qi) {
                CarryRec<MR, KD> nxt;
                read_rec(buf + min(qi + 1, cnt - 1) * RS, nxt);
                if (storer)
#pragma unroll
                    for (int k = 0; k < KD; ++k)
                        if (rowok[k]) a.entry[(base + q0 + qi) * D + d0 + k] = e[k];
                const int rk = __builtin_amdgcn_readfirstlane(cur.r);
                float cf[MR];
#pragma unroll
                for (int j = 0; j < MR; ++j) {
                    float rj[KD];
#pragma unroll
                    for (int k = 0; k < KD; ++k) rj[k] = (rowok[k] && j < rk) ? cur.R[j][k] : 0.0f;
                    cf[j] = dot<KD>(rj, e);
                }
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    float ne = cur.p * e[k];
#pragma unroll
                    for (int j = 0; j < MR; ++j) ne += (j < rk) ? cur.L[j][k] * cf[j] : 0.0f;
                    e[k] = rowok[k] ? ne + cur.b[k] : 0.0f;
                }
                cur = nxt;
            }
        }
        __syncthreads();
    }
    if (storer)
#pragma unroll
        for (int k = 0; k < KD; ++k)
            if (rowok[k]) a.entry[(base + nq) * D + d0 + k] = e[k];
}

// ------------------------------------------------------------------ replay
template <int MR, int KD>
__global__ __launch_bounds__(kThreads) void dplr_replay_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63, row4 = lane >> 4, li = lane & 15;
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const long long nch = static_cast<long long>(a.B) * a.nchunk;
    if (w * kRows >= nch) return;
    StepView sv;
    if (!step_view(a, sv)) return;
    const long long cid0 = w * kRows + row4;
    const bool rvalid = cid0 < nch;
    const long long cid = rvalid ? cid0 : nch - 1;
    const int bseq = static_cast<int>(cid / a.nchunk), q = static_cast<int>(cid % a.nchunk);
    const bool rlive = rvalid && !(a.ctl && a.skip && a.skip[bseq]);
    const int D = a.D, m = a.m, n = sv.n;
    const int t0 = q * a.chunk, t1 = min(t0 + a.chunk, a.T);
    const size_t seq = static_cast<size_t>(bseq) * a.T;
    bool rowok[KD];
    int dd[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = li + 16 * k;
        rowok[k] = d < D;
        dd[k] = min(d, D - 1);
    }
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_c = a.ctl ? sv.f_cur : a.c;
    const float *src_u = n > 0 ? a.U : src_s;
    const float *src_v = n > 0 ? a.V : src_s;
    const int nn = max(n, 1);
    float dl[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const float e0 = a.entry[cid * D + dd[k]];
        dl[k] = rowok[k] ? e0 : 0.0f;
    }
    const int len = min(a.chunk, a.T);
    for (int s = 0; s < len; ++s) {
        const int t = t0 + s;
        const bool ract = rlive && t < t1;
        const size_t pos = seq + min(t, a.T - 1);
        float u[MR][KD], v[MR][KD], c[KD], sc[KD];
#pragma unroll
        for (int k = 0; k < KD; ++k) {
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const size_t o = n > 0 ? (pos * m + min(j, nn - 1)) * D + dd[k] : pos * D + dd[k];
                const bool have = rowok[k] && j < n;
                const float uu = src_u[o], vv = src_v[o];
                u[j][k] = have ? uu * a.shrink : 0.0f;
                v[j][k] = have ? vv : 0.0f;
            }
            const float s_ = src_s[pos * D + dd[k]], c_ = src_c[pos * D + dd[k]];
            sc[k] = rowok[k] ? s_ : 0.0f;
            c[k] = rowok[k] ? (a.ctl ? c_ - s_ : c_) : 0.0f;
        }
        float y[KD];
        dplr_apply<MR, KD>(a.alpha, u, v, n, dl, y);
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            dl[k] = y[k] + c[k];
            if (ract && rowok[k]) {
                const size_t o = pos * D + li + 16 * k;
                if (a.ctl) sv.s_next[o] = sc[k] + dl[k];
                else a.out[o] = dl[k];
            }
        }
    }
}

template <int MR, int KD>
int launch_dplr(const DplrArgs &a, hipStream_t stream)
{
    const long long chunks = static_cast<long long>(a.B) * a.nchunk;
    const long long wc = (chunks + kRows - 1) / kRows;
    const unsigned gc = static_cast<unsigned>((wc + kWavesPerBlock - 1) / kWavesPerBlock);
    if (a.multisecant) DEER_LAUNCH((dplr_fold_kernel<MR, KD, true>), dim3(gc), dim3(kThreads), 0, stream, a);
    else DEER_LAUNCH((dplr_fold_kernel<MR, KD, false>), dim3(gc), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    const int nb = carry_batch(a.m, a.D, a.nchunk);
    const size_t lds = 2 * sizeof(float) * static_cast<size_t>(nb) * dplr_record_floats(a.m, a.D);
    DEER_LAUNCH((dplr_carry_kernel<MR, KD>), dim3(a.B), dim3(kThreads), lds, stream, a, nb);
    DEER_HIP(hipGetLastError());
    DEER_LAUNCH((dplr_replay_kernel<MR, KD>), dim3(gc), dim3(kThreads), 0, stream, a);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

template <int MR>
int launch_dplr_mr(const DplrArgs &a, hipStream_t stream)
{
    if (a.D <= 16) return launch_dplr<MR, 1>(a, stream);
    if (a.D <= 32) return launch_dplr<MR, 2>(a, stream);
    return launch_dplr<MR, 4>(a, stream);
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
