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
#include <type_traits>

#include "internal.h"

namespace deer {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kRows = 4;                   // chunks (or sequences) per wavefront
constexpr float kQrDrop = 1e-5f;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ void block_update(const DplrArgs &a, int m, int i, const float (&ds)[KD],
                                             const float (&df)[KD], float (&u)[MR][KD], float (&v)[MR][KD],
                                             float (&fs)[MR][KD])
{
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
// A load from a wavefront-uniform base plus a 32-bit lane byte offset (the
// global_load form with a scalar base: no 64-bit address arithmetic per load).
__device__ __forceinline__ float ldu(const float *base, unsigned off)
{
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + off);
}

// KD consecutive floats from a uniform base plus a lane byte offset (one
// 4-, 8- or 16-byte load; the offset is KD-float aligned).
template <int KD>
__device__ __forceinline__ void ldv(const float *base, unsigned off, float (&o)[KD])
{
    const char *p = reinterpret_cast<const char *>(base) + off;
    if constexpr (KD == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (KD == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
        o[0] = *reinterpret_cast<const float *>(p);
    }
}

// Lane rows: with D = 16 KD (FULL) lane i of a DPP row holds the KD
// consecutive rows KD i .. KD i + KD - 1 (vector loads, no row masks);
// otherwise rows i, i + 16, ... with rows past D masked.
template <int KD, bool FULL>
__device__ __forceinline__ int lane_row(int li, int k)
{
    return FULL ? KD * li + k : li + 16 * k;
}

// Inputs of one position for the lane's rows, as loaded (masked when used).
template <int MR, int KD>
struct FoldIn {
    float u[MR][KD], v[MR][KD], fs[MR][KD];
    float s[KD], f[KD], fp[KD], sp[KD];
};

// Positions are processed in two loops: a general one while the aggregate
// holds fewer than m columns (or fewer than m block columns exist yet), then,
// when r = n = m = MR, one whose column counts are compile-time constants
// (every step then re-compresses 2m columns to m).
template <int MR, int KD, bool MS, bool FULL>
__global__ __launch_bounds__(kThreads) void dplr_fold_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63, row4 = lane >> 4, li = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + wv;
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
    unsigned ddb[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = lane_row<KD, FULL>(li, k);
        rowok[k] = FULL || d < D;
        dd[k] = FULL ? d : min(d, D - 1);
        ddb[k] = 4u * dd[k];
    }
    float om[MR][KD];
#pragma unroll
    for (int j = 0; j < MR; ++j)
#pragma unroll
        for (int k = 0; k < KD; ++k) om[j][k] = (rowok[k] && j < m) ? a.omega[dd[k] * m + j] : 0.0f;

    // Addressing: position index P = b T + t.  The wavefront's four chunks are
    // consecutive, so every row's positions lie within 4 chunk lengths of the
    // first row's first position P0; bases are uniform, lane offsets 32-bit.
    // Loads are branch-free from always-valid sources (an unused buffer stands in).
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_f = a.ctl ? sv.f_cur : a.c;
    const float *src_fp = a.ctl ? sv.f_prev : a.c;
    const float *src_sp = a.ctl ? sv.s_prev : a.c;
    const float *src_u = m > 0 ? a.U : src_s;
    const float *src_v = m > 0 ? a.V : src_s;
    const float *src_F = (m > 0 && MS) ? a.F : src_v;
    const int mm = max(m, 1);
    const long long cw = w * kRows;
    const size_t P0 = static_cast<size_t>(cw / a.nchunk) * a.T + static_cast<size_t>(cw % a.nchunk) * a.chunk;
    const int sh = P0 > 0 ? 1 : 0;                 // s^(i-1)_{t-1} may sit one position before P0
    const int rel0 = static_cast<int>(seq + t0 - P0), relmax = static_cast<int>(seq + a.T - 1 - P0);
    const float *bs = src_s + P0 * D, *bf = src_f + P0 * D, *bfp = src_fp + P0 * D;
    const float *bsp = src_sp + (P0 - sh) * D;
    const float *bu[MR], *bv[MR], *bF[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) {
        const size_t o = (P0 * m + min(j, mm - 1)) * D;
        bu[j] = src_u + o;
        bv[j] = src_v + o;
        bF[j] = src_F + o;
    }
    auto load = [&](int s, FoldIn<MR, KD> &in) {
        // position clamped to the sequence; s^(i-1) one position earlier unless it is t = 0
        const int relc = min(rel0 + s, relmax);
        const int tc = t0 + (relc - rel0);
        const unsigned osd = 4u * static_cast<unsigned>(relc * D);
        const unsigned osp = 4u * static_cast<unsigned>((relc + sh - (tc > 0 ? 1 : 0)) * D);
        const unsigned ouv = 4u * static_cast<unsigned>(relc * m * D);
        if constexpr (FULL) {
            ldv<KD>(bs, osd + ddb[0], in.s);
            ldv<KD>(bf, osd + ddb[0], in.f);
            ldv<KD>(bfp, osd + ddb[0], in.fp);
            ldv<KD>(bsp, osp + ddb[0], in.sp);
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                ldv<KD>(bu[j], ouv + ddb[0], in.u[j]);
                ldv<KD>(bv[j], ouv + ddb[0], in.v[j]);
                if constexpr (MS) ldv<KD>(bF[j], ouv + ddb[0], in.fs[j]);
                else
#pragma unroll
                    for (int k = 0; k < KD; ++k) in.fs[j][k] = 0.0f;
            }
        } else {
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                in.s[k] = ldu(bs, osd + ddb[k]);
                in.f[k] = ldu(bf, osd + ddb[k]);
                in.fp[k] = ldu(bfp, osd + ddb[k]);
                in.sp[k] = ldu(bsp, osp + ddb[k]);
#pragma unroll
                for (int j = 0; j < MR; ++j) {
                    in.u[j][k] = ldu(bu[j], ouv + ddb[k]);
                    in.v[j][k] = ldu(bv[j], ouv + ddb[k]);
                    in.fs[j][k] = MS ? ldu(bF[j], ouv + ddb[k]) : 0.0f;
                }
            }
        }
    };

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

    // one position; STEADY: r = n = m = MR known at compile time
    auto step = [&](auto steady, const FoldIn<MR, KD> &in, int s) {
        constexpr bool S = decltype(steady)::value;
        const int n_ = S ? MR : n, m_ = S ? MR : m;
        const int t = t0 + s;
        const bool ract = rlive && t < t1;
        float u[MR][KD], v[MR][KD], fs[MR][KD], c[KD], sc[KD], ds[KD], df[KD];
#pragma unroll
        for (int k = 0; k < KD; ++k) {
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const bool have = rowok[k] && j < m_;
                u[j][k] = have ? in.u[j][k] : 0.0f;
                v[j][k] = have ? in.v[j][k] : 0.0f;
                fs[j][k] = have ? in.fs[j][k] : 0.0f;
            }
            sc[k] = rowok[k] ? in.s[k] : 0.0f;
            c[k] = rowok[k] ? (a.ctl ? in.f[k] - in.s[k] : in.s[k]) : 0.0f;   // standalone: src_s is c
            ds[k] = (rowok[k] && t > 0) ? s_before[k] - in.sp[k] : 0.0f;
            df[k] = rowok[k] ? in.f[k] - in.fp[k] : 0.0f;
        }
        if (a.ctl && sv.update) {
            block_update<MR, KD, MS>(a, m_, sv.i, ds, df, u, v, fs);
            if (ract) {
                // the slot's column is picked by selects (a runtime index into the
                // register arrays would move them to the stack)
                const int slot = (sv.i - 1) % m_;
                const size_t pos = seq + t;
                const size_t so = (pos * m_ + slot) * D;
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
                    a.V[so + dd[k]] = sv_;
                    if (MS) {
                        a.F[so + dd[k]] = sf;
#pragma unroll
                        for (int j = 0; j < MR; ++j)
                            if (j < m_) a.U[(pos * m_ + j) * D + dd[k]] = u[j][k];
                    } else {
                        a.U[so + dd[k]] = su;
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KD; ++k) s_before[k] = sc[k];
        }
        if (!wave_agg) return;                      // the rows' last chunks only update their blocks
#pragma unroll
        for (int j = 0; j < MR; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) u[j][k] *= a.shrink;

        // A_t P: the r aggregate columns, then the n block columns
        const int r_ = S ? MR : r;
        float Lf[2 * MR][KD], Rf[2 * MR][KD];
#pragma unroll
        for (int e = 0; e < MR; ++e) {
            float y[KD];
            dplr_apply<MR, KD>(a.alpha, u, v, n_, PL[e], y);
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                Lf[e][k] = (e < r_) ? y[k] : 0.0f;
                Rf[e][k] = (e < r_) ? PR[e][k] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < MR; ++j)
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                Lf[MR + j][k] = p * u[j][k];
                Rf[MR + j][k] = v[j][k];
            }
        auto col_ok = [&](int e) { return e < MR ? e < r_ : (e - MR) < n_; };
        const int K = r_ + n_;
        p = a.alpha * p;
        if (!S && K <= m) {
            // column j of the result: aggregate column j for j < r, else block column j - r
            // (selects on uniform conditions; no runtime array index)
#pragma unroll
            for (int j = 0; j < MR; ++j)
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    float nl = (j < r_) ? Lf[j][k] : 0.0f, nr = (j < r_) ? Rf[j][k] : 0.0f;
#pragma unroll
                    for (int jj = 0; jj <= j; ++jj) {
                        const bool pick = j - r_ == jj && jj < n_;
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
                if (j >= m_) {
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
                for (int e = 0; e < 2 * MR; ++e) lq[e] = (j < m_ && col_ok(e)) ? dot<KD>(Lf[e], Q[j]) : 0.0f;
#pragma unroll
                for (int k = 0; k < KD; ++k) {
                    float rr = 0.0f;
#pragma unroll
                    for (int e = 0; e < 2 * MR; ++e)
                        if (j < m_ && col_ok(e)) rr += Rf[e][k] * lq[e];
                    PL[j][k] = Q[j][k];
                    PR[j][k] = rr;
                }
            }
            r = m_;
        }
        float nb[KD];
        dplr_apply<MR, KD>(a.alpha, u, v, n_, Pb, nb);
#pragma unroll
        for (int k = 0; k < KD; ++k) Pb[k] = nb[k] + c[k];
    };

    const int len = min(a.chunk, a.T);             // only a sequence's last chunk can be shorter
    const bool steady_ok = n == MR && m == MR;
    FoldIn<MR, KD> cur;
    load(0, cur);
    int s = 0;
    for (; s < len && !(steady_ok && r == MR); ++s) {
        FoldIn<MR, KD> nxt;
        load(s + 1, nxt);                           // clamped past the chunk: a harmless extra load
        step(std::false_type{}, cur, s);
        cur = nxt;
    }
    for (; s < len; ++s) {                          // reached only with steady_ok and r = MR
        FoldIn<MR, KD> nxt;
        load(s + 1, nxt);
        step(std::true_type{}, cur, s);
        cur = nxt;
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
        const int d = dd[k];
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
struct ReplayIn {
    float u[MR][KD], v[MR][KD], s[KD], c[KD];
};

// Four chunks per wavefront replay the exact recurrence from their entries.
// The addressing is the fold's (uniform bases, 32-bit lane offsets); the
// inputs of positions s + 1 and s + 2 are in flight while position s runs.
template <int MR, int KD, bool FULL>
__global__ __launch_bounds__(kThreads) void dplr_replay_kernel(DplrArgs a)
{
    const int lane = threadIdx.x & 63, row4 = lane >> 4, li = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long w = static_cast<long long>(blockIdx.x) * kWavesPerBlock + wv;
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
    unsigned ddb[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = lane_row<KD, FULL>(li, k);
        rowok[k] = FULL || d < D;
        dd[k] = FULL ? d : min(d, D - 1);
        ddb[k] = 4u * dd[k];
    }
    const float *src_s = a.ctl ? sv.s_cur : a.c;
    const float *src_c = a.ctl ? sv.f_cur : a.c;
    const float *src_u = n > 0 ? a.U : src_s;
    const float *src_v = n > 0 ? a.V : src_s;
    const int mu = n > 0 ? m : 0;                  // column stride of the U/V stand-in
    const int nn = max(n, 1);
    const long long cw = w * kRows;
    const size_t P0 = static_cast<size_t>(cw / a.nchunk) * a.T + static_cast<size_t>(cw % a.nchunk) * a.chunk;
    const int rel0 = static_cast<int>(seq + t0 - P0), relmax = static_cast<int>(seq + a.T - 1 - P0);
    const float *bs = src_s + P0 * D, *bc = src_c + P0 * D;
    const float *bu[MR], *bv[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) {
        const size_t o = (P0 * mu + (n > 0 ? min(j, nn - 1) : 0)) * D;
        bu[j] = src_u + o;
        bv[j] = src_v + o;
    }
    auto load = [&](int s, ReplayIn<MR, KD> &in) {
        const int relc = min(rel0 + s, relmax);
        const unsigned osd = 4u * static_cast<unsigned>(relc * D);
        const unsigned ouv = 4u * static_cast<unsigned>(relc * mu * D);
        if constexpr (FULL) {
            ldv<KD>(bs, osd + ddb[0], in.s);
            ldv<KD>(bc, osd + ddb[0], in.c);
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                ldv<KD>(bu[j], ouv + ddb[0], in.u[j]);
                ldv<KD>(bv[j], ouv + ddb[0], in.v[j]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                in.s[k] = ldu(bs, osd + ddb[k]);
                in.c[k] = ldu(bc, osd + ddb[k]);
#pragma unroll
                for (int j = 0; j < MR; ++j) {
                    in.u[j][k] = ldu(bu[j], ouv + ddb[k]);
                    in.v[j][k] = ldu(bv[j], ouv + ddb[k]);
                }
            }
        }
    };
    float dl[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const float e0 = a.entry[cid * D + dd[k]];
        dl[k] = rowok[k] ? e0 : 0.0f;
    }
    const int len = min(a.chunk, a.T);
    ReplayIn<MR, KD> in0, in1;
    load(0, in0);
    load(1, in1);
    for (int s = 0; s < len; ++s) {
        ReplayIn<MR, KD> in2;
        load(s + 2, in2);                           // clamped past the chunk: harmless extra loads
        const int t = t0 + s;
        const bool ract = rlive && t < t1;
        const size_t pos = seq + min(t, a.T - 1);
        float u[MR][KD], v[MR][KD], c[KD], sc[KD];
#pragma unroll
        for (int k = 0; k < KD; ++k) {
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const bool have = rowok[k] && j < n;
                u[j][k] = have ? in0.u[j][k] * a.shrink : 0.0f;
                v[j][k] = have ? in0.v[j][k] : 0.0f;
            }
            sc[k] = rowok[k] ? in0.s[k] : 0.0f;
            c[k] = rowok[k] ? (a.ctl ? in0.c[k] - in0.s[k] : in0.c[k]) : 0.0f;
        }
        float y[KD];
        dplr_apply<MR, KD>(a.alpha, u, v, n, dl, y);
#pragma unroll
        for (int k = 0; k < KD; ++k) {
            dl[k] = y[k] + c[k];
            if (ract && rowok[k]) {
                const size_t o = pos * D + dd[k];
                if (a.ctl) sv.s_next[o] = sc[k] + dl[k];
                else a.out[o] = dl[k];
            }
        }
        in0 = in1;
        in1 = in2;
    }
}

template <int MR, int KD>
int launch_dplr(const DplrArgs &a, hipStream_t stream)
{
    const long long chunks = static_cast<long long>(a.B) * a.nchunk;
    const long long wc = (chunks + kRows - 1) / kRows;
    const unsigned gc = static_cast<unsigned>((wc + kWavesPerBlock - 1) / kWavesPerBlock);
    const bool full = a.D == 16 * KD;
    if (a.multisecant) {
        if (full) DEER_LAUNCH((dplr_fold_kernel<MR, KD, true, true>), dim3(gc), dim3(kThreads), 0, stream, a);
        else DEER_LAUNCH((dplr_fold_kernel<MR, KD, true, false>), dim3(gc), dim3(kThreads), 0, stream, a);
    } else {
        if (full) DEER_LAUNCH((dplr_fold_kernel<MR, KD, false, true>), dim3(gc), dim3(kThreads), 0, stream, a);
        else DEER_LAUNCH((dplr_fold_kernel<MR, KD, false, false>), dim3(gc), dim3(kThreads), 0, stream, a);
    }
    DEER_HIP(hipGetLastError());
    const int nb = carry_batch(a.m, a.D, a.nchunk);
    const size_t lds = 2 * sizeof(float) * static_cast<size_t>(nb) * dplr_record_floats(a.m, a.D);
    DEER_LAUNCH((dplr_carry_kernel<MR, KD>), dim3(a.B), dim3(kThreads), lds, stream, a, nb);
    DEER_HIP(hipGetLastError());
    if (full) DEER_LAUNCH((dplr_replay_kernel<MR, KD, true>), dim3(gc), dim3(kThreads), 0, stream, a);
    else DEER_LAUNCH((dplr_replay_kernel<MR, KD, false>), dim3(gc), dim3(kThreads), 0, stream, a);
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
