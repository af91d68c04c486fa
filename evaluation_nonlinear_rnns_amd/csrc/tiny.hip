// Whole-solve kernel for small tanh problems ("Parallel Broyden Methods",
// section 2: the Newton / diagonal quasi-Newton iteration; merge rule of
// appendix C.2).  When the state is tiny (D <= 4) and a sequence fits one
// workgroup (T <= 256 P), launch and polling latency dominate the multi-launch
// loop; here one workgroup per sequence runs every iteration on chip: the
// evaluation of f and of the block A_t at the thread's P positions, the
// residual test, and the linear step as an inclusive scan of the threads'
// affine maps (each thread composes its P positions, then a Hillis-Steele scan
// over the 256 thread maps in LDS), so a whole solve is one launch.  Arithmetic
// and the stopping rule are those of the multi-launch path: f = tanh(W s + p)
// with ROCm's tanhf, d = 1 - f^2, dense A_t = shrink d W, diagonal and
// Jacobi / Picard blocks from the same linearisation, b_t = f_t - A_t s_{t-1};
// a sequence stops when max |s_t - f_t| <= tol (NaN never passes) or at
// max_iter.  The input projection is formed in the same launch.
#include "internal.h"

namespace deer {
namespace {

constexpr int kTinyThreads = 256;
constexpr int kTinyD = 4;                         // state rows held per map (D <= 4)

// x -> A x + b on the padded 4-vector
struct Aff {
    float A[kTinyD][kTinyD];
    float b[kTinyD];
};

__device__ __forceinline__ void set_identity(Aff &m)
{
#pragma unroll
    for (int i = 0; i < kTinyD; ++i) {
        m.b[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < kTinyD; ++j) m.A[i][j] = (i == j) ? 1.0f : 0.0f;
    }
}

// out = later o earlier: A = A_l A_e, b = A_l b_e + b_l (the later map on the left)
__device__ __forceinline__ Aff compose(const Aff &l, const Aff &e)
{
    Aff o;
#pragma unroll
    for (int i = 0; i < kTinyD; ++i) {
        float bi = l.b[i];
#pragma unroll
        for (int k = 0; k < kTinyD; ++k) bi = __builtin_fmaf(l.A[i][k], e.b[k], bi);
        o.b[i] = bi;
#pragma unroll
        for (int j = 0; j < kTinyD; ++j) {
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < kTinyD; ++k) a = __builtin_fmaf(l.A[i][k], e.A[k][j], a);
            o.A[i][j] = a;
        }
    }
    return o;
}

__device__ __forceinline__ void store_aff(float *dst, const Aff &m)
{
#pragma unroll
    for (int i = 0; i < kTinyD; ++i) {
#pragma unroll
        for (int j = 0; j < kTinyD; ++j) dst[i * kTinyD + j] = m.A[i][j];
        dst[kTinyD * kTinyD + i] = m.b[i];
    }
}

__device__ __forceinline__ Aff load_aff(const float *src)
{
    Aff m;
#pragma unroll
    for (int i = 0; i < kTinyD; ++i) {
#pragma unroll
        for (int j = 0; j < kTinyD; ++j) m.A[i][j] = src[i * kTinyD + j];
        m.b[i] = src[kTinyD * kTinyD + i];
    }
    return m;
}

constexpr int kAffWords = kTinyD * kTinyD + kTinyD;

// One workgroup per sequence; thread k owns positions k P .. k P + P - 1.
// The input projection p_t = U x_t + b is formed here too, and the results
// go straight to the caller's host-visible words (one per sequence each).
template <int P>
__global__ __launch_bounds__(kTinyThreads) void tiny_solve_kernel(const float *__restrict__ W,
                                                                  const float *__restrict__ U,
                                                                  const float *__restrict__ bias,
                                                                  const float *__restrict__ x, int M,
                                                                  const float *__restrict__ s0,
                                                                  const float *init, float *traj, int T, int D,
                                                                  int dense, Linearization lz, float tol,
                                                                  int max_iter, int stall_window, int *iters,
                                                                  int *status, float *resid)
{
    __shared__ float S[kTinyThreads * P * kTinyD];   // the iterate s^(i), rows padded to 4
    __shared__ float agg[kTinyThreads * kAffWords];  // inclusive prefixes of the thread maps
    __shared__ unsigned red[kTinyThreads / 64];
    __shared__ unsigned fred[kTinyThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x;
    const size_t seq = static_cast<size_t>(b) * T;

    float w[kTinyD][kTinyD], x0[kTinyD];
#pragma unroll
    for (int i = 0; i < kTinyD; ++i) {
        x0[i] = (s0 && i < D) ? s0[static_cast<size_t>(b) * D + i] : 0.0f;
#pragma unroll
        for (int j = 0; j < kTinyD; ++j) w[i][j] = (i < D && j < D) ? W[i * D + j] : 0.0f;
    }
    for (int e = tid; e < T * kTinyD; e += kTinyThreads) {
        const int t = e / kTinyD, i = e % kTinyD;
        S[e] = (init && i < D) ? init[(seq + t) * D + i] : 0.0f;
    }
    float pr[P][kTinyD];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int t = tid * P + q;
#pragma unroll
        for (int i = 0; i < kTinyD; ++i) pr[q][i] = (bias && i < D) ? bias[i] : 0.0f;
        if (t >= T) continue;
        const float *xr = x + (seq + t) * M;
        for (int k = 0; k < M; ++k) {
            const float xv = xr[k];
#pragma unroll
            for (int i = 0; i < kTinyD; ++i)
                if (i < D) pr[q][i] = __builtin_fmaf(U[static_cast<size_t>(i) * M + k], xv, pr[q][i]);
        }
    }
    __syncthreads();

    int it = 0;
    float r = 0.0f;
    bool stalled = false;
    int best = -1, last_adv = 0;        // finite-step front bookkeeping (same in every thread)
    for (;; ++it) {
        // blocks and offsets at the thread's positions, composed left to right
        Aff m[P];
        unsigned rm = 0u, fm = kNoFront;
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int t = tid * P + q;
            set_identity(m[q]);
            if (t >= T) continue;                    // positions past the end stay identity maps
            float sp[kTinyD], f[kTinyD];
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) sp[i] = (t == 0) ? x0[i] : S[(t - 1) * kTinyD + i];
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) {
                float h = pr[q][i];
#pragma unroll
                for (int j = 0; j < kTinyD; ++j) h += w[i][j] * sp[j];
                f[i] = (i < D) ? tanhf(h) : 0.0f;
                if (i < D) {
                    const float ra = fabsf(S[t * kTinyD + i] - f[i]);
                    rm = max(rm, __float_as_uint(ra));
                    fm = min(fm, front_of(ra, tol, t));
                }
            }
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) {
                const float d = 1.0f - f[i] * f[i];
                float Asp = 0.0f;
                if (dense && lz.kind == kLinJacobian) {
#pragma unroll
                    for (int j = 0; j < kTinyD; ++j) {
                        m[q].A[i][j] = (i < D) ? lz.shrink * d * w[i][j] : 0.0f;
                        Asp += m[q].A[i][j] * sp[j];
                    }
                } else {
                    const float a = (i < D) ? lin_diag(lz, d * w[i][i]) : 0.0f;
#pragma unroll
                    for (int j = 0; j < kTinyD; ++j) m[q].A[i][j] = (i == j) ? a : 0.0f;
                    Asp = a * sp[i];
                }
                m[q].b[i] = (i < D) ? f[i] - Asp : 0.0f;
            }
        }
        // residual of s^(i): maximum over the workgroup on the float bits
        for (int o = 32; o > 0; o >>= 1) rm = max(rm, static_cast<unsigned>(__shfl_xor(static_cast<int>(rm), o, 64)));
        fm = wave_min_u32(fm);
        if ((tid & 63) == 0) {
            red[tid >> 6] = rm;
            fred[tid >> 6] = fm;
        }
        __syncthreads();
        unsigned rb = red[0], fb = fred[0];
#pragma unroll
        for (int k = 1; k < kTinyThreads / 64; ++k) {
            rb = max(rb, red[k]);
            fb = min(fb, fred[k]);
        }
        r = __uint_as_float(rb);
        if (r <= tol || it >= max_iter) break;       // same decision in every thread
        if (stall_window > 0) {
            // the first `it` states are exact in exact arithmetic, so the front is never below it
            const int f = fb > 0x7FFFFFFFu ? 0x7FFFFFFF : static_cast<int>(fb);
            if (f > best) {
                best = f;
                last_adv = it;
            } else if (best < it && it - last_adv >= stall_window) {
                stalled = true;
                break;
            }
        }

        // linear step: thread map, then the inclusive scan over the threads
        Aff loc = m[0];
#pragma unroll
        for (int q = 1; q < P; ++q) loc = compose(m[q], loc);
        store_aff(agg + tid * kAffWords, loc);
        __syncthreads();
        for (int off = 1; off < kTinyThreads; off <<= 1) {
            Aff prev;
            const bool has = tid >= off;
            if (has) prev = load_aff(agg + (tid - off) * kAffWords);
            __syncthreads();
            if (has) {
                loc = compose(loc, prev);
                store_aff(agg + tid * kAffWords, loc);
            }
            __syncthreads();
        }
        // state entering the thread's positions, then the exact replay
        float x[kTinyD];
        if (tid == 0) {
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) x[i] = x0[i];
        } else {
            const Aff e = load_aff(agg + (tid - 1) * kAffWords);
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) {
                float v = e.b[i];
#pragma unroll
                for (int k = 0; k < kTinyD; ++k) v = __builtin_fmaf(e.A[i][k], x0[k], v);
                x[i] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int t = tid * P + q;
            float y[kTinyD];
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) {
                float v = m[q].b[i];
#pragma unroll
                for (int k = 0; k < kTinyD; ++k) v = __builtin_fmaf(m[q].A[i][k], x[k], v);
                y[i] = v;
            }
#pragma unroll
            for (int i = 0; i < kTinyD; ++i) {
                x[i] = y[i];
                if (t < T) S[t * kTinyD + i] = y[i];
            }
        }
        __syncthreads();
    }

    for (int e = tid; e < T * D; e += kTinyThreads) {
        const int t = e / D, i = e % D;
        traj[(seq + t) * D + i] = S[t * kTinyD + i];
    }
    if (tid == 0) {
        iters[b] = it;
        status[b] = (r <= tol) ? DEER_SEQ_CONVERGED
                    : stalled      ? DEER_SEQ_STALLED
                                   : (__builtin_isfinite(r) ? DEER_SEQ_NOT_CONVERGED : DEER_SEQ_NONFINITE);
        resid[b] = r;
        __threadfence_system();
    }
}

}  // namespace

bool tiny_solve_fits(int D, int T) { return D >= 1 && D <= kTinyD && T >= 1 && T <= 4 * kTinyThreads; }

int launch_tiny_solve(const float *W, const float *U, const float *bias, const float *x, int M, const float *s0,
                      const float *init, float *traj, int B, int T, int D, bool dense, Linearization lz, float tol,
                      int max_iter, int stall_window, int *iters, int *status, float *resid, hipStream_t stream)
{
    if (B == 0) return DEER_OK;
    const int P = (T + kTinyThreads - 1) / kTinyThreads;
    const int dn = dense ? 1 : 0;
    if (P <= 1)
        DEER_LAUNCH(tiny_solve_kernel<1>, dim3(B), dim3(kTinyThreads), 0, stream, W, U, bias, x, M, s0, init, traj, T,
                    D, dn, lz, tol, max_iter, stall_window, iters, status, resid);
    else if (P <= 2)
        DEER_LAUNCH(tiny_solve_kernel<2>, dim3(B), dim3(kTinyThreads), 0, stream, W, U, bias, x, M, s0, init, traj, T,
                    D, dn, lz, tol, max_iter, stall_window, iters, status, resid);
    else
        DEER_LAUNCH(tiny_solve_kernel<4>, dim3(B), dim3(kTinyThreads), 0, stream, W, U, bias, x, M, s0, init, traj, T,
                    D, dn, lz, tol, max_iter, stall_window, iters, status, resid);
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}

}  // namespace deer
