/*
 * CPU oracle for the parallel Newton / quasi-Newton (DEER, quasi-DEER)
 * evaluation of nonlinear recurrences.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code with
 * the GPU library (no header, helper, table or constant) and the GPU library
 * never calls it.
 *
 * What it computes, plainly and slowly:
 *   - the sequential rollout s_t = f(s_{t-1}, x_t): the exact answer the
 *     parallel methods reach ("Parallel Broyden Methods" page, section 2 and
 *     Table 1 "Sequential");
 *   - the Newton (dense Jacobian) and diagonal quasi-Newton fixed-point
 *     iterations on the residual r_t = s_t - f(s_{t-1}), each linear step solved
 *     by sequential forward substitution (same page, appendix B.3 "exact
 *     sequential forward substitution");
 *   - sequential solvers of the linear recurrence s_t = A_t s_{t-1} + b_t in
 *     diagonal and dense form;
 *   - the residual r_t = s_t - f(s_{t-1}) of a given trajectory;
 *   - the largest Lyapunov exponent ("Predictability Enables Parallelization"
 *     page, rebuttal "LLE computation cost", Algorithm 1);
 *   - the parallel Broyden iteration with diagonal-plus-low-rank blocks and
 *     its chunked, randomly compressed scan ("Parallel Broyden Methods" page,
 *     section 3; its formulas were lost in extraction, so orc_impl.h states
 *     the reading it implements).
 * Each function is given in double precision (_f64) and in single precision
 * (_f32, the arithmetic a float32 run of the same algorithm performs).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared (no
 * fast-math).  OpenMP only spreads independent sequences over threads.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_CELL_TANH = 0, ORC_CELL_GRU = 1, ORC_CELL_LINEAR = 2 };
enum { ORC_MODE_DENSE = 0, ORC_MODE_DIAG = 1, ORC_MODE_JACOBI = 2, ORC_MODE_PICARD = 3 };

typedef struct {
    int cell;        /* ORC_CELL_* */
    int D, M;        /* state and input sizes */
    const float *W;  /* tanh/linear: [D,D];  GRU: W_hh [3D,D], gate order (r,z,n) */
    const float *U;  /* tanh/linear: [D,M];  GRU: W_ih [3D,M] */
    const float *b;  /* tanh/linear: [D];    GRU: b_ih [3D]; may be NULL (zeros) */
    const float *b2; /* tanh/linear: unused; GRU: b_hh [3D]; may be NULL (zeros) */
} orc_cell;

#define REAL double
#define SUF _f64
#define RTANH tanh
#define REXP exp
#include "orc_impl.h"
#undef REAL
#undef SUF
#undef RTANH
#undef REXP

#define REAL float
#define SUF _f32
#define RTANH tanhf
#define REXP expf
#include "orc_impl.h"
#undef REAL
#undef SUF
#undef RTANH
#undef REXP

static int orc_threads(int requested, int units)
{
    int n = requested;
#ifdef _OPENMP
    if (n <= 0) n = omp_get_max_threads();
#else
    n = 1;
#endif
    if (n > units) n = units;
    if (n < 1) n = 1;
    return n;
}

/* ------------------------------------------------------------ wrappers */
/* The public entry points take float32 parameters and inputs (the arrays both
 * paths read) and write results in the working precision of their suffix.
 * Return 0 on success, -1 on a bad argument or allocation failure. */

#define ORC_WRAPPERS(REAL, SUF)                                                                  \
int ORC_CAT(orc_step, SUF)(const orc_cell *c, const REAL *s, const float *x, REAL *f, REAL *J,   \
                           REAL *jd)                                                             \
{                                                                                                \
    if (!c || !s || !f || c->D <= 0) return -1;                                                  \
    REAL *tmp = (REAL *)malloc(sizeof(REAL) * 6 * (size_t)c->D);                                 \
    if (!tmp) return -1;                                                                         \
    ORC_CAT(o_step, SUF)(c, s, x, f, J, jd, tmp);                                                \
    free(tmp);                                                                                   \
    return 0;                                                                                    \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_rollout, SUF)(const orc_cell *c, const float *x, const float *s0, int B, int T,  \
                              REAL *out, int threads)                                            \
{                                                                                                \
    if (!c || !out || B < 0 || T < 0 || c->D <= 0) return -1;                                    \
    int err = 0;                                                                                 \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *tmp = (REAL *)malloc(sizeof(REAL) * 7 * (size_t)c->D);                             \
        if (!tmp) { err |= 1; continue; }                                                        \
        ORC_CAT(o_rollout_one, SUF)(c, x + (size_t)b * T * c->M, s0 ? s0 + (size_t)b * c->D : NULL, \
                                    T, out + (size_t)b * T * c->D, tmp);                         \
        free(tmp);                                                                               \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
/* Residual r_t = s_t - f(s_{t-1}, x_t) of a given trajectory (s_{-1} = s0),   \
 * the quantity the parallel methods drive to zero ("Predictability" page,     \
 * rebuttal, restating its equation 2).  traj, r: [B,T,D]. */                   \
int ORC_CAT(orc_residual, SUF)(const orc_cell *c, const float *x, const float *s0, const REAL *traj, \
                               int B, int T, REAL *r, int threads)                               \
{                                                                                                \
    if (!c || !traj || !r || B < 0 || T < 0 || c->D <= 0) return -1;                             \
    int err = 0;                                                                                 \
    const int D = c->D;                                                                          \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *buf = (REAL *)malloc(sizeof(REAL) * 8 * (size_t)D);                                \
        if (!buf) { err |= 1; continue; }                                                        \
        REAL *sp0 = buf, *f = buf + D, *tmp = buf + 2 * D;                                       \
        for (int d = 0; d < D; ++d) sp0[d] = s0 ? (REAL)s0[(size_t)b * D + d] : (REAL)0;         \
        const REAL *sb = traj + (size_t)b * T * D;                                               \
        for (int t = 0; t < T; ++t) {                                                            \
            const REAL *sp = (t == 0) ? sp0 : sb + (size_t)(t - 1) * D;                          \
            ORC_CAT(o_step, SUF)(c, sp, x + ((size_t)b * T + t) * c->M, f, NULL, NULL, tmp);     \
            for (int d = 0; d < D; ++d)                                                          \
                r[((size_t)b * T + t) * D + d] = sb[(size_t)t * D + d] - f[d];                   \
        }                                                                                        \
        free(buf);                                                                               \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_solve_diag, SUF)(const float *a, const float *bv, const float *s0, int B, int T, \
                                 int D, REAL *out, int threads)                                  \
{                                                                                                \
    if (!a || !bv || !out || B < 0 || T < 0 || D <= 0) return -1;                                \
    int err = 0;                                                                                 \
    const size_t TD = (size_t)T * D;                                                             \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *buf = (REAL *)malloc(sizeof(REAL) * (2 * TD + (size_t)D));                         \
        if (!buf) { err |= 1; continue; }                                                        \
        REAL *ar = buf, *br = buf + TD, *s0r = buf + 2 * TD;                                     \
        for (size_t e = 0; e < TD; ++e) {                                                        \
            ar[e] = (REAL)a[(size_t)b * TD + e];                                                 \
            br[e] = (REAL)bv[(size_t)b * TD + e];                                                \
        }                                                                                        \
        for (int d = 0; d < D; ++d) s0r[d] = s0 ? (REAL)s0[(size_t)b * D + d] : (REAL)0;         \
        ORC_CAT(o_solve_diag_one, SUF)(ar, br, s0r, T, D, out + (size_t)b * TD);                 \
        free(buf);                                                                               \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_solve_dense, SUF)(const float *A, const float *bv, const float *s0, int B, int T,\
                                  int D, REAL *out, int threads)                                 \
{                                                                                                \
    if (!A || !bv || !out || B < 0 || T < 0 || D <= 0) return -1;                                \
    int err = 0;                                                                                 \
    const size_t TD = (size_t)T * D, TDD = (size_t)T * D * D;                                    \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *buf = (REAL *)malloc(sizeof(REAL) * (TDD + TD + (size_t)D));                       \
        if (!buf) { err |= 1; continue; }                                                        \
        REAL *Ar = buf, *br = buf + TDD, *s0r = buf + TDD + TD;                                  \
        for (size_t e = 0; e < TDD; ++e) Ar[e] = (REAL)A[(size_t)b * TDD + e];                   \
        for (size_t e = 0; e < TD; ++e) br[e] = (REAL)bv[(size_t)b * TD + e];                    \
        for (int d = 0; d < D; ++d) s0r[d] = s0 ? (REAL)s0[(size_t)b * D + d] : (REAL)0;         \
        ORC_CAT(o_solve_dense_one, SUF)(Ar, br, s0r, T, D, out + (size_t)b * TD);                \
        free(buf);                                                                               \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_newton, SUF)(const orc_cell *c, const float *x, const float *s0, int B, int T,   \
                             int mode, double damp, double tol, int max_iter, const float *init, \
                             REAL *traj, int *iters, double *resid, int *status, double *hist,   \
                             int threads)                                                        \
{                                                                                                \
    if (!c || !traj || !iters || !resid || !status || B < 0 || T < 0 || c->D <= 0 ||            \
        max_iter < 0 || mode < ORC_MODE_DENSE || mode > ORC_MODE_PICARD ||                       \
        !(damp >= 0.0 && damp <= 1.0) ||                                                         \
        (damp != 0.0 && mode != ORC_MODE_DENSE && mode != ORC_MODE_DIAG)) return -1;            \
    int err = 0;                                                                                 \
    const int D = c->D;                                                                          \
    const size_t TD = (size_t)T * D;                                                             \
    const size_t asz = (mode == ORC_MODE_DENSE) ? TD * D : TD;                                   \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *work = (REAL *)malloc(sizeof(REAL) * (3 * TD + 7 * (size_t)D + asz));              \
        if (!work) { err |= 1; continue; }                                                       \
        status[b] = ORC_CAT(o_newton_one, SUF)(c, x + (size_t)b * T * c->M,                     \
                                               s0 ? s0 + (size_t)b * D : NULL, T, mode, damp,    \
                                               tol,                                              \
                                               max_iter, init ? init + (size_t)b * TD : NULL,    \
                                               traj + (size_t)b * TD, iters + b, resid + b,      \
                                               hist ? hist + (size_t)b * (max_iter + 1) : NULL,  \
                                               work);                                            \
        free(work);                                                                              \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_lle, SUF)(const orc_cell *c, const float *x, const float *s0, const REAL *traj,  \
                          int B, int T, const float *v0, double *out, int threads)               \
{                                                                                                \
    if (!c || !traj || !v0 || !out || B < 0 || T <= 0 || c->D <= 0) return -1;                   \
    int err = 0;                                                                                 \
    const int D = c->D;                                                                          \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *work = (REAL *)malloc(sizeof(REAL) * ((size_t)D * D + 10 * (size_t)D));            \
        if (!work) { err |= 1; continue; }                                                       \
        out[b] = ORC_CAT(o_lle_one, SUF)(c, x + (size_t)b * T * c->M,                            \
                                         s0 ? s0 + (size_t)b * D : NULL,                         \
                                         traj + (size_t)b * T * D, T, v0 + (size_t)b * D, work); \
        free(work);                                                                              \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}

#define ORC_BROYDEN_WRAPPERS(REAL, SUF)                                                          \
int ORC_CAT(orc_broyden, SUF)(const orc_cell *c, const float *x, const float *s0, int B, int T,  \
                              int rank, int multisecant, double alpha, double damp,              \
                              double gram_reg, int chunk, const float *sketch, double tol,       \
                              int max_iter, const float *init, REAL *traj, int *iters,           \
                              double *resid, int *status, double *hist, int threads)             \
{                                                                                                \
    if (!c || !traj || !iters || !resid || !status || B < 0 || T < 0 || c->D <= 0 ||            \
        max_iter < 0 || rank < 0 || rank > 8 || (rank > 0 && !sketch) || chunk < 1 ||            \
        !(damp >= 0.0 && damp <= 1.0) || !(gram_reg >= 0.0) || !isfinite(alpha)) return -1;      \
    int err = 0;                                                                                 \
    const int D = c->D, m = rank;                                                                \
    const size_t TD = (size_t)T * D, TMD = (size_t)T * m * D;                                    \
    const size_t wsz = 5 * TD + 4 * TMD + (size_t)D * m + 9 * (size_t)D                          \
                     + (4 * (size_t)D + 7 * (size_t)m * D + 2 * (size_t)m * m + (size_t)m);       \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        REAL *work = (REAL *)malloc(sizeof(REAL) * wsz);                                         \
        if (!work) { err |= 1; continue; }                                                       \
        status[b] = ORC_CAT(o_broyden_one, SUF)(c, x + (size_t)b * T * c->M,                    \
                                                s0 ? s0 + (size_t)b * D : NULL, T, rank,         \
                                                multisecant, alpha, damp, gram_reg, chunk,       \
                                                sketch, tol, max_iter,                           \
                                                init ? init + (size_t)b * TD : NULL,             \
                                                traj + (size_t)b * TD, iters + b, resid + b,     \
                                                hist ? hist + (size_t)b * (max_iter + 1) : NULL, \
                                                work);                                           \
        free(work);                                                                              \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_dplr_scan, SUF)(double alpha, const float *U, const float *V, const float *cvec, \
                                const float *sketch, int B, int T, int D, int m, int n,          \
                                int chunk, REAL *delta, int threads)                             \
{                                                                                                \
    if (!U || !V || !cvec || !delta || (m > 0 && !sketch) || B < 0 || T < 0 || D <= 0 ||        \
        m < 0 || m > 8 || n < 0 || n > m || chunk < 1) return -1;                                \
    int err = 0;                                                                                 \
    const size_t TD = (size_t)T * D, TMD = (size_t)T * m * D;                                    \
    const int nt = orc_threads(threads, B);                                                      \
    _Pragma("omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(|:err)")            \
    for (int b = 0; b < B; ++b) {                                                                \
        const size_t wsz = 2 * TMD + TD + (size_t)D * m                                          \
                         + 3 * (size_t)D + 7 * (size_t)m * D + 2 * (size_t)m * m;                \
        REAL *buf = (REAL *)malloc(sizeof(REAL) * wsz);                                          \
        if (!buf) { err |= 1; continue; }                                                        \
        REAL *Ur = buf, *Vr = buf + TMD, *cr = buf + 2 * TMD, *Om = cr + TD, *w = Om + (size_t)D * m; \
        for (size_t e = 0; e < TMD; ++e) {                                                       \
            Ur[e] = (REAL)U[(size_t)b * TMD + e];                                                \
            Vr[e] = (REAL)V[(size_t)b * TMD + e];                                                \
        }                                                                                        \
        for (size_t e = 0; e < TD; ++e) cr[e] = (REAL)cvec[(size_t)b * TD + e];                  \
        for (size_t e = 0; e < (size_t)D * m; ++e) Om[e] = (REAL)sketch[e];                      \
        ORC_CAT(o_dplr_scan_one, SUF)((REAL)alpha, Ur, Vr, n, m, cr, T, D, chunk, Om,            \
                                      delta + (size_t)b * TD, w);                                \
        free(buf);                                                                               \
    }                                                                                            \
    return err ? -1 : 0;                                                                         \
}                                                                                                \
                                                                                                 \
int ORC_CAT(orc_broyden_update, SUF)(int multisecant, double alpha, double gram_reg, int it,     \
                                     int m, int D, REAL *U, REAL *V, REAL *F, const REAL *ds,    \
                                     const REAL *df)                                             \
{                                                                                                \
    if (!U || !V || !F || !ds || !df || m < 1 || m > 8 || D <= 0 || it < 1) return -1;           \
    REAL *scr = (REAL *)malloc(sizeof(REAL) * ((size_t)D + 2 * (size_t)m * m + (size_t)m));      \
    if (!scr) return -1;                                                                         \
    ORC_CAT(o_broyden_update_one, SUF)(multisecant, (REAL)alpha, (REAL)gram_reg, it, m, D, U, V, \
                                       F, ds, df, scr);                                          \
    free(scr);                                                                                   \
    return 0;                                                                                    \
}

ORC_WRAPPERS(double, _f64)
ORC_WRAPPERS(float, _f32)
ORC_BROYDEN_WRAPPERS(double, _f64)
ORC_BROYDEN_WRAPPERS(float, _f32)

/* Threads an OpenMP region would use by default (reported with CPU timings). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
