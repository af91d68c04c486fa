/*
 * Oracle arithmetic, instantiated twice by oracle.c: REAL = double (suffix
 * _f64) and REAL = float (suffix _f32).  Test infrastructure only; see the
 * header of oracle.c.
 *
 * Every loop runs in the order its definition reads: time steps one after the
 * other, sums over k = 0, 1, ..., in REAL arithmetic, no blocking, no fusion
 * and no reassociation (the file is built without fast-math and with
 * -ffp-contract=off).
 */

#define ORC_CAT2(a, b) a##b
#define ORC_CAT(a, b) ORC_CAT2(a, b)
#define FN(name) ORC_CAT(name, SUF)

/*
 * One transition s' = f(s, x) of a cell and its Jacobian d f / d s.
 *   f  : D outputs
 *   J  : D*D row-major (J[i*D+k] = d f_i / d s_k), or NULL
 *   jd : the diagonal of J (D values), or NULL
 *
 * tanh cell (the vector form of the scalar tanh model on the "Predictability
 * Enables Parallelization" page, rebuttal "Application to RNN training
 * efficiency"):  f = tanh(W s + U x + b),  J = diag(1 - f^2) W.
 * linear cell (the same without the tanh):  f = W s + U x + b,  J = W.
 * GRU cell (textbook equations; gate order r, z, n):
 *   gi = W_ih x + b_ih,  gh = W_hh s + b_hh
 *   r = sigma(gi_r + gh_r),  z = sigma(gi_z + gh_z),  n = tanh(gi_n + r * gh_n)
 *   f = (1 - z) * n + z * s
 *   J[i,k] = z_i [i==k] + (s_i - n_i) z_i (1 - z_i) Wz[i,k]
 *          + (1 - z_i)(1 - n_i^2) (r_i Wn[i,k] + r_i (1 - r_i) Wr[i,k] gh_n[i])
 */
static void FN(o_step)(const orc_cell *c, const REAL *s, const float *x,
                         REAL *f, REAL *J, REAL *jd, REAL *tmp /* 6*D scratch */)
{
    const int D = c->D, M = c->M;
    if (c->cell == ORC_CELL_TANH || c->cell == ORC_CELL_LINEAR) {
        for (int i = 0; i < D; ++i) {
            REAL h = 0;
            for (int k = 0; k < D; ++k) h += (REAL)c->W[(size_t)i * D + k] * s[k];
            for (int j = 0; j < M; ++j) h += (REAL)c->U[(size_t)i * M + j] * (REAL)x[j];
            if (c->b) h += (REAL)c->b[i];
            const REAL fi = (c->cell == ORC_CELL_TANH) ? RTANH(h) : h;
            const REAL g = (c->cell == ORC_CELL_TANH) ? ((REAL)1 - fi * fi) : (REAL)1;
            f[i] = fi;
            if (J)
                for (int k = 0; k < D; ++k) J[(size_t)i * D + k] = g * (REAL)c->W[(size_t)i * D + k];
            if (jd) jd[i] = g * (REAL)c->W[(size_t)i * D + i];
        }
        return;
    }
    /* GRU */
    REAL *gi = tmp, *gh = tmp + 3 * D;
    for (int g = 0; g < 3 * D; ++g) {
        REAL a = 0, h = 0;
        for (int j = 0; j < M; ++j) a += (REAL)c->U[(size_t)g * M + j] * (REAL)x[j];
        if (c->b) a += (REAL)c->b[g];
        for (int k = 0; k < D; ++k) h += (REAL)c->W[(size_t)g * D + k] * s[k];
        if (c->b2) h += (REAL)c->b2[g];
        gi[g] = a;
        gh[g] = h;
    }
    for (int i = 0; i < D; ++i) {
        const REAL r = (REAL)1 / ((REAL)1 + REXP(-(gi[i] + gh[i])));
        const REAL z = (REAL)1 / ((REAL)1 + REXP(-(gi[D + i] + gh[D + i])));
        const REAL n = RTANH(gi[2 * D + i] + r * gh[2 * D + i]);
        f[i] = ((REAL)1 - z) * n + z * s[i];
        const REAL dz = z * ((REAL)1 - z);          /* d sigma at the z gate */
        const REAL dr = r * ((REAL)1 - r);          /* d sigma at the r gate */
        const REAL dn = (REAL)1 - n * n;            /* d tanh at the n gate  */
        const float *Wr = c->W + (size_t)i * D;
        const float *Wz = c->W + (size_t)(D + i) * D;
        const float *Wn = c->W + (size_t)(2 * D + i) * D;
        if (J) {
            for (int k = 0; k < D; ++k) {
                REAL v = (s[i] - n) * dz * (REAL)Wz[k]
                       + ((REAL)1 - z) * dn * (r * (REAL)Wn[k] + dr * (REAL)Wr[k] * gh[2 * D + i]);
                if (k == i) v += z;
                J[(size_t)i * D + k] = v;
            }
        }
        if (jd) {
            jd[i] = z + (s[i] - n) * dz * (REAL)Wz[i]
                  + ((REAL)1 - z) * dn * (r * (REAL)Wn[i] + dr * (REAL)Wr[i] * gh[2 * D + i]);
        }
    }
}

/* Sequential rollout s_t = f(s_{t-1}, x_t), t = 1..T, from s_0 (zeros if NULL). */
static void FN(o_rollout_one)(const orc_cell *c, const float *x /*[T,M]*/, const float *s0 /*[D]*/,
                                int T, REAL *out /*[T,D]*/, REAL *tmp /*7*D*/)
{
    const int D = c->D, M = c->M;
    REAL *prev = tmp + 6 * D;
    for (int d = 0; d < D; ++d) prev[d] = s0 ? (REAL)s0[d] : (REAL)0;
    for (int t = 0; t < T; ++t) {
        const REAL *sp = (t == 0) ? prev : out + (size_t)(t - 1) * D;
        FN(o_step)(c, sp, x + (size_t)t * M, out + (size_t)t * D, NULL, NULL, tmp);
    }
}

/* Forward substitution of s_t = a_t * s_{t-1} + b_t (elementwise), from s_0. */
static void FN(o_solve_diag_one)(const REAL *a, const REAL *b, const REAL *s0, int T, int D, REAL *out)
{
    for (int t = 0; t < T; ++t) {
        for (int d = 0; d < D; ++d) {
            const REAL prev = (t == 0) ? s0[d] : out[(size_t)(t - 1) * D + d];
            out[(size_t)t * D + d] = a[(size_t)t * D + d] * prev + b[(size_t)t * D + d];
        }
    }
}

/* Forward substitution of s_t = A_t s_{t-1} + b_t with dense D x D blocks A_t. */
static void FN(o_solve_dense_one)(const REAL *A, const REAL *b, const REAL *s0, int T, int D, REAL *out)
{
    for (int t = 0; t < T; ++t) {
        const REAL *sp = (t == 0) ? s0 : out + (size_t)(t - 1) * D;
        const REAL *At = A + (size_t)t * D * D;
        for (int i = 0; i < D; ++i) {
            REAL acc = 0;
            for (int k = 0; k < D; ++k) acc += At[(size_t)i * D + k] * sp[k];
            out[(size_t)t * D + i] = acc + b[(size_t)t * D + i];
        }
    }
}

/*
 * Fixed-point iteration of a chosen linearisation for one sequence, with the
 * linear recurrence solved by sequential forward substitution.
 *
 * Residual r_t(s) = s_t - f(s_{t-1}, x_t) (the "Predictability Enables
 * Parallelization" page, rebuttal, where it restates its equation 2); the
 * trajectory is its root.  Each iteration i:
 *   f_t (and J_t where the mode needs it) at the current guess s^(i)  (s^(i)_0 := s_0)
 *   res = max_{t,d} |s^(i)_t - f_t|      (NaN counts as not converged)
 *   stop if res <= tol (iters = i), or if i == max_iter (not converged)
 *   A_t by mode, b_t = f_t - A_t s^(i)_{t-1}, and s^(i+1) solves
 *   s_t = A_t s_{t-1} + b_t from s_0.
 * The modes are the approximate linearisations the pages compare (the first
 * page's thread: every method linearises the dynamics, then evaluates the
 * linear recurrence in parallel; "Parallel Broyden Methods", section 2):
 *   dense  : A_t = (1 - k) J_t              (Newton / DEER; k = 0 undamped)
 *   diag   : A_t = (1 - k) diag(J_t)        (diagonal quasi-Newton)
 *   jacobi : A_t = 0, so s^(i+1)_t = f_t
 *   picard : A_t = I, so s^(i+1)_t = s^(i+1)_{t-1} + (f_t - s^(i)_{t-1})
 * k is the damping of the scale-ELK method: the full Jacobian block shrunk by
 * the factor 1 - k ("Parallel Broyden Methods", appendix E.4; its Gibbs
 * appendix damps Newton this way to avoid float32 overflow).  The offsets use
 * the same A_t, so every mode keeps the trajectory as its fixed point.
 *
 * hist (optional, max_iter+1 entries) receives res at every iteration (NaN
 * after the stop).  Returns the status: 0 converged, 1 not converged within
 * max_iter, 2 the residual is not finite when the cap is reached.
 */
static int FN(o_newton_one)(const orc_cell *c, const float *x, const float *s0, int T, int mode,
                              double damp, double tol, int max_iter, const float *init,
                              REAL *s /*[T,D] in: ignored, out: final iterate*/,
                              int *iters_out, double *resid_out, double *hist,
                              REAL *work)
{
    const int D = c->D;
    const size_t TD = (size_t)T * D;
    REAL *f = work;                       /* [T,D] */
    REAL *bb = f + TD;                    /* [T,D] */
    REAL *sn = bb + TD;                   /* [T,D] */
    REAL *s0r = sn + TD;                  /* [D]   */
    REAL *tmp = s0r + D;                  /* [6D]  */
    REAL *A = tmp + 6 * D;                /* [T,D,D] dense or [T,D] diag */

    for (int d = 0; d < D; ++d) s0r[d] = s0 ? (REAL)s0[d] : (REAL)0;
    for (size_t e = 0; e < TD; ++e) s[e] = init ? (REAL)init[e] : (REAL)0;
    if (hist)
        for (int i = 0; i <= max_iter; ++i) hist[i] = NAN;

    const REAL shrink = (REAL)(1.0 - damp);
    for (int it = 0;; ++it) {
        double res = 0.0;
        int nonfinite = 0;
        for (int t = 0; t < T; ++t) {
            const REAL *sp = (t == 0) ? s0r : s + (size_t)(t - 1) * D;
            REAL *At = (mode == ORC_MODE_DENSE) ? A + (size_t)t * D * D : A + (size_t)t * D;
            FN(o_step)(c, sp, x + (size_t)t * c->M, f + (size_t)t * D,
                         mode == ORC_MODE_DENSE ? At : NULL, mode == ORC_MODE_DIAG ? At : NULL, tmp);
            for (int d = 0; d < D; ++d) {
                const double r = fabs((double)(s[(size_t)t * D + d] - f[(size_t)t * D + d]));
                if (!(r == r) || isinf(r)) nonfinite = 1;
                if (r > res) res = r;
            }
        }
        if (nonfinite) res = NAN;
        if (hist) hist[it] = res;
        if ((REAL)res <= (REAL)tol) {
            *iters_out = it;
            *resid_out = res;
            return 0;
        }
        if (it >= max_iter) {
            *iters_out = max_iter;
            *resid_out = res;
            return (res == res && !isinf(res)) ? 1 : 2;
        }
        if (mode == ORC_MODE_JACOBI) {          /* A_t = 0: the next iterate is f itself */
            memcpy(s, f, TD * sizeof(REAL));
            continue;
        }
        if (mode == ORC_MODE_PICARD) {          /* A_t = I: accumulate the one-step corrections */
            for (int t = 0; t < T; ++t)
                for (int d = 0; d < D; ++d) {
                    const REAL prev_old = (t == 0) ? s0r[d] : s[(size_t)(t - 1) * D + d];
                    bb[(size_t)t * D + d] = f[(size_t)t * D + d] - prev_old;
                }
            for (int t = 0; t < T; ++t)
                for (int d = 0; d < D; ++d) {
                    const REAL prev_new = (t == 0) ? s0r[d] : sn[(size_t)(t - 1) * D + d];
                    sn[(size_t)t * D + d] = prev_new + bb[(size_t)t * D + d];
                }
            memcpy(s, sn, TD * sizeof(REAL));
            continue;
        }
        /* damping: A_t = (1 - k) J_t (or its diagonal) */
        {
            const size_t na = (mode == ORC_MODE_DENSE) ? TD * D : TD;
            for (size_t e = 0; e < na; ++e) A[e] = shrink * A[e];
        }
        /* offsets b_t = f_t - A_t s_{t-1}, with the same A_t the solve uses */
        for (int t = 0; t < T; ++t) {
            const REAL *sp = (t == 0) ? s0r : s + (size_t)(t - 1) * D;
            for (int i = 0; i < D; ++i) {
                REAL as = 0;
                if (mode == ORC_MODE_DENSE) {
                    const REAL *Ai = A + (size_t)t * D * D + (size_t)i * D;
                    for (int k = 0; k < D; ++k) as += Ai[k] * sp[k];
                } else {
                    as = A[(size_t)t * D + i] * sp[i];
                }
                bb[(size_t)t * D + i] = f[(size_t)t * D + i] - as;
            }
        }
        if (mode == ORC_MODE_DENSE) FN(o_solve_dense_one)(A, bb, s0r, T, D, sn);
        else FN(o_solve_diag_one)(A, bb, s0r, T, D, sn);
        memcpy(s, sn, TD * sizeof(REAL));
    }
}

/*
 * Largest Lyapunov exponent along a given trajectory: push a unit vector
 * through the Jacobians J_t = d f / d s at (s_{t-1}, x_t), t = 1..T,
 * renormalising after every step, and average the log growth ("Predictability"
 * page, rebuttal "LLE computation cost", Algorithm 1 of its appendix J.5).
 * Natural log, per step, no burn-in; v0 is normalised first.
 */
static double FN(o_lle_one)(const orc_cell *c, const float *x, const float *s0, const REAL *traj,
                              int T, const float *v0, REAL *work)
{
    const int D = c->D;
    REAL *J = work;                      /* D*D */
    REAL *f = J + (size_t)D * D;         /* D   */
    REAL *v = f + D;                     /* D   */
    REAL *w = v + D;                     /* D   */
    REAL *sp0 = w + D;                   /* D   */
    REAL *tmp = sp0 + D;                 /* 6D  */
    double nrm = 0.0;
    for (int d = 0; d < D; ++d) {
        v[d] = (REAL)v0[d];
        nrm += (double)v[d] * (double)v[d];
        sp0[d] = s0 ? (REAL)s0[d] : (REAL)0;
    }
    nrm = sqrt(nrm);
    for (int d = 0; d < D; ++d) v[d] = (REAL)((double)v[d] / nrm);
    double sum = 0.0;
    for (int t = 0; t < T; ++t) {
        const REAL *sp = (t == 0) ? sp0 : traj + (size_t)(t - 1) * D;
        FN(o_step)(c, sp, x + (size_t)t * c->M, f, J, NULL, tmp);
        double g = 0.0;
        for (int i = 0; i < D; ++i) {
            REAL acc = 0;
            for (int k = 0; k < D; ++k) acc += J[(size_t)i * D + k] * v[k];
            w[i] = acc;
            g += (double)acc * (double)acc;
        }
        g = sqrt(g);
        sum += log(g);
        for (int i = 0; i < D; ++i) v[i] = (REAL)((double)w[i] / g);
    }
    return sum / (double)T;
}

#undef FN
