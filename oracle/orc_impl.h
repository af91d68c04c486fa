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


/*
 * ---------------------------------------------------------------- Broyden
 * Parallel Broyden iteration ("Parallel Broyden Methods" page, sections 3.1
 * and 3.2, appendices E.1-E.4).  The page's formulas did not survive
 * extraction; what follows is the reading stated with the build's design notes.
 *
 * Block approximation at position t: a diagonal-plus-low-rank (DPLR) matrix
 *     J^_t = alpha I + sum_j u_j v_j^T      (at most m columns)
 * with the identity-scaled diagonal baseline alpha of appendix H.5 (0 for the
 * Gibbs appendix, the leak for the RNN appendix).  The solver uses the damped
 * block A_t = alpha I + (1 - k) sum_j u_j v_j^T (appendix E.4: damping on the
 * low-rank correction only).
 *
 * Secant pair at iteration i >= 1 and position t:
 *     ds = s^(i)_{t-1} - s^(i-1)_{t-1},   df = f(s^(i)_{t-1}) - f(s^(i-1)_{t-1}).
 * Column slot of iteration i: (i - 1) mod m; after the update min(i, m)
 * columns are valid.
 *   rank-one ("good" Broyden, limited memory by simple truncation, E.1-E.2):
 *     the column in the slot (the oldest once m are stored) is dropped, then
 *     u = (df - J^' ds) / (ds.ds), v = ds, so the new block meets the secant
 *     exactly; a zero ds gives a zero column.
 *   multisecant (E.3): the slot takes (ds, df); with S, F the valid secant
 *     columns, G = S^T S + lambda I and
 *         U = (F - alpha S) G^{-1},  V = S,
 *     so J^ S = F when lambda = 0.  A failed Cholesky factorisation of G
 *     (a pivot <= 0 or not finite) leaves U = 0 at that position.
 *
 * Linear step in increment form: with c_t = f_t - s_t (minus the residual),
 *     delta_t = A_t delta_{t-1} + c_t,  delta_0 = 0,   s^(i+1) = s^(i) + delta,
 * solved by a chunked scan: chunks of L positions are replayed exactly from
 * their entry value, and the entry of chunk q+1 is the aggregate of chunk q
 * applied to the entry of chunk q.  The aggregate P = p I + sum_a l_a r_a^T,
 * with offset Pb, is folded left to right over the chunk,
 *     A_t P = alpha p I + [alpha l_a + sum_j u~_j (v_j.l_a) | p u~_j] [r_a | v_j]^T,
 *     Pb   <- A_t Pb + c_t,
 * and whenever the low-rank part has more than m columns it is re-compressed
 * to m by the randomized scheme of section 3.2: Y = L (R^T Omega) with the
 * fixed sketch Omega [D, m], Q an orthonormal basis of Y's columns (modified
 * Gram-Schmidt; a column whose remaining norm is at most 1e-5 of its original
 * norm is dropped as zero), then L <- Q, R <- R (L^T Q), i.e. the correction
 * becomes Q Q^T L R^T.  Exact zeros stay exact: where c_t = 0 on a prefix,
 * delta_t = 0 there, which keeps finite-step recovery under compression.
 */
#define ORC_QR_DROP 1e-5

/* y = alpha x + sum_{j<n} u_j (v_j . x);  u, v: n columns of D */
static void FN(o_dplr_apply)(REAL alpha, const REAL *u, const REAL *v, int n, int D, const REAL *x, REAL *y)
{
    for (int d = 0; d < D; ++d) y[d] = alpha * x[d];
    for (int j = 0; j < n; ++j) {
        REAL dot = 0;
        for (int d = 0; d < D; ++d) dot += v[(size_t)j * D + d] * x[d];
        for (int d = 0; d < D; ++d) y[d] += u[(size_t)j * D + d] * dot;
    }
}

/* Re-compress the K-column correction sum_a Lf_a Rf_a^T to m columns. */
static void FN(o_compress)(const REAL *Lf, const REAL *Rf, int K, const REAL *Om, int m, int D,
                             REAL *Lo, REAL *Ro, REAL *scr /* m*K + m*D */)
{
    REAL *RtO = scr;                 /* [K][m]: R^T Omega */
    REAL *Y = scr + (size_t)m * K;   /* [m][D] */
    for (int a = 0; a < K; ++a)
        for (int j = 0; j < m; ++j) {
            REAL acc = 0;
            for (int d = 0; d < D; ++d) acc += Rf[(size_t)a * D + d] * Om[(size_t)d * m + j];
            RtO[(size_t)a * m + j] = acc;
        }
    for (int j = 0; j < m; ++j)
        for (int d = 0; d < D; ++d) {
            REAL acc = 0;
            for (int a = 0; a < K; ++a) acc += Lf[(size_t)a * D + d] * RtO[(size_t)a * m + j];
            Y[(size_t)j * D + d] = acc;
        }
    /* modified Gram-Schmidt: Q into Lo */
    for (int j = 0; j < m; ++j) {
        REAL *q = Lo + (size_t)j * D;
        REAL ny = 0;
        for (int d = 0; d < D; ++d) {
            q[d] = Y[(size_t)j * D + d];
            ny += q[d] * q[d];
        }
        for (int l = 0; l < j; ++l) {
            const REAL *ql = Lo + (size_t)l * D;
            REAL cf = 0;
            for (int d = 0; d < D; ++d) cf += ql[d] * q[d];
            for (int d = 0; d < D; ++d) q[d] -= cf * ql[d];
        }
        REAL nq = 0;
        for (int d = 0; d < D; ++d) nq += q[d] * q[d];
        nq = (REAL)sqrt((double)nq);
        ny = (REAL)sqrt((double)ny);
        if (!(nq > (REAL)ORC_QR_DROP * ny)) {
            for (int d = 0; d < D; ++d) q[d] = 0;
        } else {
            for (int d = 0; d < D; ++d) q[d] = q[d] / nq;
        }
    }
    /* Ro_j = sum_a Rf_a (Lf_a . Q_j) */
    for (int j = 0; j < m; ++j) {
        for (int d = 0; d < D; ++d) Ro[(size_t)j * D + d] = 0;
        for (int a = 0; a < K; ++a) {
            REAL cf = 0;
            for (int d = 0; d < D; ++d) cf += Lf[(size_t)a * D + d] * Lo[(size_t)j * D + d];
            for (int d = 0; d < D; ++d) Ro[(size_t)j * D + d] += Rf[(size_t)a * D + d] * cf;
        }
    }
}

/*
 * Chunked compressed scan of delta_t = A_t delta_{t-1} + c_t, delta_0 = 0, for
 * one sequence.  A_t = alpha I + sum_{j<n} U[t][j] V[t][j]^T (U already damped);
 * U, V: [T][m][D]; c, delta: [T][D].
 */
static void FN(o_dplr_scan_one)(REAL alpha, const REAL *U, const REAL *V, int n, int m, const REAL *c, int T,
                                  int D, int L, const REAL *Om, REAL *delta, REAL *work)
{
    REAL *entry = work;                   /* D */
    REAL *Pb = entry + D;                 /* D */
    REAL *tmpv = Pb + D;                  /* D */
    REAL *PL = tmpv + D;                  /* m*D */
    REAL *PR = PL + (size_t)m * D;        /* m*D */
    REAL *Lf = PR + (size_t)m * D;        /* 2m*D */
    REAL *Rf = Lf + (size_t)2 * m * D;    /* 2m*D */
    REAL *scr = Rf + (size_t)2 * m * D;   /* 2m*m + m*D */
    for (int d = 0; d < D; ++d) entry[d] = 0;
    for (int t0 = 0; t0 < T; t0 += L) {
        const int t1 = (t0 + L < T) ? t0 + L : T;
        /* exact replay of the chunk from its entry */
        for (int t = t0; t < t1; ++t) {
            const REAL *prev = (t == t0) ? entry : delta + (size_t)(t - 1) * D;
            FN(o_dplr_apply)(alpha, U + (size_t)t * m * D, V + (size_t)t * m * D, n, D, prev, delta + (size_t)t * D);
            for (int d = 0; d < D; ++d) delta[(size_t)t * D + d] += c[(size_t)t * D + d];
        }
        if (t1 >= T) break;
        /* aggregate of the chunk, folded left to right */
        REAL p = 1;
        int r = 0;
        for (int d = 0; d < D; ++d) Pb[d] = 0;
        for (int t = t0; t < t1; ++t) {
            const REAL *u = U + (size_t)t * m * D, *v = V + (size_t)t * m * D;
            const int K = r + n;
            for (int a = 0; a < r; ++a) {
                FN(o_dplr_apply)(alpha, u, v, n, D, PL + (size_t)a * D, Lf + (size_t)a * D);
                for (int d = 0; d < D; ++d) Rf[(size_t)a * D + d] = PR[(size_t)a * D + d];
            }
            for (int j = 0; j < n; ++j)
                for (int d = 0; d < D; ++d) {
                    Lf[(size_t)(r + j) * D + d] = p * u[(size_t)j * D + d];
                    Rf[(size_t)(r + j) * D + d] = v[(size_t)j * D + d];
                }
            p = alpha * p;
            if (K <= m) {
                memcpy(PL, Lf, sizeof(REAL) * (size_t)K * D);
                memcpy(PR, Rf, sizeof(REAL) * (size_t)K * D);
                r = K;
            } else {
                FN(o_compress)(Lf, Rf, K, Om, m, D, PL, PR, scr);
                r = m;
            }
            FN(o_dplr_apply)(alpha, u, v, n, D, Pb, tmpv);
            for (int d = 0; d < D; ++d) Pb[d] = tmpv[d] + c[(size_t)t * D + d];
        }
        /* entry of the next chunk */
        FN(o_dplr_apply)(p, PL, PR, r, D, entry, tmpv);
        for (int d = 0; d < D; ++d) entry[d] = tmpv[d] + Pb[d];
    }
}

/* Block update of one position at iteration it >= 1 (see above).
 * U, V (and F for the multisecant variant): [m][D], updated in place. */
static void FN(o_broyden_update_one)(int multisecant, REAL alpha, REAL lambda, int it, int m, int D,
                                       REAL *U, REAL *V, REAL *F, const REAL *ds, const REAL *df,
                                       REAL *scr /* D + 2 m m + m */)
{
    if (m <= 0 || it < 1) return;
    const int slot = (it - 1) % m;
    if (!multisecant) {
        const int nb = (it - 1 < m) ? it - 1 : m;     /* valid before the update */
        REAL *jds = scr;
        for (int d = 0; d < D; ++d) jds[d] = alpha * ds[d];
        for (int j = 0; j < nb; ++j) {
            if (j == slot) continue;
            REAL dot = 0;
            for (int d = 0; d < D; ++d) dot += V[(size_t)j * D + d] * ds[d];
            for (int d = 0; d < D; ++d) jds[d] += U[(size_t)j * D + d] * dot;
        }
        REAL ss = 0;
        for (int d = 0; d < D; ++d) ss += ds[d] * ds[d];
        for (int d = 0; d < D; ++d) {
            if (ss > 0) {
                U[(size_t)slot * D + d] = (df[d] - jds[d]) / ss;
                V[(size_t)slot * D + d] = ds[d];
            } else {
                U[(size_t)slot * D + d] = 0;
                V[(size_t)slot * D + d] = 0;
            }
        }
        return;
    }
    for (int d = 0; d < D; ++d) {
        V[(size_t)slot * D + d] = ds[d];
        F[(size_t)slot * D + d] = df[d];
    }
    const int n = (it < m) ? it : m;
    REAL *G = scr, *C = scr + (size_t)m * m, *y = C + (size_t)m * m;
    for (int a = 0; a < n; ++a)
        for (int b = 0; b < n; ++b) {
            REAL acc = 0;
            for (int d = 0; d < D; ++d) acc += V[(size_t)a * D + d] * V[(size_t)b * D + d];
            G[(size_t)a * m + b] = acc + ((a == b) ? lambda : (REAL)0);
        }
    /* Cholesky G = C C^T (C lower triangular) */
    int ok = 1;
    for (int a = 0; a < n && ok; ++a) {
        for (int b = 0; b <= a; ++b) {
            REAL acc = G[(size_t)a * m + b];
            for (int e = 0; e < b; ++e) acc -= C[(size_t)a * m + e] * C[(size_t)b * m + e];
            if (a == b) {
                if (!(acc > 0) || isinf((double)acc)) { ok = 0; break; }
                C[(size_t)a * m + a] = (REAL)sqrt((double)acc);
            } else {
                C[(size_t)a * m + b] = acc / C[(size_t)b * m + b];
            }
        }
    }
    for (int d = 0; d < D; ++d) {
        if (!ok) {
            for (int a = 0; a < m; ++a) U[(size_t)a * D + d] = 0;
            continue;
        }
        /* solve G y = F_d - alpha S_d: forward then backward substitution */
        for (int a = 0; a < n; ++a) {
            REAL acc = F[(size_t)a * D + d] - alpha * V[(size_t)a * D + d];
            for (int e = 0; e < a; ++e) acc -= C[(size_t)a * m + e] * y[e];
            y[a] = acc / C[(size_t)a * m + a];
        }
        for (int a = n - 1; a >= 0; --a) {
            REAL acc = y[a];
            for (int e = a + 1; e < n; ++e) acc -= C[(size_t)e * m + a] * y[e];
            y[a] = acc / C[(size_t)a * m + a];
        }
        for (int a = 0; a < n; ++a) U[(size_t)a * D + d] = y[a];
        for (int a = n; a < m; ++a) U[(size_t)a * D + d] = 0;
    }
}

/*
 * The parallel Broyden iteration for one sequence.  Iteration i:
 *   f_t = f(s^(i)_{t-1}, x_t);  res = max |s^(i)_t - f_t|;  stop as the Newton
 *   iteration does (converged at res <= tol, iters = i; else at the cap);
 *   for i >= 1 update every block from the secants against iteration i-1;
 *   delta from the compressed scan with c_t = f_t - s^(i)_t;  s^(i+1) = s^(i) + delta.
 * Iteration 0 has no secant yet: A_t = alpha I.
 */
static int FN(o_broyden_one)(const orc_cell *c, const float *x, const float *s0, int T, int rank,
                               int multisecant, double alpha_d, double damp, double lambda_d, int L,
                               const float *omega, double tol, int max_iter, const float *init,
                               REAL *s /*[T,D] out*/, int *iters_out, double *resid_out, double *hist,
                               REAL *work)
{
    const int D = c->D, m = rank;
    const size_t TD = (size_t)T * D, TMD = (size_t)T * m * D;
    REAL *f = work;                   /* [T,D] */
    REAL *fp = f + TD;                /* [T,D] previous f */
    REAL *sp = fp + TD;               /* [T,D] previous iterate */
    REAL *cc = sp + TD;               /* [T,D] */
    REAL *dl = cc + TD;               /* [T,D] */
    REAL *U = dl + TD;                /* [T,m,D] */
    REAL *V = U + TMD;                /* [T,m,D] */
    REAL *F = V + TMD;                /* [T,m,D] */
    REAL *Ud = F + TMD;               /* [T,m,D] damped */
    REAL *Om = Ud + TMD;              /* [D,m] */
    REAL *s0r = Om + (size_t)D * m;   /* D */
    REAL *ds = s0r + D, *df = ds + D; /* D each */
    REAL *tmp = df + D;               /* 6D */
    REAL *scr = tmp + 6 * D;          /* scan: 3 D + 7 m D + 2 m m; update: D + 2 m m + m */
    const REAL alpha = (REAL)alpha_d, lambda = (REAL)lambda_d, shrink = (REAL)(1.0 - damp);

    for (int d = 0; d < D; ++d) s0r[d] = s0 ? (REAL)s0[d] : (REAL)0;
    for (size_t e = 0; e < (size_t)D * m; ++e) Om[e] = (REAL)omega[e];
    for (size_t e = 0; e < TD; ++e) s[e] = init ? (REAL)init[e] : (REAL)0;
    for (size_t e = 0; e < TMD; ++e) U[e] = V[e] = F[e] = Ud[e] = 0;
    if (hist)
        for (int i = 0; i <= max_iter; ++i) hist[i] = NAN;

    for (int it = 0;; ++it) {
        double res = 0.0;
        int nonfinite = 0;
        for (int t = 0; t < T; ++t) {
            const REAL *sprev = (t == 0) ? s0r : s + (size_t)(t - 1) * D;
            FN(o_step)(c, sprev, x + (size_t)t * c->M, f + (size_t)t * D, NULL, NULL, tmp);
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
        if (it >= 1 && m > 0) {
            for (int t = 0; t < T; ++t) {
                for (int d = 0; d < D; ++d) {
                    const REAL a = (t == 0) ? s0r[d] : s[(size_t)(t - 1) * D + d];
                    const REAL b = (t == 0) ? s0r[d] : sp[(size_t)(t - 1) * D + d];
                    ds[d] = a - b;
                    df[d] = f[(size_t)t * D + d] - fp[(size_t)t * D + d];
                }
                FN(o_broyden_update_one)(multisecant, alpha, lambda, it, m, D, U + (size_t)t * m * D,
                                           V + (size_t)t * m * D, F + (size_t)t * m * D, ds, df, scr);
            }
        }
        const int n = (it < m) ? it : m;
        for (size_t e = 0; e < TMD; ++e) Ud[e] = shrink * U[e];
        for (size_t e = 0; e < TD; ++e) cc[e] = f[e] - s[e];
        FN(o_dplr_scan_one)(alpha, Ud, V, n, m, cc, T, D, L, Om, dl, scr);
        memcpy(sp, s, TD * sizeof(REAL));
        memcpy(fp, f, TD * sizeof(REAL));
        for (size_t e = 0; e < TD; ++e) s[e] = s[e] + dl[e];
    }
}

#undef FN
