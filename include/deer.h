/*
 * deer.h -- C interface of the MI355X (gfx950) parallel Newton solver for
 * nonlinear recurrences.
 *
 * The problem ("Parallel Broyden Methods for Efficiently Evaluating Nonlinear
 * State Space Models", section 2, problem statement): given a transition
 * s_t = f(s_{t-1}, x_t), inputs x_1..x_T and a fixed s_0, find the trajectory
 * s_1..s_T as the root of the residual r_t(s) = s_t - f(s_{t-1}, x_t)
 * ("Predictability Enables Parallelization of Nonlinear State Space Models",
 * rebuttal, its equation 2).  Each Newton iteration linearises f around the
 * current guess, s_t ~ A_t s_{t-1} + b_t, and solves that linear recurrence
 * with a parallel associative scan; A_t is the full Jacobian (DEER, dense
 * mode) or its diagonal (quasi-DEER, diag mode).
 *
 * Conventions for every call:
 *   - float32, row-major, contiguous; sequences are laid out [B, T, D] with D
 *     fastest.  Time index t = 0..T-1 holds the state after step t+1.
 *   - Pointers named "device" must be device memory of the current HIP device
 *     (hipMalloc / torch CUDA tensors); "host" pointers are ordinary memory.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All work
 *     is enqueued on it; outputs are complete once the stream is synchronised.
 *   - The library never allocates or frees caller memory and keeps no pointer
 *     after a call returns.  Scratch memory comes from the caller's workspace
 *     (linear_scan_diag_noalloc: from a static device array instead).
 *   - Return value: DEER_OK (0) on success, DEER_NOT_CONVERGED (1) when
 *     deer_solve or deer_solve_broyden stopped at least one sequence without
 *     converging (a result, not an error), a negative DEER_ERR_* code
 *     otherwise.  After a negative return
 *     deer_last_error() describes the problem.  Nothing is thrown across the
 *     interface.
 *   - One workspace must not be used by two calls that may run at the same
 *     time (different streams or threads).
 */
#ifndef DEER_H_
#define DEER_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Linearisation used by each iteration (the first page's thread: every method
 * linearises the dynamics, then evaluates the linear recurrence in parallel;
 * "Parallel Broyden Methods", section 2 and the Picard paragraph of its
 * diffusion experiment):
 *   DENSE   A_t = (1 - k) J_t, the full Jacobian   (Newton / DEER)
 *   DIAG    A_t = (1 - k) diag(J_t)                (diagonal quasi-Newton)
 *   JACOBI  A_t = 0: the next iterate is f of the current one, shifted by one step
 *   PICARD  A_t = I: the next iterate accumulates the one-step corrections
 * with offsets b_t = f_t - A_t s_{t-1}, so every mode keeps the trajectory as
 * its fixed point and recovers it exactly within T iterations.  k is the
 * damping option of deer_solve (scale-ELK: "Parallel Broyden Methods",
 * appendix E.4).
 */
enum deer_mode { DEER_MODE_DENSE = 0, DEER_MODE_DIAG = 1, DEER_MODE_JACOBI = 2, DEER_MODE_PICARD = 3 };

enum deer_cell { DEER_CELL_TANH = 0, DEER_CELL_GRU = 1 };

enum deer_status {
    DEER_OK = 0,
    DEER_NOT_CONVERGED = 1,
    DEER_ERR_INVALID = -1,      /* bad pointer, size or flag */
    DEER_ERR_UNSUPPORTED = -2,  /* shape or cell/mode pair outside the supported set */
    DEER_ERR_WORKSPACE = -3,    /* workspace missing, too small or misaligned */
    DEER_ERR_HIP = -4,          /* a HIP runtime call failed */
    DEER_ERR_DEVICE = -5        /* a kernel reported an internal failure (see deer_last_error) */
};

/* Per-sequence outcome written to status_out[b] by deer_solve. */
enum deer_seq_status {
    DEER_SEQ_CONVERGED = 0,      /* residual <= tol after iters_out[b] iterations */
    DEER_SEQ_NOT_CONVERGED = 1,  /* max_iter reached with a finite residual */
    DEER_SEQ_NONFINITE = 2,      /* max_iter reached with a NaN / Inf residual */
    DEER_SEQ_STALLED = 3         /* rounding stopped the finite-step progress (see deer_solve_opts_t) */
};

/*
 * Cell parameters (device pointers, float32).
 *   tanh:  f(s, x) = tanh(W s + U x + b)   -- the vector form of the scalar
 *          tanh model on the "Predictability" page (rebuttal, "Application to
 *          RNN training efficiency").  W [D,D], U [D,M], b [D] or NULL (zeros);
 *          b2 unused.
 *   GRU:   gate order (r, z, n); W = W_hh [3D,D], U = W_ih [3D,M],
 *          b = b_ih [3D] or NULL, b2 = b_hh [3D] or NULL:
 *            r = sigmoid(W_ih,r x + b_ih,r + W_hh,r s + b_hh,r)
 *            z = sigmoid(W_ih,z x + b_ih,z + W_hh,z s + b_hh,z)
 *            n = tanh(W_ih,n x + b_ih,n + r * (W_hh,n s + b_hh,n))
 *            f = (1 - z) * n + z * s
 *          (the GRU is only cited on the pages; these are its textbook
 *          equations).
 * Supported: 1 <= D <= 64, 1 <= M <= 1024.  tanh in every mode, GRU in the
 * diag, Jacobi and Picard modes.
 */
typedef struct {
    int cell;        /* enum deer_cell */
    int D;           /* state size */
    int M;           /* input size */
    const float *W;
    const float *U;
    const float *b;
    const float *b2;
} deer_cell_params_t;

/*
 * Options of deer_solve.  Passing NULL means DEER_SOLVE_OPTS_DEFAULT.
 *
 *   damping         k in [0, 1]: the blocks become (1 - k) J_t (dense) or
 *                   (1 - k) diag(J_t) (diag); must be 0 for Jacobi and Picard.
 *                   k = 0 is the undamped method, k = 1 turns it into Jacobi.
 *                   Damping keeps Newton's float32 iterates finite on
 *                   unpredictable dynamics ("Parallel Broyden Methods",
 *                   appendix E.4 and its full-rank RNN experiment).
 *   scan_f64        dense mode only: the linear solve accumulates its chunk
 *                   products, offsets and carried states in double precision
 *                   from the first iteration (inputs, outputs and the cell
 *                   evaluation stay float32).
 *   multi_launch    1: always run the multi-launch iteration loop.  Otherwise
 *                   tanh problems with D <= 4 and T <= 1024 run as one launch in
 *                   which one workgroup per sequence performs every iteration on
 *                   chip (same arithmetic and stopping rule; the scan tree
 *                   differs, so results differ only by rounding).
 *   stall_window    the finite-step check, 0 = off.  After i iterations the
 *                   first i states are exact in exact arithmetic ("Parallel
 *                   Broyden Methods", Theorem 1), so the first position whose
 *                   residual exceeds tol (the front) is never below i.  When a
 *                   sequence's best front stays below i and has not advanced for
 *                   stall_window iterations, rounding has stopped its progress:
 *                   it is stopped with DEER_SEQ_STALLED, unless escalation applies.
 *                   The check is off when tol < 0 (nothing passes; the call runs
 *                   exactly max_iter iterations).
 *   stall_escalate  dense mode, 1: the first stall switches the whole solve's
 *                   linear solve to double accumulation (as scan_f64) and the
 *                   stalled sequences go on; a stall after that stops them.  With
 *                   float32 products of many Jacobians of unpredictable dynamics,
 *                   rounding breaks the step-to-step consistency of the solved
 *                   trajectory at chunk boundaries; this is the stall it repairs.
 */
typedef struct {
    float damping;
    int scan_f64;
    int multi_launch;
    int stall_window;
    int stall_escalate;
} deer_solve_opts_t;
#define DEER_SOLVE_OPTS_DEFAULT {0.0f, 0, 0, 16, 1}

/*
 * Bytes of device workspace deer_solve needs for this problem and options
 * (opts may be NULL; host output).  Returns DEER_OK, or an error for an
 * unsupported problem.
 */
int deer_workspace_size(const deer_cell_params_t *p, int B, int T, int mode, const deer_solve_opts_t *opts,
                        size_t *bytes_out);

/*
 * Zero-fill a workspace on `stream`.  Every workspace (for deer_solve,
 * linear_scan_diag or linear_scan_dense) must be zero-filled once before its
 * first use -- by this call or any other zero fill; the calls themselves leave
 * it ready for the next call.  `workspace` device, 256-byte aligned.
 */
int deer_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * Solve for the trajectory by parallel Newton (mode DEER_MODE_DENSE), diagonal
 * quasi-Newton (DEER_MODE_DIAG), Jacobi or Picard iterations ("Parallel
 * Broyden Methods", section 2: exact parallel Newton and diagonal
 * quasi-Newton; finite-step recovery, Theorem 1 of section 3.2).
 *
 *   p           cell parameters (host struct holding device pointers)
 *   x           device [B,T,M] inputs
 *   s0          device [B,D] initial states, or NULL for zeros
 *   mode        enum deer_mode
 *   tol         stop when max_{t,d} |s_t - f(s_{t-1}, x_t)| <= tol for a
 *               sequence (absolute L-infinity residual, tested on each iterate
 *               before it is refined; NaN never passes)
 *   max_iter    iteration cap (>= 0); at most T iterations are ever needed in
 *               exact arithmetic
 *   opts        deer_solve_opts_t, or NULL for the defaults
 *   init_guess  device [B,T,D] starting trajectory, or NULL for zeros
 *   traj_out    device [B,T,D]: per sequence the first iterate that passed the
 *               test, or the iterate after max_iter iterations (or at the stall)
 *   iters_out   host [B]: iterations (linearise + solve steps) applied
 *   resid_out   host [B] or NULL: the L-infinity residual of the returned iterate
 *   rms_out     host [B] or NULL: its root-mean-square residual
 *               ||r||_2 / sqrt(T D) ("Parallel Broyden Methods", appendix D.2),
 *               computed by one more evaluation after the solve (only when asked)
 *   status_out  host [B] or NULL: enum deer_seq_status per sequence
 *   workspace   device, >= deer_workspace_size bytes, 256-byte aligned,
 *               zero-filled before its first use (deer_workspace_init)
 * Sequences are independent: each stops on its own and is frozen there.
 * The call enqueues its kernels on `stream`, polls a convergence flag on the
 * device once per batch of iterations (no per-iteration host sync), and
 * returns after the outputs are complete.  Returns DEER_NOT_CONVERGED when any
 * sequence did not converge (status 1, 2 or 3).
 *
 * The diagonal-block modes run the single-pass scan of linear_scan_diag,
 * whose progress does not depend on how much of its grid is resident (see
 * there).  The GRU's fused iteration (D = 32, 64) runs a single-pass scan over
 * a persistent grid sized to the device's resident capacity with a fixed tile
 * stride per workgroup, and tanh problems with D <= 16 and T <= 8192 whose
 * grid the device holds at once run the whole solve in one launch whose
 * workgroups wait on each other once per iteration.  Those two assume the
 * whole grid is resident at once: another kernel occupying compute units on a
 * concurrent stream can delay them; the waits are bounded, and if a bound is
 * hit the call returns DEER_ERR_DEVICE.
 */
int deer_solve(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T, int mode, float tol,
               int max_iter, const deer_solve_opts_t *opts, const float *init_guess, float *traj_out,
               int *iters_out, float *resid_out, float *rms_out, int *status_out, void *workspace, size_t ws_bytes,
               void *stream);

/*
 * Bytes of workspace linear_scan_diag / linear_scan_dense need (host output).
 */
int linear_scan_workspace_size(int B, int T, int D, int dense, size_t *bytes_out);

/*
 * Inclusive scan of the diagonal affine recurrence s_t = a_t * s_{t-1} + b_t
 * (elementwise per channel), s_{-1} = s0 ("Parallel Broyden Methods",
 * section 2, diagonal quasi-Newton: diagonal blocks stay diagonal under
 * composition; merge rule of appendix C.2).
 *   a, b   device [B,T,D];  s0 device [B,D] or NULL (zeros);  s device [B,T,D]
 *   (s may alias neither a nor b).  One pass: reads a and b once, writes s once.
 *   Any B, T >= 0, 1 <= D.
 * Tiles wait on earlier tiles of their channels (decoupled look-back) over a
 * persistent grid sized to the device's resident capacity.  Tiles are handed
 * out in index order from counters in the workspace, and only to running
 * workgroups, so every tile a workgroup waits on is held by a running one:
 * the scan completes whatever part of its grid is resident (a kernel
 * occupying compute units on a concurrent stream only slows it).  The waits
 * are bounded all the same; if a bound is hit the affected outputs are NaN.
 */
int linear_scan_diag(const float *a, const float *b, const float *s0, float *s, int B, int T, int D,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * linear_scan_diag for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same scan and the same results bit for bit, with the look-back state in
 * a static device array of DEER_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.  Neither this call nor
 * the kernels it launches allocate anything.
 *   Arguments as linear_scan_diag, without the workspace.
 *   Size limit: linear_scan_workspace_size(B, T, D, 0) must not exceed
 *   DEER_NOALLOC_SCRATCH_BYTES (about 3.5e8 elements for D a multiple of 4,
 *   a quarter of that otherwise); larger problems return
 *   DEER_ERR_UNSUPPORTED.
 *   The first call on a device clears the array and synchronises `stream`
 *   once.  All calls on one device share the array: calls that may overlap on
 *   one GPU (different streams or host threads) race and must be serialised
 *   by the caller.
 */
#define DEER_NOALLOC_SCRATCH_BYTES (64u << 20)
int linear_scan_diag_noalloc(const float *a, const float *b, const float *s0, float *s, int B, int T, int D,
                             void *stream);

/*
 * Scan of the dense affine recurrence s_t = A_t s_{t-1} + b_t, s_{-1} = s0,
 * with D x D blocks A_t (row-major, A_t[i][k] multiplies s_{t-1}[k]); later
 * blocks multiply on the left when segments merge ("Parallel Broyden
 * Methods", appendix C.2).
 *   A device [B,T,D,D];  b device [B,T,D];  s0 device [B,D] or NULL;
 *   s device [B,T,D].  1 <= D <= 64.
 */
int linear_scan_dense(const float *A, const float *b, const float *s0, float *s, int B, int T,
                      int D, void *workspace, size_t ws_bytes, void *stream);

/*
 * Sequential rollout s_t = f(s_{t-1}, x_t) on the GPU, one step after the
 * other (the evaluation the parallel methods are timed against on the
 * "Predictability" page, rebuttal "Comparison with sequential speed").  The
 * input projection U x_t + b runs first over all positions at once (it does
 * not depend on the state); then one workgroup per sequence steps the
 * recurrence.
 *   x device [B,T,M];  s0 device [B,D] or NULL;  traj_out device [B,T,D].
 *   workspace device, >= deer_rollout_workspace_size bytes, 256-byte aligned
 *   (no zero fill needed).
 */
int deer_rollout_workspace_size(const deer_cell_params_t *p, int B, int T, size_t *bytes_out);
int deer_rollout(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T,
                 float *traj_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Largest Lyapunov exponent of the dynamics along a given trajectory, per
 * sequence: a probe vector is pushed through the Jacobians J_t = d f / d s at
 * (s_{t-1}, x_t), renormalised after every step, and the log growth is
 * averaged over the T steps (natural log, per step, no burn-in).  This is the
 * estimator of the "Predictability Enables Parallelization" page (rebuttal,
 * "LLE computation cost"; its appendix's Algorithm 1); a negative value
 * predicts that parallel Newton converges in few iterations.
 *   p       cell parameters (any supported cell)
 *   x       device [B,T,M] inputs;  s0 device [B,D] or NULL (zeros)
 *   traj    device [B,T,D], the trajectory (traj[t] = state after step t+1)
 *   v0      device [B,D] probe vectors (need not be normalised; not all zero)
 *   lle_out device [B] float64
 *   workspace device, >= deer_lle_workspace_size bytes, 256-byte aligned
 * T must be positive.  The vector chain is sequential in t (one wavefront per
 * sequence); the Jacobian factors are evaluated in parallel beforehand.
 */
int deer_lle_workspace_size(const deer_cell_params_t *p, int B, int T, size_t *bytes_out);
int deer_lle(const deer_cell_params_t *p, const float *x, const float *s0, const float *traj, const float *v0,
             int B, int T, double *lle_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * Parallel Broyden ("Parallel Broyden Methods", sections 3.1-3.2, appendix E):
 * quasi-Newton blocks built from trajectory secants, no Jacobian evaluated.
 * Block at position t: A_t = alpha I + (1 - damping) U_t V_t^T with at most
 * `rank` columns; each iteration i >= 1 folds in the secant pair
 * (s^(i)_{t-1} - s^(i-1)_{t-1}, f^(i)_t - f^(i-1)_t) into column slot
 * (i - 1) mod rank, by a rank-one "good Broyden" update after dropping that
 * slot's column (multisecant = 0) or by refitting all stored secants,
 * U = (F - alpha S)(S^T S + gram_reg I)^{-1}, V = S (multisecant = 1).  The
 * linear step solves the increment recurrence delta_t = A_t delta_{t-1} +
 * (f_t - s_t) by a chunked scan: chunks of `chunk` positions are replayed
 * exactly; chunk carries go through chunk aggregates whose low-rank part is
 * re-compressed to `rank` columns with the random sketch (range of
 * L (R^T sketch), modified Gram-Schmidt).  Exact zeros stay exact, so the
 * first i positions are exact after i iterations (finite-step recovery).
 */
typedef struct {
    int rank;             /* columns per block, 0..8 (0: A_t = alpha I) */
    int multisecant;      /* 0: rank-one updates with truncation; 1: multisecant refit */
    float alpha;          /* diagonal baseline alpha I (finite) */
    float damping;        /* in [0, 1]: the low-rank correction is scaled by 1 - damping */
    float gram_reg;       /* >= 0, added to the diagonal of S^T S (multisecant) */
    int chunk;            /* positions per scan chunk, 1..4096 */
    const float *sketch;  /* device [D, rank] random sketch; may be NULL when rank = 0 (and for the size query) */
    int stall_window;     /* finite-step check as in deer_solve_opts_t (0 = off); a stall stops the sequence */
} deer_broyden_opts_t;

/* Bytes of workspace deer_solve_broyden needs (host output). */
int deer_broyden_workspace_size(const deer_cell_params_t *p, int B, int T, const deer_broyden_opts_t *opts,
                                size_t *bytes_out);

/*
 * Solve for the trajectory with parallel Broyden iterations.  Arguments, the
 * stopping rule, freezing, outputs and polling are those of deer_solve; the
 * workspace (>= deer_broyden_workspace_size bytes, 256-byte aligned) needs no
 * zero fill.  Cells: tanh and GRU.  Iteration 0 uses A_t = alpha I.
 */
int deer_solve_broyden(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T,
                       const deer_broyden_opts_t *opts, float tol, int max_iter, const float *init_guess,
                       float *traj_out, int *iters_out, float *resid_out, int *status_out, void *workspace,
                       size_t ws_bytes, void *stream);

/* Bytes of workspace linear_scan_dplr needs (host output). */
int linear_scan_dplr_workspace_size(int B, int T, int D, int rank, int chunk, size_t *bytes_out);

/*
 * The chunked compressed scan alone: delta_t = (alpha I + U_t V_t^T) delta_{t-1} + c_t,
 * delta_{-1} = 0, with the chunk carries re-compressed as deer_solve_broyden does.
 *   U, V    device [B,T,rank,D] (column j of position t contiguous)
 *   c       device [B,T,D];  delta device [B,T,D] (aliases none of the inputs)
 *   sketch  device [D, rank];  1 <= D <= 64, 0 <= rank <= 8, 1 <= chunk <= 4096
 */
int linear_scan_dplr(float alpha, const float *U, const float *V, const float *c, const float *sketch,
                     float *delta, int B, int T, int D, int rank, int chunk, void *workspace, size_t ws_bytes,
                     void *stream);

/*
 * Per-kernel timing of deer_solve, for measurement.  While enabled, deer_solve
 * records a pair of HIP events on its stream around every launch of the named
 * kernel class and accumulates the elapsed time; reading returns the number of
 * launches timed and their summed milliseconds and resets the counters.
 *   which: 0 = cell evaluation (f and Jacobian), 1 = linear scan,
 *          2 = input projection, 3 = convergence check, 4 = the dense
 *          scan's chunk compose alone (a part of 1; dense tanh at D = 32 in
 *          float also evaluates the cell for the next iteration inside 1,
 *          so 0 counts only the first evaluation there).  deer_solve_broyden
 *          times its cell evaluation (0), block updates with the compressed
 *          scan (1), projection (2) and check (3) the same way.  Solves that
 *          run in one launch count it as 0 (the dense one-launch solve its
 *          double-precision continuation as 1).
 */
int deer_profile_enable(int enable);
int deer_profile_read(int which, long long *launches, double *milliseconds);

/*
 * Measurement utility, not part of the method: the HBM rate a plain streaming
 * kernel reaches on this device for a given read / write mix (the bench
 * reports its kernels against it next to the datasheet peak).  Reads all of
 * src and writes all of dst once, both as contiguous streams of 16-byte
 * non-temporal accesses: with k = src_bytes / dst_bytes, output vector
 * 64 g + l (16 bytes) is the XOR of input vectors 64 (k g + j) + l, j < k
 * (a last partial group of r < 64 outputs: input vectors
 * 64 k G + r j + l, G full groups); k = 1 is a copy.
 * Device pointers; dst_bytes and the addresses multiples of 16, k in
 * {1, 2, 4, 8}, buffers not overlapping (DEER_ERR_INVALID otherwise).
 * Asynchronous on the stream.
 */
int deer_bandwidth_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes, void *stream);

/* Thread-local description of the last failure (never NULL). */
const char *deer_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DEER_H_ */
