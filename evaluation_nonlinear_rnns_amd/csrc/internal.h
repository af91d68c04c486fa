// Internal declarations shared by the HIP translation units of libdeer.
// Not part of the public interface (include/deer.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/deer.h"

namespace deer {

// ----------------------------------------------------------------- errors
void set_error(const std::string &msg);
int fail(int code, const std::string &msg);
int hip_fail(hipError_t e, const char *what);

#define DEER_HIP(call)                                       \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return ::deer::hip_fail(e_, #call); \
    } while (0)

// --------------------------------------------------------------- constants
constexpr int kWave = 64;
constexpr int kMaxD = 64;
constexpr int kMaxM = 1024;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// Cursor that hands out 256-byte aligned regions of a workspace.
struct Carve {
    char *base;
    size_t off = 0;
    explicit Carve(void *p) : base(static_cast<char *>(p)) {}
    template <class T>
    T *take(size_t count) {
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += align_up(count * sizeof(T));
        return p;
    }
};

// ------------------------------------------------------ diagonal scan state
// Look-back state kept in a workspace between launches.  Zero-filled once by
// the caller; every launch leaves done = 0 and advances epoch.
struct ScanHeader {
    unsigned reserved;
    unsigned done;     // workgroups finished in the current launch
    unsigned epoch;    // tags descriptors of the current launch
    unsigned abort;    // set if a bounded wait gave up (should never happen)
    unsigned pad[60];
};
static_assert(sizeof(ScanHeader) == 256, "header is one alignment unit");

// Geometry of one diagonal-scan launch.
struct DiagScanPlan {
    int B, T, D;
    int vec;        // 4 when D % 4 == 0, else 1
    int ch;         // channels per tile
    int chunk_len;  // time steps per chunk
    int groups;     // channel tiles per sequence
    int chains;     // B * groups
    int nchunk;     // chunks per chain
    size_t desc_words;
};
DiagScanPlan diag_scan_plan(int B, int T, int D);
size_t diag_scan_state_bytes(int B, int T, int D);

// Enqueue the single-pass diagonal scan.  `out_sel` (device int or null)
// selects out1 when odd, out0 otherwise; `skip` (device int[B] or null)
// skips sequences whose flag is set; `all_done` (device int or null) skips
// the whole launch when set.
int launch_diag_scan(const float *a, const float *b, const float *s0, float *out0, float *out1,
                     const int *out_sel, const int *skip, const int *all_done, int B, int T, int D,
                     void *state, hipStream_t stream);

// ---------------------------------------------------------- dense scan
struct DenseScanPlan {
    int B, T, D;
    int chunk_len;
    int nchunk;     // chunks per sequence
};
DenseScanPlan dense_scan_plan(int B, int T, int D);
size_t dense_scan_state_bytes(int B, int T, int D);

// Dense scan s_t = A_t s_{t-1} + b_t.  Either A (materialised [B,T,D,D]) or
// the factored form A_t = diag(d_t) W (d [B,T,D], W [D,D]) is given.
int launch_dense_scan(const float *A, const float *d, const float *W, const float *b,
                      const float *s0, float *out0, float *out1, const int *out_sel,
                      const int *skip, const int *all_done, int B, int T, int D, void *state,
                      hipStream_t stream);

// ---------------------------------------------------------- cell kernels
// p = U x + bias for every position, O outputs.  `tiled` writes the layout
// the matrix-core GRU evaluation reads (see cell_mfma.hip); row-major [B,T,O]
// otherwise.
int launch_projection(const float *x, const float *U, const float *bias, float *p, int B, int T, int M,
                      int O, bool tiled, hipStream_t stream);
size_t projection_floats(int B, int T, int O);

// tanh cell: f_t = tanh(W s_{t-1} + p_t).  Dense mode writes the factored
// leaf d_t = 1 - f_t^2 into `lin` and b_t = f_t - d_t * (W s_{t-1}); diag mode
// writes a_t = d_t * diag(W) into `lin` and b_t = f_t - a_t * s_{t-1}.
// res_bits[b] receives atomic max of |s_t - f_t| (float bits).
int launch_tanh_eval(const float *W, const float *p, const float *s0, const float *s_even,
                     const float *s_odd, const int *sel, const int *skip, const int *all_done,
                     float *lin, float *bvec, unsigned *res_bits, int B, int T, int D, int dense,
                     hipStream_t stream);

// GRU cell, diagonal Jacobian: writes a_t = diag(d f / d s) and
// b_t = f_t - a_t * s_{t-1}.  With gru_fast_path(D, M) the projection is
// tiled and the evaluation runs on the matrix cores.
bool gru_fast_path(int D, int M);
int launch_gru_eval(const float *Whh, const float *bhh, const float *p, const float *s0,
                    const float *s_even, const float *s_odd, const int *sel, const int *skip,
                    const int *all_done, float *a, float *bvec, unsigned *res_bits, int B, int T,
                    int D, int M, hipStream_t stream);

// Matrix-core versions (cell_mfma.hip) for the supported sizes.
bool gru_mfma_supported(int D);
int launch_gru_eval_mfma(const float *Whh, const float *bhh, const float *p, const float *s0,
                         const float *s_even, const float *s_odd, const int *sel, const int *skip,
                         const int *all_done, float *a, float *bvec, unsigned *res_bits, int B, int T,
                         int D, hipStream_t stream);
bool proj_mfma_supported(int M, int O);
size_t proj_tiled_floats(int B, int T, int O);
int launch_projection_mfma(const float *x, const float *U, const float *bias, float *p, int B, int T,
                           int M, int O, bool tiled, hipStream_t stream);

// Fused quasi-DEER iteration for the GRU on the matrix cores: evaluation and
// diagonal scan in one persistent launch, writing s^(i+1) into the buffer
// that does not hold s^(i).  res_tile[tile] receives the residual maximum of
// every TP-position tile (gru_step_tile(D) positions).
int gru_step_tile(int D);
size_t gru_step_state_bytes(int B, int T, int D);
int launch_gru_quasi_step(const float *Whh, const float *bhh, const float *pt, const float *s0, float *s_even,
                          float *s_odd, const int *sel, const int *skip, const int *all_done,
                          unsigned *res_tile, int B, int T, int D, void *state, hipStream_t stream);

int launch_rollout(const deer_cell_params_t *p, const float *x, const float *s0, int B, int T,
                   float *traj, hipStream_t stream);

}  // namespace deer
