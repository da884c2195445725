/*
 * qc_scan.h — a scan over per-column carries and its VJP on MI355X (gfx950),
 * with the saved trajectory either kept whole or replaced by k snapshots and
 * recomputation (binomial checkpointing).
 *
 * Operation (rlx-autodiff source page "src/decompose_backward.rs": the Scan,
 * ScanBackward and ScanBackwardXs ops, their lowering, and the tests
 * "decompose_scan_backward_length_129" and "decompose_scan_backward_griewank"):
 *
 *     c[-1] = init,   c[t] = f(c[t-1], x[t])   (t = 0 .. s-1),   ys[t] = c[t]
 *
 * and, given an upstream cotangent u[t] for every saved carry, the VJP
 *
 *     g[s-1] = u[s-1],   d_x[t] = J_x(c[t-1], x[t])^T g[t],
 *     g[t-1] = u[t-1] + J_c(c[t-1], x[t])^T g[t],   d_init = g[-1].
 *
 * Bodies (QC_SCAN_BODY_*), each with its carry width w (floats per element):
 *   ADD  (w = 1): f(c, x) = c + x, the body of the page's scan tests.
 *   QUAT (w = 4): f(c, x) = x (x) c, Hamilton product, scalar first: the
 *        quaternion cumulative product of the burn-mamba source page
 *        "burn_mamba/mamba3/quat_scan/backward.rs" ("Gradient math"), whose
 *        per-factor VJPs give J_c^T g = conj(x) (x) g and J_x^T g = g (x) conj(c).
 *
 * Layout: xs, ys, upstream, d_xs are [b][s][m][w] float32, row-major;
 * init, d_init are [b][m][w] float32.  A column is one (b, m) sequence; the
 * device code runs one column per thread, sequentially in t, in float64, so
 * it fills the GPU only with many columns (b*m in the hundreds of thousands).
 * Snapshots are [k][b*m][w] float64.
 *
 * Checkpointing: with k snapshot slots (slot 0 holds init), the schedule from
 * qc_scan_schedule reverses the s steps with the least number of recomputed
 * forward steps (Griewank's binomial checkpointing, the "Griewank" case of
 * the page: a trajectory of k checkpoints instead of all s carries).  The
 * schedule is built on the host, once per (s, k), copied by the caller to
 * device memory, and interpreted by every column alike.
 *
 * Conventions: all pointers except the schedule's host buffer are device
 * pointers owned by the caller; the library never allocates, frees or keeps a
 * pointer.  Calls validate on the host before any HIP call and return 0 or a
 * negative QC_ERR_* code from quat_cumprod.h; launches are asynchronous on
 * `stream` (a hipStream_t as void*).  Float32 tensors need 4-byte alignment
 * (ADD) or 16-byte alignment (QUAT); snapshots 16 bytes.  Outputs must not
 * overlap inputs or each other.
 */
#ifndef QC_SCAN_H
#define QC_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QC_SCAN_BODY_ADD = 0, QC_SCAN_BODY_QUAT = 1 };

/* Schedule actions: records of four int32 {op, a, b, 0}. */
enum {
    QC_SCAN_STORE = 1,    /* snapshot[a] = current carry                         */
    QC_SCAN_LOAD = 2,     /* current carry = snapshot[a]                         */
    QC_SCAN_ADVANCE = 3,  /* apply steps a .. b-1 to the current carry           */
    QC_SCAN_REVERSE = 4   /* VJP of step a; the current carry must be c[a-1]     */
};

typedef struct {
    int64_t n_actions;      /* records written                                          */
    int64_t bwd_start;      /* first record not done by qc_scan_fwd with the schedule    */
    int64_t forward_steps;  /* body evaluations in records [0, n_actions)                */
    int64_t prefix_steps;   /* body evaluations in records [0, bwd_start)                */
} qc_scan_plan;

/* Carry width w of a body, or 0 for an unknown body. */
int32_t qc_scan_width(int32_t body);

/* Records a schedule for s steps and k snapshots can need (4 s + 2); 0 if s < 1. */
int64_t qc_scan_schedule_capacity(int64_t s);

/* Host only.  Writes the binomial-checkpointing schedule for s steps (1 <= s
 * < 2^31) and k snapshot slots (1 <= k <= 4096, slot 0 = init) into `actions`
 * (host memory, `capacity` records; NULL to only fill `plan`).  The records
 * [0, bwd_start) are STORE and ADVANCE only, end with a STORE, and form the
 * forward sweep's part.  Returns QC_ERR_SHAPE for bad s or k, QC_ERR_WORKSPACE
 * if `capacity` is too small. */
int qc_scan_schedule(int64_t s, int32_t k, int32_t* actions, int64_t capacity, qc_scan_plan* plan);

/* ys = the scan of xs from init (every carry).  If `schedule` (device copy of
 * the records) is non-NULL, the records [0, bwd_start) are carried out on the
 * way, which fills the snapshots a later qc_scan_bwd_checkpointed started at
 * bwd_start needs; `snaps` (k * b * m * w doubles) is then required.  ys may be
 * NULL when only the snapshots are wanted. */
int qc_scan_fwd(int32_t body, const float* xs, const float* init, float* ys,
                int64_t b, int64_t s, int64_t m,
                const int32_t* schedule, int64_t bwd_start, double* snaps, int32_t k,
                void* stream);

/* VJP from the whole saved trajectory ys (the page's ScanBackward with every
 * carry saved): reads xs, init, ys, upstream; writes d_xs and d_init (each may
 * be NULL, not both). */
int qc_scan_bwd_trajectory(int32_t body, const float* xs, const float* init, const float* ys,
                           const float* upstream, float* d_xs, float* d_init,
                           int64_t b, int64_t s, int64_t m, void* stream);

/* VJP from k snapshots: interprets records [start, n_actions) of the device
 * schedule (start = 0: from init alone, the snapshots are scratch; start =
 * bwd_start: after qc_scan_fwd filled them).  Every record is checked on the
 * device; a record out of range (slot >= k, step outside [0, s)) stops the
 * column and sets bit 1 of *status (device word, may be NULL).  The snapshot
 * buffer is overwritten. */
int qc_scan_bwd_checkpointed(int32_t body, const float* xs, const float* init, const float* upstream,
                             float* d_xs, float* d_init, int64_t b, int64_t s, int64_t m,
                             const int32_t* schedule, int64_t n_actions, int64_t start,
                             double* snaps, int32_t k, uint32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QC_SCAN_H */
