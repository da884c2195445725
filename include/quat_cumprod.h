/*
 * quat_cumprod.h -- C ABI of the MI355X (gfx950) quaternion cumulative-product
 * scan and its vector-Jacobian product.
 *
 * What is computed (burn-mamba source page
 * "burn_mamba/mamba3/quat_scan/backward.rs", module doc "Gradient math"):
 *
 *   forward   cum[t] = q_t (x) cum[t-1],  cum[-1] = init,  t = 0 .. s-1
 *             (equivalently cum[t] = P_t (x) init with P_t = q_t (x) ... (x) q_0)
 *   backward  given the cotangent d_cum of cum:
 *             S[t]   = sum_{u >= t} conj(P_u) (x) d_cum[u]     (reverse cumsum)
 *             G[t]   = P_t (x) S[t] / |P_t|^2
 *             d_q[t] = G[t] (x) conj(cum[t-1])                 (cum[-1] = init)
 *             d_init = S[0]
 *
 * (x) is the Hamilton product on scalar-first quaternions (w, x, y, z) with
 * i^2 = j^2 = k^2 = ijk = -1; conj(w, x, y, z) = (w, -x, -y, -z).  The page
 * states the closed form for unit quaternions (|P_t| = 1); the division by
 * |P_t|^2 keeps it the exact VJP of the given, rounded inputs, which are never
 * exactly unit.  It requires every prefix product P_t to be non-zero in the
 * working precision (no exactly-zero step q_t); otherwise the backward's
 * results are not finite and the workspace status reports QC_STATUS_ZERO (the
 * forward is exact for any input).
 *
 * Any gradient of the final carry cum[:, s-1] must already be added into
 * d_cum[:, s-1]: the page folds it there before the backward node runs, so the
 * node has a single cotangent input.
 *
 * Tensor layout (row-major, contiguous, no strides):
 *   q, cum, d_cum, d_q : [b, s, h, j, 4]    init, d_init : [b, h, j, 4]
 * The quaternion columns of one (b, t) row are the h*j contiguous entries.
 *
 * Storage dtypes: QC_DTYPE_F32 (float32 I/O, float64 arithmetic inside) and
 * QC_DTYPE_BF16 (bfloat16 I/O as raw 16-bit patterns, float32 arithmetic
 * inside, round-to-nearest-even stores).
 *
 * Pointers:
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     owned by the caller.  The library never allocates, frees or keeps a
 *     pointer after a call returns.
 *   - Alignment: 16 bytes for float32 tensors, 8 bytes for bfloat16 tensors,
 *     16 bytes for ckpt and workspace.
 *   - Outputs must not overlap any input, the workspace or each other.
 *   - stream is a hipStream_t passed as void*; NULL is the null stream.
 *
 * Calls are asynchronous: arguments are validated on the host before any HIP
 * call, then kernels are enqueued on `stream`.  A negative return value means
 * nothing was enqueued (except QC_ERR_HIP, which means a launch failed).
 *
 * Workspace: a device buffer of at least quat_cumprod_workspace_bytes(...)
 * bytes, holding a status word, a launch counter, self-validating cross-block
 * carries and (for a backward without saved boundary state) re-derived
 * boundary products.  Zero it once after allocation
 * (quat_cumprod_workspace_init does so on a stream; hipMemset also works);
 * every call leaves it ready for the next one, whatever the shape.  Calls
 * sharing one workspace must be ordered (same stream or synchronised);
 * concurrent calls need separate workspaces.
 *
 * HIP graphs: quat_cumprod_fwd/_bwd (and the _ex forms) may be called on a
 * stream that is capturing.  They then also capture a one-thread kernel that
 * advances the workspace's launch counter, so every replay of the graph gets
 * carries of its own; replays must be ordered like any other calls on that
 * workspace.  Capture calls no HIP function other than kernel launches and
 * hipStreamIsCapturing; quat_cumprod_workspace_status synchronises and must
 * not be captured.
 */
#ifndef QUAT_CUMPROD_H
#define QUAT_CUMPROD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of q, init, cum, d_cum, d_q, d_init. */
enum {
    QC_DTYPE_F32 = 0,
    QC_DTYPE_BF16 = 1
};

/* Return codes. */
enum {
    QC_OK = 0,
    QC_ERR_NULL = -1,       /* a required pointer is NULL */
    QC_ERR_SHAPE = -2,      /* a dimension < 1, or sizes overflow the library's limits */
    QC_ERR_ALIGN = -3,      /* a pointer is not aligned as required */
    QC_ERR_DTYPE = -4,      /* unknown dtype */
    QC_ERR_ALIAS = -5,      /* an output overlaps an input, another output or the workspace */
    QC_ERR_WORKSPACE = -6,  /* workspace or ckpt buffer NULL or too small */
    QC_ERR_HIP = -7,        /* a HIP runtime call failed (see quat_cumprod_last_hip_error) */
    QC_ERR_OPTION = -8      /* invalid qc_options field */
};

/* Execution-path choice for the *_ex entry points. */
enum {
    QC_PATH_AUTO = 0,       /* library heuristic */
    QC_PATH_COLUMN = 1,     /* one lane walks a whole column sequentially */
    QC_PATH_CHUNKED = 2,    /* sequence-parallel tiles with cross-block carries (one pass, look-back) */
    QC_PATH_RSCAN = 3       /* the same tiles, reduce-then-scan: tile aggregates, a scan of them, a
                               fix-up pass that re-reads the tile's inputs (never chosen by AUTO) */
};

/* Cross-tile carry scheme of the look-back path (QC_PATH_AUTO / QC_PATH_CHUNKED). */
enum {
    QC_LOOKBACK_AUTO = 0,     /* library heuristic */
    QC_LOOKBACK_FENWICK = 1,  /* each tile reads about log2(position) published partial products */
    QC_LOOKBACK_GROUPED = 2   /* tiles and groups of about sqrt(tiles) publish their aggregates; a
                                 tile reads its group's earlier tiles and the earlier groups (two
                                 publish-to-read round trips deep; AUTO takes it for launches of
                                 at most a few thousand tiles) */
};

/* How a backward without saved boundary state (ckpt = NULL) obtains the
 * prefix products before its tiles (QC_PATH_AUTO / QC_PATH_CHUNKED). */
enum {
    QC_LEAVES_AUTO = 0,       /* library heuristic */
    QC_LEAVES_PREPASS = 1,    /* a forward pass over q writes them into the workspace first (one more
                                 read of q) */
    QC_LEAVES_CORESIDENT = 2  /* one cooperative pass: groups of blocks that hold a whole chain's tiles
                                 at once also run a forward look-back among themselves, so q is read
                                 once.  Taken when at least one chain fits on the device at once and
                                 the stream is not capturing a graph; otherwise the pre-pass runs.
                                 Never chosen by AUTO (slower than the pre-pass where measured). */
};

/* What the forward saves into the ckpt buffer and the backward reads from it.
 * Forward and backward of one scan must use the same kind.  The backward's
 * formula is the one stated at the top either way; with QC_SAVED_FINAL it is
 * evaluated from the end of the sequence: G[t] by the page's reverse
 * recurrence G[t] = d_cum[t] + conj(q_{t+1}) (x) G[t+1], and cum[t-1] as
 * q_t^-1 (x) cum[t] from the final carry (products over later steps, inverted;
 * the same non-zero precondition as above). */
enum {
    QC_SAVED_BOUNDARY = 0,  /* the prefix products at a fixed stride of steps (quat_cumprod_ckpt_bytes):
                               the backward reads q and d_cum once */
    QC_SAVED_FINAL = 1      /* only the final carry cum[:, s-1] of every column, in the internal
                               precision (b*h*j quaternions): the backward still reads q and d_cum
                               once, from this alone (look-back paths; with QC_PATH_COLUMN the
                               column backward recomputes from q and ignores it; QC_PATH_RSCAN
                               refuses it) */
};

typedef struct {
    int32_t path;           /* QC_PATH_* */
    int32_t lookback;       /* QC_LOOKBACK_*; ignored by the other paths */
    int32_t leaves;         /* QC_LEAVES_*; ignored when a ckpt is given */
    int32_t saved;          /* QC_SAVED_*: the kind of the ckpt buffer, if one is given */
    int32_t reserved[4];    /* must be zero */
} qc_options;

/* Bytes of workspace that quat_cumprod_fwd and quat_cumprod_bwd need for this
 * shape and dtype (one workspace serves both).  Returns 0 for invalid
 * arguments. */
size_t quat_cumprod_workspace_bytes(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype);

/* Bytes of the optional saved boundary state ("ckpt") that the forward can
 * write and the backward can read: the prefix products P at a fixed stride
 * of sequence steps, kept in the internal precision.  Its contents are
 * internal to this library; only its size is part of the ABI.  Returns 0 for
 * invalid arguments. */
size_t quat_cumprod_ckpt_bytes(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype);

/* Same for the ckpt kind that opts->saved names (opts may be NULL = the
 * boundary state); QC_SAVED_FINAL needs b*h*j quaternions in the internal
 * precision, whatever s.  Returns 0 for invalid arguments or options. */
size_t quat_cumprod_ckpt_bytes_ex(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                                  const qc_options* opts);

/* Zero a workspace on `stream` with a fill kernel (so it may be captured in a
 * HIP graph).  Needed once per allocation. */
int quat_cumprod_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Forward scan (the page's Mamba3QuatScanBackendExt::quat_cumprod).
 *   q      [b,s,h,j,4] in      init [b,h,j,4] in      cum [b,s,h,j,4] out
 *   ckpt   optional out (NULL = none): saved state for the backward,
 *          ckpt_bytes >= quat_cumprod_ckpt_bytes(...) (the _ex form: of the
 *          kind opts->saved, sized by quat_cumprod_ckpt_bytes_ex). */
int quat_cumprod_fwd(const void* q, const void* init, void* cum,
                     void* ckpt, size_t ckpt_bytes,
                     int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward (the page's quat_scan_backward): recomputes the prefix products
 * from the saved leaves q and init, never from stored scan intermediates.
 *   q, init, d_cum   in
 *   ckpt             optional in (NULL = none): the state written by
 *                    quat_cumprod_fwd for the same q, init, shape, dtype (and,
 *                    for the _ex forms, the same opts->saved).  With it the
 *                    backward reads q and d_cum once; without it the backward
 *                    first re-derives the boundary prefix products from q (one
 *                    more read of q).
 *   d_q [b,s,h,j,4], d_init [b,h,j,4]   out, each optional (NULL = not
 *                    wanted, as for an untracked input); both NULL is a no-op. */
int quat_cumprod_bwd(const void* q, const void* init, const void* d_cum,
                     const void* ckpt, size_t ckpt_bytes,
                     void* d_q, void* d_init,
                     int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Same as above with an explicit path choice (opts may be NULL = defaults). */
int quat_cumprod_fwd_ex(const void* q, const void* init, void* cum,
                        void* ckpt, size_t ckpt_bytes,
                        int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const qc_options* opts);
int quat_cumprod_bwd_ex(const void* q, const void* init, const void* d_cum,
                        const void* ckpt, size_t ckpt_bytes,
                        void* d_q, void* d_init,
                        int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const qc_options* opts);

/* Backward without a caller workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as quat_cumprod_bwd, bit for bit,
 * except that the workspace is a fixed device array of this library: 64 MiB
 * per GPU, held by each GPU the library runs on until the process ends.  It
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   status   optional out (NULL = not wanted): a device int32 that receives
 *            the QC_STATUS_* bits raised by this call (0 = normal), written
 *            on `stream` after the backward; 4-byte aligned, not overlapping
 *            any tensor of the call.
 * Shapes whose quat_cumprod_workspace_bytes exceeds 64 MiB are rejected with
 * QC_ERR_WORKSPACE before any HIP call (float32, b8 s4096 h32 j32 with 33.5
 * million quaternions needs 56.5 MiB; the workspace grows with the number of
 * quaternions and of columns).  The first call on a device (with that device current) looks up
 * the array's device address and zeroes its header on `stream`; make it
 * outside a graph capture to keep that fill out of the graph.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU race
 * (order them on one stream, or synchronise).  Each call leaves the array's
 * status word cleared. */
int quat_cumprod_bwd_noalloc(const void* q, const void* init, const void* d_cum,
                             const void* ckpt, size_t ckpt_bytes,
                             void* d_q, void* d_init,
                             int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                             int32_t* status, void* stream);

/* Synchronise `stream`, then read the workspace's device-side status word, a
 * bit mask accumulated over the calls since it was last cleared:
 *   0                   every call completed normally;
 *   QC_STATUS_TIMEOUT   a cross-block wait hit its spin limit: results of some
 *                       call since the last clear are invalid;
 *   QC_STATUS_ZERO      a backward met a prefix product that is exactly zero
 *                       (a zero step q_t, or an underflow to zero), outside the
 *                       documented precondition: its d_q / d_init hold
 *                       non-finite values.
 * clear != 0 resets the word to 0. */
enum {
    QC_STATUS_TIMEOUT = 1,
    QC_STATUS_ZERO = 2
};
int quat_cumprod_workspace_status(void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t clear, int32_t* status_out);

/* Static description of a return code. */
const char* quat_cumprod_strerror(int32_t code);

/* Text of the last HIP error this library saw on the calling thread ("" if none). */
const char* quat_cumprod_last_hip_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t quat_cumprod_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QUAT_CUMPROD_H */
