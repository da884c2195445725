/*
 * gdn2.h — the Gated DeltaNet-2 recurrence and its VJP on MI355X (gfx950).
 *
 * Operation (burn_gdn source page "src/chunk_wy/custom_backward.rs": the direct
 * graph forward_impl, the chunk-boundary recompute recompute_chunk_states and
 * the generic recompute backward backward_impl).  Per batch entry and head,
 * a state S of shape [L, D] (latent x dense) evolves over t = 0 .. T-1 from
 * S = initial_state:
 *
 *     a = exp(log_decay_t)              (one factor per latent row)
 *     Dd = diag(a) S
 *     u = write_t * value_t - Dd^T (erase_t * key_t)
 *     S = Dd + key_t u^T
 *     context_t = S^T query_t / sqrt(L)
 *
 * The VJP takes the context's cotangent (and optionally the final state's)
 * and returns the cotangents of all seven inputs.
 *
 * Layout (row-major float32): query, key, erase, log_decay [B, H, T, L];
 * value, write, context [B, H, T, D]; initial_state, final state [B, H, L, D].
 * The saved state for the backward (`boundary`) and the backward's scratch
 * are internal formats whose sizes gdn2_boundary_bytes and gdn2_scratch_bytes
 * give; both must be 16-byte aligned.  LP is L rounded up to 16, 32 or 64.
 *
 * Two device forms, selected by `chunk`; the results agree to rounding.
 *
 * chunk 16 or 32: the chunk-WY form (the same page's tensor-core backward,
 * backward_chunk_wy_tensor_core_impl, and the factors it consumes), on
 * float32 MFMA.  Within a chunk, with c_t the cumulative decay from the chunk
 * start, the updates solve the unit-lower-triangular system
 * (I + A) U = write.value - M S0 (A = strictly lower (b k c)(k / c)^T); the
 * context, the end state and the VJP are chunk-sized matrix products.  The
 * forward writes, in `boundary`: the state before every chunk [B, H, chunks,
 * LP, D], one factor record per chunk, and the chunks' updates U [B, H,
 * chunks * chunk, D].  The backward carries the state cotangent through the
 * chunks in reverse (saving it per chunk in `scratch`, with the chunks' solved
 * right-hand sides), then forms every cotangent of every chunk in parallel.
 * Requires each chunk's cumulative decay to stay above about 1e-37 per latent
 * row (float32 range), as the page's form does.
 *
 * Any other chunk: the step-by-step recurrence.  A dense column's rows are
 * spread over 8 lanes (4 when L <= 16) and columns evolve independently, so
 * the forward runs one-wave blocks over a head's columns, with the step's
 * latent vectors broadcast through LDS; it saves the state every `chunk`
 * steps ([B, H, ceil(T / chunk), D, LP]).  The backward runs blocks of 8
 * waves (64 columns, 128 when L <= 16), several per head: it walks the chunks
 * in reverse, recomputes each chunk's states from its saved boundary (in
 * registers when chunk is 8, else into `scratch`), then reverses the chunk
 * step by step.  The latent-vector cotangents (query, key, erase, log_decay)
 * are sums over the dense axis, reduced across each block; with several
 * blocks per head their shares go through `scratch` and a second kernel adds
 * them in block order.  Results of this form do not depend on the chunk, bit
 * for bit.
 *
 * Arithmetic is float32.
 *
 * Limits: B, H, T, D, chunk >= 1; 1 <= L <= 64; D <= 1024; element counts
 * below 2^40.
 *
 * Conventions: device pointers owned by the caller; the library never
 * allocates, frees or keeps a pointer.  Validation happens on the host before
 * any HIP call; the return value is 0 or a negative QC_ERR_* code of
 * quat_cumprod.h (QC_ERR_NULL for a missing required pointer, QC_ERR_SHAPE for
 * sizes out of range, QC_ERR_ALIGN for a tensor pointer not 4-byte aligned or
 * a boundary or scratch pointer not 16-byte aligned,
 * QC_ERR_ALIAS for an output overlapping another buffer, QC_ERR_WORKSPACE for
 * a too-small scratch, QC_ERR_HIP for a failed launch).  Launches are
 * asynchronous on `stream` (a hipStream_t as void*).
 */
#ifndef QC_GDN2_H
#define QC_GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the saved state the forward writes for the backward (boundary
 * states, and for the chunk-WY form also the factor records and updates;
 * 0 if out of range). */
size_t gdn2_boundary_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk);

/* Bytes of the backward's scratch (0 if out of range). */
size_t gdn2_scratch_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk);

/* context (required), final_state (may be NULL) and the boundary states the
 * backward needs (may be NULL when no backward follows). */
int gdn2_fwd(const float* query, const float* key, const float* value, const float* erase, const float* write,
             const float* log_decay, const float* initial_state, float* context, float* final_state,
             float* boundary, int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk,
             void* stream);

/* VJP.  `boundary` is what gdn2_fwd wrote for the same inputs and chunk;
 * d_context is required, d_state (cotangent of the final state) may be NULL
 * (zero).  Each of the seven cotangent outputs may be NULL; if all are, the
 * call does nothing.  `scratch` holds gdn2_scratch_bytes and is overwritten. */
int gdn2_bwd(const float* query, const float* key, const float* value, const float* erase, const float* write,
             const float* log_decay, const float* boundary, const float* d_context, const float* d_state,
             float* d_query, float* d_key, float* d_value, float* d_erase, float* d_write, float* d_log_decay,
             float* d_initial_state, float* scratch, size_t scratch_bytes,
             int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QC_GDN2_H */
