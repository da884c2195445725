// gdn2_internal.hpp -- declarations shared by the Gated DeltaNet-2 entry
// points (gdn2.hip) and its chunk-WY kernels (gdn2_wy.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace qc {

// Chunk sizes that select the chunk-WY path (fp32 MFMA); every other chunk
// runs the step-by-step recurrent kernels.
constexpr bool wy_chunk(int64_t chunk) { return chunk == 16 || chunk == 32; }

// Dense columns per block of the sequential chunk-WY kernels.
constexpr int kWyDense = 32;

// Floats of one chunk's factor record (M, Qc, Kt [cp][lp]; T, Bq [cp][cp];
// c_last [lp]), rounded up to 256 bytes.  The chunk-WY forward keeps these
// records after the boundary states, for the backward.
constexpr int64_t wy_record_floats(int64_t cp, int64_t lp) { return (3 * cp * lp + 2 * cp * cp + lp + 63) / 64 * 64; }

struct WyArgs {
    const float *q, *k, *v, *b, *w, *g, *s0;   // inputs
    float *ctx, *state, *bnd;                   // forward outputs (bnd: [BH, n_chunks, LP, D])
    float* rec;                                 // factor records [BH, n_chunks, wy_record_floats] (after the states), or null
    float* ubuf;                                // the chunks' updates U [BH, n_chunks * chunk, D] (after the records), or null
    float* drhs;                                // backward scratch after dbnd: drhs [BH, n_chunks * chunk, D]
    const float *bnd_in, *dctx, *dstate;        // backward inputs
    float *dq, *dk, *dv, *db, *dw, *dg, *ds0;   // backward outputs (each may be null)
    float* dbnd;                                // backward scratch: [BH, n_chunks, LP, D], the state cotangent entering each chunk from later ones
    int64_t BH, T, L, D, n_chunks;
    int n_dt;                                   // dense tiles per head: ceil(D / kWyDense)
    float scale;                                // 1 / sqrt(L)
};

hipError_t launch_wy_forward(int chunk, int lp, const WyArgs& a, hipStream_t st);
hipError_t launch_wy_backward(int chunk, int lp, const WyArgs& a, hipStream_t st);

}  // namespace qc
