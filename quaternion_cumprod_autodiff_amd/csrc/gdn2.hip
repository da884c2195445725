// gdn2.hip -- gfx950 kernels and C-ABI entry points of include/gdn2.h: the
// Gated DeltaNet-2 recurrence (the direct graph of the burn_gdn source page
// "src/chunk_wy/custom_backward.rs") and its VJP (the page's generic
// recompute backward: chunk boundary states, in-chunk recompute, per-step
// reverse sweep).
//
// Forward: one thread per dense column d of one (batch, head); the column
// S[:, d] of the state lives in registers (columns never interact: the
// read-out u[d] and the write S[:, d] += k u[d] only touch column d).  The
// step's latent vectors (q, k, decay, erased key) are the same for every
// column, so one wave stages them in LDS and every lane reads them as
// broadcasts; the next step's vectors are loaded while this step computes.
//
// Backward: one block per (batch, head), one thread per dense column (D <= 256,
// so 4 waves at most and the whole register file of a SIMD per wave).  Chunks
// are taken in reverse; each is recomputed from its saved boundary state, the
// state before every step going to a per-head scratch slot (each thread
// writes and reads back only its own column), then reversed step by step.
// The cotangents of the dense vectors (value, write) and of the state are
// per column; those of the latent vectors (query, key, erase, log_decay) are
// sums over the dense axis: every lane holds one contribution per latent row,
// a transpose-reduce across the wave (log2(64) shuffle stages that halve the
// rows each lane carries) leaves every lane with one row's wave sum, and the
// waves' sums meet in LDS.
#include "gdn2.h"
#include "qc_internal.hpp"
#include "quat_cumprod.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace qc {
namespace {

constexpr int kMaxLatent = 64;
constexpr int kMaxDense = 256;
constexpr int64_t kMaxElems = int64_t(1) << 40;

struct Gdn2Args {
    const float *q, *k, *v, *b, *w, *g, *s0;
    float *ctx, *state, *bnd;   // forward outputs
    const float* bnd_in;        // boundary states read by the backward
    const float *dctx, *dstate;
    float *dq, *dk, *dv, *db, *dw, *dg, *ds0;
    float* scratch;
    int64_t T, L, D, chunk, n_chunks, scratch_steps;
    float scale;
};

// Step vectors in LDS, by row l: query, key, erase, decay = exp(log_decay),
// erased key = erase * key.  Rows L .. LM-1 are zero (decay 1), so padded
// rows of the state stay zero and contribute nothing.
enum { kVq = 0, kVk = 1, kVb = 2, kVa = 3, kVe = 4, kNVec = 5 };

// Loads row `row` (< LM) of step t's vectors into r[0..3] (q, k, b, g).
__device__ __forceinline__ void load_step_row(const Gdn2Args& a, int64_t bh, int64_t t, int row, float* r) {
    if (row < a.L) {
        const int64_t i = (bh * a.T + t) * a.L + row;
        r[0] = a.q[i];
        r[1] = a.k[i];
        r[2] = a.b[i];
        r[3] = a.g[i];
    } else {
        r[0] = r[1] = r[2] = r[3] = 0.0f;
    }
}

template <int LM>
__device__ __forceinline__ void put_step_row(float (*s)[LM], int row, const float* r) {
    s[kVq][row] = r[0];
    s[kVk][row] = r[1];
    s[kVb][row] = r[2];
    s[kVa][row] = expf(r[3]);
    s[kVe][row] = r[2] * r[1];
}

// Sum of x[0..N) over the wave's lanes, transposed: stage by stage (xor
// offsets O = 32, 16, ...), each lane keeps the half of its rows selected by
// its lane bit O and adds the partner's copy of those rows, so after
// log2(N) stages it holds one row; the remaining offsets sum the lanes that
// hold the same row.  Lane l ends with the sum of row l >> (6 - log2(LM)).
template <int N, int O>
__device__ __forceinline__ float wave_row_sum(const float (&x)[N], int lane) {
    if constexpr (N == 1) {
        float s = x[0];
#pragma unroll
        for (int o = O; o >= 1; o >>= 1) s += __shfl_xor(s, o);
        return s;
    } else {
        float y[N / 2];
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            const float keep = up ? x[j + N / 2] : x[j];
            const float send = up ? x[j] : x[j + N / 2];
            y[j] = keep + __shfl_xor(send, O);
        }
        return wave_row_sum<N / 2, O / 2>(y, lane);
    }
}

template <int LM>
constexpr int row_shift() {
    return LM == 64 ? 0 : LM == 32 ? 1 : LM == 16 ? 2 : 3;
}

// The boundary states and the backward's scratch keep each dense column's LM
// rows contiguous ([.., d, LM]), so a column moves as LM/4 float4 at
// immediate offsets from one per-thread address (a [L, D] layout would need
// a separate uniform base per row).
template <int LM>
__device__ __forceinline__ void store_column(float* p, const float (&x)[LM]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int i = 0; i < LM / 4; ++i) q[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}

template <int LM>
__device__ __forceinline__ void load_column(const float* p, float (&x)[LM]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < LM / 4; ++i) {
        const float4 v = q[i];
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
    }
}

// ------------------------------------------------------------------ forward

template <int LM>
__global__ void __launch_bounds__(64) gdn2_fwd_kernel(Gdn2Args a) {
    __shared__ float s_vec[2][kNVec][LM];
    const int lane = threadIdx.x;
    const int64_t n_db = (a.D + 63) / 64;
    const int64_t bh = blockIdx.x / n_db;
    const int64_t d = (blockIdx.x % n_db) * 64 + lane;
    const bool dok = d < a.D;

    float S[LM];
#pragma unroll
    for (int l = 0; l < LM; ++l) S[l] = (dok && l < a.L) ? a.s0[(bh * a.L + l) * a.D + d] : 0.0f;

    float r[4];
    if (lane < LM) {
        load_step_row(a, bh, 0, lane, r);
        put_step_row<LM>(s_vec[0], lane, r);
    }
    __syncthreads();
    for (int64_t t = 0; t < a.T; ++t) {
        const int buf = int(t & 1);
        const bool more = t + 1 < a.T;
        if (more && lane < LM) load_step_row(a, bh, t + 1, lane, r);   // in flight during this step
        if (a.bnd != nullptr && t % a.chunk == 0 && dok)
            store_column<LM>(a.bnd + ((bh * a.n_chunks + t / a.chunk) * a.D + d) * LM, S);
        const int64_t e = (bh * a.T + t) * a.D + d;
        const float vv = dok ? a.v[e] : 0.0f, ww = dok ? a.w[e] : 0.0f;
        float read = 0.0f;
#pragma unroll
        for (int l = 0; l < LM; ++l) {
            S[l] *= s_vec[buf][kVa][l];
            read = fmaf(s_vec[buf][kVe][l], S[l], read);
        }
        const float u = ww * vv - read;
        float o = 0.0f;
#pragma unroll
        for (int l = 0; l < LM; ++l) {
            S[l] = fmaf(s_vec[buf][kVk][l], u, S[l]);
            o = fmaf(s_vec[buf][kVq][l], S[l], o);
        }
        if (dok) a.ctx[e] = o * a.scale;
        if (more && lane < LM) put_step_row<LM>(s_vec[buf ^ 1], lane, r);
        __syncthreads();
    }
    if (a.state != nullptr && dok) {
#pragma unroll
        for (int l = 0; l < LM; ++l)
            if (l < a.L) a.state[(bh * a.L + l) * a.D + d] = S[l];
    }
}

// ----------------------------------------------------------------- backward

template <int LM>
__global__ void __launch_bounds__(kMaxDense) gdn2_bwd_kernel(Gdn2Args a) {
    constexpr int kWaves = kMaxDense / 64;
    __shared__ float s_vec[2][kNVec][LM];
    __shared__ float s_red[2][kWaves][4][LM];   // per wave: query, key (outer part), erased key, decay
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_waves = int(blockDim.x >> 6);
    const int64_t bh = blockIdx.x;
    const int64_t d = tid;
    const bool dok = d < a.D;
    constexpr int kShift = row_shift<LM>();
    const int row = lane >> kShift;
    const bool row_writer = (lane & ((1 << kShift) - 1)) == 0;

    float G[LM];   // cotangent reaching the current state, column d
#pragma unroll
    for (int l = 0; l < LM; ++l)
        G[l] = (a.dstate != nullptr && dok && l < a.L) ? a.dstate[(bh * a.L + l) * a.D + d] : 0.0f;

    // Per-head scratch: the state before each step of the current chunk.
    float* scr = a.scratch + (bh * a.scratch_steps * a.D + (dok ? d : 0)) * LM;
    const int64_t scr_step = a.D * LM;
    int it = 0;   // step counter over both sweeps: alternates the LDS buffers
    for (int64_t c = a.n_chunks - 1; c >= 0; --c) {
        const int64_t t0 = c * a.chunk;
        const int64_t t1 = t0 + a.chunk < a.T ? t0 + a.chunk : a.T;

        // Recompute the chunk from its boundary; keep the state before each
        // step.  The next step's vectors and dense values load while this one
        // computes.
        float S[LM];
        if (dok) {
            load_column<LM>(a.bnd_in + ((bh * a.n_chunks + c) * a.D + d) * LM, S);
        } else {
#pragma unroll
            for (int l = 0; l < LM; ++l) S[l] = 0.0f;
        }
        float r[4];
        float vv = 0.0f, ww = 0.0f;
        if (tid < LM) load_step_row(a, bh, t0, tid, r);
        if (dok) {
            vv = a.v[(bh * a.T + t0) * a.D + d];
            ww = a.w[(bh * a.T + t0) * a.D + d];
        }
        for (int64_t t = t0; t < t1; ++t, ++it) {
            const int buf = it & 1;
            if (tid < LM) put_step_row<LM>(s_vec[buf], tid, r);
            __syncthreads();
            const float v_now = vv, w_now = ww;
            if (t + 1 < t1) {
                if (tid < LM) load_step_row(a, bh, t + 1, tid, r);
                if (dok) {
                    vv = a.v[(bh * a.T + t + 1) * a.D + d];
                    ww = a.w[(bh * a.T + t + 1) * a.D + d];
                }
            }
            if (dok) store_column<LM>(scr + (t - t0) * scr_step, S);
            float read = 0.0f;
#pragma unroll
            for (int l = 0; l < LM; ++l) {
                S[l] *= s_vec[buf][kVa][l];
                read = fmaf(s_vec[buf][kVe][l], S[l], read);
            }
            const float u = w_now * v_now - read;
#pragma unroll
            for (int l = 0; l < LM; ++l) S[l] = fmaf(s_vec[buf][kVk][l], u, S[l]);
        }

        // Reverse the chunk, prefetching one step ahead (downwards) likewise.
        float dd = 0.0f;
        if (tid < LM) load_step_row(a, bh, t1 - 1, tid, r);
        if (dok) {
            const int64_t e = (bh * a.T + t1 - 1) * a.D + d;
            vv = a.v[e];
            ww = a.w[e];
            dd = a.dctx[e];
        }
        for (int64_t t = t1 - 1; t >= t0; --t, ++it) {
            const int buf = it & 1;
            if (tid < LM) put_step_row<LM>(s_vec[buf], tid, r);
            __syncthreads();
            const float(*sv)[LM] = s_vec[buf];
            const int64_t e = (bh * a.T + t) * a.D + d;
            float Sp[LM];   // state before step t, column d
            if (dok) {
                load_column<LM>(scr + (t - t0) * scr_step, Sp);
            } else {
#pragma unroll
                for (int l = 0; l < LM; ++l) Sp[l] = 0.0f;
            }
            const float v_now = vv, w_now = ww, dov = dd * a.scale;
            if (t > t0) {
                if (tid < LM) load_step_row(a, bh, t - 1, tid, r);
                if (dok) {
                    vv = a.v[e - a.D];
                    ww = a.w[e - a.D];
                    dd = a.dctx[e - a.D];
                }
            }
            float read = 0.0f;
#pragma unroll
            for (int l = 0; l < LM; ++l) read = fmaf(sv[kVe][l], sv[kVa][l] * Sp[l], read);
            const float u = w_now * v_now - read;

            // Read-out: the state after the step, and G += q do^T / sqrt(L).
            float x[LM];
#pragma unroll
            for (int l = 0; l < LM; ++l) {
                x[l] = fmaf(sv[kVa][l], Sp[l], sv[kVk][l] * u) * dov;   // S_t[l] * do / sqrt(L)
                G[l] = fmaf(sv[kVq][l], dov, G[l]);
            }
            const float r_q = wave_row_sum<LM, 32>(x, lane);
            // Rank-1 write: d u = G^T k, and G u (the key's outer-product part).
            float du = 0.0f;
#pragma unroll
            for (int l = 0; l < LM; ++l) {
                du = fmaf(G[l], sv[kVk][l], du);
                x[l] = G[l] * u;
            }
            const float r_k = wave_row_sum<LM, 32>(x, lane);
            if (dok) {
                if (a.dw != nullptr) a.dw[e] = du * v_now;
                if (a.dv != nullptr) a.dv[e] = du * w_now;
            }
            // Erased read-out: its cotangent is -du; the erased key gets
            // (decayed state) (-du), the decayed state gets e (-du).
            const float dr = -du;
#pragma unroll
            for (int l = 0; l < LM; ++l) x[l] = sv[kVa][l] * Sp[l] * dr;
            const float r_e = wave_row_sum<LM, 32>(x, lane);
#pragma unroll
            for (int l = 0; l < LM; ++l) {
                const float dD = fmaf(sv[kVe][l], dr, G[l]);   // cotangent of the decayed state
                x[l] = dD * Sp[l];
                G[l] = sv[kVa][l] * dD;                         // cotangent of the state before step t
            }
            const float r_a = wave_row_sum<LM, 32>(x, lane);
            if (row_writer) {
                s_red[buf][wave][0][row] = r_q;
                s_red[buf][wave][1][row] = r_k;
                s_red[buf][wave][2][row] = r_e;
                s_red[buf][wave][3][row] = r_a;
            }
            __syncthreads();
            if (tid < a.L) {
                float sq = 0.0f, sk = 0.0f, se = 0.0f, sa = 0.0f;
                for (int wv = 0; wv < n_waves; ++wv) {
                    sq += s_red[buf][wv][0][tid];
                    sk += s_red[buf][wv][1][tid];
                    se += s_red[buf][wv][2][tid];
                    sa += s_red[buf][wv][3][tid];
                }
                const int64_t i = (bh * a.T + t) * a.L + tid;
                if (a.dq != nullptr) a.dq[i] = sq;
                if (a.dk != nullptr) a.dk[i] = fmaf(se, sv[kVb][tid], sk);
                if (a.db != nullptr) a.db[i] = se * sv[kVk][tid];
                if (a.dg != nullptr) a.dg[i] = sa * sv[kVa][tid];
            }
        }
    }
    if (a.ds0 != nullptr && dok) {
#pragma unroll
        for (int l = 0; l < LM; ++l)
            if (l < a.L) a.ds0[(bh * a.L + l) * a.D + d] = G[l];
    }
}

// ------------------------------------------------------------ host helpers

struct Sizes {
    int64_t BH, T, L, D, chunk, n_chunks, scratch_steps;
    int lm;
};

int check_sizes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk, Sizes* z) {
    if (B < 1 || H < 1 || T < 1 || L < 1 || D < 1 || chunk < 1) return QC_ERR_SHAPE;
    if (L > kMaxLatent || D > kMaxDense) return QC_ERR_SHAPE;
    if (B > kMaxElems / H) return QC_ERR_SHAPE;
    z->BH = B * H;
    if (z->BH > (int64_t(1) << 31) / ((D + 63) / 64)) return QC_ERR_SHAPE;
    if (T > kMaxElems / z->BH || z->BH * T > kMaxElems / (L > D ? L : D)) return QC_ERR_SHAPE;
    z->T = T; z->L = L; z->D = D; z->chunk = chunk;
    z->n_chunks = (T + chunk - 1) / chunk;
    z->scratch_steps = chunk < T ? chunk : T;
    if (z->BH * z->n_chunks > kMaxElems / (L * D)) return QC_ERR_SHAPE;
    z->lm = L <= 8 ? 8 : L <= 16 ? 16 : L <= 32 ? 32 : 64;
    if (z->BH * (z->n_chunks > z->scratch_steps ? z->n_chunks : z->scratch_steps) > kMaxElems / (z->lm * D))
        return QC_ERR_SHAPE;
    return QC_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

struct Span {
    const void* p;
    size_t n;
};

bool overlaps(Span x, Span y) {
    if (!x.p || !y.p || !x.n || !y.n) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x.p), b = reinterpret_cast<uintptr_t>(y.p);
    return a < b + y.n && b < a + x.n;
}

// The first n_out spans are outputs: each must miss every other span.
bool any_overlap(const Span* s, int n_out, int n) {
    for (int i = 0; i < n_out; ++i)
        for (int j = 0; j < n; ++j)
            if (i != j && overlaps(s[i], s[j])) return true;
    return false;
}

template <class F>
hipError_t by_latent(int lm, F&& f) {
    switch (lm) {
        case 8: return f(std::integral_constant<int, 8>{});
        case 16: return f(std::integral_constant<int, 16>{});
        case 32: return f(std::integral_constant<int, 32>{});
        default: return f(std::integral_constant<int, 64>{});
    }
}

}  // namespace
}  // namespace qc

extern "C" {

size_t gdn2_boundary_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk) {
    qc::Sizes z;
    if (qc::check_sizes(B, H, T, L, D, chunk, &z) != QC_OK) return 0;
    return size_t(z.BH * z.n_chunks * D * z.lm) * sizeof(float);
}

size_t gdn2_scratch_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk) {
    qc::Sizes z;
    if (qc::check_sizes(B, H, T, L, D, chunk, &z) != QC_OK) return 0;
    return size_t(z.BH * z.scratch_steps * D * z.lm) * sizeof(float);
}

int gdn2_fwd(const float* query, const float* key, const float* value, const float* erase, const float* write,
             const float* log_decay, const float* initial_state, float* context, float* final_state,
             float* boundary, int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk,
             void* stream) {
    qc::Sizes z;
    int rc = qc::check_sizes(B, H, T, L, D, chunk, &z);
    if (rc != QC_OK) return rc;
    if (!query || !key || !value || !erase || !write || !log_decay || !initial_state || !context) return QC_ERR_NULL;
    for (const void* p : {static_cast<const void*>(query), static_cast<const void*>(key),
                          static_cast<const void*>(value), static_cast<const void*>(erase),
                          static_cast<const void*>(write), static_cast<const void*>(log_decay),
                          static_cast<const void*>(initial_state), static_cast<const void*>(context),
                          static_cast<const void*>(final_state), static_cast<const void*>(boundary)})
        if (p && !qc::aligned4(p)) return QC_ERR_ALIGN;
    const size_t f = sizeof(float);
    const size_t nl = size_t(z.BH * T * L) * f, nd = size_t(z.BH * T * D) * f, ns = size_t(z.BH * L * D) * f;
    const size_t nb = size_t(z.BH * z.n_chunks * D * z.lm) * f;
    if (boundary && (reinterpret_cast<uintptr_t>(boundary) & 15)) return QC_ERR_ALIGN;
    const qc::Span sp[] = {{context, nd}, {final_state, ns}, {boundary, nb},
                           {query, nl}, {key, nl}, {value, nd}, {erase, nl}, {write, nd}, {log_decay, nl},
                           {initial_state, ns}};
    if (qc::any_overlap(sp, 3, 10)) return QC_ERR_ALIAS;
    qc::Gdn2Args a{};
    a.q = query; a.k = key; a.v = value; a.b = erase; a.w = write; a.g = log_decay; a.s0 = initial_state;
    a.ctx = context; a.state = final_state; a.bnd = boundary;
    a.T = T; a.L = L; a.D = D; a.chunk = chunk; a.n_chunks = z.n_chunks; a.scratch_steps = z.scratch_steps;
    a.scale = 1.0f / sqrtf(float(L));
    const unsigned blocks = unsigned(z.BH * ((D + 63) / 64));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = qc::by_latent(z.lm, [&](auto lm) {
        void* params[] = {&a};
        return hipLaunchKernel(reinterpret_cast<const void*>(&qc::gdn2_fwd_kernel<decltype(lm)::value>),
                               dim3(blocks), dim3(64), params, 0, st);
    });
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

int gdn2_bwd(const float* query, const float* key, const float* value, const float* erase, const float* write,
             const float* log_decay, const float* boundary, const float* d_context, const float* d_state,
             float* d_query, float* d_key, float* d_value, float* d_erase, float* d_write, float* d_log_decay,
             float* d_initial_state, float* scratch, size_t scratch_bytes,
             int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk, void* stream) {
    qc::Sizes z;
    int rc = qc::check_sizes(B, H, T, L, D, chunk, &z);
    if (rc != QC_OK) return rc;
    if (!query || !key || !value || !erase || !write || !log_decay || !boundary || !d_context) return QC_ERR_NULL;
    if (!d_query && !d_key && !d_value && !d_erase && !d_write && !d_log_decay && !d_initial_state) return QC_OK;
    const size_t f = sizeof(float);
    const size_t nl = size_t(z.BH * T * L) * f, nd = size_t(z.BH * T * D) * f, ns = size_t(z.BH * L * D) * f;
    const size_t nb = size_t(z.BH * z.n_chunks * D * z.lm) * f;
    const size_t nscr = size_t(z.BH * z.scratch_steps * D * z.lm) * f;
    if (!scratch || scratch_bytes < nscr) return QC_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(boundary) & 15) || (reinterpret_cast<uintptr_t>(scratch) & 15)) return QC_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(query), static_cast<const void*>(key),
                          static_cast<const void*>(value), static_cast<const void*>(erase),
                          static_cast<const void*>(write), static_cast<const void*>(log_decay),
                          static_cast<const void*>(boundary), static_cast<const void*>(d_context),
                          static_cast<const void*>(d_state), static_cast<const void*>(d_query),
                          static_cast<const void*>(d_key), static_cast<const void*>(d_value),
                          static_cast<const void*>(d_erase), static_cast<const void*>(d_write),
                          static_cast<const void*>(d_log_decay), static_cast<const void*>(d_initial_state),
                          static_cast<const void*>(scratch)})
        if (p && !qc::aligned4(p)) return QC_ERR_ALIGN;
    const qc::Span sp[] = {{d_query, nl}, {d_key, nl}, {d_value, nd}, {d_erase, nl}, {d_write, nd},
                           {d_log_decay, nl}, {d_initial_state, ns}, {scratch, nscr},
                           {query, nl}, {key, nl}, {value, nd}, {erase, nl}, {write, nd}, {log_decay, nl},
                           {boundary, nb}, {d_context, nd}, {d_state, ns}};
    if (qc::any_overlap(sp, 8, 17)) return QC_ERR_ALIAS;
    qc::Gdn2Args a{};
    a.q = query; a.k = key; a.v = value; a.b = erase; a.w = write; a.g = log_decay; a.bnd_in = boundary;
    a.dctx = d_context; a.dstate = d_state;
    a.dq = d_query; a.dk = d_key; a.dv = d_value; a.db = d_erase; a.dw = d_write; a.dg = d_log_decay;
    a.ds0 = d_initial_state; a.scratch = scratch;
    a.T = T; a.L = L; a.D = D; a.chunk = chunk; a.n_chunks = z.n_chunks; a.scratch_steps = z.scratch_steps;
    a.scale = 1.0f / sqrtf(float(L));
    const unsigned threads = unsigned((D + 63) / 64 * 64);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = qc::by_latent(z.lm, [&](auto lm) {
        void* params[] = {&a};
        return hipLaunchKernel(reinterpret_cast<const void*>(&qc::gdn2_bwd_kernel<decltype(lm)::value>),
                               dim3(unsigned(z.BH)), dim3(threads), params, 0, st);
    });
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

}  // extern "C"
