// gdn2_wy.hip -- the Gated DeltaNet-2 recurrence and its VJP in chunk-WY form
// on gfx950 float32 MFMA (v_mfma_f32_16x16x4_f32).
//
// The form (burn_gdn source page "src/chunk_wy/custom_backward.rs", the
// tensor-core backward backward_chunk_wy_tensor_core_impl and the factors it
// consumes: the cumulative decay, the m/w bases and the unit-lower-triangular
// WY system).  Inside a chunk of C steps with state S0 at its start, let
// c_t = exp(g_0 + ... + g_t) per latent row (g = log_decay, t local), and
//   Qc_t = q_t c_t,   M_t = b_t k_t c_t,   Wb_t = k_t / c_t      (rows of [C, L])
//   A  = strictly lower part of M Wb^T,   Bq = lower part (with diagonal) of Qc Wb^T
// The recurrence u_t = w_t v_t - (diag(a_t) S_{t-1})^T (b_t k_t) unrolls to
// (I + A) U = w.v - M S0, so with T = (I + A)^-1
//   U     = T (w.v - M S0)                       (the chunk's updates, [C, D])
//   O     = (Qc S0 + Bq U) / sqrt(L)             (the chunk's context)
//   S_end = diag(c_last) S0 + Kt^T U,  Kt_t = k_t c_last / c_t
// and the VJP, given dO and the cotangent dS of S_end (dSc = diag(c_last) dS):
//   dU   = Bq^T dO / sqrt(L) + Wb dSc,   drhs = T^T dU
//   dS0  = Qc^T dO / sqrt(L) + dSc - M^T drhs           (carried to the previous chunk)
//   dw = drhs . v,  dv = drhs . w
//   dBq  = lower(dO U^T) / sqrt(L),      dA = -strictly lower(drhs U^T)
//   dQc  = dO S0^T / sqrt(L) + dBq Wb,   dM = -drhs S0^T + dA Wb
//   dWb  = dBq^T Qc + U dSc^T + dA^T M
//   dq = dQc c,  db = dM k c,  dk = dM b c + dWb / c,
//   dg_t = sum_{u >= t} (dQc.Qc + dM.M - dWb.Wb)_u  (+ rowsum(dSc . (S0 + Wb^T U)) at the last step)
// The products with c and 1/c stay in range while a chunk's cumulative decay
// stays above about 1e-37 per latent row.
//
// Kernels (256 threads = 4 waves; chunks of CP = 16 or 32 steps; latent
// rows padded to LP = 16, 32 or 64; every matrix product is 16x16 output
// tiles of the f32 MFMA, operands read from LDS):
//   wy_fwd_kernel       one block per (head, 32 dense columns): the chunks in
//                       order, the state tile in LDS; saves the state at every
//                       chunk start (the boundary states).
//   wy_bwd_carry_kernel one block per (head, 32 dense columns): the chunks in
//                       reverse, carrying dS; saves the dS entering every
//                       chunk from later ones (scratch), and d initial_state.
//   wy_bwd_grad_kernel  one block per (head, chunk), all chunks at once: from
//                       the chunk's boundary state and its dS, every
//                       cotangent of the chunk's steps; the sums over the
//                       dense axis stay in MFMA accumulators across the
//                       block's walk over 32-column dense tiles.
// Each kernel recomputes the chunk's factors (c, Qc, M, Wb, Kt, A, T, Bq)
// from the inputs with the same code, so all three see the same bits.
// Padded steps (past T in the last chunk) have k = q = b = v = w = g = 0: they
// leave the state unchanged and get no output.
#include "gdn2_internal.hpp"
#include "qc_internal.hpp"

namespace qc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kDN = kWyDense;   // dense columns per tile
constexpr int kDS = kDN + 4;    // LDS row stride of [rows][kDN] tiles

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A(m0 + 0..15, k0 + 0..K) B(k0 + 0..K, n0 + 0..15) on one wave, K a
// multiple of 4.  `a` points at A(m0, k0) and `b` at B(k0, n0); A(m, k) is
// a[m * SAM + k * SAK] and B(k, n) is b[k * SBK + n * SBN] (strides select
// transposes).  Lane l feeds A(l % 16, 4i + l / 16) and B(4i + l / 16, l % 16)
// to step i and ends with rows 4 (l / 16) + r, column l % 16 in acc[r].
template <int SAM, int SAK, int SBK, int SBN>
__device__ __forceinline__ void mma(f32x4& acc, const float* a, const float* b, int K, int lane) {
    const int i = lane & 15, kq = lane >> 4;
    a += i * SAM + kq * SAK;
    b += kq * SBK + i * SBN;
#pragma unroll 4
    for (int k = 0; k < K; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k * SAK], b[k * SBK], acc, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int lane, int r) { return 4 * (lane >> 4) + r; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

// Lower-triangle tile (ti >= tj) number j of an NT x NT tile grid, row by row.
__device__ __forceinline__ void lower_tile(int j, int& ti, int& tj) {
    ti = 0;
    while (j > ti) {
        j -= ti + 1;
        ++ti;
    }
    tj = j;
}

// One chunk's factors in LDS.  Thread (rg, l), rg = tid / LP, owns latent row
// l of the chunk's steps rg*RPT .. rg*RPT + RPT - 1.
template <int CP, int LP, bool kKt>
struct Factors {
    static constexpr int LS = LP + 4;    // row stride of [CP][LP]
    static constexpr int CS = CP + 4;    // row stride of [CP][CP]
    static constexpr int RG = kThreads / LP;
    static constexpr int RPT = CP / RG;
    static constexpr int NT = CP / 16;
    float Qc[CP * LS], M[CP * LS], Wb[CP * LS];
    float Kt[kKt ? CP * LS : 1];
    float Tm[CP * CS];     // A, then T = (I + A)^-1 (upper part zero)
    float Bq[CP * CS];     // lower part of Qc Wb^T (upper part zero)
    float tot[RG * LP];    // per-group sums of log_decay
    float clast[LP];       // c at the chunk's last (padded) step
    float tmp[16 * 20];
};

template <int RPT>
struct LatIn {
    float q[RPT], k[RPT], b[RPT], g[RPT];
};

// Latent inputs of chunk rows rg*RPT + i (zero past T or past L).
template <int CP, int LP, int RPT>
__device__ __forceinline__ void load_latent(const WyArgs& a, int64_t head, int64_t t0, int tid, LatIn<RPT>& in) {
    constexpr int RG = kThreads / LP;
    static_assert(RG * RPT == CP, "rows per thread");
    const int l = tid % LP, rg = tid / LP;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t t = t0 + rg * RPT + i;
        in.q[i] = in.k[i] = in.b[i] = in.g[i] = 0.f;
        if (t < a.T && l < a.L) {
            const int64_t idx = (head * a.T + t) * a.L + l;
            in.q[i] = a.q[idx];
            in.k[i] = a.k[idx];
            in.b[i] = a.b[idx];
            in.g[i] = a.g[idx];
        }
    }
}

// Builds Qc, M, Wb (and Kt), A, Bq in LDS, then T in place of A (wave 0,
// without a closing barrier: callers reach one before reading T).  e and ie
// receive c and 1/c of this thread's rows.  Starts and ends reading nothing
// that the caller may still be writing: the first barrier comes after the
// group sums are stored.
template <int CP, int LP, bool kKt, int RPT>
__device__ void make_factors(Factors<CP, LP, kKt>& f, const LatIn<RPT>& in, int tid, float* e, float* ie) {
    using F = Factors<CP, LP, kKt>;
    constexpr int LS = F::LS, CS = F::CS, RG = F::RG, NT = F::NT;
    const int lane = tid & 63, wave = tid >> 6;
    const int l = tid % LP, rg = tid / LP;

    float G[RPT];
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        run += in.g[i];
        G[i] = run;
    }
    f.tot[rg * LP + l] = run;
    __syncthreads();
    float off = 0.f, Gl = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const float v = f.tot[r * LP + l];
        if (r < rg) off += v;
        Gl += v;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float Gt = off + G[i];
        e[i] = __expf(Gt);
        ie[i] = __expf(-Gt);
        const int row = rg * RPT + i;
        f.Qc[row * LS + l] = in.q[i] * e[i];
        f.M[row * LS + l] = (in.b[i] * in.k[i]) * e[i];
        f.Wb[row * LS + l] = in.k[i] * ie[i];
        if constexpr (kKt) f.Kt[row * LS + l] = in.k[i] * __expf(Gl - Gt);
    }
    if (rg == 0) f.clast[l] = __expf(Gl);
    __syncthreads();

    // A = strictly lower(M Wb^T), Bq = lower(Qc Wb^T): lower 16x16 tiles only.
    constexpr int NJ = NT * (NT + 1) / 2;
    for (int job = wave; job < 2 * NJ; job += 4) {
        const bool isA = job >= NJ;
        int ti, tj;
        lower_tile(isA ? job - NJ : job, ti, tj);
        f32x4 acc = zero4();
        mma<LS, 1, 1, LS>(acc, (isA ? f.M : f.Qc) + ti * 16 * LS, f.Wb + tj * 16 * LS, LP, lane);
        float* dst = (isA ? f.Tm : f.Bq) + ti * 16 * CS + tj * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gi = ti * 16 + acc_row(lane, r), gj = tj * 16 + acc_col(lane);
            const bool keep = isA ? gi > gj : gi >= gj;
            dst[acc_row(lane, r) * CS + acc_col(lane)] = keep ? acc[r] : 0.f;
        }
    }
    if constexpr (NT > 1) {   // the upper tile (0, 1) of both
        for (int idx = tid; idx < 256; idx += kThreads) {
            const int rr = idx / 16, cc = idx % 16;
            f.Tm[rr * CS + 16 + cc] = 0.f;
            f.Bq[rr * CS + 16 + cc] = 0.f;
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by wave 0: each 16x16 diagonal block by substitution
    // (lane = block * 16 + column), then T10 = -T11 A10 T00.
    if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        if (blk < NT) {
            float x[16];
            const float* arow = f.Tm + blk * 16 * CS + blk * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = i == j ? 1.f : 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) s -= arow[i * CS + kk] * x[kk];
                x[i] = s;
            }
            float* trow = f.Tm + blk * 16 * CS + blk * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) trow[i * CS + j] = x[i];
        }
        if constexpr (NT == 2) {
            f32x4 acc = zero4();
            mma<CS, 1, CS, 1>(acc, f.Tm + 16 * CS, f.Tm, 16, lane);             // A10 T00
#pragma unroll
            for (int r = 0; r < 4; ++r) f.tmp[acc_row(lane, r) * 20 + acc_col(lane)] = acc[r];
            f32x4 acc2 = zero4();
            mma<CS, 1, 20, 1>(acc2, f.Tm + 16 * CS + 16, f.tmp, 16, lane);     // T11 (A10 T00)
#pragma unroll
            for (int r = 0; r < 4; ++r) f.Tm[(16 + acc_row(lane, r)) * CS + acc_col(lane)] = -acc2[r];
        }
    }
}

// --------------------------------------------------------------- forward

template <int CP, int LP>
__global__ void __launch_bounds__(kThreads, 2) wy_fwd_kernel(WyArgs a) {
    using F = Factors<CP, LP, true>;
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT, RPT = F::RPT;
    constexpr int NS = (LP / 16) * (kDN / 16);        // state tiles
    constexpr int NSW = (NS + 3) / 4;                   // state tiles per wave
    __shared__ F f;
    __shared__ float sX[CP * kDS], sU[CP * kDS], sS[LP * kDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t head = blockIdx.x / a.n_dt;
    const int64_t d0 = int64_t(blockIdx.x % a.n_dt) * kDN;
    const int64_t nb = a.n_chunks;

    for (int idx = tid; idx < LP * kDN; idx += kThreads) {
        const int l = idx / kDN, n = idx % kDN;
        float v = 0.f;
        if (l < a.L && d0 + n < a.D) {
            v = a.s0[(head * a.L + l) * a.D + d0 + n];
            if (a.bnd) a.bnd[((head * nb) * LP + l) * a.D + d0 + n] = v;
        }
        sS[l * kDS + n] = v;
    }

    for (int64_t c = 0; c < nb; ++c) {
        const int64_t t0 = c * CP;
        LatIn<RPT> in;
        load_latent<CP, LP>(a, head, t0, tid, in);
        constexpr int EPT = CP * kDN / kThreads;
        float wv[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
            const int64_t t = t0 + row;
            wv[i] = 0.f;
            if (t < a.T && d0 + n < a.D) {
                const int64_t gi = (head * a.T + t) * a.D + d0 + n;
                wv[i] = a.w[gi] * a.v[gi];
            }
        }
        float e[RPT], ie[RPT];
        // sX (this chunk's w.v) is free: its last reader (the previous U) is
        // behind the previous chunk's barriers, and make_factors' first
        // barrier orders this store before the rhs below.
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads;
            sX[(idx / kDN) * kDS + idx % kDN] = wv[i];
        }
        make_factors<CP, LP, true>(f, in, tid, e, ie);

        // rhs = w.v - M S0 (in place in sX), while wave 0 finishes T.
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<LS, 1, kDS, 1>(acc, f.M + ti * 16 * LS, sS + tj * 16, LP, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* p = sX + (ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane);
                *p = *p - acc[r];
            }
        }
        __syncthreads();
        // U = T rhs (T lower triangular).
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<CS, 1, kDS, 1>(acc, f.Tm + ti * 16 * CS, sX + tj * 16, (ti + 1) * 16, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sU[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = acc[r];
        }
        __syncthreads();
        // O = (Qc S0 + Bq U) / sqrt(L).
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<LS, 1, kDS, 1>(acc, f.Qc + ti * 16 * LS, sS + tj * 16, LP, lane);
            mma<CS, 1, kDS, 1>(acc, f.Bq + ti * 16 * CS, sU + tj * 16, (ti + 1) * 16, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + ti * 16 + acc_row(lane, r), d = d0 + tj * 16 + acc_col(lane);
                if (t < a.T && d < a.D) a.ctx[(head * a.T + t) * a.D + d] = acc[r] * a.scale;
            }
        }
        // S_end = diag(c_last) S0 + Kt^T U.
        f32x4 snew[NSW];
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int job = wave + 4 * s;
            if (job < NS) {
                const int ti = job >> 1, tj = job & 1;
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = ti * 16 + acc_row(lane, r);
                    acc[r] = f.clast[l] * sS[l * kDS + tj * 16 + acc_col(lane)];
                }
                mma<1, LS, kDS, 1>(acc, f.Kt + ti * 16, sU + tj * 16, CP, lane);
                snew[s] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int job = wave + 4 * s;
            if (job < NS) {
                const int ti = job >> 1, tj = job & 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = ti * 16 + acc_row(lane, r), n = tj * 16 + acc_col(lane);
                    sS[l * kDS + n] = snew[s][r];
                    if (l < a.L && d0 + n < a.D) {
                        if (c + 1 < nb) {
                            if (a.bnd) a.bnd[((head * nb + c + 1) * LP + l) * a.D + d0 + n] = snew[s][r];
                        } else if (a.state) {
                            a.state[(head * a.L + l) * a.D + d0 + n] = snew[s][r];
                        }
                    }
                }
            }
        }
    }
}

// ----------------------------------------------------- backward: the carry

template <int CP, int LP>
__global__ void __launch_bounds__(kThreads, 2) wy_bwd_carry_kernel(WyArgs a) {
    using F = Factors<CP, LP, false>;
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT, RPT = F::RPT;
    constexpr int NS = (LP / 16) * (kDN / 16);
    constexpr int NSW = (NS + 3) / 4;
    __shared__ F f;
    __shared__ float sX[CP * kDS], sU[CP * kDS], sR[CP * kDS], sS[LP * kDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t head = blockIdx.x / a.n_dt;
    const int64_t d0 = int64_t(blockIdx.x % a.n_dt) * kDN;
    const int64_t nb = a.n_chunks;
    const float s = a.scale;

    for (int idx = tid; idx < LP * kDN; idx += kThreads) {
        const int l = idx / kDN, n = idx % kDN;
        float v = 0.f;
        if (l < a.L && d0 + n < a.D) {
            if (a.dstate) v = a.dstate[(head * a.L + l) * a.D + d0 + n];
            a.dbnd[((head * nb + nb - 1) * LP + l) * a.D + d0 + n] = v;
        }
        sS[l * kDS + n] = v;
    }

    for (int64_t c = nb - 1; c >= 0; --c) {
        const int64_t t0 = c * CP;
        LatIn<RPT> in;
        load_latent<CP, LP>(a, head, t0, tid, in);
        constexpr int EPT = CP * kDN / kThreads;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
            const int64_t t = t0 + row;
            float v = 0.f;
            if (t < a.T && d0 + n < a.D) v = a.dctx[(head * a.T + t) * a.D + d0 + n];
            sX[row * kDS + n] = v;
        }
        float e[RPT], ie[RPT];
        make_factors<CP, LP, false>(f, in, tid, e, ie);

        // dSc = diag(c_last) dS, in place (sS was last read before the previous
        // chunk's final barrier); the barrier after it also publishes T.
        for (int idx = tid; idx < LP * kDN; idx += kThreads) {
            const int l = idx / kDN, n = idx % kDN;
            sS[l * kDS + n] *= f.clast[l];
        }
        __syncthreads();
        // dU = Bq^T dO / sqrt(L) + Wb dSc.
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 a1 = zero4(), a2 = zero4();
            mma<1, CS, kDS, 1>(a1, f.Bq + ti * 16 * CS + ti * 16, sX + ti * 16 * kDS + tj * 16, CP - ti * 16, lane);
            mma<LS, 1, kDS, 1>(a2, f.Wb + ti * 16 * LS, sS + tj * 16, LP, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sU[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = a1[r] * s + a2[r];
        }
        __syncthreads();
        // drhs = T^T dU.
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<1, CS, kDS, 1>(acc, f.Tm + ti * 16 * CS + ti * 16, sU + ti * 16 * kDS + tj * 16, CP - ti * 16, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sR[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = acc[r];
        }
        __syncthreads();
        // dS0 = Qc^T dO / sqrt(L) + dSc - M^T drhs.
        f32x4 dnew[NSW];
#pragma unroll
        for (int sl = 0; sl < NSW; ++sl) {
            const int job = wave + 4 * sl;
            if (job < NS) {
                const int ti = job >> 1, tj = job & 1;
                f32x4 aq = zero4(), am = zero4();
                mma<1, LS, kDS, 1>(aq, f.Qc + ti * 16, sX + tj * 16, CP, lane);
                mma<1, LS, kDS, 1>(am, f.M + ti * 16, sR + tj * 16, CP, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = ti * 16 + acc_row(lane, r);
                    dnew[sl][r] = sS[l * kDS + tj * 16 + acc_col(lane)] + aq[r] * s - am[r];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < NSW; ++sl) {
            const int job = wave + 4 * sl;
            if (job < NS) {
                const int ti = job >> 1, tj = job & 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = ti * 16 + acc_row(lane, r), n = tj * 16 + acc_col(lane);
                    sS[l * kDS + n] = dnew[sl][r];
                    if (l < a.L && d0 + n < a.D) {
                        if (c > 0)
                            a.dbnd[((head * nb + c - 1) * LP + l) * a.D + d0 + n] = dnew[sl][r];
                        else if (a.ds0)
                            a.ds0[(head * a.L + l) * a.D + d0 + n] = dnew[sl][r];
                    }
                }
            }
        }
    }
}

// ------------------------------------------------ backward: the gradients

template <int CP, int LP>
struct GradTiles {
    // The walk over dense tiles; reused for the final per-chunk matrices.
    union {
        struct {
            float S[LP * kDS];    // boundary state tile S0
            float D[LP * kDS];    // dSc = diag(c_last) dS tile
            float X[CP * kDS];    // w.v, then rhs
            float O[CP * kDS];    // dO
            float U[CP * kDS];    // U, then (after drhs) free
            float dU[CP * kDS];   // dU
            float R[CP * kDS];    // drhs
        } t;
        struct {
            float dQc[CP * (LP + 4)], dM[CP * (LP + 4)], dWb[CP * (LP + 4)], P[CP * (LP + 4)];
            float xl[kThreads];
            float red[2 * kThreads];
        } m;
    };
};

template <int CP, int LP>
__global__ void __launch_bounds__(kThreads, 2) wy_bwd_grad_kernel(WyArgs a) {
    using F = Factors<CP, LP, false>;
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT, RPT = F::RPT, RG = F::RG;
    constexpr int NJ = NT * (NT + 1) / 2;            // lower tiles of a CP x CP matrix
    constexpr int NL = NT * (LP / 16);               // tiles of a CP x LP matrix
    constexpr int NCC = (2 * NJ + 3) / 4;            // CP x CP accumulator tiles per wave (dBq then dA)
    constexpr int NCL = (NL + 3) / 4;                // CP x LP tiles per wave (dQc, dM, P each)
    __shared__ F f;
    __shared__ GradTiles<CP, LP> g;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t head = blockIdx.x / a.n_chunks;
    const int64_t c = blockIdx.x % a.n_chunks;
    const int64_t t0 = c * CP;
    const int64_t nb = a.n_chunks;
    const float s = a.scale;

    LatIn<RPT> in;
    load_latent<CP, LP>(a, head, t0, tid, in);
    float e[RPT], ie[RPT];
    make_factors<CP, LP, false>(f, in, tid, e, ie);

    f32x4 accC[NCC], accQ[NCL], accM[NCL], accP[NCL];
#pragma unroll
    for (int i = 0; i < NCC; ++i) accC[i] = zero4();
#pragma unroll
    for (int i = 0; i < NCL; ++i) accQ[i] = accM[i] = accP[i] = zero4();
    // rowsum(dSc . S0) partials: thread (l = tid / (256 / LP) ...) over its elements.
    constexpr int TPL = kThreads / LP;               // threads per latent row
    constexpr int EPL = kDN / TPL;                   // elements per thread per tile
    float xl = 0.f;

    constexpr int EPT = CP * kDN / kThreads;
    for (int dt = 0; dt < a.n_dt; ++dt) {
        const int64_t d0 = int64_t(dt) * kDN;
        // Loads: S0 and dS (scaled by c_last), w.v, dO, and v, w for this thread's drhs elements.
        {
            const int l = tid / TPL, n0 = (tid % TPL) * EPL;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int n = n0 + i;
                float sv = 0.f, dv = 0.f;
                if (l < a.L && d0 + n < a.D) {
                    const int64_t gi = ((head * nb + c) * LP + l) * a.D + d0 + n;
                    sv = a.bnd_in[gi];
                    dv = a.dbnd[gi];
                }
                dv *= f.clast[l];
                g.t.S[l * kDS + n] = sv;
                g.t.D[l * kDS + n] = dv;
                xl += dv * sv;
            }
        }
        float vv[EPT], ww[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
            const int64_t t = t0 + row;
            float o = 0.f;
            vv[i] = ww[i] = 0.f;
            if (t < a.T && d0 + n < a.D) {
                const int64_t gi = (head * a.T + t) * a.D + d0 + n;
                vv[i] = a.v[gi];
                ww[i] = a.w[gi];
                o = a.dctx[gi];
            }
            g.t.X[row * kDS + n] = ww[i] * vv[i];
            g.t.O[row * kDS + n] = o;
        }
        __syncthreads();
        // rhs = w.v - M S0;  dU = Bq^T dO / sqrt(L) + Wb dSc.
        for (int job = wave; job < NT * 4; job += 4) {
            const int ti = (job >> 1) % NT, tj = job & 1;
            if (job < NT * 2) {
                f32x4 acc = zero4();
                mma<LS, 1, kDS, 1>(acc, f.M + ti * 16 * LS, g.t.S + tj * 16, LP, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float* p = g.t.X + (ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane);
                    *p = *p - acc[r];
                }
            } else {
                f32x4 a1 = zero4(), a2 = zero4();
                mma<1, CS, kDS, 1>(a1, f.Bq + ti * 16 * CS + ti * 16, g.t.O + ti * 16 * kDS + tj * 16, CP - ti * 16,
                                   lane);
                mma<LS, 1, kDS, 1>(a2, f.Wb + ti * 16 * LS, g.t.D + tj * 16, LP, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    g.t.dU[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = a1[r] * s + a2[r];
            }
        }
        __syncthreads();
        // U = T rhs;  drhs = T^T dU.
        for (int job = wave; job < NT * 4; job += 4) {
            const int ti = (job >> 1) % NT, tj = job & 1;
            f32x4 acc = zero4();
            if (job < NT * 2) {
                mma<CS, 1, kDS, 1>(acc, f.Tm + ti * 16 * CS, g.t.X + tj * 16, (ti + 1) * 16, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) g.t.U[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = acc[r];
            } else {
                mma<1, CS, kDS, 1>(acc, f.Tm + ti * 16 * CS + ti * 16, g.t.dU + ti * 16 * kDS + tj * 16, CP - ti * 16,
                                   lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) g.t.R[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = acc[r];
            }
        }
        __syncthreads();
        // dw = drhs . v, dv = drhs . w.
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
            const int64_t t = t0 + row;
            if (t < a.T && d0 + n < a.D) {
                const int64_t gi = (head * a.T + t) * a.D + d0 + n;
                const float r = g.t.R[row * kDS + n];
                if (a.dw) a.dw[gi] = r * vv[i];
                if (a.dv) a.dv[gi] = r * ww[i];
            }
        }
        // Sums over the dense axis: dO U^T, drhs U^T (lower tiles), dO S0^T, drhs S0^T, U dSc^T.
#pragma unroll
        for (int sl = 0; sl < NCC; ++sl) {
            const int job = wave + 4 * sl;
            if (job < 2 * NJ) {
                const bool isA = job >= NJ;
                int ti, tj;
                lower_tile(isA ? job - NJ : job, ti, tj);
                mma<kDS, 1, 1, kDS>(accC[sl], (isA ? g.t.R : g.t.O) + ti * 16 * kDS, g.t.U + tj * 16 * kDS, kDN, lane);
            }
        }
#pragma unroll
        for (int sl = 0; sl < NCL; ++sl) {
            const int job = wave + 4 * sl;
            if (job < NL) {
                const int ti = job / (LP / 16), lj = job % (LP / 16);
                mma<kDS, 1, 1, kDS>(accQ[sl], g.t.O + ti * 16 * kDS, g.t.S + lj * 16 * kDS, kDN, lane);
                mma<kDS, 1, 1, kDS>(accM[sl], g.t.R + ti * 16 * kDS, g.t.S + lj * 16 * kDS, kDN, lane);
                mma<kDS, 1, 1, kDS>(accP[sl], g.t.U + ti * 16 * kDS, g.t.D + lj * 16 * kDS, kDN, lane);
            }
        }
        __syncthreads();
    }

    // dBq = lower(dO U^T) / sqrt(L) into f.Bq, dA = -strictly lower(drhs U^T) into f.Tm
    // (their upper tiles are already zero).
#pragma unroll
    for (int sl = 0; sl < NCC; ++sl) {
        const int job = wave + 4 * sl;
        if (job < 2 * NJ) {
            const bool isA = job >= NJ;
            int ti, tj;
            lower_tile(isA ? job - NJ : job, ti, tj);
            float* dst = (isA ? f.Tm : f.Bq) + ti * 16 * CS + tj * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gi = ti * 16 + acc_row(lane, r), gj = tj * 16 + acc_col(lane);
                const bool keep = isA ? gi > gj : gi >= gj;
                dst[acc_row(lane, r) * CS + acc_col(lane)] = keep ? (isA ? -accC[sl][r] : accC[sl][r] * s) : 0.f;
            }
        }
    }
    g.m.xl[tid] = xl;
    __syncthreads();
    // dQc = s dO S0^T + dBq Wb;  dM = -drhs S0^T + dA Wb;  dWb = U dSc^T + dBq^T Qc + dA^T M.
    // P = U dSc^T is kept apart too, for the last step's term sum_tau Wb[tau][l] P[tau][l].
#pragma unroll
    for (int sl = 0; sl < NCL; ++sl) {
        const int job = wave + 4 * sl;
        if (job < NL) {
            const int ti = job / (LP / 16), lj = job % (LP / 16);
            f32x4 q4, m4, w4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                q4[r] = accQ[sl][r] * s;
                m4[r] = -accM[sl][r];
            }
            w4 = accP[sl];
            mma<CS, 1, LS, 1>(q4, f.Bq + ti * 16 * CS, f.Wb + lj * 16, (ti + 1) * 16, lane);
            mma<CS, 1, LS, 1>(m4, f.Tm + ti * 16 * CS, f.Wb + lj * 16, (ti + 1) * 16, lane);
            mma<1, CS, LS, 1>(w4, f.Bq + ti * 16 * CS + ti * 16, f.Qc + ti * 16 * LS + lj * 16, CP - ti * 16, lane);
            mma<1, CS, LS, 1>(w4, f.Tm + ti * 16 * CS + ti * 16, f.M + ti * 16 * LS + lj * 16, CP - ti * 16, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(lane, r), col = lj * 16 + acc_col(lane);
                g.m.dQc[row * LS + col] = q4[r];
                g.m.dM[row * LS + col] = m4[r];
                g.m.dWb[row * LS + col] = w4[r];
                g.m.P[row * LS + col] = accP[sl][r];
            }
        }
    }
    __syncthreads();
    // Per (step, latent row): this thread's rows rg*RPT + i of row l.
    {
        const int l = tid % LP, rg = tid / LP;
        float dcc[RPT];
        float pp = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg * RPT + i;
            const float dQc = g.m.dQc[row * LS + l], dM = g.m.dM[row * LS + l], dWb = g.m.dWb[row * LS + l];
            const float Qc = f.Qc[row * LS + l], M = f.M[row * LS + l], Wb = f.Wb[row * LS + l];
            dcc[i] = dQc * Qc + dM * M - dWb * Wb;
            pp += Wb * g.m.P[row * LS + l];
            const int64_t t = t0 + row;
            if (t < a.T && l < a.L) {
                const int64_t gi = (head * a.T + t) * a.L + l;
                if (a.dq) a.dq[gi] = dQc * e[i];
                if (a.db) a.db[gi] = dM * in.k[i] * e[i];
                if (a.dk) a.dk[gi] = dM * in.b[i] * e[i] + dWb * ie[i];
            }
        }
        // Suffix sums of dcc over the chunk: local, then later groups' totals.
        float suf[RPT];
        float run = 0.f;
#pragma unroll
        for (int i = RPT - 1; i >= 0; --i) {
            run += dcc[i];
            suf[i] = run;
        }
        g.m.red[rg * LP + l] = run;
        g.m.red[kThreads + rg * LP + l] = pp;
        __syncthreads();
        float later = 0.f, xlt = 0.f;
#pragma unroll
        for (int r = RG - 1; r >= 0; --r) {
            if (r > rg) later += g.m.red[r * LP + l];
            xlt += g.m.red[kThreads + r * LP + l];
        }
        // The end state's term, rowsum(dSc . (S0 + Wb^T U)), enters at the
        // chunk's last step, so every step of the chunk gets it.
#pragma unroll
        for (int r = 0; r < TPL; ++r) xlt += g.m.xl[l * TPL + r];
        if (a.dg) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int64_t t = t0 + rg * RPT + i;
                if (t < a.T && l < a.L) a.dg[(head * a.T + t) * a.L + l] = suf[i] + later + xlt;
            }
        }
    }
}

template <int CP, int LP>
hipError_t launch_fwd_t(const WyArgs& a, hipStream_t st) {
    WyArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&wy_fwd_kernel<CP, LP>), dim3(unsigned(a.BH * a.n_dt)),
                           dim3(kThreads), params, 0, st);
}

template <int CP, int LP>
hipError_t launch_bwd_t(const WyArgs& a, hipStream_t st) {
    WyArgs args = a;
    void* params[] = {&args};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&wy_bwd_carry_kernel<CP, LP>),
                                   dim3(unsigned(a.BH * a.n_dt)), dim3(kThreads), params, 0, st);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void*>(&wy_bwd_grad_kernel<CP, LP>),
                           dim3(unsigned(a.BH * a.n_chunks)), dim3(kThreads), params, 0, st);
}

template <int CP>
hipError_t fwd_lp(int lp, const WyArgs& a, hipStream_t st) {
    return lp == 16 ? launch_fwd_t<CP, 16>(a, st) : lp == 32 ? launch_fwd_t<CP, 32>(a, st) : launch_fwd_t<CP, 64>(a, st);
}
template <int CP>
hipError_t bwd_lp(int lp, const WyArgs& a, hipStream_t st) {
    return lp == 16 ? launch_bwd_t<CP, 16>(a, st) : lp == 32 ? launch_bwd_t<CP, 32>(a, st) : launch_bwd_t<CP, 64>(a, st);
}

}  // namespace

hipError_t launch_wy_forward(int chunk, int lp, const WyArgs& a, hipStream_t st) {
    return chunk == 16 ? fwd_lp<16>(lp, a, st) : fwd_lp<32>(lp, a, st);
}

hipError_t launch_wy_backward(int chunk, int lp, const WyArgs& a, hipStream_t st) {
    return chunk == 16 ? bwd_lp<16>(lp, a, st) : bwd_lp<32>(lp, a, st);
}

}  // namespace qc
