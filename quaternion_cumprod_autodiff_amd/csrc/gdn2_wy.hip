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
// Kernels (256 threads = 4 waves unless stated; chunks of CP = 16 or 32
// steps; latent rows padded to LP = 16, 32 or 64; every matrix product is
// 16x16 output tiles of the f32 MFMA, A operands read from LDS, B operands
// from LDS or straight from the accumulators of the product before):
//   wy_factor_kernel    one block per (head, chunk), all chunks at once: the
//                       chunk's factors M, Qc, Kt, T, Bq and c_last, written
//                       as one record per chunk after the boundary states
//                       (the forward's saved state for the backward).
//   wy_fwd_strip_kernel 512 threads: one chain wave per (head, 16 dense
//                       columns), four to a block, each carrying its strip
//                       of the state through the chunks in order, and one
//                       memory wave per strip that streams the records
//                       through two LDS copies and stores the strip's
//                       results; saves the state at every chunk start and U.
//   wy_fwd_fused_kernel without a boundary buffer (no backward to follow):
//                       one block per (head, 32 dense columns), building
//                       each chunk's factors itself.
//   wy_bwd_carry_strip_kernel  as the forward strip kernel, the chunks in
//                       reverse, carrying dS; saves the dS entering every
//                       chunk from later ones and drhs (scratch), dv, dw and
//                       d initial_state.
//   wy_bwd_grad_kernel  every (head, chunk) independently, as many blocks as
//                       the device holds at once, each looping over chunks
//                       and loading the next one's inputs during the current:
//                       from the chunk's record, boundary state and dS, every
//                       cotangent of the chunk's steps; the sums over the
//                       dense axis stay in MFMA accumulators across the
//                       block's walk over 32-column dense tiles.
// The sequential kernels deal their blocks so that all dense columns of a
// head run on one XCD (block % 8), where they share the head's records in L2.
// Padded steps (past T in the last chunk) have k = q = b = v = w = g = 0: they
// leave the state unchanged and get no output.
#include "gdn2_internal.hpp"
#include "qc_internal.hpp"

#include <cstddef>
#include <type_traits>

namespace qc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kDN = kWyDense;   // dense columns per tile
constexpr int kDS = kDN + 4;    // LDS row stride of [rows][kDN] tiles read both ways (gradient kernel)
constexpr int kSeqDS = kDN + 16;  // the same for tiles read only as row-major B operands: conflict-free

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A(m0 + 0..15, k0 + 0..K) B(k0 + 0..K, n0 + 0..15) on one wave, K a
// multiple of 4 known at compile time, so that every operand read is issued
// ahead of the MFMA chain.  `a` points at A(m0, k0) and `b` at B(k0, n0);
// A(m, k) is a[m * SAM + k * SAK] and B(k, n) is b[k * SBK + n * SBN]
// (strides select transposes).  Lane l feeds A(l % 16, 4i + l / 16) and
// B(4i + l / 16, l % 16) to step i and ends with rows 4 (l / 16) + r, column
// l % 16 in acc[r].
template <int K, int SAM, int SAK, int SBK, int SBN>
__device__ __forceinline__ void mma(f32x4& acc, const float* a, const float* b, int lane) {
    const int i = lane & 15, kq = lane >> 4;
    a += i * SAM + kq * SAK;
    b += kq * SBK + i * SBN;
    float av[K / 4], bv[K / 4];
#pragma unroll
    for (int k = 0; k < K / 4; ++k) {
        av[k] = a[4 * k * SAK];
        bv[k] = b[4 * k * SBK];
    }
#pragma unroll
    for (int k = 0; k < K / 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], bv[k], acc, 0, 0, 0);
}

// acc += A B over K with both operands stored contiguously along K:
// A(m, k) = a[m * SA + k], B(k, n) = bt[n * SB + k] (a and bt point at row
// m0 and row n0).  Lane group kq = l / 16 takes k = kq * K/4 + j at step j,
// so a lane's operands for four steps are one 16-byte LDS read each (the
// same reordering of the sum for A and B, so the product is unchanged up to
// rounding).  SA and SB multiples of 4 with SA / 4 and SB / 4 odd keep the
// 16 lanes of a row group on distinct banks.
template <int K, int SA, int SB>
__device__ __forceinline__ void mma_kc(f32x4& acc, const float* a, const float* bt, int lane) {
    static_assert(K % 16 == 0 && SA % 4 == 0 && SB % 4 == 0, "16-byte operand reads");
    constexpr int KQ = K / 4;
    const int i = lane & 15, kq = lane >> 4;
    const f32x4* pa = reinterpret_cast<const f32x4*>(a + i * SA + kq * KQ);
    const f32x4* pb = reinterpret_cast<const f32x4*>(bt + i * SB + kq * KQ);
    f32x4 av[KQ / 4], bv[KQ / 4];
#pragma unroll
    for (int j = 0; j < KQ / 4; ++j) {
        av[j] = pa[j];
        bv[j] = pb[j];
    }
#pragma unroll
    for (int j = 0; j < KQ / 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][e], bv[j][e], acc, 0, 0, 0);
}

// N independent products acc[c] += A_c B whose B is another product's
// result as the accumulators hold it: K / 16 row tiles, lane l holding
// B(16 t + 4 (l / 16) + r, l % 16) in b[t][r].  Lane group kq takes
// k = 16 t + 4 kq + r at step (t, r) (the same reordering for A), so B goes
// from one product to the next without a transpose through LDS.
// acc_a reads the A operands, A_c(m, k) = a[c][m * SAM + k * SAK] (with
// SAK = 1 and SAM a multiple of 4, a lane's four operands of a tile are one
// 16-byte read), so that they can be read ahead of the product that needs
// them; acc_mma runs the chains with the MFMAs of the N chains interleaved.
template <int N, int K, int SAM, int SAK>
__device__ __forceinline__ void acc_a(f32x4 (&av)[N][K / 16], const float* const (&a)[N], int lane) {
    static_assert(K % 16 == 0, "whole accumulator tiles");
    const int i = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int t = 0; t < K / 16; ++t)
#pragma unroll
        for (int c = 0; c < N; ++c) {
            const float* p = a[c] + i * SAM + (16 * t + 4 * kq) * SAK;
            if constexpr (SAK == 1) {
                static_assert(SAM % 4 == 0, "16-byte operand reads");
                av[c][t] = *reinterpret_cast<const f32x4*>(p);
            } else {
                av[c][t] = f32x4{p[0], p[SAK], p[2 * SAK], p[3 * SAK]};
            }
        }
}

template <int N, int K>
__device__ __forceinline__ void acc_mma(f32x4 (&acc)[N], const f32x4 (&av)[N][K / 16], const f32x4* b) {
#pragma unroll
    for (int t = 0; t < K / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < N; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c][t][r], b[t][r], acc[c], 0, 0, 0);
}

// The same with K = 16 * k16, k16 wave-uniform in 1 .. KMAX / 16 (the
// triangular ranges of the chunk's lower-triangular factors; KMAX <= 32).
template <int KMAX, int SAM, int SAK, int SBK, int SBN>
__device__ __forceinline__ void mma16(f32x4& acc, const float* a, const float* b, int k16, int lane) {
    static_assert(KMAX == 16 || KMAX == 32, "chunk of 16 or 32 steps");
    if constexpr (KMAX == 32) {
        if (k16 == 2) {
            mma<32, SAM, SAK, SBK, SBN>(acc, a, b, lane);
            return;
        }
    }
    mma<16, SAM, SAK, SBK, SBN>(acc, a, b, lane);
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

// Row stride of the LDS [CP][LP] factor matrices.  Latent rows are read both
// row-major (A operands) and transposed (A^T operands); with 64 LDS banks a
// stride of 76 for 64 rows keeps the first conflict-free and the second at
// two-way, where 68 would make the second four-way.
constexpr int factor_stride(int lp) { return lp == 64 ? 76 : lp + 4; }

// One chunk's factors in LDS.  Thread (rg, l), rg = tid / LP, owns latent row
// l of the chunk's steps rg*RPT .. rg*RPT + RPT - 1.  kWb, kKt: whether Wb
// and Kt are held; kScratch: the group sums and the inversion scratch (for
// building the factors).
template <int CP, int LP, int LSV, bool kWb, bool kKt, bool kScratch>
struct alignas(16) FactorsT {
    static constexpr int LS = LSV;        // row stride of [CP][LP]
    static constexpr int CS = CP + 4;     // row stride of [CP][CP]
    static constexpr int RG = kThreads / LP;
    static constexpr int RPT = CP / RG;
    static constexpr int NT = CP / 16;
    static constexpr bool kHasKt = kKt;
    float Qc[CP * LS], M[CP * LS];
    float Wb[kWb ? CP * LS : 4];
    float Kt[kKt ? CP * LS : 4];
    float Tm[CP * CS];     // A, then T = (I + A)^-1 (upper part zero)
    float Bq[CP * CS];     // lower part of Qc Wb^T (upper part zero)
    float tot[kScratch ? RG * LP : 4];    // per-group sums of log_decay
    float clast[LP];       // c at the chunk's last (padded) step
    float tmp[kScratch ? 16 * 20 : 4];
};
template <int CP, int LP>
using BuildFactors = FactorsT<CP, LP, factor_stride(LP), true, true, true>;     // factor kernel, fused forward
template <int CP, int LP>
using StagedFactors = FactorsT<CP, LP, factor_stride(LP), false, true, false>;  // record-streaming kernels

template <int RPT>
struct LatIn {
    float q[RPT], k[RPT], b[RPT], g[RPT];
};

// Loads are unconditional, from indices clamped into range; the values are
// masked only where they are consumed.  A load under a branch makes the
// compiler wait for every outstanding load where the branch rejoins, and any
// use of a loaded register (a masking select included) waits for it, either
// of which would turn the prefetches below into synchronous loads.

// Latent inputs of chunk rows rg*RPT + i (rows past T and columns past L
// hold clamped copies: mask with latent_ok).
template <int CP, int LP, int RPT>
__device__ __forceinline__ void load_latent(const WyArgs& a, int64_t head, int64_t t0, int tid, LatIn<RPT>& in) {
    constexpr int RG = kThreads / LP;
    static_assert(RG * RPT == CP, "rows per thread");
    const int l = tid % LP, rg = tid / LP;
    const int64_t lc = l < a.L ? l : a.L - 1;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t t = t0 + rg * RPT + i;
        const int64_t idx = (head * a.T + (t < a.T ? t : a.T - 1)) * a.L + lc;
        in.q[i] = a.q[idx];
        in.k[i] = a.k[idx];
        in.b[i] = a.b[idx];
        in.g[i] = a.g[idx];
    }
}

// Whether this thread's latent row i of the chunk at t0 is a real entry.
template <int CP, int LP, int RPT>
__device__ __forceinline__ bool latent_ok(const WyArgs& a, int64_t t0, int tid, int i) {
    return t0 + (tid / LP) * RPT + i < a.T && tid % LP < a.L;
}

// One or two [B, H, T, D] tensors' values of a chunk's dense tile, element
// tid + i * kThreads of the [CP][kDN] tile (clamped copies past T or past D:
// mask with dense_ok).
// Addressing of the per-chunk tiles: one block-uniform 64-bit base (the
// tile's first element), then 32-bit offsets row * D + column per element,
// clamped in 32 bits.  Per-element 64-bit index arithmetic (multiplies,
// compares, selects) had made issuing a chunk's prefetch take about as long
// as the chunk's first matrix product.
__device__ __forceinline__ int64_t tile_base(const WyArgs& a, int64_t head, int64_t t0, int64_t d0) {
    return (head * a.T + t0) * a.D + d0;
}
__device__ __forceinline__ int last_row(const WyArgs& a, int64_t t0, int rows) {
    return a.T - t0 < rows ? int(a.T - t0) - 1 : rows - 1;
}
__device__ __forceinline__ int last_col(const WyArgs& a, int64_t d0) {
    return a.D - d0 < kDN ? int(a.D - d0) - 1 : kDN - 1;
}

template <int CP, bool kTwo>
__device__ __forceinline__ void load_dense(const float* x, const float* y, const WyArgs& a, int64_t head, int64_t t0,
                                           int64_t d0, int tid, float* xv, float* yv) {
    constexpr int EPT = CP * kDN / kThreads;
    const int64_t base = tile_base(a, head, t0, d0);
    const float* xb = x + base;
    const float* yb = kTwo ? y + base : nullptr;
    const int lr = last_row(a, t0, CP), lc = last_col(a, d0), D = int(a.D);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
        const int off = (row < lr ? row : lr) * D + (n < lc ? n : lc);
        xv[i] = xb[off];
        if constexpr (kTwo) yv[i] = yb[off];
    }
}

__device__ __forceinline__ bool dense_ok(const WyArgs& a, int64_t t0, int64_t d0, int tid, int i) {
    const int idx = tid + i * kThreads;
    return t0 + idx / kDN < a.T && d0 + idx % kDN < a.D;
}

// Builds Qc, M, Wb (and Kt), A, Bq in LDS, then T in place of A (wave 0,
// without a closing barrier: callers reach one before reading T).  e and ie
// receive c and 1/c of this thread's rows.  Starts and ends reading nothing
// that the caller may still be writing: the first barrier comes after the
// group sums are stored.
template <int CP, int LP, class F, int RPT>
__device__ void make_factors(F& f, const LatIn<RPT>& raw, const WyArgs& a, int64_t t0, int tid, float* e, float* ie) {
    constexpr int LS = F::LS, CS = F::CS, RG = F::RG, NT = F::NT;
    const int lane = tid & 63, wave = tid >> 6;
    const int l = tid % LP, rg = tid / LP;
    LatIn<RPT> in;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const bool ok = latent_ok<CP, LP, RPT>(a, t0, tid, i);
        in.q[i] = ok ? raw.q[i] : 0.f;
        in.k[i] = ok ? raw.k[i] : 0.f;
        in.b[i] = ok ? raw.b[i] : 0.f;
        in.g[i] = ok ? raw.g[i] : 0.f;
    }

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
        if constexpr (F::kHasKt) f.Kt[row * LS + l] = in.k[i] * __expf(Gl - Gt);
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
        mma_kc<LP, LS, LS>(acc, (isA ? f.M : f.Qc) + ti * 16 * LS, f.Wb + tj * 16 * LS, lane);
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
            // Column-oriented (right-looking): once x[k] is final it updates
            // every later row, so the dependent chain is 16 steps long.
            float x[16];
            const float* arow = f.Tm + blk * 16 * CS + blk * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == j ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < 15; ++kk)
#pragma unroll
                for (int i = kk + 1; i < 16; ++i) x[i] -= arow[i * CS + kk] * x[kk];
            float* trow = f.Tm + blk * 16 * CS + blk * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) trow[i * CS + j] = x[i];
        }
        if constexpr (NT == 2) {
            f32x4 acc = zero4();
            mma<16, CS, 1, CS, 1>(acc, f.Tm + 16 * CS, f.Tm, lane);             // A10 T00
#pragma unroll
            for (int r = 0; r < 4; ++r) f.tmp[acc_row(lane, r) * 20 + acc_col(lane)] = acc[r];
            f32x4 acc2 = zero4();
            mma<16, CS, 1, 20, 1>(acc2, f.Tm + 16 * CS + 16, f.tmp, lane);     // T11 (A10 T00)
#pragma unroll
            for (int r = 0; r < 4; ++r) f.Tm[(16 + acc_row(lane, r)) * CS + acc_col(lane)] = -acc2[r];
        }
    }
}

// ---------------------------------------------------------- factor records
//
// One chunk's record, floats: M, Qc, Kt [CP][LP] (row = step, unpadded),
// T, Bq [CP][CP], c_last [LP]; kSize rounds it up to 256 bytes.
template <int CP, int LP>
struct Rec {
    static constexpr int kM = 0, kQc = CP * LP, kKt = 2 * CP * LP, kT = 3 * CP * LP;
    static constexpr int kBq = kT + CP * CP, kCl = kBq + CP * CP, kUsed = kCl + LP;
    static constexpr int kSize = wy_record_floats(CP, LP);
    static constexpr int kN4 = kUsed / 4;                          // float4 per record
    static constexpr int kPer = (kN4 + kThreads - 1) / kThreads;   // float4 per thread
    static_assert(kUsed <= kSize && LP % 4 == 0 && CP % 4 == 0, "record layout");
};

// LDS address of record element e (a multiple of 4: a float4 never spans two
// rows or two sections).
template <int CP, int LP, class F>
__device__ __forceinline__ float* rec_lds(F& f, int e) {
    using R = Rec<CP, LP>;
    constexpr int LS = F::LS, CS = F::CS;
    if (e < R::kQc) return f.M + (e / LP) * LS + e % LP;
    if (e < R::kKt) return f.Qc + ((e - R::kQc) / LP) * LS + (e - R::kQc) % LP;
    if (e < R::kT) return f.Kt + ((e - R::kKt) / LP) * LS + (e - R::kKt) % LP;
    if (e < R::kBq) return f.Tm + ((e - R::kT) / CP) * CS + (e - R::kT) % CP;
    if (e < R::kCl) return f.Bq + ((e - R::kBq) / CP) * CS + (e - R::kBq) % CP;
    return f.clast + (e - R::kCl);
}

template <int CP, int LP>
struct RecRegs {
    f32x4 v[Rec<CP, LP>::kPer];
};

template <int CP, int LP>
__device__ __forceinline__ void load_rec(RecRegs<CP, LP>& r, const float* rec, int tid) {
    using R = Rec<CP, LP>;
#pragma unroll
    for (int i = 0; i < R::kPer; ++i) {
        const int j = tid + i * kThreads;
        r.v[i] = reinterpret_cast<const f32x4*>(rec)[j < R::kN4 ? j : R::kN4 - 1];   // unconditional (see load_latent)
    }
}

// Where this thread's float4 of a record land in staged factors F: offsets
// in floats from the start of F (-1: none), formed once per kernel, so that
// staging a record is a run of 16-byte LDS stores.
template <int CP, int LP, class F>
struct RecStage {
    using R = Rec<CP, LP>;
    int off[R::kPer];
    __device__ explicit RecStage(int tid) {
        constexpr int LS = F::LS, CS = F::CS;
#pragma unroll
        for (int i = 0; i < R::kPer; ++i) {
            const int j = tid + i * kThreads, e = 4 * j;
            off[i] = j >= R::kN4  ? -1
                   : e < R::kQc  ? int(offsetof(F, M) / 4) + (e / LP) * LS + e % LP
                   : e < R::kKt  ? int(offsetof(F, Qc) / 4) + ((e - R::kQc) / LP) * LS + (e - R::kQc) % LP
                   : e < R::kT   ? int(offsetof(F, Kt) / 4) + ((e - R::kKt) / LP) * LS + (e - R::kKt) % LP
                   : e < R::kBq  ? int(offsetof(F, Tm) / 4) + ((e - R::kT) / CP) * CS + (e - R::kT) % CP
                   : e < R::kCl  ? int(offsetof(F, Bq) / 4) + ((e - R::kBq) / CP) * CS + (e - R::kBq) % CP
                                 : int(offsetof(F, clast) / 4) + (e - R::kCl);
        }
    }
    __device__ void stage(F& f, const RecRegs<CP, LP>& r) const {
        float* base = reinterpret_cast<float*>(&f);
#pragma unroll
        for (int i = 0; i < R::kPer; ++i)
            if (off[i] >= 0) *reinterpret_cast<f32x4*>(base + off[i]) = r.v[i];
    }
};

template <int CP, int LP>
__global__ void __launch_bounds__(kThreads, 2) wy_factor_kernel(WyArgs a) {
    using F = BuildFactors<CP, LP>;
    using R = Rec<CP, LP>;
    __shared__ F f;
    const int tid = threadIdx.x;
    const int64_t head = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
    LatIn<F::RPT> in;
    load_latent<CP, LP>(a, head, c * CP, tid, in);
    float e[F::RPT], ie[F::RPT];
    make_factors<CP, LP>(f, in, a, c * CP, tid, e, ie);
    __syncthreads();
    f32x4* rec = reinterpret_cast<f32x4*>(a.rec + (head * a.n_chunks + c) * R::kSize);
    for (int j = tid; j < R::kN4; j += kThreads) rec[j] = *reinterpret_cast<const f32x4*>(rec_lds<CP, LP>(f, 4 * j));
}

// Blocks of the sequential kernels: block b runs dense tile dt of head
// (b / 8 / n_dt) * 8 + b % 8, so a head's tiles share one XCD (b % 8) and its
// records in that XCD's L2.  Returns false for the grid's padding blocks.
__device__ __forceinline__ bool seq_block(const WyArgs& a, int64_t* head, int64_t* d0) {
    const int64_t xcd = blockIdx.x % 8, rest = blockIdx.x / 8;
    *d0 = (rest % a.n_dt) * kDN;
    *head = (rest / a.n_dt) * 8 + xcd;
    return *head < a.BH;
}

// --------------------------------------------------------------- forward

// Stores without branches.  Loads and stores share one counter on gfx950,
// and where a store sits under a branch (a lane mask, an optional output) the
// compiler assumes, when it later waits for a load issued before the store,
// that the branch skipped it: the wait then also covers every store issued
// after that load.  A buffer resource over the output region drops stores at
// offsets past its size, so masked lanes (and an output that is not wanted,
// a region of size zero) store to an offset out of range instead, and every
// store instruction issues on every path.
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 buffer resource: 32-bit elements, no swizzle
struct OutRegion {
    static constexpr int kDrop = 0x7ffffffc;   // a byte offset past every region
    __amdgpu_buffer_rsrc_t r;
    // floats: the region's size (at most 64 rows of the API's largest D, 1024).
    __device__ OutRegion(float* base, int64_t floats)
        : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, base ? int(floats * 4) : 0, kRsrcWord3)) {}
    __device__ void store(float v, bool ok, int idx) const {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, ok ? idx * 4 : kDrop, 0, 0);
    }
    // Four floats from idx (a multiple of 4 in a 16-byte aligned region).
    __device__ void store4(const f32x4& v, bool ok, int idx) const {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(x, r, ok ? idx * 4 : kDrop & ~15, 0, 0);
    }
};


// The forward without a boundary buffer (no backward to follow, so nowhere
// to keep records): each chunk's factors are built here, one block per
// (head, 32 dense columns), the chunks in order.
template <int CP, int LP>
__global__ void __launch_bounds__(kThreads, 2) wy_fwd_fused_kernel(WyArgs a) {
    using F = BuildFactors<CP, LP>;
    constexpr int kDS = kSeqDS;   // dense tiles here are read only as row-major B operands
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT, RPT = F::RPT;
    constexpr int NS = (LP / 16) * (kDN / 16);        // state tiles
    constexpr int NSW = (NS + 3) / 4;                   // state tiles per wave
    __shared__ F f;
    __shared__ float sX[CP * kDS], sU[CP * kDS], sS[LP * kDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t head, d0;
    if (!seq_block(a, &head, &d0)) return;
    const int64_t nb = a.n_chunks;

    for (int idx = tid; idx < LP * kDN; idx += kThreads) {
        const int l = idx / kDN, n = idx % kDN;
        sS[l * kDS + n] = l < a.L && d0 + n < a.D ? a.s0[(head * a.L + l) * a.D + d0 + n] : 0.f;
    }

    // The next chunk's inputs are loaded into registers while this chunk
    // computes (barriers wait for LDS traffic only, not for these loads).
    constexpr int EPT = CP * kDN / kThreads;
    LatIn<RPT> in;
    float vv[EPT], ww[EPT];
    load_latent<CP, LP>(a, head, 0, tid, in);
    load_dense<CP, true>(a.v, a.w, a, head, 0, d0, tid, vv, ww);
    for (int64_t c = 0; c < nb; ++c) {
        const int64_t t0 = c * CP;
        // sX (this chunk's w.v) and the factors are free: their last readers
        // are behind the previous chunk's final barrier.
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int idx = tid + i * kThreads;
            sX[(idx / kDN) * kDS + idx % kDN] = dense_ok(a, t0, d0, tid, i) ? ww[i] * vv[i] : 0.f;
        }
        // Prefetches are unconditional: the last chunk reloads its own inputs
        // (dense loads past T are clamped and masked); a branch around them
        // would make the compiler wait for them where it rejoins.
        const int64_t cn = c + 1 < nb ? c + 1 : c;
        {
            float e[RPT], ie[RPT];
            make_factors<CP, LP>(f, in, a, t0, tid, e, ie);   // its barriers also order the stores above
        }
        load_latent<CP, LP>(a, head, cn * CP, tid, in);
        load_dense<CP, true>(a.v, a.w, a, head, cn * CP, d0, tid, vv, ww);

        // rhs = w.v - M S0 (in place in sX); wave 0 may still be finishing T.
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<LP, LS, 1, kDS, 1>(acc, f.M + ti * 16 * LS, sS + tj * 16, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* p = sX + (ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane);
                *p = *p - acc[r];
            }
        }
        __syncthreads();
        // U = T rhs (T lower triangular).
        const int lr = last_row(a, t0, CP), lc = last_col(a, d0), D = int(a.D);
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma16<CP, CS, 1, kDS, 1>(acc, f.Tm + ti * 16 * CS, sX + tj * 16, ti + 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sU[(ti * 16 + acc_row(lane, r)) * kDS + tj * 16 + acc_col(lane)] = acc[r];
        }
        __syncthreads();
        // O = (Qc S0 + Bq U) / sqrt(L).
        const OutRegion ob(a.ctx + tile_base(a, head, t0, 0), (lr + 1) * a.D);
        for (int job = wave; job < NT * 2; job += 4) {
            const int ti = job >> 1, tj = job & 1;
            f32x4 acc = zero4();
            mma<LP, LS, 1, kDS, 1>(acc, f.Qc + ti * 16 * LS, sS + tj * 16, lane);
            mma16<CP, CS, 1, kDS, 1>(acc, f.Bq + ti * 16 * CS, sU + tj * 16, ti + 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ti * 16 + acc_row(lane, r), col = tj * 16 + acc_col(lane);
                ob.store(acc[r] * a.scale, row <= lr && col <= lc, row * D + int(d0) + col);
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
                mma<CP, 1, LS, kDS, 1>(acc, f.Kt + ti * 16, sU + tj * 16, lane);
                snew[s] = acc;
            }
        }
        __syncthreads();
        // The state goes to the next chunk, and (last chunk) to the final state.
        const OutRegion sb(c + 1 == nb && a.state ? a.state + head * a.L * a.D : nullptr, a.L * a.D);
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int job = wave + 4 * s;
            if (job < NS) {
                const int ti = job >> 1, tj = job & 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = ti * 16 + acc_row(lane, r), n = tj * 16 + acc_col(lane);
                    sS[l * kDS + n] = snew[s][r];
                    sb.store(snew[s][r], l < a.L && n <= lc, l * D + int(d0) + n);
                }
            }
        }
    }
}

// The forward over saved records, one wave per 16-column strip of the dense
// axis: a block takes 64 dense columns of one head, and each of its first
// four waves (the chain waves) carries its strip's state S[:, strip] through
// the chunks alone.  Within a chunk no strip needs another's results:
// rhs = w.v - M S, U = T rhs, O and S_end of a strip use only that strip's
// columns, and every product takes its B operand straight from the
// accumulators of the one before (acc_mma), so the chain from S to S_end
// passes through no LDS (a chain wave loads only its w and v).  The block's
// other four waves (the memory waves, one per strip) stage the next chunk's
// record into the other of two LDS copies, load the one after, and store the
// previous chunk's U, context and state, which the chain wave left in LDS
// (two copies per strip, as for the records).  The two kinds of wave share
// each SIMD, so one's memory waits and the other's MFMA chains overlap, and a
// chunk costs one barrier.  LDS operations of one wave complete in order, so
// wave_sync (wavefront-scope fences around a wave barrier: no instructions,
// only no compiler reordering) orders a wave's own transposes.
constexpr int kStrip = 16;                 // dense columns per strip
constexpr int kStripBlock = 4 * kStrip;    // dense columns per block
constexpr int kStripThreads = 2 * kThreads;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CP, int LP>
struct alignas(16) StripOut {              // one strip's chunk results, transposed: U^T, O^T [16][CP + 4], S^T [16][LP + 4]
    float ut[16 * (CP + 4)], ot[16 * (CP + 4)], st[16 * (LP + 4)];
};

// kVec: dense rows 16-byte aligned (D a multiple of 4; w, v, the context,
// the final state, the saved state and U aligned): w and v are loaded, and U,
// the context and the state stored, as 16-byte row pieces (lane: rows
// vr + 16 k, columns vn .. vn + 3 of its strip), a quarter of the memory
// instructions; w.v reaches the accumulator layout through the chain wave's
// own transpose.
template <int CP, int LP, bool kVec>
__global__ void __launch_bounds__(kStripThreads, 1) wy_fwd_strip_kernel(WyArgs a) {
    using F = StagedFactors<CP, LP>;
    using R = Rec<CP, LP>;
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT;
    constexpr int NL = LP / 16;            // 16-row tiles of the state
    constexpr int SST = LP + 4;            // row stride of S^T [16][LP]
    constexpr int SCT = CP + 4;            // row stride of U^T, O^T and x^T [16][CP]
    static_assert((SST / 4) % 2 == 1 && (SCT / 4) % 2 == 1 && (LS / 4) % 2 == 1 && (CS / 4) % 2 == 1,
                  "16-byte operand reads on distinct banks");
    __shared__ F f[2];
    __shared__ StripOut<CP, LP> out[2][4];
    __shared__ float xt[4][16 * SCT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool chain = wave < 4;           // wave-uniform role
    const int strip = wave & 3;
    const int g4 = 4 * (lane >> 4), col = lane & 15;   // accumulator rows g4 + r, column col
    // Blocks as the other sequential kernels deal them: a head's column groups on one XCD.
    const int64_t n_dg = (a.D + kStripBlock - 1) / kStripBlock;
    const int64_t xcd = blockIdx.x % 8, rest = blockIdx.x / 8;
    const int64_t head = (rest / n_dg) * 8 + xcd;
    if (head >= a.BH) return;
    const int64_t d0 = (rest % n_dg) * kStripBlock + kStrip * strip;   // the strip's first column
    const int64_t nb = a.n_chunks;
    const int D = int(a.D);
    const bool col_ok = d0 + col < a.D;
    const int cc = int(d0 + col < a.D ? d0 + col : a.D - 1);         // clamped column (absolute)
    const int vr = lane >> 2, vn = 4 * (lane & 3);                    // kVec row pieces
    const bool vcol = d0 + vn < a.D;
    const int vcc = int(vcol ? d0 + vn : a.D - 4);   // kVec: clamped first column (D >= 4)
    const float* recs = a.rec + head * nb * R::kSize;

    if (chain) {
        // ------------------------------------------------ chain wave
        float* myX = xt[strip];
        // w and v of a chunk, raw and clamped (masked where used): at this
        // lane's accumulator elements, or (kVec) row pieces.
        float wv[NT][4], vv[NT][4];
        auto load_wv = [&](int64_t c) {
            const int64_t t0 = c * CP;
            const int lr = last_row(a, t0, CP);
            const float* wb = a.w + (head * a.T + t0) * a.D;
            const float* vb = a.v + (head * a.T + t0) * a.D;
            if constexpr (kVec) {
#pragma unroll
                for (int k = 0; k < NT; ++k) {
                    const int row = vr + 16 * k;
                    const int off = (row < lr ? row : lr) * D + vcc;
                    const f32x4 w4 = *reinterpret_cast<const f32x4*>(wb + off);
                    const f32x4 v4 = *reinterpret_cast<const f32x4*>(vb + off);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wv[k][e] = w4[e];
                        vv[k][e] = v4[e];
                    }
                }
            } else {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * ti + g4 + r;
                        const int off = (row < lr ? row : lr) * D + cc;
                        wv[ti][r] = wb[off];
                        vv[ti][r] = vb[off];
                    }
            }
        };
        auto write_t = [&](float* dstT, int stride, int row0, const f32x4& v) {   // rows row0 + g4 + r, column col
            *reinterpret_cast<f32x4*>(dstT + col * stride + row0 + g4) = v;
        };

        // The state entering chunk 0, in accumulator layout: S[16 tl + g4 + r][col].
        f32x4 sc[NL];
        const float* s0 = a.s0 + head * a.L * a.D;
#pragma unroll
        for (int tl = 0; tl < NL; ++tl)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int l = 16 * tl + g4 + r;
                sc[tl][r] = s0[(l < a.L ? l : int(a.L) - 1) * D + cc];   // clamped, masked below
            }
        load_wv(0);
        // The state goes to chunk 0's boundary slot after the loads above, as
        // every chunk's stores follow its loads: the wait for w and v at the
        // top of the loop then need not cover the stores.
        {
            const OutRegion b0(a.bnd ? a.bnd + head * nb * LP * a.D : nullptr, LP * a.D);
#pragma unroll
            for (int tl = 0; tl < NL; ++tl)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = 16 * tl + g4 + r;
                    const bool ok = l < a.L && col_ok;
                    sc[tl][r] = ok ? sc[tl][r] : 0.f;
                    b0.store(sc[tl][r], ok, l * D + int(d0) + col);
                }
        }
        __syncthreads();   // record 0 staged

        for (int64_t c = 0; c < nb; ++c) {
            const int64_t t0 = c * CP;
            F& fc = f[c & 1];
            // x = w.v of this chunk (zero on padded steps), as the negated
            // initial value of M S - x.
            f32x4 nr[NT];
            if constexpr (kVec) {
                // Rows of -x into the strip's x^T, read back in the accumulator layout.
#pragma unroll
                for (int k = 0; k < NT; ++k) {
                    const int row = vr + 16 * k;
                    const bool ok = t0 + row < a.T && vcol;
#pragma unroll
                    for (int e = 0; e < 4; ++e) myX[(vn + e) * SCT + row] = ok ? -(wv[k][e] * vv[k][e]) : 0.f;
                }
                wave_sync();
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) nr[ti] = *reinterpret_cast<const f32x4*>(myX + col * SCT + 16 * ti + g4);
            } else {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool ok = t0 + 16 * ti + g4 + r < a.T && col_ok;
                        nr[ti][r] = ok ? -(wv[ti][r] * vv[ti][r]) : 0.f;
                    }
            }
            load_wv(c + 1 < nb ? c + 1 : c);   // unconditional, clamped
            __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of the chunk's products
            // Every A operand of the chunk's products (none depends on the
            // state), read before the chain from S to S_end starts.
            f32x4 amq[2 * NT][LP / 16], at[NT][1], ab[NT][1], ak[NL][CP / 16];
            {
                const float* pmq[2 * NT];
                const float* pt[NT];
                const float* pb[NT];
                const float* pk[NL];
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    pmq[2 * ti] = fc.M + 16 * ti * LS;
                    pmq[2 * ti + 1] = fc.Qc + 16 * ti * LS;
                    // Row tile 1 of T and Bq (lower triangular) sums over steps
                    // 0..15 together with row tile 0, then over 16..31 alone.
                    pt[ti] = fc.Tm + 16 * ti * CS;
                    pb[ti] = fc.Bq + 16 * ti * CS;
                }
#pragma unroll
                for (int tl = 0; tl < NL; ++tl) pk[tl] = fc.Kt + 16 * tl;
                acc_a<2 * NT, LP, LS, 1>(amq, pmq, lane);
                acc_a<NT, 16, CS, 1>(at, pt, lane);
                acc_a<NT, 16, CS, 1>(ab, pb, lane);
                acc_a<NL, CP, 1, LS>(ak, pk, lane);
            }
            f32x4 at1[1][1], ab1[1][1];
            if constexpr (NT == 2) {
                const float* pt1[1] = {fc.Tm + 16 * CS + 16};
                const float* pb1[1] = {fc.Bq + 16 * CS + 16};
                acc_a<1, 16, CS, 1>(at1, pt1, lane);
                acc_a<1, 16, CS, 1>(ab1, pb1, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
            // M S - x and Qc S (independent chains), S straight from the
            // accumulators.
            f32x4 o[NT];
            {
                f32x4 acc[2 * NT];
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    acc[2 * ti] = nr[ti];
                    acc[2 * ti + 1] = zero4();
                }
                acc_mma<2 * NT, LP>(acc, amq, sc);
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    nr[ti] = acc[2 * ti];
                    o[ti] = acc[2 * ti + 1];
                }
            }
            // U = -T (M S - x).
            f32x4 u[NT];
            {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) u[ti] = zero4();
                acc_mma<NT, 16>(u, at, nr);
                if constexpr (NT == 2) {
                    f32x4 u1[1] = {u[1]};
                    acc_mma<1, 16>(u1, at1, nr + 1);
                    u[1] = u1[0];
                }
#pragma unroll
                for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[ti][r] = -u[ti][r];
            }
            // O = (Qc S + Bq U) / sqrt(L) and S_end = diag(c_last) S + Kt^T U:
            // independent chains over U.
            {
#pragma unroll
                for (int tl = 0; tl < NL; ++tl)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[tl][r] *= fc.clast[16 * tl + g4 + r];
                acc_mma<NT, 16>(o, ab, u);
                if constexpr (NT == 2) {
                    f32x4 o1[1] = {o[1]};
                    acc_mma<1, 16>(o1, ab1, u + 1);
                    o[1] = o1[0];
                }
                acc_mma<NL, CP>(sc, ak, u);
#pragma unroll
                for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[ti][r] *= a.scale;
            }
            // The chunk's results to the strip's output copy, for its memory wave.
            StripOut<CP, LP>& so = out[c & 1][strip];
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                write_t(so.ut, SCT, 16 * ti, u[ti]);
                write_t(so.ot, SCT, 16 * ti, o[ti]);
            }
#pragma unroll
            for (int tl = 0; tl < NL; ++tl) write_t(so.st, SST, 16 * tl, sc[tl]);
            __syncthreads();   // results handed over; the next record staged, this one free
        }
    } else {
        // ------------------------------------------------ memory wave
        const int mtid = tid - kThreads;   // 0 .. 255 over the four memory waves
        // One chunk's U (all CP rows, for the backward), context (rows < T)
        // and end state (to the next chunk's boundary slot, or after the last
        // chunk to the final state), from the chain wave's output copy.
        // Every store instruction issues whether or not `live` (dropped
        // lanes): a store under a branch would make the compiler's wait for
        // the record at the top of the loop cover the stores.  `buf` is the
        // output copy read: chunk c's, or (not live) the one no chain wave
        // writes during the first chunk.
        auto store_out = [&](int64_t c, int buf, bool live) {
            const int64_t t0 = c * CP;
            const StripOut<CP, LP>& so = out[buf][strip];
            const OutRegion ub(a.ubuf ? a.ubuf + (head * nb * CP + t0) * a.D : nullptr, CP * a.D);
            const int rows = a.T - t0 < CP ? int(a.T - t0) : CP;
            const OutRegion ob(a.ctx + (head * a.T + t0) * a.D, rows * a.D);
            const OutRegion sb = c + 1 < nb
                ? OutRegion(a.bnd ? a.bnd + (head * nb + c + 1) * LP * a.D : nullptr, LP * a.D)
                : OutRegion(a.state ? a.state + head * a.L * a.D : nullptr, a.L * a.D);
            if constexpr (kVec) {
                auto row4 = [&](const float* srcT, int stride, int row) {
                    return f32x4{srcT[vn * stride + row], srcT[(vn + 1) * stride + row],
                                 srcT[(vn + 2) * stride + row], srcT[(vn + 3) * stride + row]};
                };
#pragma unroll
                for (int k = 0; k < NT; ++k) {
                    const int row = vr + 16 * k;
                    ub.store4(row4(so.ut, SCT, row), live && vcol, row * D + vcc);
                    ob.store4(row4(so.ot, SCT, row), live && vcol && row < rows, row * D + vcc);
                }
#pragma unroll
                for (int k = 0; k < NL; ++k) {
                    const int l = vr + 16 * k;
                    sb.store4(row4(so.st, SST, l), live && vcol && l < a.L, l * D + vcc);
                }
            } else {
                // Lane: column col, rows 4 k + lane / 16.
                const int rq = lane >> 4;
#pragma unroll
                for (int k = 0; k < CP / 4; ++k) {
                    const int row = 4 * k + rq;
                    ub.store(so.ut[col * SCT + row], live && col_ok, row * D + int(d0) + col);
                    ob.store(so.ot[col * SCT + row], live && col_ok && row < rows, row * D + int(d0) + col);
                }
#pragma unroll
                for (int k = 0; k < LP / 4; ++k) {
                    const int l = 4 * k + rq;
                    sb.store(so.st[col * SST + l], live && col_ok && l < a.L, l * D + int(d0) + col);
                }
            }
        };

        RecRegs<CP, LP> rr;
        const RecStage<CP, LP, F> rs(mtid);
        load_rec<CP, LP>(rr, recs, mtid);
        rs.stage(f[0], rr);
        load_rec<CP, LP>(rr, recs + (nb > 1 ? 1 : 0) * R::kSize, mtid);
        // As many (dropped) stores after that load as every chunk issues after
        // its own, so that the wait for the record at the top of the loop does
        // not cover the stores on any path into it.
        store_out(0, 1, false);
        __syncthreads();   // record 0 staged

        for (int64_t c = 0; c < nb; ++c) {
            // The next chunk's record into the other copy (its last readers
            // were behind the previous barrier), the load of the one after
            // (unconditional, clamped), then the previous chunk's results out.
            rs.stage(f[(c + 1) & 1], rr);
            const int64_t c2 = c + 2 < nb ? c + 2 : nb - 1;
            load_rec<CP, LP>(rr, recs + c2 * R::kSize, mtid);
            store_out(c > 0 ? c - 1 : 0, int((c + 1) & 1), c > 0);
            __syncthreads();
        }
        store_out(nb - 1, int((nb - 1) & 1), true);
    }
}

// ----------------------------------------------------- backward: the carry

// The reverse carry over saved records, one wave per 16-column strip: each
// wave carries its strip of dS through the chunks in reverse, the chunk's
// record the only shared operand (two LDS copies, one barrier per chunk).
// The chain from dS to the dS entering the chunk takes its B operands from
// the accumulators (acc_mma); dO^T, which the products with dO read, and
// drhs^T, on its way to 16-byte row stores, pass through the wave's own LDS
// area.
template <int CP, int LP>
struct alignas(16) CarryStripT {          // one wave's transposes: dO^T and drhs^T [16][CP + 4]
    float ot[16 * (CP + 4)], rt[16 * (CP + 4)];
};

// kVec: dense rows 16-byte aligned (D a multiple of 4; dO, w, v, dw, dv and
// drhs aligned): dO, w and v are loaded, and drhs, dw and dv stored, as
// 16-byte row pieces (lane: rows vr + 16 k, columns vn .. vn + 3 of its
// strip), dO reaching its transpose and drhs its rows through LDS.
template <int CP, int LP, bool kVec>
__global__ void __launch_bounds__(kThreads, 1) wy_bwd_carry_strip_kernel(WyArgs a) {
    using F = StagedFactors<CP, LP>;
    using R = Rec<CP, LP>;
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT;
    constexpr int NL = LP / 16;
    constexpr int SCT = CP + 4;
    static_assert((SCT / 4) % 2 == 1 && (LS / 4) % 2 == 1 && CS % 4 == 0, "16-byte operand reads on distinct banks");
    __shared__ F f[2];
    __shared__ CarryStripT<CP, LP> strip[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = 4 * (lane >> 4), col = lane & 15;
    const int64_t n_dg = (a.D + kStripBlock - 1) / kStripBlock;
    const int64_t xcd = blockIdx.x % 8, rest = blockIdx.x / 8;
    const int64_t head = (rest / n_dg) * 8 + xcd;
    if (head >= a.BH) return;
    const int64_t d0 = (rest % n_dg) * kStripBlock + kStrip * wave;
    const int64_t nb = a.n_chunks;
    const int D = int(a.D);
    const float s = a.scale;
    const bool col_ok = d0 + col < a.D;
    const int cc = int(d0 + col < a.D ? d0 + col : a.D - 1);
    float* myOT = strip[wave].ot;
    float* myRT = strip[wave].rt;
    auto write_t = [&](float* dstT, int stride, int row0, const f32x4& v) {
        *reinterpret_cast<f32x4*>(dstT + col * stride + row0 + g4) = v;
    };

    // dO, w and v of chunk c at this lane's accumulator elements, or (kVec)
    // row pieces (raw, clamped).
    float ov[NT][4], wv[NT][4], vv[NT][4];
    const int vr = lane >> 2, vn = 4 * (lane & 3);
    const bool vcol = d0 + vn < a.D;
    const int vcc = int(vcol ? d0 + vn : a.D - 4);   // kVec: clamped first column (D >= 4)
    auto load_dense3 = [&](int64_t c) {
        const int64_t t0 = c * CP;
        const int lr = last_row(a, t0, CP);
        const int64_t base = (head * a.T + t0) * a.D;
        if constexpr (kVec) {
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int row = vr + 16 * k;
                const int off = (row < lr ? row : lr) * D + vcc;
                const f32x4 o4 = *reinterpret_cast<const f32x4*>(a.dctx + base + off);
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(a.w + base + off);
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(a.v + base + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ov[k][e] = o4[e];
                    wv[k][e] = w4[e];
                    vv[k][e] = v4[e];
                }
            }
        } else {
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * ti + g4 + r;
                    const int off = (row < lr ? row : lr) * D + cc;
                    ov[ti][r] = a.dctx[base + off];
                    wv[ti][r] = a.w[base + off];
                    vv[ti][r] = a.v[base + off];
                }
        }
    };

    // The cotangent of the final state (zero if none), in accumulator layout,
    // is what enters the last chunk from later ones.
    f32x4 sc[NL];
    {
        if (a.dstate) {
            const float* ds = a.dstate + head * a.L * a.D;
#pragma unroll
            for (int tl = 0; tl < NL; ++tl)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = 16 * tl + g4 + r;
                    sc[tl][r] = ds[(l < a.L ? l : int(a.L) - 1) * D + cc];
                }
        } else {
#pragma unroll
            for (int tl = 0; tl < NL; ++tl) sc[tl] = zero4();
        }
    }

    RecRegs<CP, LP> rr;
    const RecStage<CP, LP, F> rs(tid);
    const float* recs = a.rec + head * nb * R::kSize;
    load_rec<CP, LP>(rr, recs + (nb - 1) * R::kSize, tid);
    rs.stage(f[(nb - 1) & 1], rr);
    load_rec<CP, LP>(rr, recs + (nb > 1 ? nb - 2 : 0) * R::kSize, tid);
    load_dense3(nb - 1);
    // The last chunk's slot after the loads above, as every chunk's stores
    // follow its loads (so the waits at the top of the loop need not cover
    // stores).
    {
        const OutRegion b0(a.dbnd + (head * nb + nb - 1) * LP * a.D, LP * a.D);
#pragma unroll
        for (int tl = 0; tl < NL; ++tl)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int l = 16 * tl + g4 + r;
                const bool ok = l < a.L && col_ok;
                sc[tl][r] = ok ? sc[tl][r] : 0.f;
                b0.store(sc[tl][r], ok, l * D + int(d0) + col);
            }
    }
    __syncthreads();

    for (int64_t c = nb - 1; c >= 0; --c) {
        const int64_t t0 = c * CP;
        F& fc = f[c & 1];
        const int rows = a.T - t0 < CP ? int(a.T - t0) : CP;
        // dO of this chunk (zero past T) into its transpose; w and v kept for dw, dv.
        float wc[NT][4], vc[NT][4];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            if constexpr (kVec) {
                const int row = vr + 16 * ti;
                const bool ok = row < rows && vcol;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    myOT[(vn + e) * SCT + row] = ok ? ov[ti][e] : 0.f;
                    wc[ti][e] = wv[ti][e];
                    vc[ti][e] = vv[ti][e];
                }
            } else {
                f32x4 o4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = 16 * ti + g4 + r < rows && col_ok;
                    o4[r] = ok ? ov[ti][r] : 0.f;
                    wc[ti][r] = wv[ti][r];
                    vc[ti][r] = vv[ti][r];
                }
                write_t(myOT, SCT, 16 * ti, o4);
            }
        }
        // The previous chunk's record into the other copy, then the loads for
        // earlier chunks (unconditional, clamped).
        rs.stage(f[(c + 1) & 1], rr);
        load_rec<CP, LP>(rr, recs + (c >= 2 ? c - 2 : 0) * R::kSize, tid);
        load_dense3(c >= 1 ? c - 1 : 0);
        wave_sync();

        // The chunk's loads stay ahead of its products.
        __builtin_amdgcn_sched_barrier(0);
        // The A operands of the chain from dS to the dS entering this chunk,
        // read before it starts; the chain takes every B operand from the
        // accumulators, and the products with dO (its transpose in LDS) hang
        // off it.
        f32x4 ak[NT][LP / 16], at0[1][CP / 16], at1[1][1], am[NL][CP / 16];
        {
            const float* pk[NT];
            const float* pm[NL];
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) pk[ti] = fc.Kt + 16 * ti * LS;
#pragma unroll
            for (int tl = 0; tl < NL; ++tl) pm[tl] = fc.M + 16 * tl;
            const float* pt0[1] = {fc.Tm};
            acc_a<NT, LP, LS, 1>(ak, pk, lane);
            acc_a<1, CP, 1, CS>(at0, pt0, lane);
            if constexpr (NT == 2) {
                const float* pt1[1] = {fc.Tm + 16 * CS + 16};
                acc_a<1, 16, 1, CS>(at1, pt1, lane);
            }
            acc_a<NL, CP, 1, LS>(am, pm, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tl = 0; tl < NL; ++tl)
#pragma unroll
            for (int t = 0; t < CP / 16; ++t) am[tl][t] = -am[tl][t];   // for dS0 -= M^T drhs
        // dU = Bq^T dO / sqrt(L) + Kt dS  (Bq^T upper triangular: tile ti
        // sums over steps 16 ti ..).
        f32x4 du[NT], kd[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            du[ti] = zero4();
            kd[ti] = zero4();
        }
        acc_mma<NT, LP>(kd, ak, sc);
        mma<CP, 1, CS, 1, SCT>(du[0], fc.Bq, myOT, lane);
        if constexpr (NT == 2) mma<16, 1, CS, 1, SCT>(du[1], fc.Bq + 16 * CS + 16, myOT + 16, lane);
        // diag(c_last) dS + Qc^T dO / sqrt(L), which M^T drhs is taken from below.
#pragma unroll
        for (int tl = 0; tl < NL; ++tl) {
            f32x4 aq = zero4();
            mma<CP, 1, LS, 1, SCT>(aq, fc.Qc + 16 * tl, myOT, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[tl][r] = fc.clast[16 * tl + g4 + r] * sc[tl][r] + aq[r] * s;
        }
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
            for (int r = 0; r < 4; ++r) du[ti][r] = du[ti][r] * s + kd[ti][r];
        // drhs = T^T dU (upper triangular as Bq^T); dw = drhs . v, dv = drhs . w.
        f32x4 dr[NT];
        {
            f32x4 d0a[1] = {zero4()};
            acc_mma<1, CP>(d0a, at0, du);
            dr[0] = d0a[0];
            if constexpr (NT == 2) {
                f32x4 d1a[1] = {zero4()};
                acc_mma<1, 16>(d1a, at1, du + 1);
                dr[1] = d1a[0];
            }
        }
        // dS0 = diag(c_last) dS + Qc^T dO / sqrt(L) - M^T drhs.
        acc_mma<NL, CP>(sc, am, dr);
        const OutRegion rb(a.drhs + (head * nb * CP + t0) * a.D, CP * a.D);
        const int64_t gbase = (head * a.T + t0) * a.D;
        const OutRegion dwb(a.dw ? a.dw + gbase : nullptr, rows * a.D);
        const OutRegion dvb(a.dv ? a.dv + gbase : nullptr, rows * a.D);
        if constexpr (kVec) {   // rows of drhs from its transpose; drhs, dw, dv as 16-byte pieces
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) write_t(myRT, SCT, 16 * ti, dr[ti]);
            wave_sync();
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const int row = vr + 16 * k, off = row * D + vcc;
                f32x4 d4, w4, v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    d4[e] = myRT[(vn + e) * SCT + row];
                    w4[e] = d4[e] * vc[k][e];
                    v4[e] = d4[e] * wc[k][e];
                }
                rb.store4(d4, vcol, off);   // for the gradient kernel
                dwb.store4(w4, vcol && row < rows, off);
                dvb.store4(v4, vcol && row < rows, off);
            }
        } else {
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * ti + g4 + r;
                    const int off = row * D + int(d0) + col;
                    rb.store(dr[ti][r], col_ok, off);   // for the gradient kernel
                    dwb.store(dr[ti][r] * vc[ti][r], col_ok && row < rows, off);
                    dvb.store(dr[ti][r] * wc[ti][r], col_ok && row < rows, off);
                }
        }
        // dS entering this chunk: the previous chunk's slot, or (first chunk)
        // d initial_state.
        const OutRegion db = c > 0 ? OutRegion(a.dbnd + (head * nb + c - 1) * LP * a.D, LP * a.D)
                                   : OutRegion(a.ds0 ? a.ds0 + head * a.L * a.D : nullptr, a.L * a.D);
#pragma unroll
        for (int tl = 0; tl < NL; ++tl)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int l = 16 * tl + g4 + r;
                db.store(sc[tl][r], l < a.L && col_ok, l * D + int(d0) + col);
            }
        __syncthreads();   // the previous record is staged, this one is free for the one before
    }
}

// ------------------------------------------------ backward: the gradients

template <int CP, int LP>
struct alignas(16) GradTiles {
    // The walk over dense tiles; reused for the final per-chunk matrices.
    union {
        struct {
            float S[LP * kDS];    // boundary state tile S0
            float D[LP * kDS];    // dSc = diag(c_last) dS tile
            float O[CP * kDS];    // dO
            float U[CP * kDS];    // U (saved by the forward)
            float R[CP * kDS];    // drhs (from the carry kernel)
        } t;
        struct {
            float dQc[CP * LP], dM[CP * LP], dWb[CP * LP], P[CP * LP];
            float xl[kThreads];
            float red[2 * kThreads];
        } m;
    };
};

// kVec: dense rows 16-byte aligned (D a multiple of 4, every dense base
// aligned; chunks of 32, latent rows of 32 or 64): a dense tile's loads are
// 16-byte vectors, a quarter of the load instructions, and U, drhs and dO
// are held as one float4 per thread (row tid / 8, columns 4 (tid % 8) ..).
template <int CP, int LP, bool kVec>
__global__ void __launch_bounds__(kThreads, 2) wy_bwd_grad_kernel(WyArgs a) {
    using F = FactorsT<CP, LP, LP + 4, true, false, true>;   // no Kt: the record's Kt is skipped
    constexpr int LS = F::LS, CS = F::CS, NT = F::NT, RPT = F::RPT, RG = F::RG;
    constexpr int NJ = NT * (NT + 1) / 2;            // lower tiles of a CP x CP matrix
    constexpr int NL = NT * (LP / 16);               // tiles of a CP x LP matrix
    constexpr int NCC = (2 * NJ + 3) / 4;            // CP x CP accumulator tiles per wave (dBq then dA)
    constexpr int NCL = (NL + 3) / 4;                // CP x LP tiles per wave (dQc, dM, P each)
    __shared__ F f;
    __shared__ GradTiles<CP, LP> g;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nb = a.n_chunks;
    const uint32_t nb32 = uint32_t(nb), n_items = uint32_t(a.BH * nb);   // the launch checks both fit
    const float s = a.scale;

    // rowsum(dSc . S0) partials: thread (l = tid / (256 / LP) ...) over its elements.
    constexpr int TPL = kThreads / LP;               // threads per latent row
    constexpr int EPL = kDN / TPL;                   // elements per thread per tile
    constexpr int EPT = CP * kDN / kThreads;
    // One dense tile's loads, in registers: S0 and dS (this thread's row
    // l = tid / TPL, EPL columns), and U (saved by the forward), drhs (written
    // by the carry kernel) and dO (elements tid + i * kThreads of the
    // [CP][kDN] tile).  The next tile's are issued while this one computes,
    // the next item's first tile during this item's last; values are raw
    // (clamped) and masked where consumed.
    float sv[EPL], dsv[EPL], uu[EPT], rv[EPT], oo[EPT];
    const int xl_l = tid / TPL, xl_n0 = (tid % TPL) * EPL;
    constexpr int SV = EPL < 4 ? EPL : 4;            // floats per LDS vector store of S0 and dSc
    typedef float svec __attribute__((ext_vector_type(SV)));
    static_assert(EPL % SV == 0 && kDS % SV == 0, "aligned vector stores");
    const int xl_lc = xl_l < a.L ? xl_l : int(a.L) - 1, D = int(a.D);
    static_assert(!kVec || (CP * kDN == 4 * kThreads && EPT == 4 && EPL % 4 == 0), "vector tile layout");
    const int v_row = tid / (kDN / 4), v_n = 4 * (tid % (kDN / 4));   // kVec: U, drhs, dO element of this thread
    auto load_tile = [&](int64_t head, int64_t c, int64_t d0) {
        // Block-uniform bases and 32-bit clamped offsets (see tile_base).
        const int lc = last_col(a, d0);
        const int64_t sbase = (head * nb + c) * LP * a.D + d0;
        const float* sb = a.bnd_in + sbase;
        const float* dsb = a.dbnd + sbase;
        const int64_t ubase = (head * nb + c) * CP * a.D + d0;
        const float* ub = a.ubuf + ubase;
        const float* rb = a.drhs + ubase;
        if constexpr (kVec) {
            // lc + 1 is a multiple of 4: a float4 is wholly inside or wholly past D (clamped to the last).
#pragma unroll
            for (int j = 0; j < EPL / 4; ++j) {
                const int n = xl_n0 + 4 * j;
                const int off = xl_lc * D + (n < lc ? n : lc - 3);
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(sb + off);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsb + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[4 * j + e] = s4[e];
                    dsv[4 * j + e] = d4[e];
                }
            }
            const int off = v_row * D + (v_n < lc ? v_n : lc - 3);
            const int lr = last_row(a, c * CP, CP);
            const int ooff = (v_row < lr ? v_row : lr) * D + (v_n < lc ? v_n : lc - 3);
            const f32x4 u4 = *reinterpret_cast<const f32x4*>(ub + off);
            const f32x4 r4 = *reinterpret_cast<const f32x4*>(rb + off);
            const f32x4 o4 = *reinterpret_cast<const f32x4*>(a.dctx + tile_base(a, head, c * CP, d0) + ooff);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uu[e] = u4[e];
                rv[e] = r4[e];
                oo[e] = o4[e];
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int n = xl_n0 + i;
                const int off = xl_lc * D + (n < lc ? n : lc);
                sv[i] = sb[off];
                dsv[i] = dsb[off];
            }
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int idx = tid + i * kThreads, n = idx % kDN;
                const int off = (idx / kDN) * D + (n < lc ? n : lc);
                uu[i] = ub[off];
                rv[i] = rb[off];
            }
            load_dense<CP, false>(a.dctx, nullptr, a, head, c * CP, d0, tid, oo, nullptr);
        }
    };

    // An item's other loads: its latent inputs k, b, g (raw, clamped copies
    // past T or L) and its record's M, Qc and c_last.
    using R = Rec<CP, LP>;
    constexpr int NR4 = R::kKt / 4 + LP / 4;        // float4 of M, Qc and c_last
    constexpr int RPER = (NR4 + kThreads - 1) / kThreads;
    LatIn<RPT> raw;
    f32x4 recv[RPER];
    auto load_item = [&](int64_t head, int64_t c) {
        const int l = tid % LP, rg = tid / LP;
        const int64_t lc = l < a.L ? l : a.L - 1;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int64_t t = c * CP + rg * RPT + i;
            const int64_t idx = (head * a.T + (t < a.T ? t : a.T - 1)) * a.L + lc;
            raw.k[i] = a.k[idx];
            raw.b[i] = a.b[idx];
            raw.g[i] = a.g[idx];
        }
        const f32x4* rec4 = reinterpret_cast<const f32x4*>(a.rec + (head * nb + c) * R::kSize);
#pragma unroll
        for (int i = 0; i < RPER; ++i) {
            const int j = tid + i * kThreads;
            const int jj = j < NR4 ? j : NR4 - 1;
            recv[i] = rec4[jj < R::kKt / 4 ? jj : R::kCl / 4 + (jj - R::kKt / 4)];
        }
    };

    // Items (head, chunk) = (item / n_chunks, item % n_chunks), item =
    // blockIdx.x, blockIdx.x + gridDim.x, ...: the grid is as many blocks as
    // the device holds at once, so every load of an item but the first is
    // issued during the item before (the first: before any wait).
    uint32_t item = blockIdx.x;
    load_item(item / nb32, item % nb32);
    load_tile(item / nb32, item % nb32, 0);
    for (; item < n_items; item += gridDim.x) {
        const int64_t head = item / nb32, c = item % nb32, t0 = c * CP;
        const uint32_t nxt = item + gridDim.x < n_items ? item + gridDim.x : item;
        const int64_t nhead = nxt / nb32, nc = nxt % nb32;
        LatIn<RPT> in;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const bool ok = latent_ok<CP, LP, RPT>(a, t0, tid, i);
            in.k[i] = ok ? raw.k[i] : 0.f;
            in.b[i] = ok ? raw.b[i] : 0.f;
            in.g[i] = ok ? raw.g[i] : 0.f;
        }
        // c and 1/c of this thread's rows, as the factor kernel forms them, from
        // the rows' g and the group sums in f.tot (which stay put until the next
        // item, so the epilogue forms them again instead of keeping them live).
        auto row_scales = [&](float* e, float* ie) {
            const int l = tid % LP, rg = tid / LP;
            float off = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r)
                if (r < rg) off += f.tot[r * LP + l];
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                run += in.g[i];
                e[i] = __expf(off + run);
                ie[i] = __expf(-(off + run));
            }
        };
        {
            const int l = tid % LP, rg = tid / LP;
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) run += in.g[i];
            f.tot[rg * LP + l] = run;
            __syncthreads();
            float e[RPT], ie[RPT];
            row_scales(e, ie);
#pragma unroll
            for (int i = 0; i < RPT; ++i) f.Wb[(rg * RPT + i) * LS + l] = in.k[i] * ie[i];   // Wb = k / c
        }
#pragma unroll
        for (int i = 0; i < RPER; ++i) {
            const int j = tid + i * kThreads;
            if (j < NR4) {
                const int e4 = j < R::kKt / 4 ? 4 * j : R::kCl + 4 * (j - R::kKt / 4);
                *reinterpret_cast<f32x4*>(rec_lds<CP, LP>(f, e4)) = recv[i];
            }
        }

        f32x4 accC[NCC], accQ[NCL], accM[NCL], accP[NCL];
#pragma unroll
        for (int i = 0; i < NCC; ++i) accC[i] = zero4();
#pragma unroll
        for (int i = 0; i < NCL; ++i) accQ[i] = accM[i] = accP[i] = zero4();
        float xl = 0.f;

        __syncthreads();   // the record and Wb are in LDS
        for (int dt = 0; dt < a.n_dt; ++dt) {
            const int64_t d0 = int64_t(dt) * kDN;
            // Masks in 32 bits against the tile's own extent, c_last read once
            // and unconditionally (a conditional LDS read had become a branch
            // and an LDS wait per element), and this thread's EPL adjacent
            // S0 and dSc columns stored as whole vectors.
            const int ncols = a.D - d0 < kDN ? int(a.D - d0) : kDN;
            const int nrows = a.T - t0 < CP ? int(a.T - t0) : CP;
            const float cl = f.clast[xl_l];
            const bool lok = xl_l < a.L;
#pragma unroll
            for (int j = 0; j < EPL / SV; ++j) {
                svec s4, d4;
#pragma unroll
                for (int e = 0; e < SV; ++e) {
                    const int i = j * SV + e;
                    const bool ok = lok && xl_n0 + i < ncols;
                    s4[e] = ok ? sv[i] : 0.f;
                    d4[e] = ok ? dsv[i] * cl : 0.f;
                    xl += d4[e] * s4[e];
                }
                *reinterpret_cast<svec*>(g.t.S + xl_l * kDS + xl_n0 + j * SV) = s4;
                *reinterpret_cast<svec*>(g.t.D + xl_l * kDS + xl_n0 + j * SV) = d4;
            }
            if constexpr (kVec) {
                const bool okd = v_n < ncols, oko = okd && v_row < nrows;
                f32x4 u4, r4, o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u4[e] = okd ? uu[e] : 0.f;
                    r4[e] = okd ? rv[e] : 0.f;
                    o4[e] = oko ? oo[e] : 0.f;
                }
                *reinterpret_cast<f32x4*>(g.t.U + v_row * kDS + v_n) = u4;
                *reinterpret_cast<f32x4*>(g.t.R + v_row * kDS + v_n) = r4;
                *reinterpret_cast<f32x4*>(g.t.O + v_row * kDS + v_n) = o4;
            } else {
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    const int idx = tid + i * kThreads, row = idx / kDN, n = idx % kDN;
                    const bool okd = n < ncols;
                    g.t.U[row * kDS + n] = okd ? uu[i] : 0.f;
                    g.t.R[row * kDS + n] = okd ? rv[i] : 0.f;
                    g.t.O[row * kDS + n] = okd && row < nrows ? oo[i] : 0.f;
                }
            }
            // The next dense tile, or the next item's first (unconditional: see the forward).
            const bool more = dt + 1 < a.n_dt;
            load_tile(more ? head : nhead, more ? c : nc, more ? d0 + kDN : 0);
            __syncthreads();
            // Sums over the dense axis: dO U^T, drhs U^T (lower tiles), dO S0^T, drhs S0^T, U dSc^T.
#pragma unroll
            for (int sl = 0; sl < NCC; ++sl) {
                const int job = wave + 4 * sl;
                if (job < 2 * NJ) {
                    const bool isA = job >= NJ;
                    int ti, tj;
                    lower_tile(isA ? job - NJ : job, ti, tj);
                    mma_kc<kDN, kDS, kDS>(accC[sl], (isA ? g.t.R : g.t.O) + ti * 16 * kDS, g.t.U + tj * 16 * kDS, lane);
                }
            }
#pragma unroll
            for (int sl = 0; sl < NCL; ++sl) {
                const int job = wave + 4 * sl;
                if (job < NL) {
                    const int ti = job / (LP / 16), lj = job % (LP / 16);
                    mma_kc<kDN, kDS, kDS>(accQ[sl], g.t.O + ti * 16 * kDS, g.t.S + lj * 16 * kDS, lane);
                    mma_kc<kDN, kDS, kDS>(accM[sl], g.t.R + ti * 16 * kDS, g.t.S + lj * 16 * kDS, lane);
                    mma_kc<kDN, kDS, kDS>(accP[sl], g.t.U + ti * 16 * kDS, g.t.D + lj * 16 * kDS, lane);
                }
            }
            __syncthreads();
        }

        load_item(nhead, nc);   // the next item's latents and record, consumed at its start
        // dBq = lower(dO U^T) / sqrt(L) into f.Bq, dA = -strictly lower(drhs U^T) into f.Tm
        // (their buffers are free: this kernel reads neither T nor Bq).
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
        if constexpr (NT > 1) {   // their upper tile (0, 1) is zero
            for (int idx = tid; idx < 256; idx += kThreads) {
                f.Tm[(idx / 16) * CS + 16 + idx % 16] = 0.f;
                f.Bq[(idx / 16) * CS + 16 + idx % 16] = 0.f;
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
                mma16<CP, CS, 1, LS, 1>(q4, f.Bq + ti * 16 * CS, f.Wb + lj * 16, ti + 1, lane);
                mma16<CP, CS, 1, LS, 1>(m4, f.Tm + ti * 16 * CS, f.Wb + lj * 16, ti + 1, lane);
                mma16<CP, 1, CS, LS, 1>(w4, f.Bq + ti * 16 * CS + ti * 16, f.Qc + ti * 16 * LS + lj * 16, NT - ti, lane);
                mma16<CP, 1, CS, LS, 1>(w4, f.Tm + ti * 16 * CS + ti * 16, f.M + ti * 16 * LS + lj * 16, NT - ti, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + acc_row(lane, r), col = lj * 16 + acc_col(lane);
                    g.m.dQc[row * LP + col] = q4[r];
                    g.m.dM[row * LP + col] = m4[r];
                    g.m.dWb[row * LP + col] = w4[r];
                    g.m.P[row * LP + col] = accP[sl][r];
                }
            }
        }
        __syncthreads();
        // Per (step, latent row): this thread's rows rg*RPT + i of row l.
        {
            const int l = tid % LP, rg = tid / LP;
            float e[RPT], ie[RPT];
            row_scales(e, ie);
            // Branch-free stores (see OutRegion) of the chunk's real steps.
            const int rows = a.T - t0 < CP ? int(a.T - t0) : CP;
            const int64_t lbase = (head * a.T + t0) * a.L;
            const OutRegion dq_out(a.dq ? a.dq + lbase : nullptr, rows * a.L);
            const OutRegion db_out(a.db ? a.db + lbase : nullptr, rows * a.L);
            const OutRegion dk_out(a.dk ? a.dk + lbase : nullptr, rows * a.L);
            const OutRegion dg_out(a.dg ? a.dg + lbase : nullptr, rows * a.L);
            const int Lr = int(a.L);
            float dcc[RPT];
            float pp = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg * RPT + i;
                const float dQc = g.m.dQc[row * LP + l], dM = g.m.dM[row * LP + l], dWb = g.m.dWb[row * LP + l];
                const float Qc = f.Qc[row * LS + l], M = f.M[row * LS + l], Wb = f.Wb[row * LS + l];
                dcc[i] = dQc * Qc + dM * M - dWb * Wb;
                pp += Wb * g.m.P[row * LP + l];
                const bool real = row < rows && l < Lr;
                dq_out.store(dQc * e[i], real, row * Lr + l);
                db_out.store(dM * in.k[i] * e[i], real, row * Lr + l);
                dk_out.store(dM * in.b[i] * e[i] + dWb * ie[i], real, row * Lr + l);
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
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg * RPT + i;
                dg_out.store(suf[i] + later + xlt, row < rows && l < Lr, row * Lr + l);
            }
        }
    }
}

unsigned seq_blocks(const WyArgs& a) { return unsigned((a.BH + 7) / 8 * 8 * a.n_dt); }

template <int CP, int LP>
hipError_t launch_fwd_t(const WyArgs& a, hipStream_t st) {
    WyArgs args = a;
    void* params[] = {&args};
    if (a.rec == nullptr)
        return hipLaunchKernel(reinterpret_cast<const void*>(&wy_fwd_fused_kernel<CP, LP>), dim3(seq_blocks(a)),
                               dim3(kThreads), params, 0, st);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&wy_factor_kernel<CP, LP>),
                                   dim3(unsigned(a.BH * a.n_chunks)), dim3(kThreads), params, 0, st);
    if (e != hipSuccess) return e;
    const unsigned strips = unsigned((a.BH + 7) / 8 * 8 * ((a.D + kStripBlock - 1) / kStripBlock));
    const uintptr_t dense = reinterpret_cast<uintptr_t>(a.w) | reinterpret_cast<uintptr_t>(a.v) |
                            reinterpret_cast<uintptr_t>(a.ctx) | reinterpret_cast<uintptr_t>(a.state) |
                            reinterpret_cast<uintptr_t>(a.bnd) | reinterpret_cast<uintptr_t>(a.ubuf);
    const bool vec = a.D % 4 == 0 && (dense & 15) == 0;
    return hipLaunchKernel(vec ? reinterpret_cast<const void*>(&wy_fwd_strip_kernel<CP, LP, true>)
                               : reinterpret_cast<const void*>(&wy_fwd_strip_kernel<CP, LP, false>),
                           dim3(strips), dim3(kStripThreads), params, 0, st);
}

template <int CP, int LP>
hipError_t launch_bwd_t(const WyArgs& a, hipStream_t st) {
    WyArgs args = a;
    void* params[] = {&args};
    const unsigned strips = unsigned((a.BH + 7) / 8 * 8 * ((a.D + kStripBlock - 1) / kStripBlock));
    const uintptr_t dense = reinterpret_cast<uintptr_t>(a.dctx) | reinterpret_cast<uintptr_t>(a.w) |
                            reinterpret_cast<uintptr_t>(a.v) | reinterpret_cast<uintptr_t>(a.dw) |
                            reinterpret_cast<uintptr_t>(a.dv) | reinterpret_cast<uintptr_t>(a.drhs);
    const bool cvec = a.D % 4 == 0 && (dense & 15) == 0;
    hipError_t e = hipLaunchKernel(cvec ? reinterpret_cast<const void*>(&wy_bwd_carry_strip_kernel<CP, LP, true>)
                                        : reinterpret_cast<const void*>(&wy_bwd_carry_strip_kernel<CP, LP, false>),
                                   dim3(strips), dim3(kThreads), params, 0, st);
    if (e != hipSuccess) return e;
    if (!a.dq && !a.dk && !a.dv && !a.db && !a.dw && !a.dg) return hipSuccess;
    // 16-byte dense loads where every dense row and base allows them.
    const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = CP == 32 && LP >= 32 && a.D % 4 == 0 && al16(a.bnd_in) && al16(a.dbnd) && al16(a.ubuf) &&
                     al16(a.drhs) && al16(a.dctx);
    const void* grad = vec ? reinterpret_cast<const void*>(&wy_bwd_grad_kernel<CP, LP, (CP == 32 && LP >= 32)>)
                           : reinterpret_cast<const void*>(&wy_bwd_grad_kernel<CP, LP, false>);
    int dev = 0, cus = 0, per_cu = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, grad, kThreads, 0);
    if (e != hipSuccess) return e;
    // As many blocks as the device holds at once, each looping over items.
    const int64_t items = a.BH * a.n_chunks, resident = int64_t(cus) * (per_cu > 0 ? per_cu : 1);
    if (items > int64_t(UINT32_MAX)) return hipErrorInvalidValue;   // the kernel counts items in 32 bits
    return hipLaunchKernel(grad, dim3(unsigned(items < resident ? items : resident)), dim3(kThreads), params, 0, st);
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
