// gdn2.hip -- gfx950 kernels and C-ABI entry points of include/gdn2.h: the
// Gated DeltaNet-2 recurrence (the direct graph of the burn_gdn source page
// "src/chunk_wy/custom_backward.rs") and its VJP (the page's generic
// recompute backward: chunk boundary states, in-chunk recompute, per-step
// reverse sweep).
//
// Dense columns of a head's [L, D] state never interact in the forward (the
// read-out u[d] and the write S[:, d] += k u[d] touch column d only); the
// forward saves the state every `chunk` steps.
//
// Both kernels give each dense column Q lanes (8 when L rounds up to 32 or
// 64, else 4), lane j of the group holding rows j*R .. j*R+R-1 (R = LP/Q, LP
// = L rounded up to 16, 32 or 64) in registers; a wave holds 64/Q columns.
// Sums over a column's rows (the erased read-out, the context, d u) are a
// partial per lane plus a DPP butterfly.  The step's latent vectors are
// loaded ahead and staged in LDS, where every lane reads its own rows (the
// backward's full blocks stage a whole register chunk's rows at once).
//
// The backward runs blocks of 8 waves (two per SIMD) over 8 * 64/Q columns,
// ceil(D / (8 * 64/Q)) blocks per head.  Chunks are taken in reverse; each
// is recomputed from its saved boundary state, keeping the state before
// every step (in registers for chunks of 8 steps, else in a per-head scratch
// where each lane writes and reads back only its own rows), then reversed
// step by step.  The cotangents of value, write and the state are per
// column; those of query, key, erase and log_decay are sums over the dense
// axis: the lanes holding the same rows of the wave's columns reduce them by
// a transpose-reduce (gfx950 permlane swaps and DPP), the waves' sums meet in
// LDS, and with several blocks per head a small kernel adds the blocks'
// shares in block order.
#include "gdn2.h"
#include "gdn2_internal.hpp"
#include "qc_internal.hpp"
#include "quat_cumprod.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace qc {
namespace {

constexpr int kMaxLatent = 64;
constexpr int kMaxDense = 1024;
constexpr int kBlockWaves = 8;   // backward blocks: 8 waves, two per SIMD
constexpr int kRegChunk = 8;     // chunk size whose pre-step states the backward keeps in registers
constexpr int kFwdSets = 4;      // forward input sets in flight: loads run this many steps ahead

// Lanes per dense column: 8 when that still leaves each lane 4 or more of
// the LP padded rows (LP >= 32), else 4; each lane holds LP / Q contiguous rows.
constexpr int lanes_per_col(int lp) { return lp >= 32 ? 8 : 4; }
constexpr int cols_per_wave(int lp) { return 64 / lanes_per_col(lp); }
constexpr int cols_per_block(int lp) { return kBlockWaves * cols_per_wave(lp); }
constexpr int padded_rows(int64_t L) { return L <= 16 ? 16 : L <= 32 ? 32 : 64; }
constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
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
    int n_blk;      // backward blocks per head (ceil(D / columns per block))
    float* part;    // with n_blk > 1: per-block sums of the latent-vector cotangents, [BH, T, n_blk, 4, L]
};

// Lane exchanges inside a wave without the LDS crossbar (ds_bpermute costs an
// LDS round trip per call, on the critical path of every step).  dpp_xor<O>
// returns x from lane ^ O for O <= 8: quad permutations for 1 and 2; for 4 a
// mirror of each 8-lane half-row (lane ^ 7) composed with the quad reversal
// (lane ^ 3); for 8 a rotation of each 16-lane row by 8.  None of them reads
// outside its row, so every lane gets a defined value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor3 = 0x1B;     // quad_perm [3, 2, 1, 0]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane ^ 7 within 8
constexpr int kDppRowRor8 = 0x128;     // row_ror:8: lane ^ 8 within 16

template <int O>
__device__ __forceinline__ float dpp_xor(float x) {
    static_assert(O == 1 || O == 2 || O == 4 || O == 8, "DPP exchange offsets are 1, 2, 4 and 8");
    if constexpr (O == 1) return dpp_mov<kDppQuadXor1>(x);
    if constexpr (O == 2) return dpp_mov<kDppQuadXor2>(x);
    if constexpr (O == 4) return dpp_mov<kDppQuadXor3>(dpp_mov<kDppHalfMirror>(x));
    if constexpr (O == 8) return dpp_mov<kDppRowRor8>(x);
    return x;
}

// A product the compiler may not fuse into a later add or subtract: the
// update's write * value is rounded on its own, the same way in the forward
// and in the backward's recompute, wherever the compiler schedules it.
__device__ __forceinline__ float mul_unfused(float x, float y) {
#pragma clang fp contract(off)
    return x * y;
}

// Sum over the Q lanes of one column (its row blocks), by xor butterfly
// (offsets 1, 2, 4): every lane of the group gets the same bits (additions
// commute).  After the first two stages the four lanes of a quad agree, so
// the last stage may take the 8-lane mirror instead of lane ^ 4.
template <int Q>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(Q == 4 || Q == 8, "a column spans 4 or 8 lanes");
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    if constexpr (Q == 8) x += dpp_mov<kDppHalfMirror>(x);
    return x;
}

// Sum of x[0..N) over the lanes that hold the same rows of the wave's 64/Q
// columns (lane bits log2 Q .. 5), transposed: each stage (xor offset O = 32,
// 16, ...) keeps the half of the rows selected by lane bit O and adds the
// partner's copy of them; once one row is left, the remaining offsets down to
// Q add up the lanes holding the same row.  Lane l ends with row
// (l >> (6 - log2 N)) & (N - 1) of its position's block.
//
// For O = 32 and 16 one gfx950 permlane swap does a stage for a pair of rows:
// with A = x[i] and B = x[i + N/2], swapping A's upper half (odd 16-lane rows)
// with B's lower half (even rows) leaves A' + B' = A[l] + A[l ^ O] in the lower
// lanes and B[l ^ O] + B[l] in the upper ones, which is the stage's sum.
template <int N, int O, int Q>
__device__ __forceinline__ float cols_row_sum(const float (&x)[N], int lane) {
    if constexpr (N == 1) {
        float s = x[0];
        if constexpr (O >= Q) {
            s += dpp_xor<O>(s);
            return cols_row_sum<1, O / 2, Q>({s}, lane);
        }
        return s;
    } else {
        float y[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if constexpr (O == 32 || O == 16) {
                const auto p = O == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]),
                                                                         __float_as_uint(x[i + N / 2]), false, false)
                                       : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]),
                                                                         __float_as_uint(x[i + N / 2]), false, false);
                y[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
            } else {
                const bool up = (lane & O) != 0;
                const float keep = up ? x[i + N / 2] : x[i];
                const float send = up ? x[i] : x[i + N / 2];
                y[i] = keep + dpp_xor<O>(send);
            }
        }
        return cols_row_sum<N / 2, O / 2, Q>(y, lane);
    }
}

// The boundary states and the backward's scratch keep each dense column's LP
// rows contiguous ([.., d, LP]); a lane's R rows move as R/4 float4 from one
// per-lane address.
template <int R>
__device__ __forceinline__ void store_rows(float* p, const float (&x)[R]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int i = 0; i < R / 4; ++i) q[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}

template <int R>
__device__ __forceinline__ void load_rows_of(const float* p, float (&x)[R]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
        const float4 v = q[i];
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
    }
}

// ------------------------------------------------------------------ forward
//
// Same mapping as the backward (Q lanes per column, lane j of a column's group
// holding rows j*R ..), so the forward's sums are the backward recompute's
// arithmetic exactly and the recomputed states equal the saved ones bit for
// bit.  The step's latent vectors are staged in LDS (q, k, decay, erased key,
// and for the backward the raw erase), where every lane reads its own rows.
//
// Loads run ahead into register sets taken in turn by loops unrolled over the
// sets (four in the forward, two in the backward), so a load has whole steps
// to land before its value is used and is never copied while in flight.
// Every lane loads every step: rows past L read row L-1, columns past D read
// column D-1 and steps past the range repeat its last step (values that are
// then masked or unused), so the loads are unconditional and the compiler's
// wait counts stay exact.

enum { kVq = 0, kVk = 1, kVa = 2, kVe = 3, kVb = 4, kNVec = 4, kNRow = 5 };

// One latent row of a step: raw query, key, erase and log-decay.
struct Row {
    float q, k, b, g;
};

// kFull: D is a multiple of the columns per wave, so every lane has a column
// and the per-step context store is made by all lanes of the column (the same
// value to the same address): an unconditional store keeps the compiler's
// wait counts exact, where a conditional one makes the next step wait for a
// load issued during this one.
template <int LP, bool kFull>
__global__ void __launch_bounds__(64) gdn2_fwd_kernel(Gdn2Args a) {
    constexpr int Q = lanes_per_col(LP), R = LP / Q, CPW = cols_per_wave(LP);
    __shared__ float s_vec[2][kNVec][LP];
    const int lane = threadIdx.x, j = lane & (Q - 1);
    const int r0 = j * R;
    const int64_t n_cb = (a.D + CPW - 1) / CPW;
    const int64_t bh = blockIdx.x / n_cb;
    const int64_t d = (blockIdx.x % n_cb) * CPW + (lane >> ilog2(Q));
    const bool dok = kFull || d < a.D;
    const bool live = lane < a.L;                       // this lane's staged row is a real one
    const int64_t row0 = bh * a.T * a.L + (live ? lane : a.L - 1);
    const int64_t col0 = bh * a.T * a.D + (dok ? d : a.D - 1);

    float S[R];
#pragma unroll
    for (int i = 0; i < R; ++i) S[i] = (dok && r0 + i < a.L) ? a.s0[(bh * a.L + r0 + i) * a.D + d] : 0.0f;

    // A step's inputs as this lane loads them: its row and its column's value and write.
    struct In {
        Row r;
        float v, w;
    };
    auto load_in = [&](int64_t t, In& x) {
        const int64_t tl = t < a.T ? t : a.T - 1;
        const int64_t i = row0 + tl * a.L, e = col0 + tl * a.D;
        x.r.q = a.q[i];
        x.r.k = a.k[i];
        x.r.b = a.b[i];
        x.r.g = a.g[i];
        x.v = a.v[e];
        x.w = a.w[e];
    };
    auto put_row = [&](int buf, const Row& r) {
        if (lane < LP) {
            s_vec[buf][kVq][lane] = live ? r.q : 0.0f;
            s_vec[buf][kVk][lane] = live ? r.k : 0.0f;
            s_vec[buf][kVa][lane] = live ? __expf(r.g) : 1.0f;
            s_vec[buf][kVe][lane] = live ? r.b * r.k : 0.0f;
        }
    };

    int64_t until_bnd = 0, n_bnd = 0;   // steps to the next saved boundary, boundaries saved
    // Step t: `cur` holds its inputs (its row already staged), `nxt` those of t + 1.
    auto step = [&](int64_t t, In& cur, In& nxt) {
        const int buf = int(t & 1);
        // The update's product is formed before the set is reloaded, so no
        // old value outlives the load that replaces it (the compiler would
        // copy it, and wait for the load to do so).
        float wv = mul_unfused(cur.w, cur.v);
        asm volatile("" : "+v"(wv));          // the product is formed here (no instruction) ...
        __builtin_amdgcn_sched_barrier(0);    // ... and the reload is issued after it
        load_in(t + kFwdSets, cur);
        if (until_bnd == 0) {   // t is a multiple of the chunk
            if (a.bnd != nullptr && dok) store_rows<R>(a.bnd + ((bh * a.n_chunks + n_bnd) * a.D + d) * LP + r0, S);
            ++n_bnd;
            until_bnd = a.chunk;
        }
        --until_bnd;
        const float(*sv)[LP] = s_vec[buf];
        float read = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            S[i] *= sv[kVa][r0 + i];
            read = fmaf(sv[kVe][r0 + i], S[i], read);
        }
        const float u = wv - group_sum<Q>(read);
        float o = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            S[i] = fmaf(sv[kVk][r0 + i], u, S[i]);
            o = fmaf(sv[kVq][r0 + i], S[i], o);
        }
        o = group_sum<Q>(o);
        if constexpr (kFull)
            a.ctx[bh * a.T * a.D + d + t * a.D] = o * a.scale;
        else if (dok && j == 0)
            a.ctx[bh * a.T * a.D + d + t * a.D] = o * a.scale;
        put_row(buf ^ 1, nxt.r);   // past the last step: staged but never read
        __syncthreads();
    };
    // Four input sets in turn (set i holds the steps congruent to i mod 4):
    // step t stages the row of t + 1 from its set and reloads its own set with
    // step t + 4, so a load has three steps to land.  Whole groups of four run
    // in the loop and the last steps after it, so the sets come back to their
    // registers without copies; the first group runs before the loop, so the
    // loop is entered with the same loads and stores in flight as at its back
    // edge and its wait counts need not allow for the prologue.
    static_assert(kFwdSets == 4, "the step calls below name four sets");
    In x0, x1, x2, x3;
    load_in(0, x0);
    load_in(1, x1);
    load_in(2, x2);
    load_in(3, x3);
    put_row(0, x0.r);
    __syncthreads();
    auto group = [&](int64_t t) {
        step(t, x0, x1);
        step(t + 1, x1, x2);
        step(t + 2, x2, x3);
        step(t + 3, x3, x0);
    };
    int64_t t = 0;
    if (a.T >= 4) {
        group(0);
        t = 4;
    }
    for (; t + 4 <= a.T; t += 4) group(t);
    if (t < a.T) step(t, x0, x1);
    if (t + 1 < a.T) step(t + 1, x1, x2);
    if (t + 2 < a.T) step(t + 2, x2, x3);
    if (a.state != nullptr && dok) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (r0 + i < a.L) a.state[(bh * a.L + r0 + i) * a.D + d] = S[i];
    }
}

// ----------------------------------------------------------------- backward

// KC > 0: chunks of exactly KC steps keep their pre-step states in registers
// (the recompute stores nothing, the reverse loads nothing); a shorter last
// chunk, and every chunk when KC = 0, goes through the per-head scratch.
// kFull: D is a multiple of the block's columns, so every lane has a column.
template <int LP, int KC, bool kFull>
__global__ void __launch_bounds__(kBlockWaves * 64) gdn2_bwd_kernel(Gdn2Args a) {
    static_assert(KC == 0 || (KC >= 2 && KC % 2 == 0), "register chunks are whole step pairs");
    constexpr int Q = lanes_per_col(LP), R = LP / Q, CPW = cols_per_wave(LP), CPB = cols_per_block(LP);
    constexpr int kLogR = ilog2(R), kLogQ = ilog2(Q);
    // Per step slot and wave: the column sums of query, key (outer part),
    // erased key and decay.  Two slots used in turn, each summed over the
    // waves right after its step; with register chunks, one slot per step of
    // the chunk, summed at the chunk's end.
    __shared__ float s_red[KC > 0 ? KC : 2][kBlockWaves][4][LP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, j = lane & (Q - 1);
    const int n_waves = int(blockDim.x >> 6);
    const int r0 = j * R;
    const int64_t bh = blockIdx.x / a.n_blk;
    const int blk = int(blockIdx.x % a.n_blk);
    const int64_t d = int64_t(blk) * CPB + wave * CPW + (lane >> kLogQ);
    const bool dok = kFull || d < a.D;
    // After the column reduction this lane holds row r0 + idx; lanes that
    // differ only in the bits summed by the final butterfly hold copies.
    const int idx = (lane >> (6 - kLogR)) & (R - 1);
    const bool row_writer = ((lane >> kLogQ) & ((1 << (6 - kLogR - kLogQ)) - 1)) == 0;
    const bool out_lane = tid < a.L;

    float G[R];   // cotangent reaching the current state, this lane's rows of column d
#pragma unroll
    for (int i = 0; i < R; ++i)
        G[i] = (a.dstate != nullptr && dok && r0 + i < a.L) ? a.dstate[(bh * a.L + r0 + i) * a.D + d] : 0.0f;

    float* scr = a.scratch + (bh * a.scratch_steps * a.D + (dok ? d : 0)) * LP + r0;
    const int64_t scr_step = a.D * LP;
    const int64_t col0 = bh * a.T * a.D + d;               // element (t = 0, d) of the dense tensors
    const int64_t lcol0 = bh * a.T * a.D + (dok ? d : a.D - 1);   // the column this lane loads

    // Step vectors staged in LDS, two buffers used in turn; threads < LP stage
    // row tid, which threads < L read back raw (key, erase, decay) to finish
    // the latent-vector outputs.  Every thread loads a row (clamped as in the
    // forward) so that the loads stay unconditional.
    __shared__ float s_rows[2][kNRow][LP];
    const bool live = tid < a.L;
    const int64_t row0 = bh * a.T * a.L + ((tid & (LP - 1)) < a.L ? (tid & (LP - 1)) : a.L - 1);
    auto load_row = [&](int64_t t, Row& r) {
        const int64_t i = row0 + t * a.L;
        r.q = a.q[i];
        r.k = a.k[i];
        r.b = a.b[i];
        r.g = a.g[i];
    };
    auto put_row = [&](int buf, const Row& r) {
        if (tid < LP) {
            s_rows[buf][kVq][tid] = live ? r.q : 0.0f;
            s_rows[buf][kVk][tid] = live ? r.k : 0.0f;
            s_rows[buf][kVa][tid] = live ? __expf(r.g) : 1.0f;
            s_rows[buf][kVe][tid] = live ? r.b * r.k : 0.0f;
            s_rows[buf][kVb][tid] = live ? r.b : 0.0f;
        }
    };
    // A step's dense inputs in two register sets used in turn (the step loops
    // are unrolled by two so the roles swap without copies).  Columns past D
    // load column D - 1; their context cotangent is taken as zero.
    struct Dense {
        float v, w, dc;
    };
    Dense denA{0.0f, 0.0f, 0.0f}, denB{0.0f, 0.0f, 0.0f};
    Dense denC{0.0f, 0.0f, 0.0f}, denD{0.0f, 0.0f, 0.0f};   // register chunks: four sets
    float SpA[R], SpB[R];
    auto load_dense = [&](int64_t t, bool with_dc, Dense& dn) {
        dn.v = a.v[lcol0 + t * a.D];
        dn.w = a.w[lcol0 + t * a.D];
        if (with_dc) dn.dc = a.dctx[lcol0 + t * a.D];
    };
    // Rows load two steps ahead of their use, into two sets used in turn: the
    // step that stages row t' +- 1 at its end loads row t' +- 2 into the set
    // that held its own row.
    Row rX{0.0f, 0.0f, 0.0f, 0.0f}, rY{0.0f, 0.0f, 0.0f, 0.0f};

    // The latent-vector outputs of step t for row l from the block's sums
    // (key, erase and decay of that row given): final values with one block
    // per head, else this block's share, which gdn2_sum_kernel adds up.
    auto emit = [&](int64_t t, int l, float sq, float sk, float se, float sa, float kv, float bv, float av) {
        if (a.n_blk == 1) {
            const int64_t i = (bh * a.T + t) * a.L + l;
            if (a.dq != nullptr) a.dq[i] = sq;
            if (a.dk != nullptr) a.dk[i] = fmaf(se, bv, sk);
            if (a.db != nullptr) a.db[i] = se * kv;
            if (a.dg != nullptr) a.dg[i] = sa * av;
        } else if (a.part != nullptr) {
            float* p = a.part + (((bh * a.T + t) * a.n_blk + blk) * 4) * a.L + l;
            p[0] = sq;
            p[a.L] = sk;
            p[2 * a.L] = se;
            p[3 * a.L] = sa;
        }
    };
    // Sum of the waves' shares in slot `slot`, row l, in wave order.
    auto wave_sums = [&](int slot, int l, float& sq, float& sk, float& se, float& sa) {
        sq = sk = se = sa = 0.0f;
        for (int wv = 0; wv < n_waves; ++wv) {
            sq += s_red[slot][wv][0][l];
            sk += s_red[slot][wv][1][l];
            se += s_red[slot][wv][2][l];
            sa += s_red[slot][wv][3][l];
        }
    };

    int it = 0;   // steps so far (both sweeps): alternates the LDS buffers
    // The chunk's boundary state, and whether the previous (register) chunk
    // already loaded it with the chunk's first rows and dense inputs.
    float S[R];
    auto load_boundary = [&](int64_t c) {
        if (dok) {
            load_rows_of<R>(a.bnd_in + ((bh * a.n_chunks + c) * a.D + d) * LP + r0, S);
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) S[i] = 0.0f;
        }
    };
    bool primed = false;
    // Register chunks of full blocks: a whole chunk's staged rows, two buffers used in turn.
    __shared__ float s_chunk[KC > 0 && kFull ? 2 : 1][KC > 0 ? KC : 1][kNVec][LP];
    int cb = 0;
    for (int64_t c = a.n_chunks - 1; c >= 0; --c) {
        const int64_t t0 = c * a.chunk;
        const int64_t t1 = t0 + a.chunk < a.T ? t0 + a.chunk : a.T;

        // Recompute the chunk from its boundary; keep the state before each step.
        if (!primed) load_boundary(c);
        // Step t (upwards): rl is the set to load row row_t into (it held row
        // t; row_t is t + 2 inside the chunk), rs holds row t + 1, staged at
        // the end of the step; dnxt receives the dense inputs of dense_t.
        // The state before the step goes to the scratch (to_scratch) or to
        // the registers `keep`.
        // With svx set, the step's rows come from there (a chunk staged
        // whole) and the step neither loads nor stages rows nor waits at a
        // barrier.
        auto rec_step = [&](int64_t t, Dense& dcur, Dense& dnxt, Row& rl, const Row& rs, float (&keep)[R],
                            bool to_scratch, int64_t row_t, int64_t dense_t, bool dense_dc,
                            const float (*svx)[LP]) {
            const int buf = it & 1;
            if (svx == nullptr) {
                ++it;
                load_row(row_t, rl);
            }
            load_dense(dense_t, dense_dc, dnxt);
            if (to_scratch) {
                if (dok) store_rows<R>(scr + (t - t0) * scr_step, S);
            } else {
#pragma unroll
                for (int i = 0; i < R; ++i) keep[i] = S[i];
            }
            const float(*sv)[LP] = svx != nullptr ? svx : s_rows[buf];
            float read = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                S[i] *= sv[kVa][r0 + i];
                read = fmaf(sv[kVe][r0 + i], S[i], read);
            }
            const float u = mul_unfused(dcur.w, dcur.v) - group_sum<Q>(read);
#pragma unroll
            for (int i = 0; i < R; ++i) S[i] = fmaf(sv[kVk][r0 + i], u, S[i]);
            if (svx == nullptr) {
                put_row(buf ^ 1, rs);   // after the chunk's last step: staged but never read
                __syncthreads();
            }
        };
        // Reverse the chunk (downwards): the dense inputs and the state
        // before the step load one step ahead, rows two ahead as above (rl
        // takes row t - 2, rs holds row t - 1).  Lanes past D load from
        // column 0's scratch slot, which another block may not have written
        // yet: they zero what they loaded, and with a zero context cotangent
        // their state cotangent stays zero, so they add nothing to the sums.
        // Sp is the state before step t; with from_scratch, Sn receives the
        // one before step t - 1 from the scratch.
        // The step's column sums go to s_red slot `slot`; with sum_now the
        // block adds them up after the step's barrier.
        // row_t and dense_t (t - 2 and t - 1 inside the chunk) are the row
        // and dense inputs this step loads.
        auto rev_step = [&](int64_t t, Dense& dcur, float (&Sp)[R], Dense& dnxt, float (&Sn)[R], Row& rl,
                            const Row& rs, bool from_scratch, int slot, bool sum_now, int64_t row_t,
                            int64_t dense_t, const float (*svx)[LP]) {
            const int buf = it & 1;
            if (svx == nullptr) {
                ++it;
                load_row(row_t, rl);
            }
            const int64_t tp = t > t0 ? t - 1 : t0;
            const int64_t e = col0 + t * a.D;
            load_dense(dense_t, true, dnxt);
            if (from_scratch) load_rows_of<R>(scr + (tp - t0) * scr_step, Sn);
            const float(*sv)[LP] = svx != nullptr ? svx : s_rows[buf];
            const float dov = dok ? dcur.dc * a.scale : 0.0f;
            if (!dok) {
#pragma unroll
                for (int i = 0; i < R; ++i) Sp[i] = 0.0f;
            }
            float read = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) read = fmaf(sv[kVe][r0 + i], sv[kVa][r0 + i] * Sp[i], read);
            const float u = mul_unfused(dcur.w, dcur.v) - group_sum<Q>(read);

            // Read-out: the state after the step, and G += q do^T / sqrt(L);
            // then the rank-1 write: d u = G^T k and G u (the key's outer part).
            float x1[R], x2[R];
            float du = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                x1[i] = fmaf(sv[kVa][r0 + i], Sp[i], sv[kVk][r0 + i] * u) * dov;   // S_t * do / sqrt(L)
                G[i] = fmaf(sv[kVq][r0 + i], dov, G[i]);
                du = fmaf(G[i], sv[kVk][r0 + i], du);
                x2[i] = G[i] * u;
            }
            const float r_q = cols_row_sum<R, 32, Q>(x1, lane);
            const float r_k = cols_row_sum<R, 32, Q>(x2, lane);
            du = group_sum<Q>(du);
            if (dok && j == 0) {
                if (a.dw != nullptr) a.dw[e] = du * dcur.v;
                if (a.dv != nullptr) a.dv[e] = du * dcur.w;
            }
            // Erased read-out: its cotangent is -du; the erased key gets
            // (decayed state) (-du), the decayed state gets e (-du).
            const float dr = -du;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float av = sv[kVa][r0 + i];
                x1[i] = av * Sp[i] * dr;
                const float dD = fmaf(sv[kVe][r0 + i], dr, G[i]);   // cotangent of the decayed state
                x2[i] = dD * Sp[i];
                G[i] = av * dD;                                      // cotangent of the state before step t
            }
            const float r_e = cols_row_sum<R, 32, Q>(x1, lane);
            const float r_a = cols_row_sum<R, 32, Q>(x2, lane);
            if (row_writer) {
                s_red[slot][wave][0][r0 + idx] = r_q;
                s_red[slot][wave][1][r0 + idx] = r_k;
                s_red[slot][wave][2][r0 + idx] = r_e;
                s_red[slot][wave][3][r0 + idx] = r_a;
            }
            if (svx == nullptr) {
                put_row(buf ^ 1, rs);   // after the chunk's first step: staged but never read
                __syncthreads();
            }
            if (sum_now && out_lane) {
                float sq, sk, se, sa;
                wave_sums(slot, tid, sq, sk, se, sa);
                emit(t, tid, sq, sk, se, sa, s_rows[buf][kVk][tid], s_rows[buf][kVb][tid], s_rows[buf][kVa][tid]);
            }
        };
        // Each sweep starts with its first row staged and the next loading.
        auto start_sweep = [&](int64_t t_first, int64_t t_second, bool with_dc) {
            load_row(t_first, rX);
            put_row(it & 1, rX);
            load_row(t_second, rY);
            load_dense(t_first, with_dc, denA);
        };
        if constexpr (KC > 0 && kFull) {
            if (t1 - t0 == KC) {   // whole chunk, rows staged whole: no barrier inside the chunk
                // Every thread stages one (step, row) pair of a chunk: the
                // chunk's latent vectors go to LDS at once, loaded a whole
                // chunk ahead, so the steps neither load nor stage rows and
                // each wave runs the chunk's 16 steps without a barrier (its
                // column sums go to per-step slots, added at the chunk's end).
                // The dense inputs run two steps ahead through four sets as
                // below, and the reverse's last two steps load the next
                // chunk's first dense inputs.
                static_assert(KC == 8 && KC * 64 <= kBlockWaves * 64, "one (step, row) pair per thread");
                const int pk = tid / LP, pr = tid % LP;
                const bool pair = tid < KC * LP, plive = pr < a.L;
                const int64_t prow = bh * a.T * a.L + (plive ? pr : a.L - 1);
                auto load_chunk_row = [&](int64_t cc, Row& r) {
                    const int64_t i = prow + (cc * KC + (pair ? pk : 0)) * a.L;
                    r.q = a.q[i];
                    r.k = a.k[i];
                    r.b = a.b[i];
                    r.g = a.g[i];
                };
                auto stage_chunk_row = [&](int buf, const Row& r) {
                    if (pair) {
                        s_chunk[buf][pk][kVq][pr] = plive ? r.q : 0.0f;
                        s_chunk[buf][pk][kVk][pr] = plive ? r.k : 0.0f;
                        s_chunk[buf][pk][kVa][pr] = plive ? __expf(r.g) : 1.0f;
                        s_chunk[buf][pk][kVe][pr] = plive ? r.b * r.k : 0.0f;
                    }
                };
                if (!primed) {
                    Row first{0.0f, 0.0f, 0.0f, 0.0f};
                    load_chunk_row(c, first);
                    stage_chunk_row(cb, first);
                    load_dense(t0, false, denA);
                    load_dense(t0 + 1, false, denB);
                    __syncthreads();
                }
                Row nxt{0.0f, 0.0f, 0.0f, 0.0f};
                if (c > 0) load_chunk_row(c - 1, nxt);
                const float(*sc)[kNVec][LP] = s_chunk[cb];
                float Sst[KC][R];
                rec_step(t0, denA, denC, rX, rY, Sst[0], false, 0, t0 + 2, false, sc[0]);
                rec_step(t0 + 1, denB, denD, rY, rX, Sst[1], false, 0, t0 + 3, false, sc[1]);
                rec_step(t0 + 2, denC, denA, rX, rY, Sst[2], false, 0, t0 + 4, false, sc[2]);
                rec_step(t0 + 3, denD, denB, rY, rX, Sst[3], false, 0, t0 + 5, false, sc[3]);
                rec_step(t0 + 4, denA, denC, rX, rY, Sst[4], false, 0, t0 + 6, false, sc[4]);
                rec_step(t0 + 5, denB, denD, rY, rX, Sst[5], false, 0, t0 + 7, false, sc[5]);
                rec_step(t0 + 6, denC, denA, rX, rY, Sst[6], false, 0, t1 - 1, true, sc[6]);
                rec_step(t0 + 7, denD, denB, rY, rX, Sst[7], false, 0, t1 - 2, true, sc[7]);
                if (c > 0) load_boundary(c - 1);   // S is not read again in this chunk
                const int64_t n0 = c > 0 ? t0 - KC : t0;   // next chunk's first step (or a repeat)
                const int64_t n1 = c > 0 ? n0 + 1 : t0;
                rev_step(t0 + 7, denA, Sst[7], denC, SpB, rX, rY, false, 7, false, 0, t0 + 5, sc[7]);
                rev_step(t0 + 6, denB, Sst[6], denD, SpB, rY, rX, false, 6, false, 0, t0 + 4, sc[6]);
                rev_step(t0 + 5, denC, Sst[5], denA, SpB, rX, rY, false, 5, false, 0, t0 + 3, sc[5]);
                rev_step(t0 + 4, denD, Sst[4], denB, SpB, rY, rX, false, 4, false, 0, t0 + 2, sc[4]);
                rev_step(t0 + 3, denA, Sst[3], denC, SpB, rX, rY, false, 3, false, 0, t0 + 1, sc[3]);
                rev_step(t0 + 2, denB, Sst[2], denD, SpB, rY, rX, false, 2, false, 0, t0, sc[2]);
                rev_step(t0 + 1, denC, Sst[1], denA, SpB, rX, rY, false, 1, false, 0, n0, sc[1]);
                rev_step(t0, denD, Sst[0], denB, SpB, rY, rX, false, 0, false, 0, n1, sc[0]);
                __syncthreads();   // every slot written; this chunk's staged rows no longer read
                if (lane < a.L) {
                    for (int k = wave; k < KC; k += n_waves) {
                        const int64_t t = t0 + k;
                        const int64_t i = (bh * a.T + t) * a.L + lane;
                        float sq, sk, se, sa;
                        wave_sums(k, lane, sq, sk, se, sa);
                        if (a.n_blk == 1)
                            emit(t, lane, sq, sk, se, sa, a.k[i], a.b[i], __expf(a.g[i]));
                        else
                            emit(t, lane, sq, sk, se, sa, 0.0f, 0.0f, 0.0f);
                    }
                }
                if (c > 0) stage_chunk_row(cb ^ 1, nxt);
                __syncthreads();   // the sums read before any slot is written again; next rows staged
                cb ^= 1;
                primed = c > 0;
                continue;
            }
        }
        if constexpr (KC > 0) {
            if (t1 - t0 == KC) {   // whole chunk: states in registers
                // Loads run ahead across the sweeps: the recompute's last two
                // steps load what the reverse starts with (rows and dense
                // inputs, with the context cotangent, of t1 - 1 and t1 - 2), and
                // the reverse's last two load the next chunk's start (its
                // boundary state, rows and dense inputs), so no sweep starts
                // by waiting for memory.
                // Dense inputs run two steps ahead here, through four sets
                // (step k of the chunk reads set k mod 4 and loads step k + 2
                // into set k + 2 mod 4, downwards in the reverse).
                static_assert(KC == 8, "the step calls below spell out a chunk of 8");
                float Sst[KC][R];
                if (primed) {
                    put_row(it & 1, rX);
                } else {
                    start_sweep(t0, t0 + 1, false);
                    load_dense(t0 + 1, false, denB);
                }
                __syncthreads();
                rec_step(t0, denA, denC, rX, rY, Sst[0], false, t0 + 2, t0 + 2, false, nullptr);
                rec_step(t0 + 1, denB, denD, rY, rX, Sst[1], false, t0 + 3, t0 + 3, false, nullptr);
                rec_step(t0 + 2, denC, denA, rX, rY, Sst[2], false, t0 + 4, t0 + 4, false, nullptr);
                rec_step(t0 + 3, denD, denB, rY, rX, Sst[3], false, t0 + 5, t0 + 5, false, nullptr);
                rec_step(t0 + 4, denA, denC, rX, rY, Sst[4], false, t0 + 6, t0 + 6, false, nullptr);
                rec_step(t0 + 5, denB, denD, rY, rX, Sst[5], false, t0 + 7, t0 + 7, false, nullptr);
                rec_step(t0 + 6, denC, denA, rX, rY, Sst[6], false, t1 - 1, t1 - 1, true, nullptr);
                rec_step(t0 + 7, denD, denB, rY, rX, Sst[7], false, t1 - 2, t1 - 2, true, nullptr);
                if (c > 0) load_boundary(c - 1);   // S is not read again in this chunk
                put_row(it & 1, rX);
                __syncthreads();
                const int64_t n0 = c > 0 ? t0 - KC : t0;   // next chunk's first step (or a repeat)
                const int64_t n1 = c > 0 ? n0 + 1 : t0;
                rev_step(t0 + 7, denA, Sst[7], denC, SpB, rX, rY, false, 7, false, t0 + 5, t0 + 5, nullptr);
                rev_step(t0 + 6, denB, Sst[6], denD, SpB, rY, rX, false, 6, false, t0 + 4, t0 + 4, nullptr);
                rev_step(t0 + 5, denC, Sst[5], denA, SpB, rX, rY, false, 5, false, t0 + 3, t0 + 3, nullptr);
                rev_step(t0 + 4, denD, Sst[4], denB, SpB, rY, rX, false, 4, false, t0 + 2, t0 + 2, nullptr);
                rev_step(t0 + 3, denA, Sst[3], denC, SpB, rX, rY, false, 3, false, t0 + 1, t0 + 1, nullptr);
                rev_step(t0 + 2, denB, Sst[2], denD, SpB, rY, rX, false, 2, false, t0, t0, nullptr);
                rev_step(t0 + 1, denC, Sst[1], denA, SpB, rX, rY, false, 1, false, n0, n0, nullptr);
                rev_step(t0, denD, Sst[0], denB, SpB, rY, rX, false, 0, false, n1, n1, nullptr);
                // The chunk's sums, its steps dealt over the waves (the last
                // step's barrier published every slot; the next chunk's
                // recompute barriers come before any slot is written again).
                if (lane < a.L) {
                    for (int k = wave; k < KC; k += n_waves) {
                        const int64_t t = t0 + k;
                        const int64_t i = (bh * a.T + t) * a.L + lane;
                        float sq, sk, se, sa;
                        wave_sums(k, lane, sq, sk, se, sa);
                        if (a.n_blk == 1)
                            emit(t, lane, sq, sk, se, sa, a.k[i], a.b[i], __expf(a.g[i]));
                        else
                            emit(t, lane, sq, sk, se, sa, 0.0f, 0.0f, 0.0f);
                    }
                }
                primed = c > 0;
                continue;
            }
        }
        start_sweep(t0, t0 + 1 < t1 ? t0 + 1 : t1 - 1, false);
        __syncthreads();
        for (int64_t t = t0; t < t1; t += 2) {
            rec_step(t, denA, denB, rX, rY, SpA, true, t + 2 < t1 ? t + 2 : t1 - 1, t + 1 < t1 ? t + 1 : t1 - 1,
                     false, nullptr);
            if (t + 1 < t1)
                rec_step(t + 1, denB, denA, rY, rX, SpA, true, t + 3 < t1 ? t + 3 : t1 - 1,
                         t + 2 < t1 ? t + 2 : t1 - 1, false, nullptr);
        }
        start_sweep(t1 - 1, t1 - 2 >= t0 ? t1 - 2 : t0, true);
        load_rows_of<R>(scr + (t1 - 1 - t0) * scr_step, SpA);
        __syncthreads();
        for (int64_t t = t1 - 1; t >= t0; t -= 2) {
            rev_step(t, denA, SpA, denB, SpB, rX, rY, true, it & 1, true, t - 2 >= t0 ? t - 2 : t0,
                     t - 1 >= t0 ? t - 1 : t0, nullptr);
            if (t - 1 >= t0)
                rev_step(t - 1, denB, SpB, denA, SpA, rY, rX, true, it & 1, true, t - 3 >= t0 ? t - 3 : t0,
                         t - 2 >= t0 ? t - 2 : t0, nullptr);
        }
        primed = false;
    }
    if (a.ds0 != nullptr && dok) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (r0 + i < a.L) a.ds0[(bh * a.L + r0 + i) * a.D + d] = G[i];
    }
}

// With several blocks per head: the latent-vector cotangents are the sums of
// the blocks' shares, taken in block order (so the result is deterministic).
__global__ void __launch_bounds__(256) gdn2_sum_kernel(Gdn2Args a, int64_t n_rows) {
    const int64_t n = n_rows * a.L;   // n_rows = BH * T
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t row = i / a.L, l = i - row * a.L;
        const float* p = a.part + row * a.n_blk * 4 * a.L + l;
        float sq = 0.0f, sk = 0.0f, se = 0.0f, sa = 0.0f;
        for (int b = 0; b < a.n_blk; ++b, p += 4 * a.L) {
            sq += p[0];
            sk += p[a.L];
            se += p[2 * a.L];
            sa += p[3 * a.L];
        }
        if (a.dq != nullptr) a.dq[i] = sq;
        if (a.dk != nullptr) a.dk[i] = fmaf(se, a.b[i], sk);
        if (a.db != nullptr) a.db[i] = se * a.k[i];
        if (a.dg != nullptr) a.dg[i] = sa * __expf(a.g[i]);
    }
}

// ------------------------------------------------------------ host helpers

struct Sizes {
    int64_t BH, T, L, D, chunk, n_chunks, scratch_steps;
    int lm, cpw, n_blk;   // padded rows, columns per wave, backward blocks per head
    size_t state_scratch, part_bytes, scratch_bytes;   // the backward's scratch: states, then block shares
    size_t bnd_bytes;   // the forward's saved state: boundary states (and, chunk-WY, the factor records)
};

int check_sizes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk, Sizes* z) {
    if (B < 1 || H < 1 || T < 1 || L < 1 || D < 1 || chunk < 1) return QC_ERR_SHAPE;
    if (L > kMaxLatent || D > kMaxDense) return QC_ERR_SHAPE;
    if (B > kMaxElems / H) return QC_ERR_SHAPE;
    z->BH = B * H;
    z->lm = padded_rows(L);
    z->cpw = cols_per_wave(z->lm);
    if (z->BH > (int64_t(1) << 31) / ((D + z->cpw - 1) / z->cpw)) return QC_ERR_SHAPE;
    if (T > kMaxElems / z->BH || z->BH * T > kMaxElems / (L > D ? L : D)) return QC_ERR_SHAPE;
    z->T = T; z->L = L; z->D = D; z->chunk = chunk;
    z->n_chunks = (T + chunk - 1) / chunk;
    z->scratch_steps = chunk < T ? chunk : T;
    if (z->BH * z->n_chunks > kMaxElems / (L * D)) return QC_ERR_SHAPE;
    if (z->BH * (z->n_chunks > z->scratch_steps ? z->n_chunks : z->scratch_steps) > kMaxElems / (z->lm * D))
        return QC_ERR_SHAPE;
    z->n_blk = int((D + cols_per_block(z->lm) - 1) / cols_per_block(z->lm));
    if (z->BH > (int64_t(1) << 31) / z->n_blk) return QC_ERR_SHAPE;
    if (z->BH * T > kMaxElems / (4 * L * z->n_blk)) return QC_ERR_SHAPE;
    z->state_scratch = (size_t(z->BH * z->scratch_steps * D * z->lm) * sizeof(float) + 255) / 256 * 256;
    z->part_bytes = z->n_blk > 1 ? size_t(z->BH * T * z->n_blk * 4 * L) * sizeof(float) : 0;
    z->scratch_bytes = z->state_scratch + z->part_bytes;
    z->bnd_bytes = size_t(z->BH * z->n_chunks * D * z->lm) * sizeof(float);
    if (wy_chunk(chunk)) {
        // Chunk-WY path: grids of BH * n_chunks and BH * ceil(D / kWyDense)
        // blocks; the scratch holds the state cotangent entering each chunk.
        if (z->BH > (int64_t(1) << 31) / z->n_chunks) return QC_ERR_SHAPE;
        if (z->BH > (int64_t(1) << 31) / ((D + kWyDense - 1) / kWyDense)) return QC_ERR_SHAPE;
        // Scratch: the state cotangent entering each chunk, then drhs of every
        // padded step.  Saved state: boundary states, factor records, then U of
        // every padded step.
        const int64_t tp = z->n_chunks * chunk;
        if (z->BH * z->n_chunks > kMaxElems / wy_record_floats(chunk, z->lm)) return QC_ERR_SHAPE;
        if (z->BH * tp > kMaxElems / D) return QC_ERR_SHAPE;
        z->scratch_bytes = size_t(z->BH * z->n_chunks * z->lm * D + z->BH * tp * D) * sizeof(float);
        z->bnd_bytes += size_t(z->BH * z->n_chunks * wy_record_floats(chunk, z->lm) + z->BH * tp * D) * sizeof(float);
    }
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
    return z.bnd_bytes;
}

size_t gdn2_scratch_bytes(int64_t B, int64_t H, int64_t T, int64_t L, int64_t D, int64_t chunk) {
    qc::Sizes z;
    if (qc::check_sizes(B, H, T, L, D, chunk, &z) != QC_OK) return 0;
    return z.scratch_bytes;
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
    const size_t nb = z.bnd_bytes;
    if (boundary && (reinterpret_cast<uintptr_t>(boundary) & 15)) return QC_ERR_ALIGN;
    const qc::Span sp[] = {{context, nd}, {final_state, ns}, {boundary, nb},
                           {query, nl}, {key, nl}, {value, nd}, {erase, nl}, {write, nd}, {log_decay, nl},
                           {initial_state, ns}};
    if (qc::any_overlap(sp, 3, 10)) return QC_ERR_ALIAS;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (qc::wy_chunk(chunk)) {
        qc::WyArgs w{};
        w.q = query; w.k = key; w.v = value; w.b = erase; w.w = write; w.g = log_decay; w.s0 = initial_state;
        w.ctx = context; w.state = final_state; w.bnd = boundary;
        w.rec = boundary ? boundary + z.BH * z.n_chunks * z.lm * D : nullptr;
        w.ubuf = boundary ? w.rec + z.BH * z.n_chunks * qc::wy_record_floats(chunk, z.lm) : nullptr;
        w.BH = z.BH; w.T = T; w.L = L; w.D = D; w.n_chunks = z.n_chunks;
        w.n_dt = int((D + qc::kWyDense - 1) / qc::kWyDense);
        w.scale = 1.0f / sqrtf(float(L));
        const hipError_t e = qc::launch_wy_forward(int(chunk), z.lm, w, st);
        return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
    }
    qc::Gdn2Args a{};
    a.q = query; a.k = key; a.v = value; a.b = erase; a.w = write; a.g = log_decay; a.s0 = initial_state;
    a.ctx = context; a.state = final_state; a.bnd = boundary;
    a.T = T; a.L = L; a.D = D; a.chunk = chunk; a.n_chunks = z.n_chunks; a.scratch_steps = z.scratch_steps;
    a.scale = 1.0f / sqrtf(float(L));
    const unsigned blocks = unsigned(z.BH * ((D + z.cpw - 1) / z.cpw));
    const bool full = D % z.cpw == 0;
    const hipError_t e = qc::by_latent(z.lm, [&](auto lm) {
        constexpr int kLP = decltype(lm)::value;
        void* params[] = {&a};
        const void* kern = full ? reinterpret_cast<const void*>(&qc::gdn2_fwd_kernel<kLP, true>)
                                : reinterpret_cast<const void*>(&qc::gdn2_fwd_kernel<kLP, false>);
        return hipLaunchKernel(kern, dim3(blocks), dim3(64), params, 0, st);
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
    const size_t nb = z.bnd_bytes;
    const size_t nscr = z.scratch_bytes;
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
    if (qc::wy_chunk(chunk)) {
        qc::WyArgs w{};
        w.q = query; w.k = key; w.v = value; w.b = erase; w.w = write; w.g = log_decay;
        w.bnd_in = boundary; w.dctx = d_context; w.dstate = d_state;
        w.rec = const_cast<float*>(boundary) + z.BH * z.n_chunks * z.lm * D;
        w.ubuf = w.rec + z.BH * z.n_chunks * qc::wy_record_floats(chunk, z.lm);
        w.drhs = scratch + z.BH * z.n_chunks * z.lm * D;
        w.dq = d_query; w.dk = d_key; w.dv = d_value; w.db = d_erase; w.dw = d_write; w.dg = d_log_decay;
        w.ds0 = d_initial_state; w.dbnd = scratch;
        w.BH = z.BH; w.T = T; w.L = L; w.D = D; w.n_chunks = z.n_chunks;
        w.n_dt = int((D + qc::kWyDense - 1) / qc::kWyDense);
        w.scale = 1.0f / sqrtf(float(L));
        const hipError_t e = qc::launch_wy_backward(int(chunk), z.lm, w, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
    }
    qc::Gdn2Args a{};
    a.q = query; a.k = key; a.v = value; a.b = erase; a.w = write; a.g = log_decay; a.bnd_in = boundary;
    a.dctx = d_context; a.dstate = d_state;
    a.dq = d_query; a.dk = d_key; a.dv = d_value; a.db = d_erase; a.dw = d_write; a.dg = d_log_decay;
    a.ds0 = d_initial_state; a.scratch = scratch;
    a.T = T; a.L = L; a.D = D; a.chunk = chunk; a.n_chunks = z.n_chunks; a.scratch_steps = z.scratch_steps;
    a.scale = 1.0f / sqrtf(float(L));
    a.n_blk = z.n_blk;
    const bool want_latent = d_query || d_key || d_erase || d_log_decay;
    a.part = (z.n_blk > 1 && want_latent) ? reinterpret_cast<float*>(reinterpret_cast<char*>(scratch) + z.state_scratch)
                                          : nullptr;
    const unsigned threads = z.n_blk > 1 ? unsigned(qc::kBlockWaves * 64)
                                         : unsigned((D + z.cpw - 1) / z.cpw * 64);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = qc::by_latent(z.lm, [&](auto lm) {
        constexpr int kLP = decltype(lm)::value;
        void* params[] = {&a};
        const bool reg = chunk == qc::kRegChunk, full = D % qc::cols_per_block(kLP) == 0;
        const void* kern =
            reg ? (full ? reinterpret_cast<const void*>(&qc::gdn2_bwd_kernel<kLP, qc::kRegChunk, true>)
                        : reinterpret_cast<const void*>(&qc::gdn2_bwd_kernel<kLP, qc::kRegChunk, false>))
                : (full ? reinterpret_cast<const void*>(&qc::gdn2_bwd_kernel<kLP, 0, true>)
                        : reinterpret_cast<const void*>(&qc::gdn2_bwd_kernel<kLP, 0, false>));
        return hipLaunchKernel(kern, dim3(unsigned(z.BH * z.n_blk)), dim3(threads), params, 0, st);
    });
    if (e == hipSuccess && a.part != nullptr) {
        int64_t rows = z.BH * T;
        const int64_t want = (rows * L + 255) / 256;
        const unsigned blocks = unsigned(want < (int64_t(1) << 20) ? want : (int64_t(1) << 20));
        void* params[] = {&a, &rows};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&qc::gdn2_sum_kernel), dim3(blocks), dim3(256), params, 0,
                            st);
    }
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

}  // extern "C"
