// qc_kernels.hip -- gfx950 (CDNA4) kernels of the quaternion cumulative-product
// scan and its recompute-based VJP.
//
// Method (burn-mamba source page "burn_mamba/mamba3/quat_scan/backward.rs",
// module doc "Gradient math"):
//   forward   cum[t] = q_t (x) cum[t-1], cum[-1] = init; cum[t] = P_t (x) init
//   backward  S[t] = sum_{u>=t} conj(P_u) (x) d_cum[u]; G[t] = P_t (x) S[t] / |P_t|^2;
//             d_q[t] = G[t] (x) conj(cum[t-1]); d_init = S[0]
// (the division by |P_t|^2 is the exact form off the unit sphere; it is a
// no-op for exactly unit steps, which is where the page states the form).
//
// Two execution paths:
//   column   one lane walks one whole column (batch entry, h*j index) through
//            the sequence.  Forward: one read of q, one write of cum.  Backward:
//            one pass accumulates S[0], a second pass emits d_q.
//   chunked  sequence-parallel tiles.  A tile is WC adjacent columns x T steps;
//            each lane owns L consecutive steps of one column in registers.
//            The carry of the non-commutative product is combined in
//            left-multiply order (later factor on the left) across lanes
//            (ds_bpermute shuffles), across waves (LDS) and across blocks
//            (a Fenwick tree of per-tile carries in the workspace, see below).
//            The backward runs its tiles in reverse time order and carries the
//            plain (commutative) sum S in the same way.
//
// Cross-block carries.  Tiles of one column group form a chain; tile i
// (1-based, in chain order) publishes node i of a Fenwick tree: the combined
// carry of tiles (i - lowbit(i), i].  Node i only needs nodes i-1, i-2, ...,
// i-lowbit(i)/2 (ranges inside it), and the exclusive prefix of tile i is the
// ordered combination of the nodes on the Fenwick query path from i-1 down.
// Waits therefore form chains of depth log2(tiles), every tile reads and
// combines O(log tiles) values, and the association of every floating-point
// combine is fixed, so results are bitwise reproducible run to run.  Block
// ids come from an atomic ticket, so a block only waits on blocks that
// started before it; every wait is bounded (kSpinLimit) and raises a status
// word instead of hanging.  Before every scan kernel a small kernel clears
// the ticket and that launch's flags: the flag and carry areas of different
// problem shapes overlap in the workspace, so nothing is assumed about what
// earlier calls left there.
//
// Arithmetic: float64 for float32 storage, float32 for bfloat16 storage.
#include "qc_internal.hpp"

namespace qc {
namespace {

// --------------------------------------------------------------- quaternions

template <typename T>
struct alignas(16) Q4 {
    T w, x, y, z;
};

template <typename T>
__device__ __forceinline__ Q4<T> q_one() { return {T(1), T(0), T(0), T(0)}; }
template <typename T>
__device__ __forceinline__ Q4<T> q_zero() { return {T(0), T(0), T(0), T(0)}; }

// a (x) b, Hamilton product, scalar first.
template <typename T>
__device__ __forceinline__ Q4<T> qmul(const Q4<T>& a, const Q4<T>& b) {
    Q4<T> r;
    r.w = a.w * b.w - a.x * b.x - a.y * b.y - a.z * b.z;
    r.x = a.w * b.x + a.x * b.w + a.y * b.z - a.z * b.y;
    r.y = a.w * b.y - a.x * b.z + a.y * b.w + a.z * b.x;
    r.z = a.w * b.z + a.x * b.y - a.y * b.x + a.z * b.w;
    return r;
}

// conj(a) (x) b
template <typename T>
__device__ __forceinline__ Q4<T> qcmul(const Q4<T>& a, const Q4<T>& b) {
    Q4<T> r;
    r.w = a.w * b.w + a.x * b.x + a.y * b.y + a.z * b.z;
    r.x = a.w * b.x - a.x * b.w - a.y * b.z + a.z * b.y;
    r.y = a.w * b.y + a.x * b.z - a.y * b.w - a.z * b.x;
    r.z = a.w * b.z - a.x * b.y + a.y * b.x - a.z * b.w;
    return r;
}

// a (x) conj(b)
template <typename T>
__device__ __forceinline__ Q4<T> qmulc(const Q4<T>& a, const Q4<T>& b) {
    Q4<T> r;
    r.w = a.w * b.w + a.x * b.x + a.y * b.y + a.z * b.z;
    r.x = a.x * b.w - a.w * b.x - a.y * b.z + a.z * b.y;
    r.y = a.y * b.w - a.w * b.y + a.x * b.z - a.z * b.x;
    r.z = a.z * b.w - a.w * b.z - a.x * b.y + a.y * b.x;
    return r;
}

template <typename T>
__device__ __forceinline__ Q4<T> qadd(const Q4<T>& a, const Q4<T>& b) {
    return {a.w + b.w, a.x + b.x, a.y + b.y, a.z + b.z};
}
template <typename T>
__device__ __forceinline__ Q4<T> qsub(const Q4<T>& a, const Q4<T>& b) {
    return {a.w - b.w, a.x - b.x, a.y - b.y, a.z - b.z};
}
template <typename T>
__device__ __forceinline__ Q4<T> qscale(const Q4<T>& a, T s) {
    return {a.w * s, a.x * s, a.y * s, a.z * s};
}
template <typename T>
__device__ __forceinline__ T qnorm2(const Q4<T>& a) {
    return a.w * a.w + a.x * a.x + a.y * a.y + a.z * a.z;
}

template <typename T>
__device__ __forceinline__ Q4<T> shfl_up_q(const Q4<T>& v, int delta) {
    return {__shfl_up(v.w, delta), __shfl_up(v.x, delta), __shfl_up(v.y, delta), __shfl_up(v.z, delta)};
}
template <typename T>
__device__ __forceinline__ Q4<T> shfl_down_q(const Q4<T>& v, int delta) {
    return {__shfl_down(v.w, delta), __shfl_down(v.x, delta), __shfl_down(v.y, delta), __shfl_down(v.z, delta)};
}
template <typename T>
__device__ __forceinline__ Q4<T> shfl_q(const Q4<T>& v, int src) {
    return {__shfl(v.w, src), __shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src)};
}

// ------------------------------------------------------------ storage dtypes

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;  // NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                              // nearest, ties even
    return u >> 16;
}

// float32 storage: one float4 (16 B) per quaternion; float64 arithmetic.
struct IoF32 {
    using CT = double;
    using Raw = float4;
    static __device__ __forceinline__ Raw load(const void* base, int64_t idx) {
        return reinterpret_cast<const float4*>(base)[idx];
    }
    static __device__ __forceinline__ Raw one_raw() { return make_float4(1.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ Raw zero_raw() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ Q4<CT> ct(const Raw& v) {
        return {double(v.x), double(v.y), double(v.z), double(v.w)};
    }
    // Same as ct(), but hides the register's provenance so the compiler
    // re-converts here instead of keeping float64 copies of every step alive
    // between the two sweeps (twice the registers).
    static __device__ __forceinline__ Q4<CT> ct_fresh(Raw v) {
        asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
        return ct(v);
    }
    static __device__ __forceinline__ void store(void* base, int64_t idx, const Q4<CT>& v) {
        reinterpret_cast<float4*>(base)[idx] = make_float4(float(v.w), float(v.x), float(v.y), float(v.z));
    }
};

// bfloat16 storage: 4 x 16-bit patterns (8 B) per quaternion; float32 arithmetic.
struct IoBF16 {
    using CT = float;
    using Raw = uint2;
    static __device__ __forceinline__ Raw load(const void* base, int64_t idx) {
        return reinterpret_cast<const uint2*>(base)[idx];
    }
    static __device__ __forceinline__ Raw one_raw() { return make_uint2(0x3f80u, 0u); }
    static __device__ __forceinline__ Raw zero_raw() { return make_uint2(0u, 0u); }
    static __device__ __forceinline__ Q4<CT> ct(const Raw& v) {
        return {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ Q4<CT> ct_fresh(Raw v) {
        asm volatile("" : "+v"(v.x), "+v"(v.y));
        return ct(v);
    }
    static __device__ __forceinline__ void store(void* base, int64_t idx, const Q4<CT>& v) {
        const uint32_t lo = f32_to_bf16_bits(v.w) | (f32_to_bf16_bits(v.x) << 16);
        const uint32_t hi = f32_to_bf16_bits(v.y) | (f32_to_bf16_bits(v.z) << 16);
        reinterpret_cast<uint2*>(base)[idx] = make_uint2(lo, hi);
    }
};

// ------------------------------------------------- cross-block carry helpers

// Wait until a tile's ready flag is set, then make its carry values visible.
// The wave polls one address uniformly; the wait is bounded.
__device__ __forceinline__ void wait_ready(const KernelArgs& a, const uint32_t* flag) {
    uint32_t polls = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls > a.spin_limit) {
            __hip_atomic_store(&a.hdr[kHdrStatus], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Store a tile's carry values (lanes with `writer`), then release the flag.
// Called by the whole wave: the fence covers every lane's stores.
template <typename T>
__device__ __forceinline__ void publish(const KernelArgs& a, Q4<T>* slot, uint32_t* flag,
                                        const Q4<T>& v, bool writer, bool flag_writer) {
    if (writer) *slot = v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (flag_writer) __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fenwick look-back for tile `pos` (0-based) of `chain`, run by one wave.
// `own` is this tile's aggregate.  Combine(later, earlier) is
//   product:  later (x) earlier           (forward carry P)
//   sum:      later + earlier             (backward carry S, "later" = earlier in time)
// Returns the exclusive prefix (identity / zero for the first tile).
template <typename T, int WC, bool kProduct>
__device__ Q4<T> fenwick_exclusive(const KernelArgs& a, int64_t chain, int64_t pos,
                                   const Q4<T>& own, int c, bool writer, bool flag_writer) {
    const int64_t i = pos + 1;
    const int64_t low = i & (-i);
    const int64_t node0 = chain * a.n_tiles;   // node n lives at node0 + n - 1
    Q4<T>* desc = reinterpret_cast<Q4<T>*>(a.desc);
    Q4<T> acc = kProduct ? q_one<T>() : q_zero<T>();
    bool published = (i == a.n_tiles);        // nothing reads the last node
    int64_t jn = i - 1;
    for (;;) {
        if (!published && jn <= i - low) {
            const Q4<T> node = kProduct ? qmul(own, acc) : qadd(own, acc);
            publish(a, desc + (node0 + i - 1) * WC + c, a.flags + node0 + i - 1, node, writer, flag_writer);
            published = true;
        }
        if (jn == 0) break;
        wait_ready(a, a.flags + node0 + jn - 1);
        const Q4<T> v = desc[(node0 + jn - 1) * WC + c];
        acc = kProduct ? qmul(acc, v) : qadd(acc, v);
        jn -= jn & (-jn);
    }
    return acc;
}

// Tile coordinates shared by the chunked kernels.
struct TileCoord {
    int64_t chain, pos, bi, m, t0, base;
    bool col_ok, full;
};

template <int WC, int L, int NW>
__device__ __forceinline__ TileCoord tile_coord(const KernelArgs& a, uint32_t id, bool reverse, int k, int c) {
    constexpr int T = (64 / WC) * NW * L;
    TileCoord tc;
    tc.chain = id % a.n_chains;
    tc.pos = id / a.n_chains;
    const int64_t tile = reverse ? a.n_tiles - 1 - tc.pos : tc.pos;
    tc.bi = tc.chain / a.n_cg;
    const int64_t cg = tc.chain % a.n_cg;
    tc.m = cg * WC + c;
    tc.col_ok = tc.m < a.M;
    tc.t0 = tile * T + int64_t(k) * L;
    tc.base = (tc.bi * a.s + tc.t0) * a.M + tc.m;
    tc.full = (tile + 1) * T <= a.s && (cg + 1) * WC <= a.M;   // block-uniform
    return tc;
}

// In-tile exclusive prefix product of slice aggregates (left-multiply order).
// Slice k = wave*R + r.  Returns F = product of slices before k in this tile;
// `tile_agg` receives the tile's full product (valid in the last wave).
template <typename T, int WC, int NW>
__device__ __forceinline__ Q4<T> tile_scan_product(const Q4<T>& A, Q4<T> (*s_wagg)[WC], int wave, int r, int c,
                                                   Q4<T>* tile_agg) {
    constexpr int R = 64 / WC;
    Q4<T> inc = A;
#pragma unroll
    for (int d = 1; d < R; d <<= 1) {
        const Q4<T> o = shfl_up_q(inc, d * WC);
        if (r >= d) inc = qmul(inc, o);
    }
    Q4<T> exw = shfl_up_q(inc, WC);
    if (r == 0) exw = q_one<T>();
    if (r == R - 1) s_wagg[wave][c] = inc;
    __syncthreads();
    Q4<T> wex = q_one<T>();
    for (int w2 = wave - 1; w2 >= 0; --w2) wex = qmul(wex, s_wagg[w2][c]);
    const Q4<T> last = shfl_q(inc, (R - 1) * WC + c);
    *tile_agg = qmul(last, wex);
    return qmul(exw, wex);
}

// ------------------------------------------------------------ forward, chunked

template <class IO, int WC, int L, int NW>
__global__ void __launch_bounds__(NW * 64) fwd_chunked_kernel(KernelArgs a) {
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    constexpr int R = 64 / WC;
    __shared__ Q4<CT> s_wagg[NW][WC];
    __shared__ Q4<CT> s_carry[WC];
    __shared__ uint32_t s_id;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / WC, c = lane % WC;
    if (tid == 0) s_id = __hip_atomic_fetch_add(&a.hdr[kHdrTicket], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_id >= a.n_blocks) {   // ticket not cleared: refuse to index with it
        if (tid == 0) __hip_atomic_store(&a.hdr[kHdrStatus], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const TileCoord tc = tile_coord<WC, L, NW>(a, s_id, false, wave * R + r, c);

    Raw qv[L];
    if (tc.full) {
#pragma unroll
        for (int i = 0; i < L; ++i) qv[i] = IO::load(a.q, tc.base + int64_t(i) * a.M);
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i)
            qv[i] = (tc.col_ok && tc.t0 + i < a.s) ? IO::load(a.q, tc.base + int64_t(i) * a.M) : IO::one_raw();
    }
    Raw init_raw = IO::one_raw();
    if (a.out != nullptr && tc.col_ok) init_raw = IO::load(a.init, tc.bi * a.M + tc.m);

    // Slice product: A = q_{t0+L-1} (x) ... (x) q_{t0}.
    Q4<CT> A = IO::ct(qv[0]);
#pragma unroll
    for (int i = 1; i < L; ++i) A = qmul(IO::ct(qv[i]), A);

    Q4<CT> tile_agg;
    const Q4<CT> F = tile_scan_product<CT, WC, NW>(A, s_wagg, wave, r, c, &tile_agg);
    if (wave == NW - 1) {
        const Q4<CT> E = fenwick_exclusive<CT, WC, true>(a, tc.chain, tc.pos, tile_agg, c, r == 0, lane == 0);
        if (r == 0) s_carry[c] = E;
    }
    __syncthreads();
    const Q4<CT> Ps = qmul(F, s_carry[c]);   // P_{t0-1}: prefix product before this slice

    if (a.ckpt != nullptr && tc.col_ok && tc.t0 < a.s && (tc.t0 % kCkptStride) == 0)
        reinterpret_cast<Q4<CT>*>(a.ckpt)[(tc.bi * a.n_ck + tc.t0 / kCkptStride) * a.M + tc.m] = Ps;

    if (a.out != nullptr) {
        Q4<CT> cm = qmul(Ps, IO::ct(init_raw));   // cum[t0-1]
        if (tc.full) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                cm = qmul(IO::ct_fresh(qv[i]), cm);
                IO::store(a.out, tc.base + int64_t(i) * a.M, cm);
            }
        } else if (tc.col_ok) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if (tc.t0 + i < a.s) {
                    cm = qmul(IO::ct_fresh(qv[i]), cm);
                    IO::store(a.out, tc.base + int64_t(i) * a.M, cm);
                }
            }
        }
    }
}

// ----------------------------------------------------------- backward, chunked
//
// Per slice (L steps from t0, E = P_{t0-1} from the saved boundary state and
// the in-tile scan), with local products Lc_t = q_t (x) ... (x) q_{t0}:
//   P_t = Lc_t (x) E,   conj(P_t) (x) d_t = conj(E) (x) [conj(Lc_t) (x) d_t]
//   Yh  = sum_{t in slice} conj(Lc_t) (x) d_t            (local frame)
//   S[t] = conj(E) (x) Sh_t + S_after,   Sh_t = sum_{u>=t in slice} conj(Lc_u) (x) d_u
//   G[t] = P_t (x) S[t] / |P_t|^2 = Lc_t (x) (Sh_t + Z) / |Lc_t|^2,  Z = E (x) S_after / |E|^2
//   cum[t-1] = Lc_{t-1} (x) (E (x) init)
// so the long-range quantities enter once per slice and the per-step
// arithmetic stays in the well-conditioned local frame.

template <class IO, int WC, int L, int NW>
__global__ void __launch_bounds__(NW * 64) bwd_chunked_kernel(KernelArgs a) {
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    constexpr int R = 64 / WC;
    __shared__ Q4<CT> s_wagg[NW][WC];
    __shared__ Q4<CT> s_wsum[NW][WC];
    __shared__ Q4<CT> s_after[WC];
    __shared__ uint32_t s_id;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / WC, c = lane % WC;
    if (tid == 0) s_id = __hip_atomic_fetch_add(&a.hdr[kHdrTicket], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_id >= a.n_blocks) {   // ticket not cleared: refuse to index with it
        if (tid == 0) __hip_atomic_store(&a.hdr[kHdrStatus], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const TileCoord tc = tile_coord<WC, L, NW>(a, s_id, true, wave * R + r, c);

    Raw qv[L], dv[L];
    if (tc.full) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            qv[i] = IO::load(a.q, tc.base + int64_t(i) * a.M);
            dv[i] = IO::load(a.d_cum, tc.base + int64_t(i) * a.M);
        }
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const bool ok = tc.col_ok && tc.t0 + i < a.s;
            qv[i] = ok ? IO::load(a.q, tc.base + int64_t(i) * a.M) : IO::one_raw();
            dv[i] = ok ? IO::load(a.d_cum, tc.base + int64_t(i) * a.M) : IO::zero_raw();
        }
    }
    // Boundary prefix product at the tile start and the initial carry.
    const int64_t tile_t0 = tc.t0 - int64_t(wave * R + r) * L;
    Q4<CT> Et = q_one<CT>();
    Raw init_raw = IO::one_raw();
    if (tc.col_ok) {
        Et = reinterpret_cast<const Q4<CT>*>(a.ckpt)[(tc.bi * a.n_ck + tile_t0 / kCkptStride) * a.M + tc.m];
        init_raw = IO::load(a.init, tc.bi * a.M + tc.m);
    }

    // Sweep 1 (local frame): slice product and Yh = sum conj(Lc_t) (x) d_t.
    Q4<CT> Lc = q_one<CT>();
    Q4<CT> Yh = q_zero<CT>();
#pragma unroll
    for (int i = 0; i < L; ++i) {
        Lc = qmul(IO::ct(qv[i]), Lc);
        Yh = qadd(Yh, qcmul(Lc, IO::ct(dv[i])));
    }

    // Forward prefix inside the tile -> E = P_{t0-1} of this slice.
    Q4<CT> tile_prod;
    const Q4<CT> F = tile_scan_product<CT, WC, NW>(Lc, s_wagg, wave, r, c, &tile_prod);
    const Q4<CT> E = qmul(F, Et);
    const Q4<CT> Y = qcmul(E, Yh);   // this slice's share of S, global frame

    // Reverse (suffix) sums of Y over the slices of the tile.
    Q4<CT> sinc = Y;   // sum over slices r' >= r of this wave
#pragma unroll
    for (int d = 1; d < R; d <<= 1) {
        const Q4<CT> o = shfl_down_q(sinc, d * WC);
        if (r + d < R) sinc = qadd(sinc, o);
    }
    Q4<CT> later_in_wave = shfl_down_q(sinc, WC);
    if (r == R - 1) later_in_wave = q_zero<CT>();
    if (r == 0) s_wsum[wave][c] = sinc;
    __syncthreads();
    Q4<CT> later_waves = q_zero<CT>();
    for (int w2 = wave + 1; w2 < NW; ++w2) later_waves = qadd(later_waves, s_wsum[w2][c]);
    if (wave == 0) {
        const Q4<CT> tile_sum = qadd(shfl_q(sinc, c), later_waves);
        const Q4<CT> Sa = fenwick_exclusive<CT, WC, false>(a, tc.chain, tc.pos, tile_sum, c, r == 0, lane == 0);
        if (r == 0) s_after[c] = Sa;
    }
    __syncthreads();
    const Q4<CT> S_after = qadd(qadd(later_in_wave, later_waves), s_after[c]);   // S at t0 + L

    if (a.d_init != nullptr && tc.t0 == 0 && tc.col_ok)
        IO::store(a.d_init, tc.bi * a.M + tc.m, qadd(Y, S_after));   // S[0]

    if (a.out != nullptr && tc.col_ok) {
        const Q4<CT> Z = qscale(qmul(E, S_after), CT(1) / qnorm2(E));
        const Q4<CT> C = qmul(E, IO::ct(init_raw));   // cum[t0-1]
        Q4<CT> Lp = q_one<CT>();
        Q4<CT> run = q_zero<CT>();
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if (!tc.full && tc.t0 + i >= a.s) break;
            const Q4<CT> Lt = qmul(IO::ct_fresh(qv[i]), Lp);
            const Q4<CT> X = qcmul(Lt, IO::ct_fresh(dv[i]));
            const Q4<CT> Sh = qsub(Yh, run);
            run = qadd(run, X);
            const Q4<CT> G = qscale(qmul(Lt, qadd(Sh, Z)), CT(1) / qnorm2(Lt));
            const Q4<CT> cprev = qmul(Lp, C);
            IO::store(a.out, tc.base + int64_t(i) * a.M, qmulc(G, cprev));
            Lp = Lt;
        }
    }
}

// ------------------------------------------------------------- column path

template <class IO, int U>
__global__ void __launch_bounds__(kColumnBlock) fwd_column_kernel(KernelArgs a) {
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    const int64_t col = int64_t(blockIdx.x) * kColumnBlock + threadIdx.x;
    if (col >= a.b * a.M) return;
    const int64_t bi = col / a.M, m = col % a.M;
    Q4<CT> cm = IO::ct(IO::load(a.init, bi * a.M + m));
    Q4<CT> P = q_one<CT>();
    const bool want_ckpt = a.ckpt != nullptr;
    Q4<CT>* ck = reinterpret_cast<Q4<CT>*>(a.ckpt);
    const int64_t base = bi * a.s * a.M + m;
    for (int64_t t0 = 0; t0 < a.s; t0 += U) {
        Raw qv[U];
#pragma unroll
        for (int i = 0; i < U; ++i)
            qv[i] = (t0 + i < a.s) ? IO::load(a.q, base + (t0 + i) * a.M) : IO::one_raw();
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t t = t0 + i;
            if (t >= a.s) break;
            const Q4<CT> qq = IO::ct(qv[i]);
            if (want_ckpt) {
                if (t % kCkptStride == 0) ck[(bi * a.n_ck + t / kCkptStride) * a.M + m] = P;
                P = qmul(qq, P);
            }
            cm = qmul(qq, cm);
            if (a.out != nullptr) IO::store(a.out, base + t * a.M, cm);
        }
    }
}

template <class IO, int U>
__global__ void __launch_bounds__(kColumnBlock) bwd_column_kernel(KernelArgs a) {
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    const int64_t col = int64_t(blockIdx.x) * kColumnBlock + threadIdx.x;
    if (col >= a.b * a.M) return;
    const int64_t bi = col / a.M, m = col % a.M;
    const int64_t base = bi * a.s * a.M + m;
    // Pass 1: S[0] = sum_t conj(P_t) (x) d_t.
    Q4<CT> P = q_one<CT>();
    Q4<CT> S0 = q_zero<CT>();
    for (int64_t t0 = 0; t0 < a.s; t0 += U) {
        Raw qv[U], dv[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool ok = t0 + i < a.s;
            qv[i] = ok ? IO::load(a.q, base + (t0 + i) * a.M) : IO::one_raw();
            dv[i] = ok ? IO::load(a.d_cum, base + (t0 + i) * a.M) : IO::zero_raw();
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            P = qmul(IO::ct(qv[i]), P);
            S0 = qadd(S0, qcmul(P, IO::ct(dv[i])));
        }
    }
    if (a.d_init != nullptr) IO::store(a.d_init, bi * a.M + m, S0);
    if (a.out == nullptr) return;
    // Pass 2: S[t] = S[0] - sum_{u<t} conj(P_u) (x) d_u, then G and d_q.
    const Q4<CT> ini = IO::ct(IO::load(a.init, bi * a.M + m));
    Q4<CT> Pp = q_one<CT>();
    Q4<CT> run = q_zero<CT>();
    for (int64_t t0 = 0; t0 < a.s; t0 += U) {
        Raw qv[U], dv[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool ok = t0 + i < a.s;
            qv[i] = ok ? IO::load(a.q, base + (t0 + i) * a.M) : IO::one_raw();
            dv[i] = ok ? IO::load(a.d_cum, base + (t0 + i) * a.M) : IO::zero_raw();
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t t = t0 + i;
            if (t >= a.s) break;
            const Q4<CT> Pt = qmul(IO::ct(qv[i]), Pp);
            const Q4<CT> X = qcmul(Pt, IO::ct(dv[i]));
            const Q4<CT> S = qsub(S0, run);
            run = qadd(run, X);
            const Q4<CT> G = qscale(qmul(Pt, S), CT(1) / qnorm2(Pt));
            IO::store(a.out, base + t * a.M, qmulc(G, qmul(Pp, ini)));
            Pp = Pt;
        }
    }
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// Runs before each scan kernel: ticket := 0 and flags[0, n) := 0; the first
// kernel of an API call also clears the status word.
__global__ void clear_launch_state_kernel(uint32_t* hdr, uint32_t* flags, size_t n, uint32_t clear_status) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[kHdrTicket] = 0u;
        if (clear_status) hdr[kHdrStatus] = 0u;
    }
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
        flags[i] = 0u;
}

// ------------------------------------------------------------------ launchers

template <class IO, int WC>
hipError_t launch_fwd_wc(const KernelArgs& a, hipStream_t st) {
    constexpr Geometry g = geometry_for(WC);
    KernelArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_chunked_kernel<IO, WC, g.fwd_l, g.fwd_nw>),
                           dim3(a.n_blocks), dim3(g.fwd_nw * 64), params, 0, st);
}

template <class IO, int WC>
hipError_t launch_bwd_wc(const KernelArgs& a, hipStream_t st) {
    constexpr Geometry g = geometry_for(WC);
    KernelArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_chunked_kernel<IO, WC, g.bwd_l, g.bwd_nw>),
                           dim3(a.n_blocks), dim3(g.bwd_nw * 64), params, 0, st);
}

template <class IO>
hipError_t launch_fwd_io(int wc, const KernelArgs& a, hipStream_t st) {
    switch (wc) {
        case 64: return launch_fwd_wc<IO, 64>(a, st);
        case 32: return launch_fwd_wc<IO, 32>(a, st);
        case 16: return launch_fwd_wc<IO, 16>(a, st);
        case 8: return launch_fwd_wc<IO, 8>(a, st);
        case 4: return launch_fwd_wc<IO, 4>(a, st);
        case 2: return launch_fwd_wc<IO, 2>(a, st);
        case 1: return launch_fwd_wc<IO, 1>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <class IO>
hipError_t launch_bwd_io(int wc, const KernelArgs& a, hipStream_t st) {
    switch (wc) {
        case 64: return launch_bwd_wc<IO, 64>(a, st);
        case 32: return launch_bwd_wc<IO, 32>(a, st);
        case 16: return launch_bwd_wc<IO, 16>(a, st);
        case 8: return launch_bwd_wc<IO, 8>(a, st);
        case 4: return launch_bwd_wc<IO, 4>(a, st);
        case 2: return launch_bwd_wc<IO, 2>(a, st);
        case 1: return launch_bwd_wc<IO, 1>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_chunked(int dtype, int wc, const KernelArgs& a, hipStream_t st) {
    return dtype == 0 ? launch_fwd_io<IoF32>(wc, a, st) : launch_fwd_io<IoBF16>(wc, a, st);
}

hipError_t launch_bwd_chunked(int dtype, int wc, const KernelArgs& a, hipStream_t st) {
    return dtype == 0 ? launch_bwd_io<IoF32>(wc, a, st) : launch_bwd_io<IoBF16>(wc, a, st);
}

hipError_t launch_fwd_column(int dtype, const KernelArgs& a, hipStream_t st) {
    KernelArgs args = a;
    void* params[] = {&args};
    const void* fn = dtype == 0 ? reinterpret_cast<const void*>(&fwd_column_kernel<IoF32, 8>)
                                : reinterpret_cast<const void*>(&fwd_column_kernel<IoBF16, 8>);
    return hipLaunchKernel(fn, dim3(a.n_blocks), dim3(kColumnBlock), params, 0, st);
}

hipError_t launch_bwd_column(int dtype, const KernelArgs& a, hipStream_t st) {
    KernelArgs args = a;
    void* params[] = {&args};
    const void* fn = dtype == 0 ? reinterpret_cast<const void*>(&bwd_column_kernel<IoF32, 8>)
                                : reinterpret_cast<const void*>(&bwd_column_kernel<IoBF16, 8>);
    return hipLaunchKernel(fn, dim3(a.n_blocks), dim3(kColumnBlock), params, 0, st);
}

hipError_t launch_clear_state(uint32_t* hdr, uint32_t* flags, size_t n_flags, bool clear_status,
                              hipStream_t st) {
    size_t blocks = (n_flags + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    uint32_t* h = hdr;
    uint32_t* f = flags;
    size_t n = n_flags;
    uint32_t cs = clear_status ? 1u : 0u;
    void* params[] = {&h, &f, &n, &cs};
    return hipLaunchKernel(reinterpret_cast<const void*>(&clear_launch_state_kernel), dim3(unsigned(blocks)),
                           dim3(256), params, 0, st);
}

hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t st) {
    if (n_words == 0) return hipSuccess;
    size_t blocks = (n_words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    uint32_t* pp = p;
    size_t nn = n_words;
    void* params[] = {&pp, &nn};
    return hipLaunchKernel(reinterpret_cast<const void*>(&zero_words_kernel), dim3(unsigned(blocks)), dim3(256),
                           params, 0, st);
}

}  // namespace qc
