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
//            (permlane swaps, or ds_bpermute shuffles for narrow column
//            groups), across waves (LDS) and across blocks
//            (a Fenwick tree of per-tile carries in the workspace, see below).
//            The backward runs its tiles in reverse time order and carries the
//            plain (commutative) sum S in the same way; without saved boundary
//            products (only the forward's final carry) it carries instead each
//            range's product and its share of S in the range's own frame.
//
// Cross-block carries.  Tiles of one column group form a chain; tile i
// (1-based, in chain order) publishes node i of a Fenwick tree: the combined
// carry of tiles (i - lowbit(i), i].  Node i only needs nodes i-1, i-2, ...,
// i-lowbit(i)/2 (ranges inside it), and the exclusive prefix of tile i is the
// ordered combination of the nodes on the Fenwick query path from i-1 down.
// Waits therefore form chains of depth log2(tiles), every tile reads and
// combines O(log tiles) values, and the association of every floating-point
// combine is fixed, so results are bitwise reproducible run to run.
//
// Publication protocol.  Each column's carry in a node is a slot of 64-bit
// words: the value bits followed by one check word, a hash of the value words
// and of the launch epoch.  The slot is written with agent-scope atomic stores
// and read with agent-scope atomic loads (coherent accesses that bypass the
// per-XCD L2, so no L2 write-back or invalidate is ever needed: on this chip
// those cost more than the scan itself).  A reader accepts a slot when its
// check word matches its value words and the current epoch.  Slots left by
// earlier launches fail (their epoch differs; a zeroed slot can never match),
// so nothing is cleared between launches, and a slot read while it is being
// written fails unless a 64-bit hash collides.  Publishing is therefore a
// handful of stores with no wait, and reading is one round trip, with no
// ready flag and no ordering between words.
//
// Ordering.  Tile ids are the block index, position-major over the chains
// (id = position * chains + chain), and a tile only ever waits on tiles of
// smaller id.  Workgroups are dispatched in increasing id order (the grid is
// dealt round-robin to the XCDs, and each dispatches its share in order), so
// every resource a pending tile needs is held by tiles of smaller id, and the
// smallest unfinished tile never waits on an unstarted one: the waits always
// drain.  Every wait is still bounded (kSpinLimit) and raises a status word
// instead of hanging.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// The [b,s,h,j,4] tensors are streamed once per kernel, so their stores and
// the cotangent loads are non-temporal (they would only evict useful lines).
// The chunked kernels read q with the default policy: the backward walks the
// sequence in reverse, so when it runs right after the forward on the same q
// (a step, or a segment recomputed for its backward) it starts on the tiles
// the forward read last, which the memory-side cache still holds, and the
// next forward starts where the backward ended (about 1% per step measured).
// float32 storage: one 16-byte vector per quaternion; float64 arithmetic.
struct IoF32 {
    static constexpr int kDtype = 0;
    using CT = double;
    using Raw = f32x4;
    static __device__ __forceinline__ Raw load(const void* base, int64_t idx) {
        return reinterpret_cast<const Raw*>(base)[idx];
    }
    static __device__ __forceinline__ Raw load_stream(const void* base, int64_t idx) {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(base) + idx);
    }
    static __device__ __forceinline__ Raw one_raw() { return Raw{1.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ Raw zero_raw() { return Raw{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ Q4<CT> ct(const Raw& v) {
        return {double(v.x), double(v.y), double(v.z), double(v.w)};
    }
    // Same as ct(), but hides the register's provenance so the compiler
    // re-converts here instead of keeping float64 copies of every step alive
    // between the two sweeps (twice the registers).
    static __device__ __forceinline__ Q4<CT> ct_fresh(Raw v) {
        asm volatile("" : "+v"(v));
        return ct(v);
    }
    static __device__ __forceinline__ Raw pack(const Q4<CT>& v) {
        return Raw{float(v.w), float(v.x), float(v.y), float(v.z)};
    }
    static __device__ __forceinline__ void store(void* base, int64_t idx, const Q4<CT>& v) {
        reinterpret_cast<Raw*>(base)[idx] = pack(v);
    }
    static __device__ __forceinline__ void store_stream(void* base, int64_t idx, const Q4<CT>& v) {
        __builtin_nontemporal_store(pack(v), reinterpret_cast<Raw*>(base) + idx);
    }
};

// bfloat16 storage: 4 x 16-bit patterns (8 B) per quaternion; float32 arithmetic.
struct IoBF16 {
    static constexpr int kDtype = 1;
    using CT = float;
    using Raw = u32x2;
    static __device__ __forceinline__ Raw load(const void* base, int64_t idx) {
        return reinterpret_cast<const Raw*>(base)[idx];
    }
    static __device__ __forceinline__ Raw load_stream(const void* base, int64_t idx) {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(base) + idx);
    }
    static __device__ __forceinline__ Raw one_raw() { return Raw{0x3f80u, 0u}; }
    static __device__ __forceinline__ Raw zero_raw() { return Raw{0u, 0u}; }
    static __device__ __forceinline__ Q4<CT> ct(const Raw& v) {
        return {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ Q4<CT> ct_fresh(Raw v) {
        asm volatile("" : "+v"(v));
        return ct(v);
    }
    static __device__ __forceinline__ Raw pack(const Q4<CT>& v) {
        return Raw{f32_to_bf16_bits(v.w) | (f32_to_bf16_bits(v.x) << 16),
                   f32_to_bf16_bits(v.y) | (f32_to_bf16_bits(v.z) << 16)};
    }
    static __device__ __forceinline__ void store(void* base, int64_t idx, const Q4<CT>& v) {
        reinterpret_cast<Raw*>(base)[idx] = pack(v);
    }
    static __device__ __forceinline__ void store_stream(void* base, int64_t idx, const Q4<CT>& v) {
        __builtin_nontemporal_store(pack(v), reinterpret_cast<Raw*>(base) + idx);
    }
};

// 1/x for the |q|^2 and |P|^2 normalisations: the hardware reciprocal
// estimate refined by Newton-Raphson, r <- r + r (1 - x r), which squares the
// relative error.  The float64 estimate is good to about 2^-23 relative, so
// one step gives about 2^-46: far below the float32 rounding of every result
// it feeds (each use passes through at most a slice's steps before a store).
__device__ __forceinline__ double recip(double x) {
    const double r = __builtin_amdgcn_rcp(x);
    const double e = __builtin_fma(-x, r, 1.0);
    return __builtin_fma(r, e, r);
}
__device__ __forceinline__ float recip(float x) {
    float r = __builtin_amdgcn_rcpf(x);
    const float e = __builtin_fmaf(-x, r, 1.0f);
    return __builtin_fmaf(r, e, r);
}

// ------------------------------------------------- cross-block carry helpers

using SlotWord = unsigned long long;

// Value words per column slot (float64: one per component; float32: two
// components per word), plus one check word.
template <typename T> struct SlotLayout;
template <> struct SlotLayout<double> { static constexpr int kValueWords = 4; };
template <> struct SlotLayout<float> { static constexpr int kValueWords = 2; };

// Check word of a slot: a multiply-xorshift hash of the value words and the
// launch epoch.  Being non-linear, a slot that mixes words of two different
// writes matches with probability about 2^-63 whatever the bit patterns; the
// low bit is forced to 1 so a zeroed slot never matches.
template <int NV>
__device__ __forceinline__ SlotWord check_word(const SlotWord* v, uint64_t epoch) {
    SlotWord h = epoch * 0x9E3779B97F4A7C15ull;   // odd multiplier: distinct epochs, distinct seeds
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        h = (h ^ v[k]) * 0xFF51AFD7ED558CCDull;
        h ^= h >> 33;
    }
    return h | 1ull;
}

__device__ __forceinline__ void pack_words(const Q4<double>& q, SlotWord* v) {
    v[0] = __builtin_bit_cast(SlotWord, q.w);
    v[1] = __builtin_bit_cast(SlotWord, q.x);
    v[2] = __builtin_bit_cast(SlotWord, q.y);
    v[3] = __builtin_bit_cast(SlotWord, q.z);
}
__device__ __forceinline__ void pack_words(const Q4<float>& q, SlotWord* v) {
    v[0] = SlotWord(__float_as_uint(q.w)) | (SlotWord(__float_as_uint(q.x)) << 32);
    v[1] = SlotWord(__float_as_uint(q.y)) | (SlotWord(__float_as_uint(q.z)) << 32);
}
__device__ __forceinline__ Q4<double> unpack_words(const SlotWord* v, double) {
    return {__builtin_bit_cast(double, v[0]), __builtin_bit_cast(double, v[1]), __builtin_bit_cast(double, v[2]),
            __builtin_bit_cast(double, v[3])};
}
__device__ __forceinline__ Q4<float> unpack_words(const SlotWord* v, float) {
    return {__uint_as_float(uint32_t(v[0])), __uint_as_float(uint32_t(v[0] >> 32)), __uint_as_float(uint32_t(v[1])),
            __uint_as_float(uint32_t(v[1] >> 32))};
}

// Carries of the look-back, as monoids over ranges of tiles.  combine(x, y)
// joins two adjacent ranges: x is the one nearer the reading tile (met first
// on its look-back path), y the farther one.
//   ProductCarry  forward prefix product P: x is later in time, so x (x) y.
//   SumCarry      backward reverse sum S (in the global frame): x + y.
//   PairCarry     backward without boundary products (only the forward's final
//                 carry saved): a range of steps a..b as (U, Y), its product
//                 U = q_b (x) ... (x) q_a and its share of S in the frame of its
//                 first step, Y = sum_t conj(q_t (x) ... (x) q_a) (x) d_t.  The
//                 reverse look-back meets x earlier in time than y, and
//                 (U, Y)_xy = (U_y (x) U_x, Y_x + conj(U_x) (x) Y_y).
template <typename T>
struct QPair {
    Q4<T> u, y;
};

template <typename T>
struct ProductCarry {
    using V = Q4<T>;
    static constexpr int kWords = SlotLayout<T>::kValueWords;
    static __device__ __forceinline__ V identity() { return q_one<T>(); }
    static __device__ __forceinline__ V combine(const V& x, const V& y) { return qmul(x, y); }
    static __device__ __forceinline__ void pack(const V& v, SlotWord* w) { pack_words(v, w); }
    static __device__ __forceinline__ V unpack(const SlotWord* w) { return unpack_words(w, T()); }
};

template <typename T>
struct SumCarry {
    using V = Q4<T>;
    static constexpr int kWords = SlotLayout<T>::kValueWords;
    static __device__ __forceinline__ V identity() { return q_zero<T>(); }
    static __device__ __forceinline__ V combine(const V& x, const V& y) { return qadd(x, y); }
    static __device__ __forceinline__ void pack(const V& v, SlotWord* w) { pack_words(v, w); }
    static __device__ __forceinline__ V unpack(const SlotWord* w) { return unpack_words(w, T()); }
};

template <typename T>
struct PairCarry {
    using V = QPair<T>;
    static constexpr int kWords = 2 * SlotLayout<T>::kValueWords;
    static __device__ __forceinline__ V identity() { return {q_one<T>(), q_zero<T>()}; }
    static __device__ __forceinline__ V combine(const V& x, const V& y) {
        return {qmul(y.u, x.u), qadd(x.y, qcmul(x.u, y.y))};
    }
    static __device__ __forceinline__ void pack(const V& v, SlotWord* w) {
        pack_words(v.u, w);
        pack_words(v.y, w + SlotLayout<T>::kValueWords);
    }
    static __device__ __forceinline__ V unpack(const SlotWord* w) {
        return {unpack_words(w, T()), unpack_words(w + SlotLayout<T>::kValueWords, T())};
    }
};

template <class C>
constexpr int carry_slot_words() { return C::kWords + 1; }

// Publish this lane's column of a node (lanes with `writer` set).
template <class C, int WC>
__device__ __forceinline__ void publish(const KernelArgs& a, SlotWord* slot, const typename C::V& v, bool writer) {
    if (writer) {
        constexpr int NV = C::kWords;
        SlotWord w[NV + 1];
        C::pack(v, w);
        w[NV] = check_word<NV>(w, a.epoch);
#pragma unroll
        for (int k = 0; k <= NV; ++k) __hip_atomic_store(slot + k * WC, w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One read attempt of this lane's column of a node: true (and *out set) if
// the slot holds a complete value of this launch.
template <class C, int WC>
__device__ __forceinline__ bool try_read(const KernelArgs& a, const SlotWord* slot, typename C::V* out) {
    constexpr int NV = C::kWords;
    SlotWord w[NV + 1];
#pragma unroll
    for (int k = 0; k <= NV; ++k) w[k] = __hip_atomic_load(slot + k * WC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *out = C::unpack(w);
    return w[NV] == check_word<NV>(w, a.epoch);
}

// Wait (bounded) until the node is published, then read this lane's column.
// Polls back off from about 30 ns to about 2 us between attempts, so a slot
// that many tiles wait on is not hammered with coherent loads.
template <class C, int WC>
__device__ __forceinline__ typename C::V wait_read(const KernelArgs& a, const SlotWord* slot) {
    typename C::V v = C::identity();
    uint32_t polls = 0;
    while (!try_read<C, WC>(a, slot, &v)) {
        if (polls < 8) {
            __builtin_amdgcn_s_sleep(1);
        } else if (polls < 64) {
            __builtin_amdgcn_s_sleep(8);
        } else {
            __builtin_amdgcn_s_sleep(64);
        }
        if (++polls > a.spin_limit) {
            __hip_atomic_fetch_or(&a.hdr[kHdrStatus], kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    return v;
}

// Fenwick look-back.  The query path of tile i (1-based) is i-1, then
// repeatedly j - lowbit(j) down to 0; lane slot `slot` = wave*R + r of round
// `round` reads the node `round*PAR + slot` steps down the path.
template <int PAR>
__device__ __forceinline__ int64_t path_node(int64_t jn, int steps) {
    for (int k = 0; k < steps && jn > 0; ++k) jn -= jn & (-jn);
    return jn;
}

// Address of column c's first slot word in carry node `node` (0-based over
// all chains).  A node stores its words word-major: word k of column c sits at
// k * WC + c, so the lanes of a column group read each word coalesced.
template <class C, int WC>
__device__ __forceinline__ SlotWord* slot_ptr(const KernelArgs& a, int64_t node, int c) {
    return reinterpret_cast<SlotWord*>(a.desc) + node * (WC * carry_slot_words<C>()) + c;
}

// First-round read attempt, issued right after the tile's data loads so that
// its latency overlaps theirs; predecessor tiles that started long enough
// before have published by then.  Slots are write-once per launch, so an
// early successful read is final; a failed one is retried in the look-back.
template <class C, int WC, int NW>
__device__ __forceinline__ bool fenwick_prefetch(const KernelArgs& a, int64_t chain, int64_t pos, int slot, int c,
                                                 typename C::V* v) {
    const int64_t node = path_node<NW * (64 / WC)>(pos, slot);   // i - 1 = pos
    if (node <= 0) return false;
    return try_read<C, WC>(a, slot_ptr<C, WC>(a, chain * a.n_tiles + node - 1, c), v);
}

// Fenwick look-back for tile `pos` (0-based) of `chain`; called by every
// thread of the block.  `own` is this tile's aggregate, valid in the wave
// `own_wave`; (pre_v, pre_ok) is this slot's first-round prefetch.  Nodes
// are combined with C::combine, nearest first.  The query path is walked in rounds of PAR = NW*R nodes: every lane slot
// makes one read attempt of one node for column c (round 0 uses the
// prefetch), so published nodes cost at most one round trip together; then
// `own_wave` combines the round in the fixed order, waiting itself (nearest
// node first) only for nodes that were not yet published, and publishes node
// i as soon as its children are in.  Returns the exclusive prefix (the
// identity for the first tile) to every thread.
template <class C, int WC, int NW, bool kStaged = false>
__device__ typename C::V fenwick_exclusive(const KernelArgs& a, int64_t chain, int64_t pos, const typename C::V& own,
                                           bool own_wave, int wave, int r, int c, const typename C::V& pre_v,
                                           bool pre_ok, typename C::V (*s_nodes)[WC], uint8_t (*s_ok)[WC],
                                           typename C::V* s_out) {
    using V = typename C::V;
    constexpr int R = 64 / WC;
    constexpr int PAR = NW * R;
    const int64_t i = pos + 1;
    const int64_t low = i & (-i);
    const int64_t node0 = chain * a.n_tiles;   // node n lives at node0 + n - 1
    const int slot = wave * R + r;
    V acc = C::identity();
    bool published = (i == a.n_tiles);        // nothing reads the last node
    int64_t jn = i - 1;                       // next node on the query path (block-uniform)
    for (int round = 0;; ++round) {
        if (own_wave && !published && jn <= i - low) {
            publish<C, WC>(a, slot_ptr<C, WC>(a, node0 + i - 1, c), C::combine(own, acc), r == 0);
            published = true;
        }
        if (jn == 0) break;
        const int64_t mine = path_node<PAR>(jn, slot);
        if (mine > 0) {
            const int64_t nd = node0 + mine - 1;
            if constexpr (kStaged) {
                if (round > 0 || !s_ok[slot][c]) {
                    V v;
                    s_ok[slot][c] = try_read<C, WC>(a, slot_ptr<C, WC>(a, nd, c), &v) ? 1 : 0;
                    s_nodes[slot][c] = v;
                }
            } else {
                V v = pre_v;
                const bool ok = round == 0 ? (pre_ok || try_read<C, WC>(a, slot_ptr<C, WC>(a, nd, c), &v))
                                           : try_read<C, WC>(a, slot_ptr<C, WC>(a, nd, c), &v);
                s_nodes[slot][c] = v;
                s_ok[slot][c] = ok ? 1 : 0;
            }
        }
        __syncthreads();
        for (int k = 0; k < PAR && jn > 0; ++k) {
            if (own_wave) {
                if (!published && jn <= i - low) {
                    publish<C, WC>(a, slot_ptr<C, WC>(a, node0 + i - 1, c), C::combine(own, acc), r == 0);
                    published = true;
                }
                const V v = s_ok[k][c] ? s_nodes[k][c] : wait_read<C, WC>(a, slot_ptr<C, WC>(a, node0 + jn - 1, c));
                acc = C::combine(acc, v);
            }
            jn -= jn & (-jn);
        }
        __syncthreads();                      // s_nodes is reused by the next round
    }
    if (own_wave && r == 0) s_out[c] = acc;
    __syncthreads();
    return s_out[c];
}

// Grouped look-back, for chains whose tiles are mostly in flight at once
// (few, long chains), where the Fenwick query's depth of about log2(tiles)
// publish-then-poll round trips is exposed instead of hidden behind other
// tiles' streaming.  Tiles form groups of G = a.group consecutive positions.
// Every tile publishes its own aggregate as soon as it has it; the last tile
// of each group (unless it is in the chain's last group) also publishes the
// group's aggregate once it has read the rest of its group.  Tile p = gG + k
// then combines, nearest first, the aggregates of tiles p-1 .. gG and of
// groups g-1 .. 0: two round trips deep, at the price of up to
// (G - 1) + (groups - 1) node reads per tile instead of about log2(p).
// Node layout: tile aggregates at chain * n_tiles + p (as the Fenwick nodes),
// group aggregates after all of those, at n_chains * n_tiles + chain * n_groups + g.
// Item t of tile p's read list is the tile node p-1-t for t < k, else the
// group node g-1-(t-k).
template <class C, int WC>
__device__ __forceinline__ SlotWord* grouped_node(const KernelArgs& a, int64_t chain, int64_t pos, int64_t t, int c) {
    const int64_t k = pos % a.group;
    const int64_t node = t < k ? chain * a.n_tiles + pos - 1 - t
                               : a.n_chains * a.n_tiles + chain * a.n_groups + pos / a.group - 1 - (t - k);
    return slot_ptr<C, WC>(a, node, c);
}

// First-round read attempt of the Fenwick look-back (the grouped one reads
// its nodes when it gets there).
template <class C, int WC, int NW, bool kGrouped>
__device__ __forceinline__ bool lookback_prefetch(const KernelArgs& a, int64_t chain, int64_t pos, int slot, int c,
                                                  typename C::V* v) {
    if constexpr (kGrouped) return false;
    return fenwick_prefetch<C, WC, NW>(a, chain, pos, slot, c, v);
}

// Combination, in list order, of items [lo, hi) of the read list: this lane
// slot takes a contiguous run of them (a few items), waiting for each in turn.
template <class C, int WC, int PAR>
__device__ typename C::V grouped_run(const KernelArgs& a, int64_t chain, int64_t pos, int64_t lo, int64_t hi,
                                     int slot, int c) {
    const int64_t per = (hi - lo + PAR - 1) / PAR;
    const int64_t r0 = lo + slot * per < hi ? lo + slot * per : hi;
    const int64_t r1 = r0 + per < hi ? r0 + per : hi;
    typename C::V part = C::identity();
    for (int64_t t = r0; t < r1; ++t) part = C::combine(part, wait_read<C, WC>(a, grouped_node<C, WC>(a, chain, pos, t, c)));
    return part;
}

// Same contract as fenwick_exclusive (pre_v / pre_ok unused).
template <class C, int WC, int NW>
__device__ typename C::V grouped_exclusive(const KernelArgs& a, int64_t chain, int64_t pos, const typename C::V& own,
                                           bool own_wave, int wave, int r, int c, typename C::V (*s_nodes)[WC],
                                           typename C::V* s_out) {
    constexpr int R = 64 / WC;
    constexpr int PAR = NW * R;
    const int64_t k = pos % a.group, g = pos / a.group;
    const int slot = wave * R + r;
    // Nothing reads the chain's last tile, nor the last group.
    if (own_wave && pos + 1 < a.n_tiles) publish<C, WC>(a, slot_ptr<C, WC>(a, chain * a.n_tiles + pos, c), own, r == 0);
    // Phase 1, the group's earlier tiles: the group's last tile publishes the
    // group aggregate from them before it waits on anything else.
    s_nodes[slot][c] = grouped_run<C, WC, PAR>(a, chain, pos, 0, k, slot, c);
    __syncthreads();
    typename C::V acc = C::identity();
    if (own_wave) {
#pragma unroll 2
        for (int j = 0; j < PAR; ++j) acc = C::combine(acc, s_nodes[j][c]);
        if (k == a.group - 1 && g + 1 < a.n_groups)
            publish<C, WC>(a, slot_ptr<C, WC>(a, a.n_chains * a.n_tiles + chain * a.n_groups + g, c),
                           C::combine(own, acc), r == 0);
    }
    __syncthreads();
    // Phase 2, the earlier groups.
    s_nodes[slot][c] = grouped_run<C, WC, PAR>(a, chain, pos, k, k + g, slot, c);
    __syncthreads();
    if (own_wave) {
#pragma unroll 2
        for (int j = 0; j < PAR; ++j) acc = C::combine(acc, s_nodes[j][c]);
        if (r == 0) s_out[c] = acc;
    }
    __syncthreads();
    return s_out[c];
}

// The two look-backs are separate kernel instances: the scan kernels hold
// their tile in registers across the look-back, and code for both would
// raise every instance's register count.
template <class C, int WC, int NW, bool kGrouped, bool kStaged = false>
__device__ __forceinline__ typename C::V lookback_exclusive(const KernelArgs& a, int64_t chain, int64_t pos,
                                                            const typename C::V& own, bool own_wave, int wave, int r,
                                                            int c, const typename C::V& pre_v, bool pre_ok,
                                                            typename C::V (*s_nodes)[WC], uint8_t (*s_ok)[WC],
                                                            typename C::V* s_out) {
    if constexpr (kGrouped)
        return grouped_exclusive<C, WC, NW>(a, chain, pos, own, own_wave, wave, r, c, s_nodes, s_out);
    else
        return fenwick_exclusive<C, WC, NW, kStaged>(a, chain, pos, own, own_wave, wave, r, c, pre_v, pre_ok, s_nodes,
                                                     s_ok, s_out);
}

// The launch epoch: from the arguments, or (launches captured in a graph,
// epoch 0) from the header counter that a one-thread kernel bumped just
// before, read coherently and made wave-uniform.
__device__ __forceinline__ uint64_t launch_epoch(const KernelArgs& a) {
    if (a.epoch != 0) return a.epoch;
    const uint64_t e = __hip_atomic_load(reinterpret_cast<const uint64_t*>(a.hdr + kHdrEpoch), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(e));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(e >> 32));
    return (uint64_t(hi) << 32) | lo;
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
    // Position-major ids; within one position the chains are rotated by the
    // position, so consecutive tiles of a chain land on different XCDs (the
    // grid is dealt round-robin to them) and no XCD streams a fixed subset of
    // column groups.  Still monotone in position within a chain.
    tc.pos = id / a.n_chains;
    const int64_t j = id % a.n_chains, rot = tc.pos % a.n_chains;
    tc.chain = j >= rot ? j - rot : j - rot + a.n_chains;
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

// Lane moves by gfx950 permlane swaps (VALU, no LDS crossbar).  For O = 32,
// lane blocks are the wave's two 32-lane halves; for O = 16, the 16-lane rows
// of each half.  Given x, *even receives in every lane the value of the even
// block of its pair (O = 32: the lower half; O = 16: rows 0, 0, 2, 2) and
// *odd that of the odd block (the upper half; rows 1, 1, 3, 3): the swap
// exchanges one operand's odd blocks with the other's even blocks, and both
// operands are x.
template <int O, typename T>
__device__ __forceinline__ void q_perm(const Q4<T>& x, Q4<T>* even, Q4<T>* odd) {
    static_assert(O == 32 || O == 16, "permlane swaps move 32 or 16 lanes");
    constexpr int N = int(sizeof(Q4<T>) / 4);
    uint32_t in[N], e[N], o[N];
    __builtin_memcpy(in, &x, sizeof(in));
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const auto p = O == 32 ? __builtin_amdgcn_permlane32_swap(in[i], in[i], false, false)
                               : __builtin_amdgcn_permlane16_swap(in[i], in[i], false, false);
        e[i] = p[0];
        o[i] = p[1];
    }
    __builtin_memcpy(even, e, sizeof(e));
    __builtin_memcpy(odd, o, sizeof(o));
}

// In-wave scan of the R slice products of a column (slice r holds A), in
// left-multiply order: *inc = A_r (x) ... (x) A_0, *exw = A_{r-1} (x) ... (x) A_0
// (identity for r = 0), *last = the wave's total A_{R-1} (x) ... (x) A_0 in every
// lane.  Two and four slices per wave (32- and 16-column groups) move lanes
// by permlane swaps; four first scans each 32-lane half, then offsets the
// upper half by the lower half's total.  Narrower groups (eight or more
// slices) use a Hillis-Steele scan over ds_bpermute shuffles.
template <typename T, int WC>
__device__ __forceinline__ void wave_scan_product(const Q4<T>& A, int r, int c, Q4<T>* inc, Q4<T>* exw,
                                                  Q4<T>* last) {
    constexpr int R = 64 / WC;
    Q4<T> even, odd;
    if constexpr (R == 1) {
        *inc = A;
        *exw = q_one<T>();
        *last = A;
    } else if constexpr (R == 2) {
        q_perm<32>(A, &even, &odd);                   // even: the lower slice's A
        *inc = r == 1 ? qmul(A, even) : A;
        *exw = r == 1 ? even : q_one<T>();
        q_perm<32>(*inc, &even, last);                // odd: the upper slice's inc
    } else if constexpr (R == 4) {
        q_perm<16>(A, &even, &odd);                   // even: rows 0, 0, 2, 2 of A
        const Q4<T> in_half = (r & 1) ? qmul(A, even) : A;
        const Q4<T> ex_half = (r & 1) ? even : q_one<T>();
        Q4<T> half_tot, lower_tot;
        q_perm<16>(in_half, &even, &half_tot);        // odd: each half's total (rows 1, 1, 3, 3)
        q_perm<32>(half_tot, &lower_tot, &odd);       // even: the lower half's total, everywhere
        const Q4<T> off = r >= 2 ? lower_tot : q_one<T>();
        *inc = qmul(in_half, off);
        *exw = qmul(ex_half, off);
        Q4<T> row_odd;
        q_perm<16>(*inc, &even, &row_odd);            // odd: rows 1, 1, 3, 3 of inc
        q_perm<32>(row_odd, &even, last);             // odd: the upper half's, i.e. row 3's
    } else {
        Q4<T> x = A;
#pragma unroll
        for (int d = 1; d < R; d <<= 1) {
            const Q4<T> o = shfl_up_q(x, d * WC);
            if (r >= d) x = qmul(x, o);
        }
        *inc = x;
        *exw = shfl_up_q(x, WC);
        if (r == 0) *exw = q_one<T>();
        *last = shfl_q(x, (R - 1) * WC + c);
    }
}

// In-tile exclusive prefix product of slice aggregates (left-multiply order).
// Slice k = wave*R + r.  Returns F = product of slices before k in this tile;
// `tile_agg` receives the tile's full product (valid in the last wave).
template <typename T, int WC, int NW>
__device__ __forceinline__ Q4<T> tile_scan_product(const Q4<T>& A, Q4<T> (*s_wagg)[WC], int wave, int r, int c,
                                                   Q4<T>* tile_agg) {
    constexpr int R = 64 / WC;
    Q4<T> inc, exw, last;
    wave_scan_product<T, WC>(A, r, c, &inc, &exw, &last);
    if (r == R - 1) s_wagg[wave][c] = inc;
    __syncthreads();
    Q4<T> wex = q_one<T>();
    for (int w2 = wave - 1; w2 >= 0; --w2) wex = qmul(wex, s_wagg[w2][c]);
    *tile_agg = qmul(last, wex);
    return qmul(exw, wex);
}

// ------------------------------------------------------------ forward, chunked

// Carries of the reduce-then-scan variant, in the workspace's carry region:
// per (chain, tile position, column) one compute-type quaternion, the tile
// aggregates first, then the scanned carries.
template <typename CT, int WC>
__device__ __forceinline__ Q4<CT>* rscan_agg(const KernelArgs& a, int64_t chain, int64_t pos, int c) {
    return reinterpret_cast<Q4<CT>*>(a.desc) + (chain * a.n_tiles + pos) * WC + c;
}
template <typename CT, int WC>
__device__ __forceinline__ Q4<CT>* rscan_carry(const KernelArgs& a, int64_t chain, int64_t pos, int c) {
    return reinterpret_cast<Q4<CT>*>(a.desc) + (a.n_chains * a.n_tiles + chain * a.n_tiles + pos) * WC + c;
}

// kStore = false is the boundary-state pass of a backward without saved
// state: no cum output, so q is dropped right after sweep 1 (fewer registers).
// kMode selects how a tile learns the product of the tiles before it:
//   kLookback  the Fenwick look-back over published carries, in one pass;
//   kGrouped   the grouped look-back, in one pass;
//   kAggregate reduce-then-scan, pass 1: only the tile's product, stored;
//   kFixup     reduce-then-scan, pass 3: the scanned carry, read.
enum : int { kLookback = 0, kAggregate = 1, kFixup = 2, kGrouped = 3 };
constexpr bool one_pass(int mode) { return mode == kLookback || mode == kGrouped; }

template <class IO, int WC, int L, int NW, bool kStore, int kMode>
__global__ void __launch_bounds__(NW * 64) fwd_chunked_kernel(KernelArgs a) {
    if constexpr (one_pass(kMode)) a.epoch = launch_epoch(a);
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    constexpr int R = 64 / WC;
    __shared__ Q4<CT> s_wagg[NW][WC];
    __shared__ Q4<CT> s_nodes[NW * R][WC];
    __shared__ uint8_t s_ok[NW * R][WC];
    __shared__ Q4<CT> s_carry[WC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / WC, c = lane % WC;
    const uint32_t s_id = blockIdx.x;
    const TileCoord tc = tile_coord<WC, L, NW>(a, s_id, false, wave * R + r, c);

    Raw qv[L];
    if (tc.full) {
#pragma unroll
        for (int i = 0; i < L; ++i) qv[i] = IO::load(a.q, tc.base + int64_t(i) * a.M);
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i)
            qv[i] = (tc.col_ok && tc.t0 + i < a.s) ? IO::load(a.q, tc.base + int64_t(i) * a.M)
                                                    : IO::one_raw();
    }
    Raw init_raw = IO::one_raw();
    if (kStore && tc.col_ok) init_raw = IO::load(a.init, tc.bi * a.M + tc.m);
    Q4<CT> pre_v = q_one<CT>();
    bool pre_ok = false;
    if constexpr (one_pass(kMode))
        pre_ok = lookback_prefetch<ProductCarry<CT>, WC, NW, kMode == kGrouped>(a, tc.chain, tc.pos, wave * R + r, c,
                                                                                &pre_v);
    Q4<CT> Et = q_one<CT>();
    if constexpr (kMode == kFixup) Et = *rscan_carry<CT, WC>(a, tc.chain, tc.pos, c);

    // Slice product: A = q_{t0+L-1} (x) ... (x) q_{t0}.
    Q4<CT> A = IO::ct(qv[0]);
#pragma unroll
    for (int i = 1; i < L; ++i) A = qmul(IO::ct(qv[i]), A);

    Q4<CT> tile_agg;
    const Q4<CT> F = tile_scan_product<CT, WC, NW>(A, s_wagg, wave, r, c, &tile_agg);
    if constexpr (kMode == kAggregate) {
        if (wave == NW - 1 && r == 0) *rscan_agg<CT, WC>(a, tc.chain, tc.pos, c) = tile_agg;
        return;
    }
    if constexpr (one_pass(kMode))
        Et = lookback_exclusive<ProductCarry<CT>, WC, NW, kMode == kGrouped>(a, tc.chain, tc.pos, tile_agg, wave == NW - 1,
                                                                             wave, r, c, pre_v, pre_ok, s_nodes, s_ok,
                                                                             s_carry);
    const Q4<CT> Ps = qmul(F, Et);   // P_{t0-1}: prefix product before this slice

    if (a.ckpt != nullptr && tc.col_ok && tc.t0 < a.s && (tc.t0 % kCkptStride) == 0)
        reinterpret_cast<Q4<CT>*>(a.ckpt)[(tc.bi * a.n_ck + tc.t0 / kCkptStride) * a.M + tc.m] = Ps;

    if (kStore) {
        Q4<CT> cm = qmul(Ps, IO::ct(init_raw));   // cum[t0-1]
        if (tc.full) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                cm = qmul(IO::ct_fresh(qv[i]), cm);
                IO::store_stream(a.out, tc.base + int64_t(i) * a.M, cm);
            }
        } else if (tc.col_ok) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if (tc.t0 + i < a.s) {
                    cm = qmul(IO::ct_fresh(qv[i]), cm);
                    IO::store_stream(a.out, tc.base + int64_t(i) * a.M, cm);
                }
            }
        }
        // The final carry cum[s-1], for a backward from it alone.
        if (a.fin != nullptr && tc.col_ok && tc.t0 < a.s && tc.t0 + L >= a.s)
            reinterpret_cast<Q4<CT>*>(a.fin)[tc.bi * a.M + tc.m] = cm;
    }
}

// ----------------------------------------------------------- backward, chunked
//
// Tiles run in reverse time order; lane slice k = wave*R + r of a tile owns
// steps t0 .. t0+L-1 of one column.  Sweep 1 (ascending) keeps only two
// quaternions per lane, in the frame of the slice start:
//   Q_k = q_{t0+L-1} (x) ... (x) q_{t0}                    (slice product)
//   Y_k = sum_t conj(q_t (x) ... (x) q_{t0}) (x) d_t         (slice's share of S)
// One LDS exchange then gives every lane, from the (Q, Y) of all slices of its
// column in the tile:
//   A_k  = Q_k (x) ... (x) Q_0                 (tile-local prefix through the slice)
//   R'_k = Y_{k+1} + conj(Q_{k+1}) (x) (Y_{k+2} + conj(Q_{k+2}) (x) ( ... ))
//          (what later slices of the tile send back to the slice's last step)
// and the tile's total conj(E) (x) (Y_0 + conj(Q_0) (x) R'_0), E = P before the
// tile (saved boundary state), enters the reverse look-back over tiles, which
// returns S_after = sum over later tiles of conj(P_u) (x) d_u.  The cotangent
// reaching the slice's last step te is then exact for any non-zero inputs:
//   G[te] = d_te + R'_k + A_k (x) Z / |A_k|^2,     Z = E (x) S_after / |E|^2
// (the later-tile part is P_te (x) S_after / |P_te|^2 written in the tile frame).
// Sweep 2 walks the slice downwards with the reverse recurrence
//   d_q[t] = G[t] (x) conj(cum[t-1]),   G[t-1] = d_{t-1} + conj(q_t) (x) G[t],
//   cum[t-1] = conj(q_t) (x) cum[t] / |q_t|^2
// from cum[te] = A_k (x) E (x) init, with cum[t0-1] taken directly as
// A_{k-1} (x) E (x) init.  Only q and d stay in registers between the sweeps, in
// storage precision.
//
// kFinal: the same tile without any prefix product saved, only the forward's
// final carry cum[s-1] (a.fin, per column, internal precision).  G needs no
// prefix product at all (it is the page's reverse recurrence), only cum does.
// The reverse look-back carries the frame-free pair of each later range
// (PairCarry): its product U and its share Y in the frame of its first step,
// which gives the tile (U_a, Y_a) over all later tiles.  With
// B_k = Q_{K-1} (x) ... (x) Q_{k+1}, the slices of the tile after k:
//   G[te]   = d_te + R'_k + conj(B_k) (x) Y_a     (the sum over u > te of
//             conj(q_u (x) ... (x) q_{te+1}) (x) d_u, which P_te (x) S / |P_te|^2
//             reduces to: P_u = (q_u (x) ... (x) q_{te+1}) (x) P_te)
//   cum[te] = B_k^-1 (x) U_a^-1 (x) cum[s-1]      (cum[s-1] = U_a (x) B_k (x) cum[te])
//   cum[t0 - 1] = Q_k^-1 (x) cum[te],    d_init = S[0] = Y of the whole sequence.
// Nothing here needs a product from the front of the sequence, so q and
// d_cum are read once and no boundary state exists.  The inverses need the
// products over later steps to be non-zero, which holds whenever no step is
// zero (else the status word reports it, as for a zero prefix product).

// Sweep 2 of a backward slice: from G[te] and cum[te] at its last step te and
// cum[t0-1] before it, walk down the slice storing d_q[t] = G[t] (x) conj(cum[t-1]).
template <class IO, int L>
__device__ __forceinline__ void sweep2_store(const KernelArgs& a, const TileCoord& tc, const typename IO::Raw (&qv)[L],
                                             const typename IO::Raw (&dv)[L], Q4<typename IO::CT> G,
                                             Q4<typename IO::CT> cm, const Q4<typename IO::CT>& c0) {
    using CT = typename IO::CT;
#pragma unroll
    for (int i = L - 1; i >= 0; --i) {
        const Q4<CT> qi = IO::ct_fresh(qv[i]);
        const Q4<CT> cprev = i == 0 ? c0 : qscale(qcmul(qi, cm), recip(qnorm2(qi)));
        if (tc.full || tc.t0 + i < a.s) IO::store_stream(a.out, tc.base + int64_t(i) * a.M, qmulc(G, cprev));
        if (i > 0) G = qadd(IO::ct_fresh(dv[i - 1]), qcmul(qi, G));
        cm = cprev;
    }
}

// Waves per SIMD to ask of the compiler: 3 while the slice's q and d_cum fit
// in 64 registers, else 2; bfloat16 slices (float32 arithmetic) fit 4.
template <class IO, int L>
constexpr int bwd_min_waves() {
    return IO::kDtype == 1 && L * 2 * int(sizeof(typename IO::Raw)) / 4 <= 64 ? 4
         : L * 2 * int(sizeof(typename IO::Raw)) / 4 <= 64 ? 3 : 2;
}

template <class IO, int WC, int L, int NW, int kMode, bool kFinal>
__global__ void __launch_bounds__(NW * 64, (bwd_min_waves<IO, L>())) bwd_chunked_kernel(KernelArgs a) {
    static_assert(!kFinal || one_pass(kMode), "the final-carry backward runs only with a look-back");
    if constexpr (one_pass(kMode)) a.epoch = launch_epoch(a);
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    using Carry = std::conditional_t<kFinal, PairCarry<CT>, SumCarry<CT>>;
    using CV = typename Carry::V;
    constexpr int R = 64 / WC;
    constexpr int K = NW * R;   // slices per column in a tile
    __shared__ Q4<CT> s_sq[K][WC];
    __shared__ Q4<CT> s_sy[K][WC];
    __shared__ CV s_nodes[K][WC];
    __shared__ uint8_t s_ok[K][WC];
    __shared__ CV s_after[WC];
    __shared__ Q4<CT> s_b[kFinal ? K : 1][WC];
    __shared__ Q4<CT> s_rp[kFinal ? K : 1][WC];
    __shared__ Q4<CT> s_fin[kFinal ? WC : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / WC, c = lane % WC;
    const int k = wave * R + r;
    const uint32_t s_id = blockIdx.x;
    const TileCoord tc = tile_coord<WC, L, NW>(a, s_id, true, k, c);

    Raw qv[L], dv[L];
    if (tc.full) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            qv[i] = IO::load(a.q, tc.base + int64_t(i) * a.M);
            // The reduce-then-scan passes read d_cum twice: keep it cached.
            dv[i] = one_pass(kMode) ? IO::load_stream(a.d_cum, tc.base + int64_t(i) * a.M)
                                       : IO::load(a.d_cum, tc.base + int64_t(i) * a.M);
        }
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const bool ok = tc.col_ok && tc.t0 + i < a.s;
            qv[i] = ok ? IO::load(a.q, tc.base + int64_t(i) * a.M) : IO::one_raw();
            dv[i] = ok ? (one_pass(kMode) ? IO::load_stream(a.d_cum, tc.base + int64_t(i) * a.M)
                                             : IO::load(a.d_cum, tc.base + int64_t(i) * a.M))
                       : IO::zero_raw();
        }
    }
    // Prefix product before the tile (saved boundary state) and the initial
    // carry.  (kFinal reads the forward's final carry after the look-back.)
    const int64_t tile_t0 = tc.t0 - int64_t(k) * L;
    Q4<CT> Et = q_one<CT>();
    Raw init_raw = IO::one_raw();
    if (!kFinal && tc.col_ok) {
        Et = reinterpret_cast<const Q4<CT>*>(a.ckpt)[(tc.bi * a.n_ck + tile_t0 / kCkptStride) * a.M + tc.m];
        init_raw = IO::load(a.init, tc.bi * a.M + tc.m);
    }
    CV pre_v = Carry::identity();
    bool pre_ok = false;
    if constexpr (one_pass(kMode))
        pre_ok = lookback_prefetch<Carry, WC, NW, kMode == kGrouped>(a, tc.chain, tc.pos, k, c, &pre_v);
    Q4<CT> fin = q_one<CT>();
    if (kFinal && k == 0 && tc.col_ok) fin = reinterpret_cast<const Q4<CT>*>(a.fin)[tc.bi * a.M + tc.m];
    CV Sa = Carry::identity();
    if constexpr (kMode == kFixup) Sa = *rscan_carry<CT, WC>(a, tc.chain, tc.pos, c);

    // Sweep 1: slice product and slice share, frame of the slice start.
    Q4<CT> Ql = IO::ct(qv[0]);
    Q4<CT> Yl = qcmul(Ql, IO::ct(dv[0]));
#pragma unroll
    for (int i = 1; i < L; ++i) {
        Ql = qmul(IO::ct(qv[i]), Ql);
        Yl = qadd(Yl, qcmul(Ql, IO::ct(dv[i])));
    }
    s_sq[k][c] = Ql;
    s_sy[k][c] = Yl;
    if constexpr (kFinal && kMode == kLookback) {
        s_nodes[k][c] = pre_v;
        s_ok[k][c] = pre_ok ? 1 : 0;
    }
    __syncthreads();

    // Exclusive prefix F (slices before k) and exclusive suffix R' (slices
    // after k); kFinal needs no F, but B = Q_{K-1} (x) ... (x) Q_{k+1}.
    Q4<CT> F = q_one<CT>(), B = q_one<CT>();
    if constexpr (!kFinal) {
        if (k > 0) {
            F = s_sq[0][c];
            for (int k2 = 1; k2 < k; ++k2) F = qmul(s_sq[k2][c], F);
        }
    }
    Q4<CT> Rp = q_zero<CT>();
    if (k < K - 1) {
        Rp = s_sy[K - 1][c];
        if constexpr (kFinal) B = s_sq[K - 1][c];
        for (int k2 = K - 2; k2 > k; --k2) {
            Rp = qadd(s_sy[k2][c], qcmul(s_sq[k2][c], Rp));
            if constexpr (kFinal) B = qmul(B, s_sq[k2][c]);
        }
    }

    // kFinal parks B and R' in LDS across the look-back, whose pair carries
    // leave no registers for them (Q_k and Y_k are still in s_sq / s_sy).
    if constexpr (kFinal) {
        s_b[k][c] = B;
        s_rp[k][c] = Rp;
        if (k == 0) s_fin[c] = fin;
    }

    // The tile's carry, meaningful in slice 0, which publishes it: its share
    // of S in the global frame, conj(E) (x) (Y_0 + conj(Q_0) (x) R'_0); kFinal:
    // the pair (U_t, Y_0 + conj(Q_0) (x) R'_0), U_t = B_0 (x) Q_0.
    CV own = Carry::identity();
    if (wave == 0) {
        if constexpr (kFinal)
            own = {qmul(B, Ql), qadd(Yl, qcmul(Ql, Rp))};
        else
            own = qcmul(Et, qadd(Yl, qcmul(Ql, Rp)));
    }
    if constexpr (kMode == kAggregate) {
        if (wave == 0 && r == 0) *rscan_agg<CT, WC>(a, tc.chain, tc.pos, c) = own;
        return;
    }
    if constexpr (one_pass(kMode))
        Sa = lookback_exclusive<Carry, WC, NW, kMode == kGrouped, kFinal>(a, tc.chain, tc.pos, own, wave == 0, wave,
                                                                          r, c, pre_v, pre_ok, s_nodes, s_ok, s_after);

    if constexpr (kFinal) {
        // Sa = (U_a, Y_a) of all later tiles.  At the slice end te,
        // cum[te] = B^-1 (x) U_a^-1 (x) cum[s-1] and the later steps' part of
        // G[te] is R' + conj(B) (x) Y_a; S[0] is the whole sequence's Y.
        const Q4<CT> Bk = s_b[k][c], Rk = s_rp[k][c], Qk = s_sq[k][c];
        if (a.d_init != nullptr && tc.t0 == 0 && tc.col_ok) {
            const Q4<CT> Ut = qmul(Bk, Qk), Yt = qadd(s_sy[k][c], qcmul(Qk, Rk));
            IO::store(a.d_init, tc.bi * a.M + tc.m, qadd(Yt, qcmul(Ut, Sa.y)));
        }
        if (a.out != nullptr && tc.col_ok) {
            const CT nU = qnorm2(Sa.u), nB = qnorm2(Bk), nQ = qnorm2(Qk);
            if (nU == CT(0) || nB == CT(0) || nQ == CT(0))
                __hip_atomic_fetch_or(&a.hdr[kHdrStatus], kStatusZeroPrefix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const Q4<CT> Ce = qscale(qcmul(Sa.u, s_fin[c]), recip(nU));   // cum at the tile's last step
            const Q4<CT> cm = qscale(qcmul(Bk, Ce), recip(nB));      // cum[t0 + L - 1]
            const Q4<CT> c0 = qscale(qcmul(Qk, cm), recip(nQ));      // cum[t0 - 1]
            const Q4<CT> G = qadd(IO::ct_fresh(dv[L - 1]), qadd(Rk, qcmul(Bk, Sa.y)));
            sweep2_store<IO, L>(a, tc, qv, dv, G, cm, c0);
        }
    } else {
        const Q4<CT> A = qmul(Ql, F);
        if (a.d_init != nullptr && tc.t0 == 0 && tc.col_ok)
            IO::store(a.d_init, tc.bi * a.M + tc.m, qadd(own, Sa));   // S[0] (slice 0 of the first tile, E = 1)
        if (a.out != nullptr && tc.col_ok) {
            const CT nE = qnorm2(Et), nA = qnorm2(A);
            // A zero step makes every later prefix product exactly zero, which shows
            // up here (E for later tiles, A for its own and later slices of this tile).
            if (nE == CT(0) || nA == CT(0))
                __hip_atomic_fetch_or(&a.hdr[kHdrStatus], kStatusZeroPrefix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const Q4<CT> Z = qscale(qmul(Et, Sa), recip(nE));
            const Q4<CT> C = qmul(Et, IO::ct(init_raw));           // cum before the tile
            const Q4<CT> c0 = qmul(F, C);                          // cum[t0 - 1]
            const Q4<CT> cm = qmul(A, C);                          // cum[t0 + L - 1]
            const Q4<CT> G = qadd(IO::ct_fresh(dv[L - 1]), qadd(Rp, qscale(qmul(A, Z), recip(nA))));
            sweep2_store<IO, L>(a, tc, qv, dv, G, cm, c0);
        }
    }
}

// Leaves-only backward in one pass, for shapes whose chains fit on the chip
// a group of blocks at a time (the page's contract: only q and init are
// saved, and no pre-pass re-reads q to rebuild the boundary products).  The
// grid is cooperative: a.n_coop groups of a.n_tiles blocks, all resident at
// once, and group g walks chains g, g + n_coop, ...  Block b of a group owns
// tile b (time order) of its chain.  A tile learns the prefix product E
// before it from a forward Fenwick look-back among its own group (nodes in
// a.desc2: the tile's product of all its slices), then runs the backward's
// reverse look-back and sweep 2 as bwd_chunked_kernel does with E from the
// saved boundary state.  Every wait is on a block of the same group in the
// same chain; the group is resident, and a block leaves a chain only after
// publishing all of its nodes of that chain, so every wait ends.
template <int WC, int L, int NW>
__device__ __forceinline__ TileCoord tile_at(const KernelArgs& a, int64_t chain, int64_t tile, int k, int c) {
    constexpr int T = (64 / WC) * NW * L;
    TileCoord tc;
    tc.chain = chain;
    tc.pos = a.n_tiles - 1 - tile;   // the reverse look-back's position
    tc.bi = chain / a.n_cg;
    const int64_t cg = chain % a.n_cg;
    tc.m = cg * WC + c;
    tc.col_ok = tc.m < a.M;
    tc.t0 = tile * T + int64_t(k) * L;
    tc.base = (tc.bi * a.s + tc.t0) * a.M + tc.m;
    tc.full = (tile + 1) * T <= a.s && (cg + 1) * WC <= a.M;
    return tc;
}

template <class IO, int WC, int L, int NW>
__global__ void __launch_bounds__(NW * 64, (bwd_min_waves<IO, L>() < 3 ? bwd_min_waves<IO, L>() : 3))
    bwd_coresident_kernel(KernelArgs a) {
    a.epoch = launch_epoch(a);
    using CT = typename IO::CT;
    using Raw = typename IO::Raw;
    constexpr int R = 64 / WC;
    constexpr int K = NW * R;
    __shared__ Q4<CT> s_sq[K][WC];
    __shared__ Q4<CT> s_sy[K][WC];
    __shared__ Q4<CT> s_nodes[K][WC];
    __shared__ uint8_t s_ok[K][WC];
    __shared__ Q4<CT> s_before[WC];
    __shared__ Q4<CT> s_after[WC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / WC, c = lane % WC;
    const int k = wave * R + r;
    const int64_t group = blockIdx.x / a.n_tiles, tile = blockIdx.x % a.n_tiles;
    KernelArgs af = a;
    af.desc = a.desc2;

    for (int64_t chain = group; chain < a.n_chains; chain += a.n_coop) {
        const TileCoord tc = tile_at<WC, L, NW>(a, chain, tile, k, c);
        Raw qv[L], dv[L];
        if (tc.full) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                qv[i] = IO::load(a.q, tc.base + int64_t(i) * a.M);
                dv[i] = IO::load_stream(a.d_cum, tc.base + int64_t(i) * a.M);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const bool ok = tc.col_ok && tc.t0 + i < a.s;
                qv[i] = ok ? IO::load(a.q, tc.base + int64_t(i) * a.M) : IO::one_raw();
                dv[i] = ok ? IO::load_stream(a.d_cum, tc.base + int64_t(i) * a.M) : IO::zero_raw();
            }
        }
        Raw init_raw = IO::one_raw();
        if (tc.col_ok) init_raw = IO::load(a.init, tc.bi * a.M + tc.m);

        // Sweep 1 and the tile's exchange, as in bwd_chunked_kernel.
        Q4<CT> Ql = IO::ct(qv[0]);
        Q4<CT> Yl = qcmul(Ql, IO::ct(dv[0]));
#pragma unroll
        for (int i = 1; i < L; ++i) {
            Ql = qmul(IO::ct(qv[i]), Ql);
            Yl = qadd(Yl, qcmul(Ql, IO::ct(dv[i])));
        }
        s_sq[k][c] = Ql;
        s_sy[k][c] = Yl;
        __syncthreads();
        Q4<CT> F = q_one<CT>();
        if (k > 0) {
            F = s_sq[0][c];
            for (int k2 = 1; k2 < k; ++k2) F = qmul(s_sq[k2][c], F);
        }
        Q4<CT> Rp = q_zero<CT>();
        if (k < K - 1) {
            Rp = s_sy[K - 1][c];
            for (int k2 = K - 2; k2 > k; --k2) Rp = qadd(s_sy[k2][c], qcmul(s_sq[k2][c], Rp));
        }
        const Q4<CT> A = qmul(Ql, F);

        // The tile's product (all K slices; wave 0 publishes it) and the
        // forward look-back for E, the prefix product before the tile.
        Q4<CT> Pt = q_one<CT>();
        if (wave == 0) {
            Pt = s_sq[0][c];
            for (int k2 = 1; k2 < K; ++k2) Pt = qmul(s_sq[k2][c], Pt);
        }
        // (No first-round prefetch: its value would be held across sweep 1,
        // and the tile's registers are full.)
        const Q4<CT> Et = fenwick_exclusive<ProductCarry<CT>, WC, NW>(af, chain, tile, Pt, wave == 0, wave, r, c,
                                                                      q_one<CT>(), false, s_nodes, s_ok, s_before);

        Q4<CT> Yg = q_zero<CT>();
        if (wave == 0) Yg = qcmul(Et, qadd(Yl, qcmul(Ql, Rp)));
        const Q4<CT> Sa = fenwick_exclusive<SumCarry<CT>, WC, NW>(a, chain, tc.pos, Yg, wave == 0, wave, r, c,
                                                                  q_zero<CT>(), false, s_nodes, s_ok, s_after);

        if (a.d_init != nullptr && tc.t0 == 0 && tc.col_ok) IO::store(a.d_init, tc.bi * a.M + tc.m, qadd(Yg, Sa));

        if (a.out != nullptr && tc.col_ok) {
            const CT nE = qnorm2(Et), nA = qnorm2(A);
            if (nE == CT(0) || nA == CT(0))
                __hip_atomic_fetch_or(&a.hdr[kHdrStatus], kStatusZeroPrefix, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            const Q4<CT> Z = qscale(qmul(Et, Sa), recip(nE));
            const Q4<CT> C = qmul(Et, IO::ct(init_raw));
            const Q4<CT> c0 = qmul(F, C);
            const Q4<CT> cm = qmul(A, C);
            const Q4<CT> G = qadd(IO::ct_fresh(dv[L - 1]), qadd(Rp, qscale(qmul(A, Z), recip(nA))));
            sweep2_store<IO, L>(a, tc, qv, dv, G, cm, c0);
        }
        __syncthreads();   // s_sq / s_sy are rewritten for the next chain
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
            qv[i] = (t0 + i < a.s) ? IO::load_stream(a.q, base + (t0 + i) * a.M) : IO::one_raw();
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
            if (a.out != nullptr) IO::store_stream(a.out, base + t * a.M, cm);
        }
    }
    if (a.fin != nullptr) reinterpret_cast<Q4<CT>*>(a.fin)[col] = cm;
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
    Q4<CT> S = q_zero<CT>();
    for (int64_t t0 = 0; t0 < a.s; t0 += U) {
        Raw qv[U], dv[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool ok = t0 + i < a.s;
            qv[i] = ok ? IO::load_stream(a.q, base + (t0 + i) * a.M) : IO::one_raw();
            dv[i] = ok ? IO::load_stream(a.d_cum, base + (t0 + i) * a.M) : IO::zero_raw();
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            P = qmul(IO::ct(qv[i]), P);
            S = qadd(S, qcmul(P, IO::ct(dv[i])));
        }
    }
    if (a.d_init != nullptr) IO::store(a.d_init, bi * a.M + m, S);
    if (a.out == nullptr) return;
    // Pass 2: the closed form step by step, S[t+1] = S[t] - conj(P_t) (x) d_t.
    Q4<CT> cm = IO::ct(IO::load(a.init, bi * a.M + m));   // cum[-1] = init
    P = q_one<CT>();
    bool zero = false;
    for (int64_t t0 = 0; t0 < a.s; t0 += U) {
        Raw qv[U], dv[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool ok = t0 + i < a.s;
            qv[i] = ok ? IO::load_stream(a.q, base + (t0 + i) * a.M) : IO::one_raw();
            dv[i] = ok ? IO::load_stream(a.d_cum, base + (t0 + i) * a.M) : IO::zero_raw();
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t t = t0 + i;
            if (t >= a.s) break;
            const Q4<CT> qq = IO::ct(qv[i]);
            P = qmul(qq, P);
            const CT nP = qnorm2(P);
            zero = zero || nP == CT(0);
            const Q4<CT> G = qscale(qmul(P, S), recip(nP));
            IO::store_stream(a.out, base + t * a.M, qmulc(G, cm));
            S = qsub(S, qcmul(P, IO::ct(dv[i])));
            cm = qmul(qq, cm);
        }
    }
    if (zero)
        __hip_atomic_fetch_or(&a.hdr[kHdrStatus], kStatusZeroPrefix, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reduce-then-scan, pass 2: one block per chain scans its tiles' aggregates
// into exclusive carries.  Thread (segment, column) walks a contiguous run of
// tiles for its column, loading them in batches so that the loads overlap;
// the runs' totals meet in LDS.  Forward: products in left-multiply order
// (later factor on the left), identity first.  Backward: plain sums (the
// tiles are already in reverse time order), zero first.
template <int WC>
constexpr int rscan_segments() { return WC >= 16 ? 1024 / WC : 64; }

template <typename CT, int WC, bool kProduct>
__global__ void __launch_bounds__(rscan_segments<WC>() * WC) rscan_kernel(KernelArgs a) {
    constexpr int NSEG = rscan_segments<WC>();
    constexpr int B = 8;
    __shared__ Q4<CT> s_run[NSEG][WC];
    const int c = threadIdx.x % WC, seg = threadIdx.x / WC;
    const int64_t chain = blockIdx.x;
    const int64_t per = (a.n_tiles + NSEG - 1) / NSEG;
    const int64_t lo = seg * per < a.n_tiles ? seg * per : a.n_tiles;
    const int64_t hi = lo + per < a.n_tiles ? lo + per : a.n_tiles;
    const Q4<CT> id = kProduct ? q_one<CT>() : q_zero<CT>();
    Q4<CT> run = id;
    for (int64_t i0 = lo; i0 < hi; i0 += B) {
        Q4<CT> v[B];
#pragma unroll
        for (int k = 0; k < B; ++k) v[k] = *rscan_agg<CT, WC>(a, chain, i0 + k < hi ? i0 + k : hi - 1, c);
#pragma unroll
        for (int k = 0; k < B; ++k)
            if (i0 + k < hi) run = kProduct ? qmul(v[k], run) : qadd(run, v[k]);
    }
    s_run[seg][c] = run;
    __syncthreads();
    Q4<CT> p = id;
    for (int k = 0; k < seg; ++k) p = kProduct ? qmul(s_run[k][c], p) : qadd(p, s_run[k][c]);
    for (int64_t i0 = lo; i0 < hi; i0 += B) {
        Q4<CT> v[B];
#pragma unroll
        for (int k = 0; k < B; ++k) v[k] = *rscan_agg<CT, WC>(a, chain, i0 + k < hi ? i0 + k : hi - 1, c);
#pragma unroll
        for (int k = 0; k < B; ++k) {
            if (i0 + k < hi) {
                *rscan_carry<CT, WC>(a, chain, i0 + k, c) = p;
                p = kProduct ? qmul(v[k], p) : qadd(p, v[k]);
            }
        }
    }
}

__global__ void bump_epoch_kernel(uint32_t* hdr) {
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(hdr + kHdrEpoch), uint64_t(1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// ------------------------------------------------------------------ launchers

template <class IO, int WC, int kMode>
hipError_t launch_fwd_mode(bool deep, const KernelArgs& a, hipStream_t st) {
    constexpr Geometry g = geometry_for(WC, IO::kDtype);
    static_assert(kCkptStride % g.fwd_l == 0 && kCkptStride % g.fwd_deep_l == 0,
                  "a forward slice must start on every saved boundary");
    KernelArgs args = a;
    void* params[] = {&args};
    const bool store = a.out != nullptr;
    const void* fn =
        deep ? (store ? reinterpret_cast<const void*>(&fwd_chunked_kernel<IO, WC, g.fwd_deep_l, g.fwd_nw, true, kMode>)
                      : reinterpret_cast<const void*>(&fwd_chunked_kernel<IO, WC, g.fwd_deep_l, g.fwd_nw, false, kMode>))
             : (store ? reinterpret_cast<const void*>(&fwd_chunked_kernel<IO, WC, g.fwd_l, g.fwd_nw, true, kMode>)
                      : reinterpret_cast<const void*>(&fwd_chunked_kernel<IO, WC, g.fwd_l, g.fwd_nw, false, kMode>));
    return hipLaunchKernel(fn, dim3(a.n_blocks), dim3(g.fwd_nw * 64), params, 0, st);
}

template <class IO, int WC, int kMode, bool kFinal = false>
hipError_t launch_bwd_mode(bool deep, const KernelArgs& a, hipStream_t st) {
    constexpr Geometry g = geometry_for(WC, IO::kDtype);
    static_assert(bwd_tile_steps(WC, IO::kDtype, false) % kCkptStride == 0, "backward tiles start on saved boundaries");
    static_assert(bwd_tile_steps(WC, IO::kDtype, true) % kCkptStride == 0, "backward tiles start on saved boundaries");
    KernelArgs args = a;
    void* params[] = {&args};
    const void* fn =
        deep ? reinterpret_cast<const void*>(&bwd_chunked_kernel<IO, WC, g.bwd_deep_l, g.bwd_nw, kMode, kFinal>)
             : reinterpret_cast<const void*>(&bwd_chunked_kernel<IO, WC, g.bwd_l, g.bwd_nw, kMode, kFinal>);
    return hipLaunchKernel(fn, dim3(a.n_blocks), dim3(g.bwd_nw * 64), params, 0, st);
}

template <class IO, int WC, bool kProduct>
hipError_t launch_rscan(const KernelArgs& a, hipStream_t st) {
    KernelArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&rscan_kernel<typename IO::CT, WC, kProduct>),
                           dim3(unsigned(a.n_chains)), dim3(rscan_segments<WC>() * WC), params, 0, st);
}

// One pass with either look-back (a.group != 0: the grouped one), or the
// three reduce-then-scan passes.
template <class IO, int WC>
hipError_t launch_fwd_wc(bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    if (!rscan)
        return a.group != 0 ? launch_fwd_mode<IO, WC, kGrouped>(deep, a, st)
                            : launch_fwd_mode<IO, WC, kLookback>(deep, a, st);
    hipError_t e = launch_fwd_mode<IO, WC, kAggregate>(deep, a, st);
    if (e == hipSuccess) e = launch_rscan<IO, WC, true>(a, st);
    if (e == hipSuccess) e = launch_fwd_mode<IO, WC, kFixup>(deep, a, st);
    return e;
}

template <class IO, int WC>
hipError_t launch_bwd_wc(bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    if (a.fin != nullptr) {
        if (rscan) return hipErrorInvalidValue;
        return a.group != 0 ? launch_bwd_mode<IO, WC, kGrouped, true>(deep, a, st)
                            : launch_bwd_mode<IO, WC, kLookback, true>(deep, a, st);
    }
    if (!rscan)
        return a.group != 0 ? launch_bwd_mode<IO, WC, kGrouped>(deep, a, st)
                            : launch_bwd_mode<IO, WC, kLookback>(deep, a, st);
    hipError_t e = launch_bwd_mode<IO, WC, kAggregate>(deep, a, st);
    if (e == hipSuccess) e = launch_rscan<IO, WC, false>(a, st);
    if (e == hipSuccess) e = launch_bwd_mode<IO, WC, kFixup>(deep, a, st);
    return e;
}

template <class IO>
hipError_t launch_fwd_io(int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    switch (wc) {
        case 64: return launch_fwd_wc<IO, 64>(deep, rscan, a, st);
        case 32: return launch_fwd_wc<IO, 32>(deep, rscan, a, st);
        case 16: return launch_fwd_wc<IO, 16>(deep, rscan, a, st);
        case 8: return launch_fwd_wc<IO, 8>(deep, rscan, a, st);
        case 4: return launch_fwd_wc<IO, 4>(deep, rscan, a, st);
        case 2: return launch_fwd_wc<IO, 2>(deep, rscan, a, st);
        case 1: return launch_fwd_wc<IO, 1>(deep, rscan, a, st);
        default: return hipErrorInvalidValue;
    }
}

// Backward column groups are at most 32 wide (the dispatcher's cap).
template <class IO>
hipError_t launch_bwd_io(int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    switch (wc) {
        case 32: return launch_bwd_wc<IO, 32>(deep, rscan, a, st);
        case 16: return launch_bwd_wc<IO, 16>(deep, rscan, a, st);
        case 8: return launch_bwd_wc<IO, 8>(deep, rscan, a, st);
        case 4: return launch_bwd_wc<IO, 4>(deep, rscan, a, st);
        case 2: return launch_bwd_wc<IO, 2>(deep, rscan, a, st);
        case 1: return launch_bwd_wc<IO, 1>(deep, rscan, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_chunked(int dtype, int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    return dtype == 0 ? launch_fwd_io<IoF32>(wc, deep, rscan, a, st) : launch_fwd_io<IoBF16>(wc, deep, rscan, a, st);
}

hipError_t launch_bwd_chunked(int dtype, int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st) {
    return dtype == 0 ? launch_bwd_io<IoF32>(wc, deep, rscan, a, st) : launch_bwd_io<IoBF16>(wc, deep, rscan, a, st);
}

namespace {

template <class IO, int WC>
const void* coresident_fn(bool deep) {
    constexpr Geometry g = geometry_for(WC, IO::kDtype);
    return deep ? reinterpret_cast<const void*>(&bwd_coresident_kernel<IO, WC, g.bwd_deep_l, g.bwd_nw>)
                : reinterpret_cast<const void*>(&bwd_coresident_kernel<IO, WC, g.bwd_l, g.bwd_nw>);
}

template <class IO>
const void* coresident_fn_io(int wc, bool deep) {
    switch (wc) {
        case 32: return coresident_fn<IO, 32>(deep);
        case 16: return coresident_fn<IO, 16>(deep);
        case 8: return coresident_fn<IO, 8>(deep);
        case 4: return coresident_fn<IO, 4>(deep);
        case 2: return coresident_fn<IO, 2>(deep);
        case 1: return coresident_fn<IO, 1>(deep);
        default: return nullptr;
    }
}

const void* coresident_kernel(int dtype, int wc, bool deep) {
    return dtype == 0 ? coresident_fn_io<IoF32>(wc, deep) : coresident_fn_io<IoBF16>(wc, deep);
}

int bwd_threads(int dtype, int wc) {
    const Geometry g = dtype == 0 ? geometry_for(wc, 0) : geometry_for(wc, 1);
    return g.bwd_nw * 64;
}

}  // namespace

int64_t coresident_blocks(int dtype, int wc, bool deep) {
    const void* fn = coresident_kernel(dtype, wc, deep);
    if (fn == nullptr) return 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, bwd_threads(dtype, wc), 0) != hipSuccess) return 0;
    return int64_t(per_cu) * cus;
}

hipError_t launch_bwd_coresident(int dtype, int wc, bool deep, const KernelArgs& a, hipStream_t st) {
    const void* fn = coresident_kernel(dtype, wc, deep);
    if (fn == nullptr) return hipErrorInvalidValue;
    KernelArgs args = a;
    void* params[] = {&args};
    return hipLaunchCooperativeKernel(fn, dim3(unsigned(a.n_coop * a.n_tiles)), dim3(bwd_threads(dtype, wc)), params, 0,
                                      st);
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

hipError_t launch_bump_epoch(uint32_t* hdr, hipStream_t st) {
    void* params[] = {&hdr};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bump_epoch_kernel), dim3(1), dim3(64), params, 0, st);
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
