// qc_scan.hip -- gfx950 kernels and C-ABI entry points of the scan VJP in
// include/qc_scan.h: a forward scan, the VJP from the whole saved trajectory,
// and the VJP from k snapshots driven by a host-built schedule.
//
// One column (one (b, m) sequence) per thread, sequential in t, float64
// arithmetic on float32 storage.  Consecutive threads own consecutive m, so
// every step's loads and stores are contiguous across a wave (4 bytes per
// lane for the add body, one 16-byte quaternion for the quaternion body).
// Steps inside an advance or a trajectory sweep are processed in groups of
// kGroup whose loads are all issued before the group's arithmetic: the
// memory latency is hidden by the loads in flight rather than by occupancy
// alone.
#include "qc_internal.hpp"
#include "qc_scan.h"
#include "quat_cumprod.h"

#include <hip/hip_runtime.h>

namespace qc {
namespace {

constexpr int kScanBlock = 256;
constexpr int kGroup = 8;

// ---------------------------------------------------------------- bodies
//
// f(c, x) and its VJP (J_c^T g, J_x^T g).  The quaternion body is the
// left-multiplying cumulative product, whose per-factor VJPs are those of the
// burn-mamba page's "Gradient math": for y = a (x) b, the cotangent of a is
// y' (x) conj(b) and that of b is conj(a) (x) y'.

struct BodyAdd {
    static constexpr int W = 1;
    struct V { double v[1]; };
    __device__ static V step(const V& c, const V& x) { return V{{c.v[0] + x.v[0]}}; }
    __device__ static void vjp(const V&, const V&, const V& g, V* dc, V* dx) {
        *dc = g;
        *dx = g;
    }
};

struct BodyQuat {
    static constexpr int W = 4;
    struct V { double v[4]; };
    // Hamilton product a (x) b, components (w, x, y, z).
    __device__ static V mul(const V& a, const V& b) {
        V r;
        r.v[0] = a.v[0] * b.v[0] - a.v[1] * b.v[1] - a.v[2] * b.v[2] - a.v[3] * b.v[3];
        r.v[1] = a.v[0] * b.v[1] + a.v[1] * b.v[0] + a.v[2] * b.v[3] - a.v[3] * b.v[2];
        r.v[2] = a.v[0] * b.v[2] - a.v[1] * b.v[3] + a.v[2] * b.v[0] + a.v[3] * b.v[1];
        r.v[3] = a.v[0] * b.v[3] + a.v[1] * b.v[2] - a.v[2] * b.v[1] + a.v[3] * b.v[0];
        return r;
    }
    __device__ static V conj(const V& a) { return V{{a.v[0], -a.v[1], -a.v[2], -a.v[3]}}; }
    __device__ static V step(const V& c, const V& x) { return mul(x, c); }
    __device__ static void vjp(const V& c, const V& x, const V& g, V* dc, V* dx) {
        *dc = mul(conj(x), g);
        *dx = mul(g, conj(c));
    }
};

// Storage access: element e of a float32 tensor of width W.
template <class B>
struct Io;

template <>
struct Io<BodyAdd> {
    using Raw = float;
    __device__ static Raw load(const float* p, int64_t e) { return p[e]; }
    __device__ static Raw load_stream(const float* p, int64_t e) { return __builtin_nontemporal_load(p + e); }
    __device__ static BodyAdd::V widen(Raw r) { return BodyAdd::V{{double(r)}}; }
    __device__ static void store(float* p, int64_t e, const BodyAdd::V& v) {
        __builtin_nontemporal_store(float(v.v[0]), p + e);
    }
};

typedef float scan_f32x4 __attribute__((ext_vector_type(4)));

template <>
struct Io<BodyQuat> {
    using Raw = scan_f32x4;
    __device__ static Raw load(const float* p, int64_t e) { return reinterpret_cast<const Raw*>(p)[e]; }
    __device__ static Raw load_stream(const float* p, int64_t e) {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(p) + e);
    }
    __device__ static BodyQuat::V widen(Raw r) { return BodyQuat::V{{double(r.x), double(r.y), double(r.z), double(r.w)}}; }
    __device__ static void store(float* p, int64_t e, const BodyQuat::V& v) {
        const Raw r = {float(v.v[0]), float(v.v[1]), float(v.v[2]), float(v.v[3])};
        __builtin_nontemporal_store(r, reinterpret_cast<Raw*>(p) + e);
    }
};

template <class B>
__device__ typename B::V zero_v() {
    typename B::V z;
#pragma unroll
    for (int i = 0; i < B::W; ++i) z.v[i] = 0.0;
    return z;
}

template <class B>
__device__ typename B::V add_v(const typename B::V& a, const typename B::V& b) {
    typename B::V r;
#pragma unroll
    for (int i = 0; i < B::W; ++i) r.v[i] = a.v[i] + b.v[i];
    return r;
}

// Snapshots: [k][n_cols][W] doubles.
template <class B>
__device__ void snap_store(double* snaps, int64_t n_cols, int slot, int64_t col, const typename B::V& v) {
    double* p = snaps + (int64_t(slot) * n_cols + col) * B::W;
#pragma unroll
    for (int i = 0; i < B::W; ++i) p[i] = v.v[i];
}

template <class B>
__device__ typename B::V snap_load(const double* snaps, int64_t n_cols, int slot, int64_t col) {
    const double* p = snaps + (int64_t(slot) * n_cols + col) * B::W;
    typename B::V v;
#pragma unroll
    for (int i = 0; i < B::W; ++i) v.v[i] = p[i];
    return v;
}

struct ScanArgs {
    const float* xs;
    const float* init;
    const float* ys;        // trajectory (backward from the trajectory)
    const float* up;
    float* out;             // ys (forward) or d_xs (backward); may be null
    float* d_init;          // may be null
    const int32_t* sched;   // device schedule records (may be null in the forward)
    int64_t n_actions, start;
    double* snaps;
    int32_t k;
    uint32_t* status;
    int64_t s, M, n_cols;
};

struct Col {
    int64_t col, base;   // base: element index of (bi, t = 0, m)
};

// Blocks are dealt to kSlices near-equal slices of the column range in turn:
// block b takes position b / kSlices of slice b % kSlices (slices of
// q + 1 blocks first, then of q, so the map is a bijection of the grid).  The
// blocks resident at once then cover kSlices separate stretches of each row
// instead of one contiguous stretch: measured +16% on both kernels for 2^20
// quaternion columns in one 16 MiB row; results are unchanged.
constexpr int64_t kSlices = 16;

__device__ int64_t spread_block(int64_t b, int64_t nb) {
    const int64_t q = nb / kSlices, r = nb % kSlices, i = b % kSlices, k = b / kSlices;
    return i * q + (i < r ? i : r) + k;
}

__device__ Col column(const ScanArgs& a) {
    const int64_t col = spread_block(blockIdx.x, gridDim.x) * kScanBlock + threadIdx.x;
    const int64_t bi = col / a.M, m = col - bi * a.M;
    return Col{col, bi * a.s * a.M + m};
}

// Applies steps t0 .. t1-1 to c, writing every new carry to ys if non-null.
template <class B>
__device__ typename B::V advance(const ScanArgs& a, const Col& cc, typename B::V c, int64_t t0, int64_t t1, float* ys) {
    using IO = Io<B>;
    int64_t t = t0;
    for (; t + kGroup <= t1; t += kGroup) {
        typename IO::Raw x[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) x[i] = IO::load(a.xs, cc.base + (t + i) * a.M);
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            c = B::step(c, IO::widen(x[i]));
            if (ys) IO::store(ys, cc.base + (t + i) * a.M, c);
        }
    }
    for (; t < t1; ++t) {
        c = B::step(c, IO::widen(IO::load(a.xs, cc.base + t * a.M)));
        if (ys) IO::store(ys, cc.base + t * a.M, c);
    }
    return c;
}

// Reads a schedule record; every lane reads the same one.
__device__ int4 record(const int32_t* sched, int64_t i) {
    const int4 r = reinterpret_cast<const int4*>(sched)[i];
    return make_int4(__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                     __builtin_amdgcn_readfirstlane(r.z), 0);
}

__device__ void flag_bad(const ScanArgs& a) {
    if (a.status) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- kernels

template <class B>
__global__ void __launch_bounds__(kScanBlock) scan_fwd_kernel(ScanArgs a) {
    const Col cc = column(a);
    if (cc.col >= a.n_cols) return;
    using IO = Io<B>;
    typename B::V c = IO::widen(IO::load(a.init, cc.col));
    int64_t pos = 0;
    if (a.sched) {
        for (int64_t i = 0; i < a.start; ++i) {
            const int4 r = record(a.sched, i);
            if (r.x == QC_SCAN_STORE && r.y >= 0 && r.y < a.k) {
                snap_store<B>(a.snaps, a.n_cols, r.y, cc.col, c);
            } else if (r.x == QC_SCAN_ADVANCE && r.y == pos && r.z >= r.y && r.z <= a.s) {
                c = advance<B>(a, cc, c, r.y, r.z, a.out);
                pos = r.z;
            } else {
                flag_bad(a);
                return;
            }
        }
    }
    if (a.out) advance<B>(a, cc, c, pos, a.s, a.out);
}

template <class B>
__global__ void __launch_bounds__(kScanBlock) scan_bwd_trajectory_kernel(ScanArgs a) {
    const Col cc = column(a);
    if (cc.col >= a.n_cols) return;
    using IO = Io<B>;
    typename B::V g = zero_v<B>(), dc, dx;
    int64_t t = a.s - 1;
    // Groups of kGroup steps, loads first: x[t], u[t] and c[t-1] for each.
    for (; t >= kGroup; t -= kGroup) {   // steps t .. t-kGroup+1, all >= 1
        typename IO::Raw x[kGroup], u[kGroup], cp[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int64_t e = cc.base + (t - i) * a.M;
            x[i] = IO::load(a.xs, e);
            u[i] = IO::load_stream(a.up, e);
            cp[i] = IO::load_stream(a.ys, e - a.M);
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            g = add_v<B>(g, IO::widen(u[i]));
            B::vjp(IO::widen(cp[i]), IO::widen(x[i]), g, &dc, &dx);
            if (a.out) IO::store(a.out, cc.base + (t - i) * a.M, dx);
            g = dc;
        }
    }
    for (; t >= 0; --t) {
        const int64_t e = cc.base + t * a.M;
        const typename B::V cprev = t > 0 ? IO::widen(IO::load_stream(a.ys, e - a.M))
                                          : IO::widen(IO::load(a.init, cc.col));
        g = add_v<B>(g, IO::widen(IO::load_stream(a.up, e)));
        B::vjp(cprev, IO::widen(IO::load(a.xs, e)), g, &dc, &dx);
        if (a.out) IO::store(a.out, e, dx);
        g = dc;
    }
    if (a.d_init) IO::store(a.d_init, cc.col, g);
}

template <class B>
__global__ void __launch_bounds__(kScanBlock) scan_bwd_checkpointed_kernel(ScanArgs a) {
    const Col cc = column(a);
    if (cc.col >= a.n_cols) return;
    using IO = Io<B>;
    typename B::V c = IO::widen(IO::load(a.init, cc.col));
    if (a.start > 0) {
        // Resume after the forward sweep's part: the carry is the last snapshot it took.
        const int4 r = record(a.sched, a.start - 1);
        if (r.x != QC_SCAN_STORE || r.y < 0 || r.y >= a.k) {
            flag_bad(a);
            return;
        }
        c = snap_load<B>(a.snaps, a.n_cols, r.y, cc.col);
    }
    typename B::V g = zero_v<B>(), dc, dx;
    for (int64_t i = a.start; i < a.n_actions; ++i) {
        const int4 r = record(a.sched, i);
        if (r.x == QC_SCAN_STORE && r.y >= 0 && r.y < a.k) {
            snap_store<B>(a.snaps, a.n_cols, r.y, cc.col, c);
        } else if (r.x == QC_SCAN_LOAD && r.y >= 0 && r.y < a.k) {
            c = snap_load<B>(a.snaps, a.n_cols, r.y, cc.col);
        } else if (r.x == QC_SCAN_ADVANCE && r.y >= 0 && r.z >= r.y && r.z <= a.s) {
            c = advance<B>(a, cc, c, r.y, r.z, nullptr);
        } else if (r.x == QC_SCAN_REVERSE && r.y >= 0 && r.y < a.s) {
            const int64_t e = cc.base + int64_t(r.y) * a.M;
            g = add_v<B>(g, IO::widen(IO::load_stream(a.up, e)));
            B::vjp(c, IO::widen(IO::load(a.xs, e)), g, &dc, &dx);
            if (a.out) IO::store(a.out, e, dx);
            g = dc;
        } else {
            flag_bad(a);
            return;
        }
    }
    if (a.d_init) IO::store(a.d_init, cc.col, g);
}

template <class B>
hipError_t launch(void (*kern)(ScanArgs), const ScanArgs& a, hipStream_t st) {
    ScanArgs args = a;
    void* params[] = {&args};
    const unsigned blocks = unsigned((a.n_cols + kScanBlock - 1) / kScanBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(blocks), dim3(kScanBlock), params, 0, st);
}

// ------------------------------------------------------------ validation

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxBlocks = int64_t(1) << 31;

struct Dims {
    int w;
    int64_t n_cols, N;   // columns, elements per [b][s][m] tensor
};

int check_dims(int32_t body, int64_t b, int64_t s, int64_t m, Dims* d) {
    d->w = qc_scan_width(body);
    if (d->w == 0) return QC_ERR_DTYPE;
    if (b < 1 || s < 1 || m < 1 || s >= (int64_t(1) << 31)) return QC_ERR_SHAPE;
    if (m > kMaxElems / b) return QC_ERR_SHAPE;
    d->n_cols = b * m;
    if (s > kMaxElems / d->n_cols) return QC_ERR_SHAPE;
    if ((d->n_cols + kScanBlock - 1) / kScanBlock >= kMaxBlocks) return QC_ERR_SHAPE;
    d->N = d->n_cols * s;
    return QC_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Span {
    const void* p;
    size_t n;
};

bool overlaps(Span x, Span y) {
    if (!x.p || !y.p || !x.n || !y.n) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x.p), b = reinterpret_cast<uintptr_t>(y.p);
    return a < b + y.n && b < a + x.n;
}

// Outputs (first n_out spans) against everything else and each other.
bool any_overlap(const Span* s, int n_out, int n) {
    for (int i = 0; i < n_out; ++i)
        for (int j = 0; j < n; ++j)
            if (i != j && overlaps(s[i], s[j])) return true;
    return false;
}

template <class F>
hipError_t dispatch(int32_t body, F&& f) {
    return body == QC_SCAN_BODY_ADD ? f(BodyAdd{}) : f(BodyQuat{});
}

}  // namespace
}  // namespace qc

using qc::BodyAdd;
using qc::BodyQuat;

extern "C" {

int qc_scan_fwd(int32_t body, const float* xs, const float* init, float* ys, int64_t b, int64_t s, int64_t m,
                const int32_t* schedule, int64_t bwd_start, double* snaps, int32_t k, void* stream) {
    qc::Dims d;
    int rc = qc::check_dims(body, b, s, m, &d);
    if (rc != QC_OK) return rc;
    if (!xs || !init) return QC_ERR_NULL;
    if (!ys && !schedule) return QC_ERR_NULL;
    if (schedule && (!snaps || k < 1 || k > 4096)) return QC_ERR_WORKSPACE;
    if (schedule && (bwd_start < 1 || bwd_start > qc_scan_schedule_capacity(s))) return QC_ERR_SHAPE;
    const size_t eb = size_t(d.w) * 4;
    if (!qc::aligned(xs, eb) || !qc::aligned(init, eb) || (ys && !qc::aligned(ys, eb))) return QC_ERR_ALIGN;
    if ((schedule && !qc::aligned(schedule, 16)) || (snaps && !qc::aligned(snaps, 16))) return QC_ERR_ALIGN;
    const size_t big = size_t(d.N) * eb, snap_bytes = schedule ? size_t(k) * d.n_cols * d.w * 8 : 0;
    const qc::Span sp[] = {{ys, big}, {snaps, snap_bytes}, {xs, big}, {init, size_t(d.n_cols) * eb},
                           {schedule, schedule ? size_t(bwd_start) * 16 : 0}};
    if (qc::any_overlap(sp, 2, 5)) return QC_ERR_ALIAS;
    qc::ScanArgs a{};
    a.xs = xs; a.init = init; a.out = ys; a.sched = schedule; a.start = schedule ? bwd_start : 0;
    a.snaps = snaps; a.k = k; a.s = s; a.M = m; a.n_cols = d.n_cols;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = qc::dispatch(body, [&](auto bd) {
        using B = decltype(bd);
        return qc::launch<B>(&qc::scan_fwd_kernel<B>, a, st);
    });
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

int qc_scan_bwd_trajectory(int32_t body, const float* xs, const float* init, const float* ys, const float* upstream,
                           float* d_xs, float* d_init, int64_t b, int64_t s, int64_t m, void* stream) {
    qc::Dims d;
    int rc = qc::check_dims(body, b, s, m, &d);
    if (rc != QC_OK) return rc;
    if (!xs || !init || !ys || !upstream) return QC_ERR_NULL;
    if (!d_xs && !d_init) return QC_OK;
    const size_t eb = size_t(d.w) * 4;
    for (const void* p : {static_cast<const void*>(xs), static_cast<const void*>(init), static_cast<const void*>(ys),
                          static_cast<const void*>(upstream), static_cast<const void*>(d_xs),
                          static_cast<const void*>(d_init)})
        if (p && !qc::aligned(p, eb)) return QC_ERR_ALIGN;
    const size_t big = size_t(d.N) * eb, small = size_t(d.n_cols) * eb;
    const qc::Span sp[] = {{d_xs, big}, {d_init, small}, {xs, big}, {init, small}, {ys, big}, {upstream, big}};
    if (qc::any_overlap(sp, 2, 6)) return QC_ERR_ALIAS;
    qc::ScanArgs a{};
    a.xs = xs; a.init = init; a.ys = ys; a.up = upstream; a.out = d_xs; a.d_init = d_init;
    a.s = s; a.M = m; a.n_cols = d.n_cols;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = qc::dispatch(body, [&](auto bd) {
        using B = decltype(bd);
        return qc::launch<B>(&qc::scan_bwd_trajectory_kernel<B>, a, st);
    });
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

int qc_scan_bwd_checkpointed(int32_t body, const float* xs, const float* init, const float* upstream, float* d_xs,
                             float* d_init, int64_t b, int64_t s, int64_t m, const int32_t* schedule,
                             int64_t n_actions, int64_t start, double* snaps, int32_t k, uint32_t* status,
                             void* stream) {
    qc::Dims d;
    int rc = qc::check_dims(body, b, s, m, &d);
    if (rc != QC_OK) return rc;
    if (!xs || !init || !upstream || !schedule) return QC_ERR_NULL;
    if (!d_xs && !d_init) return QC_OK;
    if (!snaps || k < 1 || k > 4096) return QC_ERR_WORKSPACE;
    if (n_actions < 1 || n_actions > qc_scan_schedule_capacity(s) || start < 0 || start >= n_actions)
        return QC_ERR_SHAPE;
    const size_t eb = size_t(d.w) * 4;
    for (const void* p : {static_cast<const void*>(xs), static_cast<const void*>(init),
                          static_cast<const void*>(upstream), static_cast<const void*>(d_xs),
                          static_cast<const void*>(d_init)})
        if (p && !qc::aligned(p, eb)) return QC_ERR_ALIGN;
    if (!qc::aligned(schedule, 16) || !qc::aligned(snaps, 16) || (status && !qc::aligned(status, 4)))
        return QC_ERR_ALIGN;
    const size_t big = size_t(d.N) * eb, small = size_t(d.n_cols) * eb;
    const qc::Span sp[] = {{d_xs, big},      {d_init, small}, {snaps, size_t(k) * d.n_cols * d.w * 8},
                           {status, 4},      {xs, big},       {init, small},
                           {upstream, big},  {schedule, size_t(n_actions) * 16}};
    if (qc::any_overlap(sp, 4, 8)) return QC_ERR_ALIAS;
    qc::ScanArgs a{};
    a.xs = xs; a.init = init; a.up = upstream; a.out = d_xs; a.d_init = d_init;
    a.sched = schedule; a.n_actions = n_actions; a.start = start; a.snaps = snaps; a.k = k; a.status = status;
    a.s = s; a.M = m; a.n_cols = d.n_cols;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = qc::dispatch(body, [&](auto bd) {
        using B = decltype(bd);
        return qc::launch<B>(&qc::scan_bwd_checkpointed_kernel<B>, a, st);
    });
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}

}  // extern "C"
