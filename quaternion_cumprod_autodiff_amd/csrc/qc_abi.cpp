// qc_abi.cpp -- C ABI of the quaternion cumulative-product scan (see
// include/quat_cumprod.h): argument validation, path choice, workspace
// layout and kernel launches on the caller's stream.
//
// All validation happens before the first HIP call, so a rejected call
// touches no device state.
#include "quat_cumprod.h"
#include "qc_internal.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <tuple>

namespace {

using qc::kCkptStride;

thread_local std::string g_last_hip_error;

// Epochs enter the check word of every carry slot a launch writes.  The
// 64-bit counter never wraps in practice, so a slot left by an earlier launch
// of this process can never carry the current epoch; it starts at a random
// value so that slots another process left in recycled memory are not
// expected to match either.
uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        return (static_cast<uint64_t>(rd()) << 32) ^ static_cast<uint64_t>(rd());
    }()};
    uint64_t e;
    do {
        e = counter.fetch_add(1, std::memory_order_relaxed);
    } while (e == 0);   // 0 tells the kernels to read the epoch from the workspace header
    return e;
}

int hip_fail(hipError_t e) {
    g_last_hip_error = hipGetErrorString(e);
    return QC_ERR_HIP;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;   // quaternions per tensor
constexpr size_t kAlignWs = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Chunked-path geometry of one kernel (forward or backward).
struct Tiling {
    int wc = 0;               // columns per group
    int64_t n_cg = 0;         // groups per batch entry
    int64_t n_chains = 0;     // b * n_cg
    bool deep = false;        // the deep slice length (few chains)
    int64_t n_tiles = 0;      // tiles per chain
    int64_t group = 0;        // grouped look-back: tiles per group, about sqrt(n_tiles)
    int64_t n_groups = 0;     // groups per chain
    bool grouped = false;     // AUTO takes the grouped look-back
};

struct Plan {
    int64_t b = 0, s = 0, M = 0, N = 0;
    int dtype = 0;
    size_t io_bytes = 0;      // bytes per stored quaternion
    size_t ct_bytes = 0;      // bytes per internal quaternion
    size_t slot_bytes = 0;    // bytes per carry slot (value words + check word)
    size_t pair_slot_bytes = 0;   // the same for the final-carry backward's (product, share) pairs
    Tiling fwd, bwd;
    int64_t n_ck = 0;
    size_t ckpt_bytes = 0;
    size_t final_bytes = 0;   // saved final carries (QC_SAVED_FINAL)
    size_t off_desc = 0, off_ckpt = 0, ws_bytes = 0;
    int64_t n_cols = 0;
};

// Widest column group each kernel uses.  Groups of 32 columns make 4-wave
// blocks on wide rows, so that (at 3 waves per SIMD for these register
// counts) three blocks share a compute unit and overlap their load, compute
// and carry-wait phases.
constexpr int kFwdMaxWc = 32;
constexpr int kBwdMaxWc = 32;
static_assert(kBwdMaxWc <= 32, "backward kernels exist for column groups of at most 32");

// The forward can also take 64-column groups with half-height tiles (same
// tile size, 1 KiB per row read instead of 512 B, measured a few percent
// faster), but that doubles the tiles per chain.  It is used only while
// there are at least this many chains, i.e. few tiles of each chain in
// flight at once; deep chains keep 32-column groups and their shorter
// carry look-backs.
constexpr int kFwdWideWc = 64;
constexpr int64_t kFwdWideMinChains = 64;

int column_group_width(int64_t M, int cap) {
    if (M >= cap) return cap;
    int w = 1;
    while (w < M) w <<= 1;
    return w;
}

// Deep (twice-as-tall) tiles when there are fewer chains than this: each
// chain then has many tiles in flight at once, and halving the look-backs per
// byte outweighs the lower occupancy.  The backward takes them at any depth
// (drift -2% per step, medium -5%, long-seq -6%); the forward only when its
// chains are also long (drift -2.5%, long-seq -4%; medium's 16-tile chains
// were 2% slower).  With many chains (the headline has 128 and 256) neither
// kernel does.
constexpr int64_t kDeepMaxChains = 64;
constexpr int64_t kFwdDeepMinTiles = 64;

// The grouped look-back replaces the Fenwick one where a launch's tiles are
// about as many as the chip holds at once (so most of a chain waits on its
// look-back at the same time, and the Fenwick query's log2(tiles) round trips
// are exposed) and its chains are long enough for the depth to matter.
// Measured per step: long-seq -4.5%, medium -2%.
constexpr int64_t kGroupedMaxTiles = 2048;
constexpr int64_t kGroupedMinTiles = 16;

Tiling make_tiling(int64_t b, int64_t s, int64_t M, int cap, int dtype, bool backward) {
    Tiling t;
    t.wc = column_group_width(M, cap);
    t.n_cg = (M + t.wc - 1) / t.wc;
    t.n_chains = b * t.n_cg;
    if (backward) {
        t.deep = t.n_chains < kDeepMaxChains;
    } else {
        const int64_t steps = qc::fwd_tile_steps(t.wc, dtype, false);
        t.deep = t.n_chains < kDeepMaxChains && (s + steps - 1) / steps >= kFwdDeepMinTiles;
    }
    const int64_t steps = backward ? qc::bwd_tile_steps(t.wc, dtype, t.deep) : qc::fwd_tile_steps(t.wc, dtype, t.deep);
    t.n_tiles = (s + steps - 1) / steps;
    t.group = 1;
    while (t.group * t.group < t.n_tiles) ++t.group;
    t.n_groups = (t.n_tiles + t.group - 1) / t.group;
    t.grouped = t.n_chains * t.n_tiles <= kGroupedMaxTiles && t.n_tiles >= kGroupedMinTiles;
    return t;
}

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a <= limit / b; }

int make_plan(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype, Plan* p) {
    if (dtype != QC_DTYPE_F32 && dtype != QC_DTYPE_BF16) return QC_ERR_DTYPE;
    if (b < 1 || s < 1 || h < 1 || j < 1) return QC_ERR_SHAPE;
    if (!mul_ok(h, j, int64_t(1) << 31)) return QC_ERR_SHAPE;
    const int64_t M = h * j;
    if (!mul_ok(b, M, int64_t(1) << 31)) return QC_ERR_SHAPE;
    if (!mul_ok(b * M, s, kMaxElems)) return QC_ERR_SHAPE;
    p->b = b; p->s = s; p->M = M; p->N = b * s * M; p->dtype = dtype;
    p->io_bytes = dtype == QC_DTYPE_F32 ? 16 : 8;
    p->ct_bytes = dtype == QC_DTYPE_F32 ? 32 : 16;
    p->slot_bytes = dtype == QC_DTYPE_F32 ? 40 : 24;
    p->pair_slot_bytes = dtype == QC_DTYPE_F32 ? 72 : 40;
    p->n_cols = b * M;
    p->fwd = make_tiling(b, s, M, kFwdMaxWc, dtype, false);
    if (M >= kFwdWideWc && b * ((M + kFwdWideWc - 1) / kFwdWideWc) >= kFwdWideMinChains)
        p->fwd = make_tiling(b, s, M, kFwdWideWc, dtype, false);
    p->bwd = make_tiling(b, s, M, kBwdMaxWc, dtype, true);
    // One block per tile; the grid's work-item count is a 32-bit quantity
    // (blocks have at most 512 threads).
    const int64_t max_blocks = int64_t(1) << 22;
    if (!mul_ok(p->fwd.n_chains, p->fwd.n_tiles, max_blocks)) return QC_ERR_SHAPE;
    if (!mul_ok(p->bwd.n_chains, p->bwd.n_tiles, max_blocks)) return QC_ERR_SHAPE;
    if ((p->n_cols + qc::kColumnBlock - 1) / qc::kColumnBlock > max_blocks) return QC_ERR_SHAPE;
    p->n_ck = (s + kCkptStride - 1) / kCkptStride;
    p->ckpt_bytes = size_t(b) * size_t(p->n_ck) * size_t(M) * p->ct_bytes;
    p->final_bytes = size_t(p->n_cols) * p->ct_bytes;
    // The carry region holds the look-back's slots (one node per tile, then
    // the grouped look-back's group nodes), or the reduce-then-scan variant's
    // tile aggregates and scanned carries (one internal quaternion each).
    const size_t tiles_fwd = size_t(p->fwd.n_chains * p->fwd.n_tiles) * size_t(p->fwd.wc);
    const size_t tiles_bwd = size_t(p->bwd.n_chains * p->bwd.n_tiles) * size_t(p->bwd.wc);
    const size_t nodes_fwd = tiles_fwd + size_t(p->fwd.n_chains * p->fwd.n_groups) * size_t(p->fwd.wc);
    const size_t nodes_bwd = tiles_bwd + size_t(p->bwd.n_chains * p->bwd.n_groups) * size_t(p->bwd.wc);
    // The co-resident leaves-only backward keeps two sets of tile nodes, one
    // per look-back; the final-carry backward's nodes hold pairs.
    const size_t look = std::max(std::max(std::max(nodes_fwd, nodes_bwd), 2 * tiles_bwd) * p->slot_bytes,
                                 nodes_bwd * p->pair_slot_bytes);
    const size_t agg = 2 * (tiles_fwd > tiles_bwd ? tiles_fwd : tiles_bwd) * p->ct_bytes;
    const size_t desc = look > agg ? look : agg;
    p->off_desc = round_up(size_t(qc::kHdrWords) * 4, kAlignWs);
    p->off_ckpt = round_up(p->off_desc + desc, kAlignWs);
    p->ws_bytes = round_up(p->off_ckpt + p->ckpt_bytes, kAlignWs);
    return QC_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

struct Range {
    const void* p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Ranges flagged as outputs must be disjoint from every other range.
bool any_alias(const Range* r, const bool* is_out, int n) {
    for (int i = 0; i < n; ++i)
        for (int k = i + 1; k < n; ++k)
            if ((is_out[i] || is_out[k]) && overlap(r[i], r[k])) return true;
    return false;
}

struct Options {
    int path = QC_PATH_AUTO;
    int lookback = QC_LOOKBACK_AUTO;
    int leaves = QC_LEAVES_AUTO;
    int saved = QC_SAVED_BOUNDARY;
};

int check_options(const qc_options* o, Options* out) {
    *out = Options{};
    if (!o) return QC_OK;
    if (o->path < QC_PATH_AUTO || o->path > QC_PATH_RSCAN) return QC_ERR_OPTION;
    if (o->lookback < QC_LOOKBACK_AUTO || o->lookback > QC_LOOKBACK_GROUPED) return QC_ERR_OPTION;
    if (o->leaves < QC_LEAVES_AUTO || o->leaves > QC_LEAVES_CORESIDENT) return QC_ERR_OPTION;
    if (o->saved < QC_SAVED_BOUNDARY || o->saved > QC_SAVED_FINAL) return QC_ERR_OPTION;
    for (int i = 0; i < 4; ++i)
        if (o->reserved[i] != 0) return QC_ERR_OPTION;
    out->path = o->path;
    out->lookback = o->lookback;
    out->leaves = o->leaves;
    out->saved = o->saved;
    return QC_OK;
}

// Size of the ckpt buffer of the kind o.saved names.
size_t saved_bytes(const Plan& p, const Options& o) {
    return o.saved == QC_SAVED_FINAL ? p.final_bytes : p.ckpt_bytes;
}

// The column path wins the forward when enough columns exist to fill the
// chip with one lane per column; the backward always prefers the chunked path
// (it reads q and d_cum once instead of twice).
constexpr int64_t kColumnPathMinColumns = int64_t(1) << 18;

qc::KernelArgs base_args(const Plan& p, void* ws, const Tiling& tl, int lookback = QC_LOOKBACK_AUTO) {
    qc::KernelArgs a{};
    a.b = p.b; a.s = p.s; a.M = p.M; a.n_ck = p.n_ck;
    a.n_cg = tl.n_cg; a.n_chains = tl.n_chains; a.n_tiles = tl.n_tiles;
    const bool grouped = lookback == QC_LOOKBACK_GROUPED || (lookback == QC_LOOKBACK_AUTO && tl.grouped);
    a.group = grouped ? tl.group : 0;
    a.n_groups = grouped ? tl.n_groups : 0;
    a.n_blocks = uint32_t(tl.n_chains * tl.n_tiles);
    a.hdr = reinterpret_cast<uint32_t*>(ws);
    a.desc = static_cast<char*>(ws) + p.off_desc;
    a.spin_limit = qc::kSpinLimit;
    return a;
}

// A launch captured in a HIP graph is replayed with the same arguments, so a
// host-chosen epoch would repeat and a replay could accept the carries of the
// previous one.  Captured launches therefore bump a counter in the workspace
// header (one-thread kernel, captured too) and pass epoch 0, which makes the
// kernels read the counter: every replay gets a fresh epoch.
int set_epoch(qc::KernelArgs* a, hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return hip_fail(e);
    if (cs == hipStreamCaptureStatusNone) {
        a->epoch = next_epoch();
        return QC_OK;
    }
    a->epoch = 0;
    e = qc::launch_bump_epoch(a->hdr, st);
    return e == hipSuccess ? QC_OK : hip_fail(e);
}

qc::KernelArgs column_args(const Plan& p, void* ws) {
    qc::KernelArgs a = base_args(p, ws, p.fwd);
    a.n_tiles = 1;
    a.n_blocks = uint32_t((p.n_cols + qc::kColumnBlock - 1) / qc::kColumnBlock);
    return a;
}

// The reduce-then-scan variant (three passes: tile aggregates, a scan of them,
// a fix-up that re-reads the tile's inputs) runs only when asked for.  It has
// no cross-block waits, but moves one more read of the inputs than the
// look-back, and on the long single-chain shapes where its waits-free passes
// could pay it measured slower than the look-back, so AUTO never takes it.
bool use_rscan(int path) { return path == QC_PATH_RSCAN; }

// Chains the co-resident backward can hold at once on the current device
// (occupancy of its kernel, cached per device and instance).
int64_t coresident_groups(const Plan& p) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, bool>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const auto key = std::make_tuple(dev, p.dtype, p.bwd.wc, p.bwd.deep);
    int64_t blocks = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) {
            blocks = it->second;
        } else {
            blocks = qc::coresident_blocks(p.dtype, p.bwd.wc, p.bwd.deep);
            cache[key] = blocks;
        }
    }
    return std::min(blocks / p.bwd.n_tiles, p.bwd.n_chains);
}

// Launches the co-resident leaves-only backward if the options and the shape
// allow it; *done tells whether it did.  It runs only when asked for
// (QC_LEAVES_CORESIDENT), outside graph capture, and when at least one chain
// fits on the device at once.  It reads q once, but each group of blocks
// walks its chains in lockstep with two look-backs per chain, which the other
// groups' streaming does not hide: measured slower than the pre-pass at every
// workload (headline backward 613 us against 392, medium 45.5 against 34.5,
// drift 781 against 423), so AUTO keeps the pre-pass.
int try_bwd_coresident(const Plan& p, const Options& o, const void* q, const void* init, const void* d_cum,
                       void* d_q, void* d_init, void* ws, hipStream_t st, bool* done) {
    *done = false;
    if (o.leaves != QC_LEAVES_CORESIDENT || use_rscan(o.path)) return QC_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(st, &cs);
    if (ce != hipSuccess) return hip_fail(ce);
    if (cs != hipStreamCaptureStatusNone) return QC_OK;   // graphs keep the pre-pass's plain launches
    const int64_t groups = coresident_groups(p);
    if (groups < 1) return QC_OK;
    qc::KernelArgs a = base_args(p, ws, p.bwd, QC_LOOKBACK_FENWICK);
    a.q = q; a.init = init; a.d_cum = d_cum; a.out = d_q; a.d_init = d_init;
    a.desc2 = static_cast<char*>(a.desc) + size_t(p.bwd.n_chains * p.bwd.n_tiles) * size_t(p.bwd.wc) * p.slot_bytes;
    a.n_coop = groups;
    a.n_blocks = uint32_t(groups * p.bwd.n_tiles);
    const int rc = set_epoch(&a, st);
    if (rc != QC_OK) return rc;
    const hipError_t e = qc::launch_bwd_coresident(p.dtype, p.bwd.wc, p.bwd.deep, a, st);
    if (e == hipErrorCooperativeLaunchTooLarge) {
        (void)hipGetLastError();   // the device holds fewer blocks than its occupancy said: use the pre-pass
        return QC_OK;
    }
    if (e != hipSuccess) return hip_fail(e);
    *done = true;
    return QC_OK;
}

int launch_forward(const Plan& p, const void* q, const void* init, void* cum, void* ckpt, void* fin, void* ws,
                   hipStream_t st, bool column, bool rscan, int lookback) {
    qc::KernelArgs a = column ? column_args(p, ws) : base_args(p, ws, p.fwd, lookback);
    a.q = q; a.init = init; a.out = cum; a.ckpt = ckpt; a.fin = fin;
    if (!column && !rscan) {
        const int rc = set_epoch(&a, st);
        if (rc != QC_OK) return rc;
    }
    const hipError_t e = column ? qc::launch_fwd_column(p.dtype, a, st)
                                : qc::launch_fwd_chunked(p.dtype, p.fwd.wc, p.fwd.deep, rscan, a, st);
    return e == hipSuccess ? QC_OK : hip_fail(e);
}

}  // namespace

int qc::record_hip_error(hipError_t e) { return hip_fail(e); }

extern "C" {

size_t quat_cumprod_workspace_bytes(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype) {
    Plan p;
    return make_plan(b, s, h, j, dtype, &p) == QC_OK ? p.ws_bytes : 0;
}

size_t quat_cumprod_ckpt_bytes(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype) {
    Plan p;
    return make_plan(b, s, h, j, dtype, &p) == QC_OK ? p.ckpt_bytes : 0;
}

size_t quat_cumprod_ckpt_bytes_ex(int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype, const qc_options* opts) {
    Options o;
    Plan p;
    if (check_options(opts, &o) != QC_OK || make_plan(b, s, h, j, dtype, &p) != QC_OK) return 0;
    return saved_bytes(p, o);
}

int quat_cumprod_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return QC_ERR_NULL;
    if (!aligned(workspace, 16)) return QC_ERR_ALIGN;
    if (workspace_bytes < size_t(qc::kHdrWords) * 4) return QC_ERR_WORKSPACE;
    const hipError_t e = qc::launch_zero_words(static_cast<uint32_t*>(workspace), workspace_bytes / 4,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QC_OK : hip_fail(e);
}

int quat_cumprod_fwd_ex(const void* q, const void* init, void* cum, void* ckpt, size_t ckpt_bytes,
                        int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream, const qc_options* opts) {
    Options o;
    int rc = check_options(opts, &o);
    const int path = o.path;
    if (rc != QC_OK) return rc;
    Plan p;
    rc = make_plan(b, s, h, j, dtype, &p);
    if (rc != QC_OK) return rc;
    if (!q || !init || !cum) return QC_ERR_NULL;
    if (!workspace) return QC_ERR_WORKSPACE;
    const size_t ck_bytes = saved_bytes(p, o);
    if (ckpt && ckpt_bytes < ck_bytes) return QC_ERR_WORKSPACE;
    if (workspace_bytes < p.ws_bytes) return QC_ERR_WORKSPACE;
    if (!aligned(q, p.io_bytes) || !aligned(init, p.io_bytes) || !aligned(cum, p.io_bytes)) return QC_ERR_ALIGN;
    if ((ckpt && !aligned(ckpt, 16)) || !aligned(workspace, 16)) return QC_ERR_ALIGN;
    const size_t big = size_t(p.N) * p.io_bytes, small = size_t(p.n_cols) * p.io_bytes;
    const Range rs[] = {{q, big}, {init, small}, {cum, big}, {ckpt, ck_bytes}, {workspace, p.ws_bytes}};
    const bool out[] = {false, false, true, true, true};
    if (any_alias(rs, out, 5)) return QC_ERR_ALIAS;

    const bool column = path == QC_PATH_COLUMN || (path == QC_PATH_AUTO && p.n_cols >= kColumnPathMinColumns);
    const bool final_only = o.saved == QC_SAVED_FINAL;
    return launch_forward(p, q, init, cum, final_only ? nullptr : ckpt, final_only ? ckpt : nullptr, workspace,
                          static_cast<hipStream_t>(stream), column, !column && use_rscan(path), o.lookback);
}

int quat_cumprod_fwd(const void* q, const void* init, void* cum, void* ckpt, size_t ckpt_bytes,
                     int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
    return quat_cumprod_fwd_ex(q, init, cum, ckpt, ckpt_bytes, b, s, h, j, dtype, workspace, workspace_bytes,
                               stream, nullptr);
}

int quat_cumprod_bwd_ex(const void* q, const void* init, const void* d_cum, const void* ckpt, size_t ckpt_bytes,
                        void* d_q, void* d_init,
                        int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream, const qc_options* opts) {
    Options o;
    int rc = check_options(opts, &o);
    const int path = o.path;
    if (rc != QC_OK) return rc;
    Plan p;
    rc = make_plan(b, s, h, j, dtype, &p);
    if (rc != QC_OK) return rc;
    if (!q || !init || !d_cum) return QC_ERR_NULL;
    const bool final_only = ckpt && o.saved == QC_SAVED_FINAL;
    if (final_only && use_rscan(path)) return QC_ERR_OPTION;
    if (!d_q && !d_init) return QC_OK;
    if (!workspace) return QC_ERR_WORKSPACE;
    const size_t ck_bytes = saved_bytes(p, o);
    if (ckpt && ckpt_bytes < ck_bytes) return QC_ERR_WORKSPACE;
    if (workspace_bytes < p.ws_bytes) return QC_ERR_WORKSPACE;
    if (!aligned(q, p.io_bytes) || !aligned(init, p.io_bytes) || !aligned(d_cum, p.io_bytes)) return QC_ERR_ALIGN;
    if ((d_q && !aligned(d_q, p.io_bytes)) || (d_init && !aligned(d_init, p.io_bytes))) return QC_ERR_ALIGN;
    if ((ckpt && !aligned(ckpt, 16)) || !aligned(workspace, 16)) return QC_ERR_ALIGN;
    const size_t big = size_t(p.N) * p.io_bytes, small = size_t(p.n_cols) * p.io_bytes;
    const Range rs[] = {{q, big}, {init, small}, {d_cum, big}, {ckpt, ck_bytes},
                        {d_q, big}, {d_init, small}, {workspace, p.ws_bytes}};
    const bool out[] = {false, false, false, false, true, true, true};
    if (any_alias(rs, out, 7)) return QC_ERR_ALIAS;

    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (path == QC_PATH_COLUMN) {
        qc::KernelArgs a = column_args(p, workspace);
        a.q = q; a.init = init; a.d_cum = d_cum; a.out = d_q; a.d_init = d_init;
        const hipError_t e = qc::launch_bwd_column(p.dtype, a, st);
        return e == hipSuccess ? QC_OK : hip_fail(e);
    }
    void* ck = final_only ? nullptr : const_cast<void*>(ckpt);
    if (!ckpt) {
        bool done = false;
        rc = try_bwd_coresident(p, o, q, init, d_cum, d_q, d_init, workspace, st, &done);
        if (rc != QC_OK || done) return rc;
        // Leaves-only backward: re-derive the boundary prefix products from q.
        ck = static_cast<char*>(workspace) + p.off_ckpt;
        rc = launch_forward(p, q, init, nullptr, ck, nullptr, workspace, st, false, use_rscan(path), o.lookback);
        if (rc != QC_OK) return rc;
    }
    qc::KernelArgs a = base_args(p, workspace, p.bwd, o.lookback);
    a.q = q; a.init = init; a.d_cum = d_cum; a.out = d_q; a.d_init = d_init; a.ckpt = ck;
    if (final_only) a.fin = const_cast<void*>(ckpt);
    const bool rscan = use_rscan(path);
    if (!rscan) {
        rc = set_epoch(&a, st);
        if (rc != QC_OK) return rc;
    }
    const hipError_t e = qc::launch_bwd_chunked(p.dtype, p.bwd.wc, p.bwd.deep, rscan, a, st);
    return e == hipSuccess ? QC_OK : hip_fail(e);
}

int quat_cumprod_bwd(const void* q, const void* init, const void* d_cum, const void* ckpt, size_t ckpt_bytes,
                     void* d_q, void* d_init,
                     int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
    return quat_cumprod_bwd_ex(q, init, d_cum, ckpt, ckpt_bytes, d_q, d_init, b, s, h, j, dtype, workspace,
                               workspace_bytes, stream, nullptr);
}

int quat_cumprod_workspace_status(void* workspace, size_t workspace_bytes, void* stream, int32_t clear,
                                  int32_t* status_out) {
    if (!workspace || !status_out) return QC_ERR_NULL;
    if (!aligned(workspace, 16)) return QC_ERR_ALIGN;
    if (workspace_bytes < size_t(qc::kHdrWords) * 4) return QC_ERR_WORKSPACE;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t* word = static_cast<uint32_t*>(workspace) + qc::kHdrStatus;
    uint32_t v = 0;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e);
    e = hipMemcpy(&v, word, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    if (clear && v != 0) {
        e = qc::launch_zero_words(word, 1, st);
        if (e != hipSuccess) return hip_fail(e);
        e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e);
    }
    *status_out = int32_t(v);
    return QC_OK;
}

const char* quat_cumprod_strerror(int32_t code) {
    switch (code) {
        case QC_OK: return "ok";
        case QC_ERR_NULL: return "a required pointer is NULL";
        case QC_ERR_SHAPE: return "invalid shape (a dimension < 1, or sizes beyond the library's limits)";
        case QC_ERR_ALIGN: return "misaligned pointer";
        case QC_ERR_DTYPE: return "unknown dtype";
        case QC_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
        case QC_ERR_WORKSPACE: return "workspace or ckpt buffer missing or too small";
        case QC_ERR_HIP: return "HIP runtime error";
        case QC_ERR_OPTION: return "invalid option";
        default: return "unknown error code";
    }
}

const char* quat_cumprod_last_hip_error(void) { return g_last_hip_error.c_str(); }

int32_t quat_cumprod_version(void) { return 100; }

}  // extern "C"
