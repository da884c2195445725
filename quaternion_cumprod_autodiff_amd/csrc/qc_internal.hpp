// qc_internal.hpp -- declarations shared by the gfx950 kernels and the C-ABI
// dispatcher of the quaternion cumulative-product scan.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace qc {

// Stride, in sequence steps, of the saved boundary state: entry n holds the
// prefix product P_{nK-1} (identity for n = 0) of every column.
constexpr int kCkptStride = 64;

// Bounded waits: a cross-block wait gives up after this many polls (each poll
// is a few coherent loads plus a short sleep, about a microsecond, so well
// under a second in all) and raises the workspace status word instead of
// spinning forever.
constexpr uint32_t kSpinLimit = 1u << 16;

// Workspace header words, and the bits of the sticky status word.
// kHdrEpoch holds a 64-bit launch counter (words 4-5) for launches captured
// in a HIP graph, whose arguments (and so a host-chosen epoch) are frozen.
enum : int { kHdrStatus = 2, kHdrEpoch = 4, kHdrWords = 64 };
enum : uint32_t {
    kStatusWaitTimeout = 1u,   // a cross-block wait hit kSpinLimit
    kStatusZeroPrefix = 2u,    // a prefix product was exactly zero: the backward's results are not finite
};

// Tile geometry of the chunked path, by column-group width WC (a power of two
// <= 64) and storage dtype.  A wave holds R = 64/WC time slices of WC adjacent
// columns; a block has NW waves; every lane owns L consecutive steps of one
// column.  A tile is WC columns x (R*NW*L) steps.  Backward tiles are a
// multiple of kCkptStride steps, so they start on saved boundaries, and every
// L divides kCkptStride, so some forward slice starts on each boundary.
// bfloat16 quaternions are half the size, so their slices are twice as long
// for the same registers (and half as many tiles share the fixed costs).
// Both kernels have a second, "deep" slice length for shapes with few
// chains: each chain then has many tiles in flight, and twice-as-tall tiles
// halve the carry look-backs per byte, at the price of more registers
// (float32: 2 waves per SIMD instead of 3).  bfloat16 slices are already as
// long as the registers allow.  float32 16-column groups use 4-wave blocks
// (16 slices per column): narrow shapes are usually single long chains, where
// the taller tiles pay for the longer in-tile combines (long-seq: -6% per step).
struct Geometry {
    int wc;
    int fwd_l, fwd_nw;
    int bwd_l, bwd_nw;
    int fwd_deep_l, bwd_deep_l;
};

constexpr Geometry geometry_for(int wc, int dtype) {
    return dtype == 0
        ? (wc == 64 ? Geometry{64, 16, 4, 8, 8, 32, 16}
         : wc == 32 ? Geometry{32, 16, 4, 8, 4, 32, 16}
         : wc == 16 ? Geometry{16, 16, 4, 8, 4, 32, 16}
         : wc == 8  ? Geometry{8, 16, 1, 8, 1, 32, 16}
         : wc == 4  ? Geometry{4, 8, 1, 4, 1, 16, 8}
         : wc == 2  ? Geometry{2, 4, 1, 2, 1, 8, 4}
         :            Geometry{1, 2, 1, 1, 1, 4, 2})
        : (wc == 64 ? Geometry{64, 32, 4, 16, 8, 32, 16}
         : wc == 32 ? Geometry{32, 32, 4, 16, 4, 32, 16}
         : wc == 16 ? Geometry{16, 32, 2, 16, 2, 32, 16}
         : wc == 8  ? Geometry{8, 32, 1, 16, 1, 32, 16}
         : wc == 4  ? Geometry{4, 16, 1, 8, 1, 16, 8}
         : wc == 2  ? Geometry{2, 8, 1, 4, 1, 8, 4}
         :            Geometry{1, 4, 1, 2, 1, 4, 2});
}

constexpr int fwd_tile_steps(int wc, int dtype, bool deep) {
    return (64 / wc) * geometry_for(wc, dtype).fwd_nw *
           (deep ? geometry_for(wc, dtype).fwd_deep_l : geometry_for(wc, dtype).fwd_l);
}
constexpr int bwd_tile_steps(int wc, int dtype, bool deep) {
    return (64 / wc) * geometry_for(wc, dtype).bwd_nw *
           (deep ? geometry_for(wc, dtype).bwd_deep_l : geometry_for(wc, dtype).bwd_l);
}

// Arguments of every scan kernel (passed by value).
struct KernelArgs {
    const void* q;        // [b][s][M] quaternions, storage dtype
    const void* init;     // [b][M]
    const void* d_cum;    // [b][s][M]           (backward)
    void* out;            // cum (forward, may be null) or d_q (backward, may be null)
    void* d_init;         // [b][M]              (backward, may be null)
    void* ckpt;           // [b][n_ck][M] quaternions in the compute type (may be null)
    void* fin;            // [b][M] final carries cum[s-1] in the compute type (forward: written if not
                          // null; chunked backward: not null selects the backward from them alone)
    uint32_t* hdr;        // workspace header
    void* desc;           // per-tile carry slots, WC columns each (value words + check word)
    int64_t b, s, M;
    int64_t n_ck;         // ceil(s / kCkptStride)
    int64_t n_cg;         // column groups per batch entry
    int64_t n_chains;     // b * n_cg
    int64_t n_tiles;      // tiles per chain
    int64_t group;        // grouped look-back: tiles per group (0: the Fenwick look-back)
    int64_t n_groups;     // groups per chain (grouped look-back)
    void* desc2;          // co-resident leaves-only backward: the forward look-back's carry nodes
    int64_t n_coop;       // co-resident leaves-only backward: chains in flight at once (groups of n_tiles blocks)
    uint64_t epoch;       // this launch's epoch, folded into every check word (0: read it from the header)
    uint32_t n_blocks;    // grid size
    uint32_t spin_limit;
};

// rscan: the reduce-then-scan variant (tile aggregates, a scan of them per
// chain, a fix-up pass) instead of the single pass with the look-back.
hipError_t launch_fwd_chunked(int dtype, int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st);
hipError_t launch_bwd_chunked(int dtype, int wc, bool deep, bool rscan, const KernelArgs& a, hipStream_t st);
// Co-resident leaves-only backward (cooperative launch of a.n_coop groups of
// a.n_tiles blocks), and how many of its blocks the current device holds at
// once (0 if that cannot be told).
hipError_t launch_bwd_coresident(int dtype, int wc, bool deep, const KernelArgs& a, hipStream_t st);
int64_t coresident_blocks(int dtype, int wc, bool deep);
hipError_t launch_fwd_column(int dtype, const KernelArgs& a, hipStream_t st);
hipError_t launch_bwd_column(int dtype, const KernelArgs& a, hipStream_t st);
hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t st);
hipError_t launch_bump_epoch(uint32_t* hdr, hipStream_t st);

// Records a failed HIP call for quat_cumprod_last_hip_error; returns QC_ERR_HIP.
int record_hip_error(hipError_t e);

constexpr int kColumnBlock = 256;   // threads per block on the column path

}  // namespace qc
