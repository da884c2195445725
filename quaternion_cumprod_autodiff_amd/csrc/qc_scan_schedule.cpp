// qc_scan_schedule.cpp -- host-side binomial checkpointing schedule for the
// scan VJP of include/qc_scan.h.
//
// The rlx-autodiff source page "src/decompose_backward.rs" lowers a scan
// backward whose trajectory holds k checkpoints instead of every carry (its
// test "decompose_scan_backward_griewank"); the page does not say where the
// checkpoints go.  This file places them by Griewank's binomial rule, which
// reverses s steps with k snapshot slots using the fewest recomputed forward
// steps.
//
// Cost model.  Reversing a segment of n steps whose input carry sits in a
// slot, with f further free slots, costs C(n, f) forward steps:
//   C(1, f) = 0,   C(n, 0) = n (n - 1) / 2   (recompute from the start for
//   every step),
//   C(n, f) = min over 1 <= m < n of  m + C(n - m, f - 1) + C(m, f)
//   (advance m steps, snapshot, reverse the right part with one slot fewer,
//   then the left part with the slot freed again).
// Griewank's closed form: with k = f + 1 slots and beta(k, r) = C(k + r, r),
// let r be the least integer with beta(k, r) >= n; then
//   C(n, f) = r n - beta(k + 1, r - 1).
// C(., f) is convex and piecewise linear (its slope on the r-th range is r),
// so m + C(m, f) + C(n - m, f - 1) is convex in m and its least minimiser
// is found by bisection on its forward difference.
#include "qc_scan.h"
#include "quat_cumprod.h"

#include <cstdint>
#include <vector>

namespace {

constexpr int64_t kSat = int64_t(1) << 62;

// beta(k, r) = C(k + r, r), saturated at kSat; beta(k, -1) = 0.
int64_t beta(int64_t k, int64_t r) {
    if (r < 0) return 0;
    int64_t v = 1;
    for (int64_t i = 1; i <= r; ++i) {
        // v * (k + i) / i stays an integer: v = C(k + i - 1, i - 1).
        const int64_t num = k + i;
        if (v > kSat / num) return kSat;
        v = v * num / i;
    }
    return v;
}

// Least r with beta(k, r) >= n.
int64_t repetitions(int64_t n, int64_t k) {
    int64_t r = 0, v = 1;
    while (v < n) {
        ++r;
        const int64_t num = k + r;
        v = (v > kSat / num) ? kSat : v * num / r;
    }
    return r;
}

int64_t cost(int64_t n, int64_t f) {
    if (n <= 1) return 0;
    if (f == 0) return n * (n - 1) / 2;
    const int64_t k = f + 1;
    const int64_t r = repetitions(n, k);
    return r * n - beta(k + 1, r - 1);
}

int64_t split_cost(int64_t n, int64_t f, int64_t m) { return m + cost(m, f) + cost(n - m, f - 1); }

// Least minimiser of split_cost over 1 <= m < n (n >= 2, f >= 1).
int64_t best_split(int64_t n, int64_t f) {
    int64_t lo = 1, hi = n - 1;   // answer in [lo, hi]
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (split_cost(n, f, mid + 1) - split_cost(n, f, mid) >= 0)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

struct Emitter {
    int32_t* out;
    int64_t cap, n = 0, steps = 0;
    int64_t cur = -1;   // the current carry is c[cur - 1]; -1 = unknown
    bool overflow = false;
    void put(int32_t op, int64_t a, int64_t b) {
        if (out) {
            if (n >= cap) {
                overflow = true;
            } else {
                int32_t* r = out + 4 * n;
                r[0] = op; r[1] = int32_t(a); r[2] = int32_t(b); r[3] = 0;
            }
        }
        ++n;
    }
    void load(int32_t slot, int64_t pos) {
        if (cur != pos) put(QC_SCAN_LOAD, slot, 0);
        cur = pos;
    }
    void advance(int64_t t0, int64_t t1) {
        if (t1 > t0) put(QC_SCAN_ADVANCE, t0, t1);
        steps += t1 - t0;
        cur = t1;
    }
};

struct Segment {
    int64_t l, n;     // steps l .. l + n - 1
    int32_t base;     // slot holding c[l - 1]
    int32_t free;     // free slots
};

}  // namespace

extern "C" {

int32_t qc_scan_width(int32_t body) {
    return body == QC_SCAN_BODY_ADD ? 1 : body == QC_SCAN_BODY_QUAT ? 4 : 0;
}

int64_t qc_scan_schedule_capacity(int64_t s) { return s < 1 ? 0 : 4 * s + 2; }

int qc_scan_schedule(int64_t s, int32_t k, int32_t* actions, int64_t capacity, qc_scan_plan* plan) {
    if (s < 1 || s >= (int64_t(1) << 31) || k < 1 || k > 4096) return QC_ERR_SHAPE;
    if (!plan) return QC_ERR_NULL;
    if (actions && capacity < qc_scan_schedule_capacity(s)) return QC_ERR_WORKSPACE;
    Emitter em{actions, capacity};
    int64_t bwd_start = -1, prefix_steps = 0;
    em.put(QC_SCAN_STORE, 0, 0);   // slot 0 = init
    em.cur = 0;
    std::vector<Segment> stack{{0, s, 0, k - 1}};
    // The forward sweep's part ends at the last STORE before the first LOAD
    // or REVERSE.
    auto mark = [&](bool store_follows) {
        if (bwd_start < 0 && !store_follows) {
            bwd_start = em.n;
            prefix_steps = em.steps;
        }
    };
    while (!stack.empty()) {
        const Segment g = stack.back();
        stack.pop_back();
        if (g.n == 1) {
            mark(false);
            em.load(g.base, g.l);
            em.put(QC_SCAN_REVERSE, g.l, 0);
        } else if (g.free == 0) {
            mark(false);
            for (int64_t t = g.l + g.n - 1; t >= g.l; --t) {
                em.load(g.base, g.l);
                em.advance(g.l, t);
                em.put(QC_SCAN_REVERSE, t, 0);
            }
        } else {
            const int64_t m = best_split(g.n, g.free);
            const int32_t slot = k - g.free;
            if (em.cur != g.l) mark(false);
            em.load(g.base, g.l);
            em.advance(g.l, g.l + m);
            em.put(QC_SCAN_STORE, slot, 0);
            stack.push_back({g.l, m, g.base, g.free});
            stack.push_back({g.l + m, g.n - m, slot, g.free - 1});
        }
    }
    if (em.overflow) return QC_ERR_WORKSPACE;
    plan->n_actions = em.n;
    plan->bwd_start = bwd_start;
    plan->forward_steps = em.steps;
    plan->prefix_steps = prefix_steps;
    return QC_OK;
}

}  // extern "C"
