"""Host-side checks of the scan VJP's checkpointing schedule and argument
validation (include/qc_scan.h); no GPU needed.

The schedule is pinned by (1) a brute-force dynamic program over every split
point, which gives the least number of recomputed forward steps that reversing
n steps with k snapshot slots can need (Griewank's binomial checkpointing, the
"Griewank" trajectory of the rlx-autodiff page "src/decompose_backward.rs"),
and (2) a symbolic run of every record: each reversed step must see exactly
the carry it needs, steps must be reversed from s-1 down to 0 exactly once,
and no more than k slots may be used.
"""
import ctypes
import functools
import math
import os

import pytest

from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.build import LIB_PATH

STORE, LOAD, ADVANCE, REVERSE = 1, 2, 3, 4
E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_ALIAS, E_WS = -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from quaternion_cumprod_autodiff_amd.build import build
        build()
    return capi.load()


@functools.lru_cache(maxsize=None)
def best_cost(n: int, free: int) -> int:
    """Least forward steps to reverse n steps whose input carry is in a slot,
    with `free` more slots, by trying every first snapshot position."""
    if n <= 1:
        return 0
    if free == 0:
        return n * (n - 1) // 2
    return min(m + best_cost(n - m, free - 1) + best_cost(m, free) for m in range(1, n))


def simulate(sched):
    """Runs the records symbolically; returns (forward steps, slots used)."""
    s, k = sched.s, sched.k
    acts = sched.actions.tolist()
    assert len(acts) == sched.n_actions >= s
    cur = 0            # the current carry is c[cur - 1]; init = c[-1]
    slots = {}
    steps = 0
    expect = s - 1
    used = set()
    prefix_steps = None
    for i, (op, a, b, _) in enumerate(acts):
        if i == sched.bwd_start:
            prefix_steps = steps
            assert acts[i - 1][0] == STORE
        if i < sched.bwd_start:
            assert op in (STORE, ADVANCE)
        if op == STORE:
            assert 0 <= a < k
            slots[a] = cur
            used.add(a)
        elif op == LOAD:
            assert a in slots
            cur = slots[a]
        elif op == ADVANCE:
            assert a == cur and b > a and b <= s
            steps += b - a
            cur = b
        elif op == REVERSE:
            assert a == expect and cur == a, (i, a, expect, cur)
            expect -= 1
        else:
            raise AssertionError(f"bad op {op}")
    assert expect == -1
    assert acts[0] == [STORE, 0, 0, 0]
    assert steps == sched.forward_steps
    assert prefix_steps == sched.prefix_steps
    return steps, len(used)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6])
def test_schedule_is_optimal_and_valid_small(lib, k):
    for s in range(1, 41):
        sch = capi.ScanSchedule(s, k)
        steps, used = simulate(sch)
        assert used <= k
        assert steps == best_cost(s, k - 1), (s, k, steps, best_cost(s, k - 1))


@pytest.mark.parametrize("s,k", [(4096, 8), (65536, 16), (65536, 2), (100000, 40), (1000, 1000)])
def test_schedule_valid_large_and_matches_binomial_count(lib, s, k):
    sch = capi.ScanSchedule(s, k)
    steps, used = simulate(sch)
    assert used <= k
    # Griewank's count for k slots: r n - C(k + r, r - 1), r least with C(k + r, r) >= n.
    r = 0
    while math.comb(k + r, r) < s:
        r += 1
    assert steps == r * s - (math.comb(k + r, r - 1) if r >= 1 else 0)
    assert sch.n_actions <= int(lib.qc_scan_schedule_capacity(s))


def test_griewank_page_example(lib):
    # The page's test reverses 4 steps with a trajectory of 2 checkpoints.
    sch = capi.ScanSchedule(4, 2)
    steps, used = simulate(sch)
    assert used <= 2 and steps == best_cost(4, 1) == 4


def test_schedule_arguments(lib):
    plan = capi.QcScanPlan()
    assert lib.qc_scan_schedule(0, 2, None, 0, ctypes.byref(plan)) == E_SHAPE
    assert lib.qc_scan_schedule(10, 0, None, 0, ctypes.byref(plan)) == E_SHAPE
    assert lib.qc_scan_schedule(10, 4097, None, 0, ctypes.byref(plan)) == E_SHAPE
    assert lib.qc_scan_schedule(10, 2, None, 0, None) == E_NULL
    buf = (ctypes.c_int32 * 8)()
    assert lib.qc_scan_schedule(10, 2, buf, 2, ctypes.byref(plan)) == E_WS
    assert lib.qc_scan_schedule(10, 2, None, 0, ctypes.byref(plan)) == 0 and plan.n_actions > 10
    assert lib.qc_scan_schedule_capacity(0) == 0 and lib.qc_scan_schedule_capacity(10) == 42
    assert lib.qc_scan_width(0) == 1 and lib.qc_scan_width(1) == 4 and lib.qc_scan_width(7) == 0


# Fake, suitably aligned device addresses: validation rejects these calls
# before any HIP call, so nothing is dereferenced.
A = 1 << 40
GB = 1 << 30


def test_scan_entry_points_validate_before_launching(lib):
    f = lib.qc_scan_fwd
    assert f(5, A, A + GB, A + 2 * GB, 1, 8, 8, None, 0, None, 0, None) == E_DTYPE
    assert f(1, A, A + GB, A + 2 * GB, 0, 8, 8, None, 0, None, 0, None) == E_SHAPE
    assert f(1, None, A + GB, A + 2 * GB, 1, 8, 8, None, 0, None, 0, None) == E_NULL
    assert f(1, A + 4, A + GB, A + 2 * GB, 1, 8, 8, None, 0, None, 0, None) == E_ALIGN
    assert f(1, A, A + GB, A + 64, 1, 8, 8, None, 0, None, 0, None) == E_ALIAS
    assert f(1, A, A + GB, A + 2 * GB, 1, 8, 8, A + 3 * GB, 1, None, 2, None) == E_WS
    # bwd_start must name a record inside a schedule for s steps (at most 4 s + 2 records).
    assert f(1, A, A + GB, A + 2 * GB, 1, 8, 8, A + 3 * GB, 0, A + 4 * GB, 2, None) == E_SHAPE
    assert f(1, A, A + GB, A + 2 * GB, 1, 8, 8, A + 3 * GB, 35, A + 4 * GB, 2, None) == E_SHAPE
    t = lib.qc_scan_bwd_trajectory
    assert t(1, A, A + GB, A + 2 * GB, None, A + 3 * GB, None, 1, 8, 8, None) == E_NULL
    assert t(1, A, A + GB, A + 2 * GB, A + 3 * GB, None, None, 1, 8, 8, None) == 0   # nothing wanted
    assert t(1, A, A + GB, A + 2 * GB, A + 3 * GB, A + 3 * GB + 64, None, 1, 8, 8, None) == E_ALIAS
    assert t(0, A + 4, A + GB, A + 2 * GB, A + 3 * GB, A + 4 * GB + 2, None, 1, 8, 8, None) == E_ALIGN
    c = lib.qc_scan_bwd_checkpointed
    args = lambda **kw: [kw.get(n, v) for n, v in (
        ("body", 1), ("xs", A), ("init", A + GB), ("up", A + 2 * GB), ("dxs", A + 3 * GB), ("dinit", A + 4 * GB),
        ("b", 1), ("s", 8), ("m", 8), ("sched", A + 5 * GB), ("n", 10), ("start", 0), ("snaps", A + 6 * GB),
        ("k", 2), ("status", A + 7 * GB), ("stream", None))]
    assert c(*args(sched=None)) == E_NULL
    assert c(*args(snaps=None)) == E_WS
    assert c(*args(k=0)) == E_WS
    assert c(*args(n=0)) == E_SHAPE
    assert c(*args(n=1000)) == E_SHAPE
    assert c(*args(start=10)) == E_SHAPE
    assert c(*args(sched=A + 5 * GB + 4)) == E_ALIGN
    assert c(*args(snaps=A + 3 * GB)) == E_ALIAS
    assert c(*args(dxs=None, dinit=None)) == 0


def test_spread_block_map_is_a_bijection():
    """The scan kernels deal blocks to 16 slices of the column range (block b
    takes position b // 16 of slice b % 16, slices of q + 1 blocks first);
    this restatement of that map must permute every grid size."""
    def spread(b, nb, slices=16):
        q, r, i, k = nb // slices, nb % slices, b % slices, b // slices
        return i * q + min(i, r) + k
    for nb in list(range(1, 200)) + [4095, 4096, 4097, 65537]:
        assert sorted(spread(b, nb) for b in range(nb)) == list(range(nb))
