"""Host-side checks of bench.py's accounting (no GPU): the algorithmic bytes
it counts for the checkpointed scan VJP, on the rlx-autodiff page's Griewank
case (4 steps, 2 snapshots), counted by hand from the schedule's records."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quaternion_cumprod_autodiff_amd import capi  # noqa: E402
from quaternion_cumprod_autodiff_amd.build import LIB_PATH  # noqa: E402

STORE, LOAD, ADVANCE, REVERSE = 1, 2, 3, 4


@pytest.fixture(scope="module")
def sched():
    if not os.path.exists(LIB_PATH):
        from quaternion_cumprod_autodiff_amd.build import build
        build()
    return capi.ScanSchedule(4, 2)


def test_griewank_case_records(sched):
    # Forward part: snapshot init, one step, snapshot c[0]; then the reverse
    # part advances 2 + 1 steps, reverses 4 and loads a snapshot 3 times.
    acts = sched.actions.tolist()
    assert sched.bwd_start == 3 and sched.n_actions == 12
    fwd, bwd = acts[:3], acts[3:]
    assert [r[0] for r in fwd] == [STORE, ADVANCE, STORE]
    assert sum(r[2] - r[1] for r in bwd if r[0] == ADVANCE) == 3
    assert sum(r[0] == REVERSE for r in bwd) == 4
    assert sum(r[0] == LOAD for r in bwd) == 3 and not any(r[0] == STORE for r in bwd)


@pytest.mark.parametrize("body,ebytes,w,fwd_b,bwd_b", [
    # quat: 16-byte x, u, d_x; 32-byte float64 snapshots.
    #   forward part: 1 step (16) + 2 stores (64) = 80
    #   reverse part: 3 steps (48) + 4 reversed steps x (x, u, d_x) (192) + 3 loads (96) = 336
    ("quat", 16, 4, 80, 336),
    # add: 4-byte values, 8-byte snapshots; a reversed step reads u and writes d_x only.
    #   forward part: 4 + 16 = 20;  reverse part: 12 + 4 x 8 + 24 = 68
    ("add", 4, 1, 20, 68),
])
def test_schedule_bytes_by_hand(sched, body, ebytes, w, fwd_b, bwd_b):
    cols = 3
    assert bench.scan_schedule_bytes(body, sched, 0, sched.bwd_start, ebytes, cols, w) == cols * fwd_b
    assert bench.scan_schedule_bytes(body, sched, sched.bwd_start, sched.n_actions, ebytes, cols, w) == cols * bwd_b
