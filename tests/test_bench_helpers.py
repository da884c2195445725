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


# ----------------------------------------------------------------- profiles

def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' for v in r) + "\n")


def test_profile_summary_names_every_scan_kernel(tmp_path):
    """The kernel summary gives each chunked kernel its algorithmic bytes:
    backward instances (names ending in the final-carry flag) included, the
    boundary pre-pass (a forward that stores no cum) excluded."""
    ns = "void qc::(anonymous namespace)::"
    names = {
        "bwd": ns + "bwd_chunked_kernel<qc::(anonymous namespace)::IoF32, 32, 8, 4, 0, false>(qc::KernelArgs)",
        "bwd_final": ns + "bwd_chunked_kernel<qc::(anonymous namespace)::IoF32, 32, 8, 4, 0, true>(qc::KernelArgs)",
        "fwd": ns + "fwd_chunked_kernel<qc::(anonymous namespace)::IoF32, 64, 16, 4, true, 0>(qc::KernelArgs)",
        "pre": ns + "fwd_chunked_kernel<qc::(anonymous namespace)::IoF32, 32, 16, 4, false, 0>(qc::KernelArgs)",
    }
    trace = tmp_path / "trace"
    _write_csv(str(trace / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[n, 10, 1000.0, 900.0, 1100.0] for n in names.values()])
    pmc = tmp_path / "pmc"
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        _write_csv(str(pmc / ctr / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[n, ctr, 1024.0] for n in names.values()])
    out = tmp_path / "out"
    out.mkdir()
    bench.summarize_profile(str(trace), "tiny", str(pmc), "cmd", None, "boundary", str(out))
    text = (out / "kernels_tiny.txt").read_text()
    b, s, h, j = 1, 256, 4, 8
    n, cols = b * s * h * j, b * h * j
    rows = {ln.split()[0]: ln.split() for ln in text.splitlines() if ln and not ln.startswith("#")}
    traffic = [ln for ln in text.split("# kernel")[-1].splitlines()[1:] if ln.strip()]
    algo = {ln.rsplit(None, 4)[0].strip(): int(ln.split()[-2]) for ln in traffic}
    assert algo["bwd_chunked_kernel<IoF32, 32, 8, 4, 0, false>"] == 48 * n + 32 * cols
    assert algo["bwd_chunked_kernel<IoF32, 32, 8, 4, 0, true>"] == 48 * n + 32 * cols
    assert algo["fwd_chunked_kernel<IoF32, 64, 16, 4, true, 0>"] == 32 * n + 16 * cols
    assert algo["fwd_chunked_kernel<IoF32, 32, 16, 4, false, 0>"] == 0
    assert rows  # the trace table is there too


def test_traffic_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    """The bench reports measured traffic only for the kernel sources the
    counters were taken on (their SHA-256 in the summary)."""
    good = tmp_path / "traffic.txt"
    good.write_text(f"workload = W\nkernel_source_sha256 = {bench.kernel_source_sha()}\n"
                    "bwd_hbm_bytes_per_launch = 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.load_traffic("W") == 123.0
    assert bench.load_traffic("another workload") is None
    stale = tmp_path / "stale.txt"
    stale.write_text("workload = W\nkernel_source_sha256 = 0\nbwd_hbm_bytes_per_launch = 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.load_traffic("W") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.load_traffic("W") is None
