"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_swa_pairs_closed_form():
    # brute force over positions: min(t + 1, w) keys for row t
    for T, w in ((1, 1), (5, 2), (7, 7), (9, 20), (100, 13)):
        assert bench.swa_pairs(T, w) == sum(min(t + 1, w) for t in range(T))


def test_traffic_reported_only_for_matching_sources(monkeypatch):
    sha = bench.kernel_sources_sha("band_kernel")
    monkeypatch.setattr(bench, "TRAFFIC", {"band_kernel": {"sha": sha, "bytes_per_launch": 123.0}})
    assert bench.traffic_for("band_kernel") == 123.0
    monkeypatch.setattr(bench, "TRAFFIC", {"band_kernel": {"sha": "0" * 16, "bytes_per_launch": 123.0}})
    assert bench.traffic_for("band_kernel") is None
    assert bench.traffic_for("split_rows_kernel") is None or isinstance(bench.traffic_for("split_rows_kernel"), float)


def test_gpus_other_than_one_exit_with_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_timed_keeps_events_out_of_the_timed_steps(monkeypatch):
    """bench.timed: `steps` calls with the library's per-kernel events off (the timed pass),
    then reset, then the same calls with the events on (the stage times)."""
    log = []
    state = {"events": False}
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda: None)
    monkeypatch.setattr(bench.ox, "timing_begin", lambda: state.update(events=True) or log.append("begin"))

    def end():
        state["events"] = False
        log.append("end")
        return {"band": (1.0, 3)}

    monkeypatch.setattr(bench.ox, "timing_end", end)
    ms, stages = bench.timed(lambda i: log.append(("step", i, state["events"])), 3,
                             reset=lambda: log.append("reset"))
    assert log == [("step", 0, False), ("step", 1, False), ("step", 2, False), "reset", "begin",
                   ("step", 0, True), ("step", 1, True), ("step", 2, True), "end"]
    assert stages == {"band": (1.0, 3)} and ms >= 0.0
