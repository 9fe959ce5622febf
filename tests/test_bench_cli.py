"""bench.py's host-side parts: the one-GPU guard, the counter-note reader
and the rocprofv3 CSV summaries (no GPU, no torch import)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _note(tmp_path, digest, workload="w 1", hbm="123456"):
    p = tmp_path / "note.md"
    p.write_text("# note\n\n- workload: %s\n- tile_id: 8\n- hbm_bytes_per_launch: %s\n"
                 "- consumer_sources_sha256: %s\n" % (workload, hbm, digest))
    return str(p)


def test_stored_traffic_only_for_current_sources_and_workload(tmp_path, monkeypatch):
    digest = bench.consumer_digest()
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", _note(tmp_path, digest))
    assert bench.stored_traffic("w 1") == 123456.0
    assert bench.stored_traffic("w 1", 8) == 123456.0
    assert bench.stored_traffic("w 1", 15) is None      # counters of another kernel
    assert bench.stored_traffic("another workload") is None
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", _note(tmp_path, "0" * 64))
    assert bench.stored_traffic("w 1") is None
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", str(tmp_path / "missing.md"))
    assert bench.stored_traffic("w 1") is None


def test_consumer_digest_follows_the_sources(tmp_path, monkeypatch):
    d0 = bench.consumer_digest()
    assert len(d0) == 64 and d0 == bench.consumer_digest()
    # the digest covers every listed source: dropping one changes it
    monkeypatch.setattr(bench, "CONSUMER_SOURCES", bench.CONSUMER_SOURCES[:-1])
    assert bench.consumer_digest() != d0


def test_pmc_summary_means_per_kernel_and_counter(tmp_path, capsys):
    d = tmp_path / "pmc" / "sub"
    d.mkdir(parents=True)
    rows = [("kA", "FETCH_SIZE", 10.0), ("kA", "FETCH_SIZE", 30.0), ("kB", "FETCH_SIZE", 7.0)]
    with open(d / "x_counter_collection.csv", "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f"{k},{c},{v}\n")
    bench.pmc_summary(str(tmp_path / "pmc"))
    out = capsys.readouterr().out.splitlines()
    got = {l.split()[-1]: l for l in out}
    assert set(got) == {"kA", "kB"}
    assert float(got["kA"].split()[1]) == 20.0 and "dispatches=   2" in got["kA"]
    assert float(got["kB"].split()[1]) == 7.0 and "dispatches=   1" in got["kB"]


def test_trace_summary_window_in_dispatch_order(tmp_path, capsys):
    d = tmp_path / "tr"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        # kernel k: durations 1, 2, 3, 4, 5 us, written out of dispatch order
        for i, us in [(3, 3), (1, 1), (5, 5), (2, 2), (4, 4)]:
            f.write(f"{i},k,{1000 * i},{1000 * i + 1000 * us}\n")
    bench.trace_summary(str(d), 2, 3)
    line = capsys.readouterr().out.strip()
    assert line.startswith("5 dispatches")
    assert "mean       3.0 us" in line            # all five
    assert "[3, 5): mean       4.5 us" in line    # dispatches 4 and 5
    assert "min      4.0  max      5.0" in line
    bench.trace_summary(str(d), 2, 1)
    assert "[1, 3): mean       2.5 us" in capsys.readouterr().out


@pytest.mark.parametrize("steps,expect", [(100, 20), (5, 1), (20, 4), (1, 1), (7, 2)])
def test_timed_brackets_one_call_in_five(steps, expect):
    """timed() brackets the first call of every five with the consumer's
    event pair (at least one); a stand-in for torch counts the pairs."""
    class Ev:
        def __init__(self, enable_timing=False):
            self.t = 0.0

        def record(self):
            pass

        def elapsed_time(self, other):
            return 1.0

    class Cuda:
        Event = Ev

        @staticmethod
        def synchronize():
            pass

    class Torch:
        cuda = Cuda

    made = []
    ran = []

    def make(ev):
        made.append(ev)
        return lambda: ran.append(ev)

    per = []
    t, c = bench.timed(Torch, make, steps, 3, per_call=per)
    assert len(ran) == 3 + steps
    assert all(ev is None for ev in ran[:3])
    assert sum(ev is not None for ev in ran[3:]) == expect
    assert [i for i, ev in enumerate(ran[3:]) if ev is not None] == list(range(0, steps, 5))
    assert len(per) == expect and c == 1.0


def test_consumer_digest_ignores_comments():
    import bench
    a = "int f(int x) {  // add one\n    return x + 1; /* the sum */\n}\n"
    b = "// header\nint f(int x) {\n\n    return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)
    # the stored counter note is tied to the consumer's code as it stands
    assert bench.stored_traffic("f16 8x1024 rows M=8192 K=4096 N=4096") is not None
