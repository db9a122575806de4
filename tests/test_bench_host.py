"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the t(a) = t0 + a tau fit and the
rule that the counter-derived traffic is reported only for the kernel sources it was measured on."""
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""                      # no JSON line
    assert "one GPU" in r.stderr


def _rows(t0, tau, actives, bytes_per_route=4_719_744):
    return [dict(H=2048, I=768, active=a, us_per_step_median=t0 + a * tau, bytes_streamed=a * bytes_per_route)
            for a in actives]


def test_active_fit_recovers_an_exact_line():
    fit = bench.active_fit(_rows(5.25, 1.0625, [8, 4, 2, 0]))
    assert abs(fit["t0_us"] - 5.25) < 1e-12
    assert abs(fit["tau_us_per_route"] - 1.0625) < 1e-12
    assert abs(fit["r2"] - 1.0) < 1e-12
    # tau's rate: one route's expert bytes per tau
    assert abs(fit["tau_gbs"] - 4_719_744 / 1.0625e-6 / 1e9) < 1e-6


def test_active_fit_least_squares_on_noisy_rows():
    # t = 3 + 2a plus residuals that sum to zero and are orthogonal to a: the fit is still (3, 2)
    rows = _rows(3.0, 2.0, [8, 4, 2, 0])
    for r, e in zip(rows, [0.1, -0.2, 0.0, 0.1]):
        r["us_per_step_median"] += e
    fit = bench.active_fit(rows)
    assert abs(fit["t0_us"] - 3.0) < 1e-12 and abs(fit["tau_us_per_route"] - 2.0) < 1e-12
    assert 0.0 < fit["r2"] < 1.0


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    summary = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DECODE_SOURCES", ("kernel.hip",))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.measured_traffic() is None                         # no summary
    summary.write_text("# decode counters\n\nno traffic line\n")
    assert bench.measured_traffic() is None                         # no TRAFFIC line
    sha = bench.sources_sha256(("kernel.hip",))
    summary.write_text('text\n\nTRAFFIC {"traffic_bytes_per_step": 123, "sources_sha256": "%s"}\n' % sha)
    assert bench.measured_traffic()["traffic_bytes_per_step"] == 123
    src.write_text("// kernel v2\n")                                # the kernel changed since the counters
    assert bench.measured_traffic() is None


def test_committed_traffic_summary_parses():
    """The committed decode counter summary holds a TRAFFIC line with the fields the bench reports."""
    import json
    import re
    text = open(bench.TRAFFIC_SUMMARY).read()
    m = re.search(r"^TRAFFIC (\{.*\})$", text, flags=re.M)
    assert m
    rec = json.loads(m.group(1))
    for key in ("traffic_bytes_per_step", "fetch_bytes_per_step", "write_bytes_per_step", "fetch_factor",
                "write_factor", "sources_sha256"):
        assert key in rec
    # each figure is rounded to whole bytes on its own, so the parts may sum one byte off the total
    assert abs(rec["traffic_bytes_per_step"] - rec["fetch_bytes_per_step"] - rec["write_bytes_per_step"]) <= 1
