"""bench.py's graphics-clock sampler (host logic, CPU only): statistics are
taken over the GPU metrics table's refreshes, not over repeated reads of one
table, the refresh written before the timed region is dropped, and a table
that never refreshes (as under a profiler) yields no clock at all."""
import os
import sys
import types

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


class _FakeSmi(types.ModuleType):
    """amdsmi stand-in: each read returns the next (timestamp, per-XCD clocks)
    of a scripted sequence, repeating the last one."""

    def __init__(self, seq):
        super().__init__("amdsmi")
        self.seq, self.i = list(seq), 0

    def amdsmi_init(self):
        pass

    def amdsmi_get_processor_handles(self):
        return [object()]

    def amdsmi_get_gpu_metrics_info(self, handle):
        stamp, clocks = self.seq[min(self.i, len(self.seq) - 1)]
        self.i += 1
        m = {"current_gfxclks": list(clocks)}
        if stamp is not None:
            m["system_clock_counter"] = stamp
        return m


def _sampler(monkeypatch, seq):
    monkeypatch.setitem(sys.modules, "amdsmi", _FakeSmi(seq))
    import bench
    c = bench.ClockSampler(period_s=0.0)
    assert c.ok
    return c


def _run(c, reads):
    # drive the sampler's reads directly instead of through its thread
    c.samples, c.stamps = [], {}
    for _ in range(reads):
        x = c._read()
        if x is not None:
            c.samples.append(x)
    c.ok = False            # nothing to join
    return c.stop()


def test_statistics_over_refreshes_after_the_first(monkeypatch):
    # the construction read consumes the first entry; then the table written
    # before the region (idle clock), read many times, then two refreshes
    seq = [(10, [800] * 8)] + [(10, [800] * 8)] * 50 + [(20, [1900, 1910] * 4)] * 50 + [(30, [1800] * 8)] * 50
    c = _sampler(monkeypatch, seq)
    r = _run(c, 150)
    assert r is not None
    assert r["metric_updates"] == 2
    assert r["min_mhz"] == 1800.0 and r["max_mhz"] == 1905.0
    assert r["median_mhz"] == 1905.0          # upper median of the two refreshes
    assert r["samples"] == 150


def test_stale_table_gives_no_clock(monkeypatch):
    c = _sampler(monkeypatch, [(7, [1422.6] * 8)] * 200)
    assert _run(c, 100) is None


def test_without_timestamps_a_constant_reading_is_rejected(monkeypatch):
    c = _sampler(monkeypatch, [(None, [1500] * 8)] * 200)
    assert _run(c, 100) is None
    c = _sampler(monkeypatch, [(None, [1500] * 8)] * 10 + [(None, [1700] * 8)] * 10)
    r = _run(c, 20)
    assert r is not None and r["min_mhz"] == 1500.0 and r["max_mhz"] == 1700.0


def test_clock_adjusted_fractions_and_the_stale_reading_rule():
    import bench
    clk = {"median_mhz": 1900.0, "min_mhz": 1890.0, "max_mhz": 1905.0, "samples": 300, "metric_updates": 3}
    r = bench.clock_adjusted(clk, 1300.0, 1280.0, 256)
    peak = 256 * 4096 * 1.9e9 / 1e12                          # 1,992.3 TFLOP/s
    assert r["peak_TFLOPs"] == round(peak, 1)
    assert r["frac_attention"] == round(1300.0 / peak, 4) and r["frac_step"] == round(1280.0 / peak, 4)
    assert r["median_mhz"] == 1900.0                           # the sampler's fields are kept
    # a clock whose peak is below the measured rate is rejected
    assert bench.clock_adjusted(dict(clk, median_mhz=1200.0), 1300.0, 1280.0, 256) is None
    assert bench.clock_adjusted(None, 1300.0, 1280.0, 256) is None
