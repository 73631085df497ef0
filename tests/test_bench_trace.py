"""The trace leg's timeline summary (bench.trace_summary), on hand-built stamps.

Host logic only: the summary of the tracing build's per-workgroup timestamps
(s_memrealtime ticks of 10 ns) for two consecutive launches."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _stamps(start, phases, n):
    """n workgroups starting 2 ticks apart from `start`, with the given phase lengths."""
    t = np.zeros((n, 5), dtype=np.uint64)
    for w in range(n):
        s = start + 2 * w
        t[w, :4] = [s, s + phases[0], s + phases[0] + phases[1], s + sum(phases)]
        t[w, 4] = (np.uint64(w % 8) << np.uint64(32)) | np.uint64((w % 16) << 8)  # XCC, CU id
    return t


def test_two_launches_in_either_buffer_order():
    n = 64
    first, second = _stamps(1000, (400, 100, 50), n), _stamps(1000 + 2 * (n - 1) + 550 + 170, (400, 100, 50), n)
    for order in ((first, second), (second, first)):  # which buffer holds which launch does not matter
        d = bench.trace_summary(np.stack(order), n)
        a, b = d["launches"]
        assert abs(a["start_us"]) < 1e-9
        assert abs(a["span_us"] - (2 * (n - 1) + 550) * 0.01) < 1e-9
        assert abs(d["gap_us"] - 1.7) < 1e-9                      # 170 ticks between last end and next start
        assert abs(a["phase_us_p50"]["log_coefficients"] - 4.0) < 1e-9
        assert abs(a["phase_us_p50"]["column_sums"] - 1.0) < 1e-9
        assert abs(a["phase_us_p50"]["output_append_fold"] - 0.5) < 1e-9
        assert abs(a["workgroup_us"]["p90"] - 5.5) < 1e-9
        assert abs(a["start_spread_us"]["max"] - 2 * (n - 1) * 0.01) < 1e-9
        assert a["compute_units_used"] == 16 and b["compute_units_used"] == 16
        assert d["workgroups_per_launch"] == n
