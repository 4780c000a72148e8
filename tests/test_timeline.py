"""The timeline tool's arithmetic (no GPU): figures of one launch from
synthetic stamps whose answers are known by construction.

Nine workgroups on four compute units (two XCDs of two units each): the
first four start at 0 with a 2 us prologue, 10 key-loop steps of 1.5 us and
a 1 us epilogue; the next four start 1 us later on the same units and take
2 us per step; the ninth takes the first unit's slot 3 us after the first
workgroup there ended, at 1.5 us per step. Stamps tick at 100 MHz from an
arbitrary origin, and the hardware-id words carry wave, SIMD and workgroup
fields that must not split a unit.
"""
import numpy as np
import pytest

from flashattention_tiled_amd import timeline

TICK = 100  # ticks per microsecond


def _stamps():
    origin = 123_456_789_000
    rows = []

    def wg(i, xcc, cu, start_us, per_step_us, steps=10):
        t0 = start_us * TICK
        t1 = t0 + 2 * TICK
        t2 = t1 + steps * per_step_us * TICK
        t3 = t2 + 1 * TICK
        hw = (cu << 8) | (i & 0xF) | ((i % 4) << 4) | ((i % 16) << 16)
        rows.append([origin + int(t) for t in (t0, t1, t2, t3)] +
                    [hw | (xcc << 32), i | (i << 16) | (steps << 32), 0, 0])

    for i in range(8):
        wg(i, i % 2, (i // 2) % 2, 0 if i < 4 else 1, 1.5 if i < 4 else 2.0)
    wg(8, 0, 0, 18 + 3, 1.5)
    return np.array(rows, dtype=np.uint64)


def test_summary_figures():
    fig = timeline.summarize(_stamps(), n_cu=4)
    assert fig["workgroups"] == 9 and fig["units"] == 4 and fig["steps"] == 90
    assert fig["span_us"] == pytest.approx(39.0)
    assert fig["prologue_us"] == pytest.approx(2.0)
    assert fig["epilogue_us"] == pytest.approx(1.0)
    assert fig["loop_us_per_step"] == pytest.approx((5 * 1.5 + 4 * 2.0) / 9)
    # XCD 0: workgroups 0, 2, 4, 6, 8; XCD 1: 1, 3, 5, 7
    assert sorted(fig["xcd"]) == [0, 1]
    assert fig["xcd"][0]["workgroups"] == 5
    assert fig["xcd"][0]["us_per_step"] == pytest.approx(85 / 50)
    assert fig["xcd"][0]["last_end_us"] == pytest.approx(39.0)
    assert fig["xcd"][1]["us_per_step"] == pytest.approx(70 / 40)
    assert fig["xcd"][1]["last_end_us"] == pytest.approx(24.0)
    assert fig["unit_end_us"] == pytest.approx((24.0, 24.0, 39.0))
    # the one workgroup that took a freed slot: 3 us after the end before it
    assert fig["gap_us"] == pytest.approx(3.0)
    assert fig["first_wave_us_per_step"] == pytest.approx((1.5, 2.0))


def test_report_lines():
    fig = timeline.summarize(_stamps(), n_cu=4)
    text = timeline.report("synthetic", fig, event_us=41.0)
    assert "9 workgroups on 4 compute units" in text
    assert "39.0 us from the first start to the last end (41.0 us by HIP events" in text
    assert "| 0 | 5 | 1.700 | 39.0 |" in text
    assert "| 1 | 4 | 1.750 | 24.0 |" in text
    assert "next start on its unit: 3.00 us" in text


def test_single_wave_has_no_first_wave_split():
    fig = timeline.summarize(_stamps()[:4], n_cu=4)
    assert "first_wave_us_per_step" not in fig and fig["gap_us"] is None
