"""bench.py's per-call timing: one event is recorded before each call and a
call's interval runs to the next event (the next call's, or the event that
closes the region); pairs=True brackets each call instead.  Fake events carry
a timestamp from a fake clock, so this runs on the CPU."""
import os
import sys
import types

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


class Clock:
    t = 0.0


class FakeEvent:
    def __init__(self, enable_timing=False):
        self.t = None

    def record(self):
        self.t = Clock.t

    def elapsed_time(self, other):
        return other.t - self.t


FAKE_TORCH = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=FakeEvent))


def _region(timer, calls, gap):
    """Run (label, duration) calls, with `gap` of idle time after each, then
    close the region with an event, as bench.timed does."""
    Clock.t = 0.0
    for label, d in calls:
        def fn(d=d):
            Clock.t += d
        timer.run(label, fn)
        Clock.t += gap
    end = FakeEvent()
    end.record()
    timer.collect(end)


def test_chained_intervals_cover_each_call_and_the_gap_after_it():
    timer = bench.Timer(FAKE_TORCH)
    _region(timer, [("a", 1.0), ("b", 3.0), ("a", 2.0), ("b", 5.0)], gap=0.25)
    assert timer.avg_ms("a") == 1.75
    assert timer.avg_ms("b") == 4.25
    assert timer.count == {"a": 2, "b": 2}
    assert timer.pending == []


def test_regions_accumulate():
    timer = bench.Timer(FAKE_TORCH)
    _region(timer, [("a", 1.0)], gap=0.0)
    _region(timer, [("a", 3.0)], gap=0.0)
    assert timer.avg_ms("a") == 2.0


def test_pairs_bracket_each_call():
    timer = bench.Timer(FAKE_TORCH, pairs=True)
    Clock.t = 0.0
    for d in (1.0, 2.0):
        timer.run("w", lambda d=d: setattr(Clock, "t", Clock.t + d))
        Clock.t += 10.0  # other work between calls is not counted
    timer.collect()
    assert timer.avg_ms("w") == 1.5


class FakeCuda:
    Event = FakeEvent

    @staticmethod
    def synchronize():
        pass


def test_timed_steps_hold_no_marks_and_attribution_runs_after():
    """bench.timed: warm-up, then exactly `steps` steps between two events with
    the timer disabled (no mark inside), then as many more with per-call marks,
    whose durations are attributed to the labels."""
    torch = types.SimpleNamespace(cuda=FakeCuda)
    timer = bench.Timer(torch)
    seen = []
    marks_in_timed = []

    def step(i):
        seen.append(i)
        n0 = len(timer.pending)
        timer.run("q", lambda: setattr(Clock, "t", Clock.t + 1.0))
        timer.run("g", lambda: setattr(Clock, "t", Clock.t + 4.0))
        if not timer.enabled:
            marks_in_timed.append(len(timer.pending) - n0)

    Clock.t = 0.0
    ms, _ = bench.timed(torch, timer, step, steps=3, warmup=2)
    assert seen == [0, 1, 2, 3, 4, 5, 6, 7]  # 2 warm-up, 3 timed, 3 attributed
    assert marks_in_timed == [0, 0, 0]
    assert ms == 5.0
    assert timer.count == {"q": 3, "g": 3}
    assert timer.avg_ms("q") == 1.0 and timer.avg_ms("g") == 4.0
    assert timer.enabled
