"""bench.py's timed region, checked on the CPU with a stand-in for torch.cuda:
whatever --steps is, the region is ONE graph launch holding exactly the steps
(step s on rotation copy s % copies), the graph was replayed once before it,
and a cache flush is enqueued between the opening synchronisation and the
start event."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class _Log:
    def __init__(self):
        self.events = []   # ("sync",), ("flush",), ("record", id), ("replay", gid), ("step", r), ...

    def add(self, *e):
        self.events.append(e)


class _FakeCuda:
    def __init__(self, log):
        self.log = log
        self.capturing = None
        cuda = self
        self._graphs = 0

        class Event:
            _n = 0

            def __init__(self, enable_timing=False):
                Event._n += 1
                self.id = Event._n

            def record(self):
                cuda.log.add("record", self.id)

            def elapsed_time(self, other):
                return 1.0

        class CUDAGraph:
            def __init__(self):
                cuda._graphs += 1
                self.gid = cuda._graphs
                self.nodes = []

            def replay(self):
                cuda.log.add("replay", self.gid, len(self.nodes))

        class _Ctx:
            def __init__(self, enter=None, exit_=None):
                self.enter, self.exit_ = enter, exit_

            def __enter__(self):
                if self.enter:
                    self.enter()

            def __exit__(self, *a):
                if self.exit_:
                    self.exit_()

        class Stream:
            def wait_stream(self, other):
                pass

        self.Event, self.CUDAGraph, self.Stream, self._Ctx = Event, CUDAGraph, Stream, _Ctx

    def current_stream(self):
        return self.Stream()

    def stream(self, s):
        return self._Ctx()

    def graph(self, g, stream=None):
        def enter():
            self.capturing = g

        def exit_():
            self.capturing = None
        return self._Ctx(enter, exit_)

    def synchronize(self):
        self.log.add("sync")


class _FakeTorch:
    def __init__(self, log):
        self.cuda = _FakeCuda(log)


@pytest.mark.parametrize("steps", [1, 5, 20, 40, 41, 42, 123, 2000])
def test_timed_region_is_one_graph_launch_of_exactly_the_steps(steps):
    bench = _bench()
    log = _Log()
    torch = _FakeTorch(log)
    copies = 41
    captured = []

    def step(r):
        g = torch.cuda.capturing
        if g is None:
            log.add("eager-step", r)
        else:
            g.nodes.append(r)
            captured.append(r)

    timer = bench.StepTimer(step, steps, copies, torch, flush=lambda: log.add("flush"))
    # The graph holds exactly the steps, each on copy s % copies.
    assert captured == [s % copies for s in range(steps)]
    assert timer.graph is not None and len(timer.graph.nodes) == steps
    # It was replayed once (untimed) at construction.
    assert [e for e in log.events if e[0] == "replay"] == [("replay", timer.graph.gid, steps)]
    log.events.clear()

    ms, _ = timer.time()
    ev = log.events
    starts = [i for i, e in enumerate(ev) if e[0] == "record"]
    assert len(starts) == 2
    region = ev[starts[0] + 1:starts[1]]
    # One graph launch, no eager step, nothing else between the two events.
    assert region == [("replay", timer.graph.gid, steps)]
    # sync, flush, start event ... end event, sync.
    assert ev[0] == ("sync",) and ev[1] == ("flush",) and ev[2][0] == "record"
    assert ev[-1] == ("sync",)
    assert ms == pytest.approx(1.0 / steps)
    assert not [e for e in ev if e[0] == "eager-step"]


def test_warm_timing_replays_the_same_graph_before_its_region():
    bench = _bench()
    log = _Log()
    torch = _FakeTorch(log)
    timer = bench.StepTimer(lambda r: torch.cuda.capturing.nodes.append(r), 7, 1, torch,
                            flush=lambda: log.add("flush"))
    log.events.clear()
    timer.time_warm()
    ev = log.events
    starts = [i for i, e in enumerate(ev) if e[0] == "record"]
    assert ev[starts[0] + 1:starts[1]] == [("replay", timer.graph.gid, 7)]
    # The untimed replay (not a flush) precedes the start event.
    assert ev[starts[0] - 1] == ("replay", timer.graph.gid, 7)
    assert ("flush",) not in ev


def test_median_uses_cold_regions():
    bench = _bench()
    log = _Log()
    torch = _FakeTorch(log)
    timer = bench.StepTimer(lambda r: torch.cuda.capturing.nodes.append(r), 200, 256, torch,
                            flush=lambda: log.add("flush"))
    log.events.clear()
    timer.median_ms(5)
    assert sum(1 for e in log.events if e == ("flush",)) == 5
    assert sum(1 for e in log.events if e[0] == "replay") == 5


def test_per_launch_region_sizes():
    bench = _bench()
    assert bench.per_launch_count(20) == 200
    assert bench.per_launch_count(2000) == 3000
