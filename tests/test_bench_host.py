"""Host logic of bench.py (no GPU): which timed steps carry stage events."""

import importlib.util
import math
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_event_stride_samples_every_layer_and_enough_steps():
    b = _bench()
    for steps in (5, 8, 20, 50, 99, 100, 300, 500, 2000):
        for layers in (1, 2, 3, 4, 6):
            s = b.event_stride(steps, layers, 0)
            sampled = list(range(1, steps, s))
            assert math.gcd(s, layers) == 1, (steps, layers, s)
            if steps >= 20:
                # at least 4 sampled steps (8 from 100 steps on), never all of a short run
                assert len(sampled) >= (8 if steps >= 100 else 4), (steps, layers, s)
                assert len(sampled) <= (12 if steps >= 100 else 6), (steps, layers, s)
            if steps >= 20 and layers <= 4:
                # every layer copy is sampled
                assert {i % layers for i in sampled} == set(range(layers)), (steps, layers, s)


def test_event_stride_takes_the_requested_one():
    b = _bench()
    assert b.event_stride(20, 4, 7) == 7


def test_percentiles():
    b = _bench()
    assert b.percentiles(list(range(101))) == [10.0, 50.0, 90.0]
