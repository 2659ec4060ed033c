"""Every entry point runs on the stream its caller passes (torch's current
stream in the binding): calls on non-default streams, and independent calls
on two streams at once, give the default-stream results bit for bit."""
import pytest
import torch

from tests.test_gpu_graph import _calls, _same, _scribble

pytestmark = pytest.mark.gpu


def _eager(calls):
    for fn, _ in calls:
        fn()
    torch.cuda.synchronize()
    return [[t.clone() for t in outs] for _, outs in calls]


def _check(calls, ref, what):
    torch.cuda.synchronize()
    for i, ((_, outs), r) in enumerate(zip(calls, ref)):
        for t, e in zip(outs, r):
            assert _same(t, e), f"{what}: call {i} differs from its default-stream result"


def test_calls_in_order_on_a_side_stream():
    calls = _calls()
    ref = _eager(calls)
    for _, outs in calls:
        for t in outs:
            _scribble(t)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn, _ in calls:
            fn()
    _check(calls, ref, "side stream")


def test_independent_gemvs_on_two_concurrent_streams():
    # the first calls of the table are GEMVs, each writing its own output
    calls = [c for c in _calls()[:15]]
    ref = _eager(calls)
    for _, outs in calls:
        for t in outs:
            _scribble(t)
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for x in s:
        x.wait_stream(torch.cuda.current_stream())
    for i, (fn, _) in enumerate(calls):
        with torch.cuda.stream(s[i % 2]):
            fn()
    _check(calls, ref, "two streams")
