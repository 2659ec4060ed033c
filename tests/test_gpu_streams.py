"""Every entry point runs on the stream its caller passes (torch's current
stream in the binding): calls on non-default streams, and independent calls
on two streams at once, give the default-stream results bit for bit; and no
call waits for the GPU before it returns."""
import pytest
import torch

import gemv_nvfp4_int8_amd as qp

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


def test_calls_return_before_their_kernels_finish():
    """No entry point synchronises the host: right after forty large GEMMs
    (about 9 ms of GPU work) have been enqueued, an event recorded behind
    them has not completed yet, so the host got control back while the
    kernels were still running.  The results are those of one call."""
    m, n, k = 8192, 8192, 4096                  # ~0.2 ms per call
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    a = torch.randint(0, 0x7E, (m, k), generator=g, device="cuda:0", dtype=torch.uint8)
    w = torch.randint(0, 0x7E, (n, k), generator=g, device="cuda:0", dtype=torch.uint8)
    sa = torch.rand(m, generator=g, device="cuda:0") + 0.5
    sw = torch.rand(n, generator=g, device="cuda:0") + 0.5
    ref = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(ref)
    qp.fp8_gemm_rowscale(a, sa, w, sw, ref)
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    for _ in range(40):
        qp.fp8_gemm_rowscale(a, sa, w, sw, out)
    done.record()
    still_running = not done.query()
    torch.cuda.synchronize()
    assert done.query()
    assert still_running, "the calls returned only after their kernels had finished"
    assert _same(out, ref)
