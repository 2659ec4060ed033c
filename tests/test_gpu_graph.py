"""HIP-graph capture of the library's entry points.

The stateless entry points launch kernels only: no allocation, no memset, no
synchronization.  So a sequence of calls can be captured into a HIP graph,
and every replay must reproduce the eager results bit for bit (every kernel
here is deterministic).  The replays are separated by eager work on the same
buffers (the outputs are overwritten with NaN, other kernels run) and by
synchronizations, and every replay is checked, not only the first.
"""
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


def _calls():
    """(callable, [output tensors]) pairs covering every stateless entry point
    and each GEMV kernel variant (K-split at both prefetch depths and both row
    units, row-split).  Every lambda binds its tensors as default arguments:
    the names are reused further down."""
    calls = []

    # row-scaled FP8 GEMV: narrow (depth 1), narrow (depth 2), wide
    for sid, (n, k) in enumerate([(300, 512), (12300, 1040), (70000, 512)]):
        wq, ws = _empty((n, k), torch.uint8), _empty((n,), torch.float32)
        qp.quant_rowwise_fp8(synth.gemv_weight_bf16(n, k, DEV, shape_id=sid), wq, ws)
        x = synth.gemv_acts_bf16(16, k, DEV, shape_id=sid)
        for m in (1, 3, 16):
            o = _empty((m, n), torch.bfloat16)
            calls.append((lambda x=x[:m], wq=wq, ws=ws, o=o: qp.fp8_gemv_rowscale(x, wq, ws, o), [o]))

    # block-scaled FP8 GEMV
    for sid, (n, k) in enumerate([(384, 1152), (12416, 1152)]):
        w, grid = synth.gemv_block_weight(n, k, DEV, shape_id=sid)
        x = synth.gemv_acts_bf16(16, k, DEV, shape_id=sid + 3)
        for m in (1, 4):
            o = _empty((m, n), torch.bfloat16)
            calls.append((lambda x=x[:m], w=w, g=grid, o=o: qp.fp8_gemv_blockscale(x, w, g, o), [o]))

    # NVFP4-weight GEMV
    n, k = 512, 1024
    wp, we, s2 = synth.gemv_nvfp4_weight(n, k, DEV, shape_id=0)
    x = synth.gemv_acts_bf16(8, k, DEV, shape_id=5)
    for m in (1, 8):
        o = _empty((m, n), torch.bfloat16)
        calls.append((lambda x=x[:m], o=o, wp=wp, we=we, s2=s2: qp.w4a16_gemv(x, wp, we, s2, o), [o]))

    # W4A8 prefill chain: activation requant, weight requant, int8 GEMM
    m, n, k = 130, 256, 512
    c = synth.w4a8_tiny(DEV, m=m, n=n, k=k)
    a_i8, a_s = _empty((m, k), torch.int8), _empty((m, k // 32), torch.float32)
    w_i8, w_s = _empty((n, k), torch.int8), _empty((n, k // 32), torch.float32)
    o8 = _empty((m, n), torch.bfloat16)
    calls.append((lambda c=c, a_i8=a_i8, a_s=a_s: qp.requant_a_bf16_int8(c.a_bf16, a_i8, a_s),
                  [a_i8, a_s]))
    calls.append((lambda c=c, w_i8=w_i8, w_s=w_s:
                   qp.requant_w_nvfp4_int8(c.w_packed, c.w_e4m3, c.scale2, w_i8, w_s),
                  [w_i8, w_s]))
    calls.append((lambda a_i8=a_i8, w_i8=w_i8, a_s=a_s, w_s=w_s, o8=o8:
                   qp.int8_gemm_blockscaled(a_i8, w_i8, a_s, w_s, o8), [o8]))

    # W4A4: quantize both operands to NVFP4, then the GEMM
    m, n, k = 96, 160, 512
    a = synth.gemv_acts_bf16(m, k, DEV, shape_id=6)
    wb = synth.gemv_weight_bf16(n, k, DEV, shape_id=6)
    ap, asc = _empty((m, k // 2), torch.uint8), _empty((m, k // 16), torch.uint8)
    wp4, wsc = _empty((n, k // 2), torch.uint8), _empty((n, k // 16), torch.uint8)
    o4 = _empty((m, n), torch.bfloat16)
    calls.append((lambda a=a, ap=ap, asc=asc: qp.quantize_bf16_nvfp4(a, ap, asc, 1.0), [ap, asc]))
    calls.append((lambda wb=wb, wp4=wp4, wsc=wsc: qp.quantize_bf16_nvfp4(wb, wp4, wsc, 0.25),
                  [wp4, wsc]))
    calls.append((lambda ap=ap, asc=asc, wp4=wp4, wsc=wsc, o4=o4:
                   qp.w4a4_gemm(ap, asc, wp4, wsc, o4, 1.0, 0.25), [o4]))

    # FP8 row-wise projection pieces: block-scaled weight requant, activation
    # quantizer, GEMM
    m, n, k = 64, 256, 384
    w, grid = synth.gemv_block_weight(n, k, DEV, shape_id=7)
    wr, wrs = _empty((n, k), torch.uint8), _empty((n,), torch.float32)
    a = synth.gemv_acts_bf16(m, k, DEV, shape_id=7)
    aq, aqs = _empty((m, k), torch.uint8), _empty((m,), torch.float32)
    of = _empty((m, n), torch.bfloat16)
    calls.append((lambda w=w, grid=grid, wr=wr, wrs=wrs:
                   qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, grid, wr, wrs),
                  [wr, wrs]))
    calls.append((lambda a=a, aq=aq, aqs=aqs: qp.quant_rowwise_fp8(a, aq, aqs), [aq, aqs]))
    calls.append((lambda aq=aq, aqs=aqs, wr=wr, wrs=wrs, of=of:
                   qp.fp8_gemm_rowscale(aq, aqs, wr, wrs, of), [of]))
    return calls


def _scribble(t):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(0x5A)


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_captured_calls_replay_bit_exact():
    calls = _calls()
    for fn, _ in calls:
        fn()
    torch.cuda.synchronize()
    eager = [[t.clone() for t in outs] for _, outs in calls]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn, _ in calls:
            fn()

    for rep in range(3):
        # eager work on the graph's own buffers between replays
        for _, outs in calls:
            for t in outs:
                _scribble(t)
        calls[rep][0]()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((_, outs), ref) in enumerate(zip(calls, eager)):
            for t, r in zip(outs, ref):
                assert _same(t, r), f"replay {rep}: call {i} differs from its eager result"


def test_cached_hit_replays_from_a_captured_graph():
    """A cache hit enqueues no kernel and only makes the stream wait for the
    derivation, so it may be captured (the miss, which allocates, ran
    eagerly before): every replay equals the eager stateless projection."""
    from tests.gpu_util import empty, filled
    m, n, k = 130, 384, 640
    cse = synth.fp8_block("cpu", m, n, k)
    w, g, a = cse.w_block.to(DEV), cse.block_grid.to(DEV), cse.a_bf16.to(DEV)
    aq, asc = empty((m, k), torch.uint8), empty((m,), torch.float32)
    ref = filled((m, n), torch.bfloat16)
    wr, wrs = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, w, g, wr, wrs, a, aq, asc, ref)
    c = qp.DerivedWeights()
    try:
        out = filled((m, n), torch.bfloat16)
        aq2, asc2 = empty((m, k), torch.uint8), empty((m,), torch.float32)
        c.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, w, g, a, aq2, asc2, out)      # the miss
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            c.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, w, g, a, aq2, asc2, out)  # a hit
        for rep in range(3):
            _scribble(out)
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            assert _same(out, ref), f"replay {rep}"
        assert c.stats()[0] == 1
    finally:
        torch.cuda.synchronize()
        c.close()
