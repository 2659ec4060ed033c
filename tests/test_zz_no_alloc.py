"""The no-allocation W4A8 prefill entry point against the caller-scratch one.

int8_w4a8_prefill_noalloc runs the same two kernels as int8_w4a8_prefill
with the activation scratch in the library's fixed per-GPU array, so its
output must be bit-identical.  Two calls in a row (the second smaller, so
it reads scratch the first one left behind) are each compared with the
caller-scratch call on the same inputs; a problem larger than the array is
refused on the host.
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import synth
from tests.gpu_util import dev, empty, filled, host

pytestmark = pytest.mark.gpu


def _weight(n, k, seed):
    c = synth.w4a8_tiny("cpu", m=1, n=n, k=k)
    w_i8, w_s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(dev(c.w_packed), dev(c.w_e4m3), c.scale2, w_i8, w_s)
    return w_i8, w_s


def _both(m, n, k, seed):
    a = dev(synth.bf16_normal((m, k), 1.0, seed, "cpu", outlier_frac=0.01, outlier_mult=20.0))
    w_i8, w_s = _weight(n, k, seed)
    ref = filled((m, n), torch.bfloat16)
    qp.int8_w4a8_prefill(a, w_i8, w_s, empty((m, k), torch.int8),
                         empty((m, k // 32), torch.float32), ref)
    got = filled((m, n), torch.bfloat16, byte=0x5A)
    qp.int8_w4a8_prefill_noalloc(a, w_i8, w_s, got)
    return host(got), host(ref)


def test_noalloc_prefill_matches_caller_scratch_on_two_calls():
    # first call: 4096 x 5120 activations fill 23.6 of the 24 MiB array
    m, n, k = 4096, 256, 5120
    assert (m * k + 255) // 256 * 256 + 4 * m * (k // 32) <= qp.noalloc_scratch_bytes()
    got, ref = _both(m, n, k, 71)
    assert np.array_equal(got, ref)
    # second call, smaller and ragged: it runs over the first call's leftovers
    got, ref = _both(37, 200, 1024, 72)
    assert np.array_equal(got, ref)


def test_noalloc_prefill_refuses_a_problem_beyond_its_array():
    m, n, k = 5000, 128, 5120          # 5000 x 5120 codes alone exceed 24 MiB
    a, w = empty((m, k), torch.bfloat16), empty((n, k), torch.int8)
    ws, out = empty((n, k // 32), torch.float32), empty((m, n), torch.bfloat16)
    before = qp.launch_count()
    with pytest.raises(qp.QProjError) as e:
        qp.int8_w4a8_prefill_noalloc(a, w, ws, out)
    assert e.value.status == qp.QP_ERR_SCRATCH
    assert qp.launch_count() == before
