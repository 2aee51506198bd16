"""The allocation-free GEMV entry point (slq_gemv_noalloc) against slq_gemv.

Called through the C ABI with ctypes directly.  Its result must equal the
workspace form's bit for bit (same kernels, same launch shapes) and stay
within the products' tolerance of the CPU oracle, on two calls in a row on
one GPU, the second with a smaller input (the static scratch keeps the
previous call's contents), and again after a call of the workspace form.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import qref
from helpers import rel_err

import layer_sliced_quantized_amd as slq
from layer_sliced_quantized_amd import _native

pytestmark = pytest.mark.gpu

LIMIT = 16 << 20


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _noalloc(qtype, packed, rows, cols, x):
    b = x.shape[0]
    y = torch.full((b, rows), float("nan"), dtype=torch.float32, device="cuda")
    rc = _native.lib().slq_gemv_noalloc(qtype, ctypes.c_void_p(packed.data_ptr()), rows, cols, b,
                                        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _native.check(rc)
    return y


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_noalloc_gemv_equals_workspace_gemv(qtype):
    # first call: a larger matrix and batch; second: smaller, with other row
    # groups and splits, on the scratch the first left behind
    calls = [(5120, 17408, 16), (1000, 32 * 37, 3), (200, 32 * 19, 1), (17408, 5120, 5)]
    for i, (rows, cols, batch) in enumerate(calls):
        raw = synth.quant_blocks(synth.stream(41, synth.WL_GEMV, 400 + i, qtype), qtype, rows, cols)
        packed = slq.repack(qtype, _dev(raw), rows, cols)
        x = _dev(synth.gemv_x(42, batch, cols, tag=i))
        y0 = _noalloc(qtype, packed, rows, cols, x).cpu().numpy()
        y1 = slq.gemv(qtype, packed, rows, cols, x).cpu().numpy()
        np.testing.assert_array_equal(y0, y1)
        sample = np.linspace(0, rows - 1, 64).astype(int)
        ref = qref.gemv(qtype, raw[sample], len(sample), cols, x.cpu().numpy().astype(np.float64))
        for t in range(batch):
            assert rel_err(y0[t, sample], ref[t]) <= 1e-5, (i, t)
        # again on the same scratch: the same bits
        np.testing.assert_array_equal(_noalloc(qtype, packed, rows, cols, x).cpu().numpy(), y0)


def test_noalloc_gemv_errors():
    L = _native.lib()
    need = L.slq_gemv_workspace_bytes(synth.Q4_0, 65472, 512 * 1024, 16)
    assert need > LIMIT
    x = torch.zeros(1, device="cuda")
    rc = L.slq_gemv_noalloc(synth.Q4_0, ctypes.c_void_p(x.data_ptr()), 65472, 512 * 1024, 16,
                            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), None)
    assert rc == _native.SLICE_ESHAPE
    assert b"static scratch" in L.slice_last_error()
    rc = L.slq_gemv_noalloc(synth.Q4_0, None, 64, 64, 1, None, None, None)
    assert rc == _native.SLICE_EINVAL
    rc = L.slq_gemv_noalloc(synth.Q4_0, None, 64, 64, 17, None, None, None)
    assert rc == _native.SLICE_ESHAPE
