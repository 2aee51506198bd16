"""Argument checks of the mixer entry points: rejected on the host, before any
GPU call, with the documented error codes (no device needed)."""
import ctypes

import pytest

SLICE_EINVAL, SLICE_ESHAPE, SLICE_ERANGE = -1, -2, -3
FAKE = ctypes.c_void_p(256)      # never dereferenced: every call below fails its checks first


@pytest.fixture(scope="module")
def lib():
    from layer_sliced_quantized_amd import _native
    return _native.lib()


def _desc(**kw):
    from layer_sliced_quantized_amd import AttnDesc
    d = AttnDesc()
    d.q_heads, d.kv_heads, d.head_dim, d.rope_dims = 24, 4, 256, 64
    d.rope_theta, d.qk_norm, d.has_gate, d.eps, d.max_seq = 1e7, 0, 1, 1e-6, 4096
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("args,code", [
    ((32, 128, 128, 0), SLICE_ERANGE), ((32, 128, 128, 17), SLICE_ERANGE),
    ((32, 48, 128, 1), SLICE_ESHAPE), ((32, 160, 128, 1), SLICE_ESHAPE), ((32, 128, 40, 1), SLICE_ESHAPE),
    ((0, 128, 128, 1), SLICE_ESHAPE),
])
def test_dn_step_rejects(lib, args, code):
    assert lib.slq_dn_step(*args, FAKE, FAKE, FAKE, None) == code


def test_dn_step_null_pointer(lib):
    assert lib.slq_dn_step(32, 128, 128, 1, None, FAKE, FAKE, None) == SLICE_EINVAL
    assert lib.slq_dn_state_layout(32, 128, 128, None, FAKE, 1, None) == SLICE_EINVAL
    assert lib.slq_dn_state_layout(32, 100, 128, FAKE, FAKE, 1, None) == SLICE_ESHAPE


@pytest.mark.parametrize("kw", [dict(q_heads=23), dict(head_dim=96), dict(rope_dims=300), dict(max_seq=100),
                                dict(qk_norm=1)])
def test_attn_rejects_descriptor(lib, kw):
    d = _desc(**kw)
    assert lib.slq_attn_workspace_bytes(ctypes.byref(d), 1) == 0
    assert lib.slq_attn_decode(ctypes.byref(d), 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == SLICE_ESHAPE


def test_attn_rejects_range_and_workspace(lib):
    d = _desc()
    n = lib.slq_attn_workspace_bytes(ctypes.byref(d), 16)
    assert n > lib.slq_attn_workspace_bytes(ctypes.byref(d), 1) > 0
    assert lib.slq_attn_workspace_bytes(ctypes.byref(d), 17) == 0
    call = lambda T, pos, ws: lib.slq_attn_decode(ctypes.byref(d), T, pos, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert call(0, 0, n) == SLICE_ERANGE
    assert call(17, 0, n) == SLICE_ERANGE
    assert call(16, 4096 - 15, n) == SLICE_ERANGE
    assert call(1, -1, n) == SLICE_ERANGE
    assert call(16, 4096 - 16, n - 1) == SLICE_EINVAL
    assert lib.slq_attn_decode(ctypes.byref(d), 1, 0, None, FAKE, FAKE, FAKE, FAKE, n, None) == SLICE_EINVAL
    assert lib.slq_attn_prepare(ctypes.byref(d), FAKE, 16, None) == SLICE_EINVAL


def test_kv_layout_rejects(lib):
    assert lib.slq_kv_layout(4, 4096, 96, 10, FAKE, FAKE, FAKE, FAKE, 1, None) == SLICE_ESHAPE
    assert lib.slq_kv_layout(4, 4000, 256, 10, FAKE, FAKE, FAKE, FAKE, 1, None) == SLICE_ESHAPE
    assert lib.slq_kv_layout(4, 4096, 256, 4097, FAKE, FAKE, FAKE, FAKE, 1, None) == SLICE_ERANGE
    assert lib.slq_kv_layout(4, 4096, 256, 10, None, FAKE, FAKE, FAKE, 1, None) == SLICE_EINVAL
