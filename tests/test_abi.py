"""The C ABI library loads and exports every entry point of include/slice.h (CPU only).

Only host-side calls are made here (sizes and configuration checks); nothing
touches a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slice.h")
LIB = os.path.join(ROOT, "layer_sliced_quantized_amd", "libslq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libslq.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|void|char)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for n in ("slice_load", "slice_decode", "slice_verify", "slice_commit", "slq_gemv", "slq_repack"):
        assert n in names
    assert len(names) >= 20


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert getattr(L, n) is not None


def test_binding_covers_the_header():
    from layer_sliced_quantized_amd import _native
    assert sorted(_native.exported_names()) == declared_functions()


def test_packed_sizes_match_block_bytes():
    from layer_sliced_quantized_amd import _native
    L = _native.lib()
    for rows, cols in synth.GEMV_SHAPES:
        assert L.slq_packed_bytes(2, rows, cols) == rows * cols // 32 * 18
        assert L.slq_packed_bytes(8, rows, cols) == rows * cols // 32 * 34
    # ragged rows pad to 64-row groups; ragged K adds one scale strip per row group
    assert L.slq_packed_bytes(2, 65, 256) == 2 * 64 * 8 * 18
    assert L.slq_packed_bytes(2, 64, 32 * 19) == 2 * (8 * 1024 + 1024) + (3 * 1024 + 1024)
    assert L.slq_packed_bytes(2, 64, 33) == 0
    assert L.slq_packed_bytes(5, 64, 64) == 0
    assert L.slq_gemv_workspace_bytes(2, 64, 64, 17) == 0


def test_config_validation_and_slice_sizes():
    import layer_sliced_quantized_amd as slq
    from layer_sliced_quantized_amd import _native
    L = _native.lib()
    cfg = slq.make_config(synth.HYBRID_5120, 2, 0, 64, max_seq=1024, max_verify=4)
    wb = L.slice_weights_bytes(ctypes.byref(cfg))
    # 64 layers of Q4_0 weights: 13.41 GB plus alignment and fp32 norm vectors
    mats = sum(r * c for l in range(64) for r, c in synth.matrix_shapes(synth.HYBRID_5120, l).values())
    assert mats * 18 // 32 <= wb <= mats * 18 // 32 + 64 * 6 * 4096 + 64 * 3 * 5120 * 4 + 4096
    assert 13.3e9 < wb < 13.5e9
    ws = L.slice_workspace_bytes(ctypes.byref(cfg))
    assert ws > 48 * 5 * 32 * 128 * 128 * 4      # 48 DeltaNet layers x 5 state slots
    bad = slq.make_config(synth.HYBRID_5120, 3, 0, 64)
    assert L.slice_weights_bytes(ctypes.byref(bad)) == 0
    assert b"qtype" in L.slice_last_error()
    bad = slq.make_config(synth.HYBRID_5120, 2, 0, 65)
    assert L.slice_weights_bytes(ctypes.byref(bad)) == 0
    bad = slq.make_config(synth.HYBRID_5120, 2, 0, 4, max_verify=17)
    assert L.slice_workspace_bytes(ctypes.byref(bad)) == 0
    tiny = slq.make_config(synth.TINY_LLAMA, 2, 0, 30, max_seq=256, has_embed=True, has_head=True)
    assert L.slice_weights_bytes(ctypes.byref(tiny)) > 4096 * 576 * 18 // 32
