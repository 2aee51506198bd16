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


def test_q35_tensor_shapes_and_validation():
    """The qwen3_5 DeltaNet tensors' shapes (host only) and rejected configs."""
    import dataclasses
    import layer_sliced_quantized_amd as slq
    import synth
    sh = synth.HYBRID_5120_Q35
    cfg = slq.make_config(sh, synth.Q4_0, 0, 4, max_seq=1024, max_verify=4)
    assert slq.tensor_info(cfg, 0, "dn_conv")["rows"] == sh.conv_dim * sh.dn_conv
    assert slq.tensor_info(cfg, 0, "dn_alog")["rows"] == sh.dn_heads
    assert slq.tensor_info(cfg, 0, "dn_norm")["rows"] == sh.dn_dv
    assert slq.tensor_info(cfg, 0, "dn_q")["rows"] == sh.k_heads * sh.dn_dk
    assert slq.tensor_info(cfg, 0, "dn_v")["rows"] == sh.dn_heads * sh.dn_dv
    with pytest.raises(slq.SliceError):
        slq.tensor_info(slq.make_config(synth.HYBRID_5120, synth.Q4_0, 0, 4), 0, "dn_conv")
    for bad in (dict(dn_conv=5), dict(dn_k_heads=5), dict(dn_dv=32, dn_dk=128), dict(dn_variant=2)):
        with pytest.raises(slq.SliceError):
            slq.tensor_info(slq.make_config(dataclasses.replace(sh, **bad), synth.Q4_0, 0, 4), 0, "dn_q")


def test_draft_head_tensor_shapes_and_validation():
    """The draft head's tensors (host only): the 2H-wide input projection and
    the two input norms; a draft head needs the embedding; a plain slice
    holds none of them."""
    import dataclasses
    import layer_sliced_quantized_amd as slq
    import synth
    base = dataclasses.replace(synth.HYBRID_5120, vocab=2048)
    sh = synth.mtp_shape(base)
    cfg = slq.make_config(sh, synth.Q4_0, 0, 1, max_seq=1024, max_verify=1, has_embed=True, has_head=True,
                          has_mtp=True)
    fc = slq.tensor_info(cfg, 0, "mtp_fc")
    assert (fc["rows"], fc["cols"], fc["kind"]) == (5120, 10240, synth.Q4_0)
    assert fc["src_bytes"] == 5120 * 10240 // 32 * 18
    for n in ("mtp_norm_e", "mtp_norm_h"):
        assert slq.tensor_info(cfg, 0, n) == {"rows": 5120, "cols": 1, "kind": 0, "src_bytes": 4 * 5120}
    assert slq.tensor_info(cfg, 0, "wq")["rows"] == sh.q_heads * sh.head_dim     # its layer is attention
    with pytest.raises(slq.SliceError):   # no embedding
        slq.tensor_info(slq.make_config(sh, synth.Q4_0, 0, 1, has_head=True, has_mtp=True), 0, "mtp_fc")
    with pytest.raises(slq.SliceError):   # not a draft head
        slq.tensor_info(slq.make_config(sh, synth.Q4_0, 0, 1, has_embed=True), 0, "mtp_fc")
    # the weights buffer holds the projection and the norms on top of a plain slice's tensors
    plain = slq.make_config(sh, synth.Q4_0, 0, 1, max_seq=1024, max_verify=1, has_embed=True, has_head=True)
    extra = slq.lib().slice_weights_bytes(ctypes.byref(cfg)) - slq.lib().slice_weights_bytes(ctypes.byref(plain))
    assert fc["src_bytes"] <= extra <= fc["src_bytes"] + 2 * 4 * 5120 + 3 * 256


def test_prompt_pass_width_validation():
    """max_prefill (tokens per prompt pass) is 0..64; past 16 the DeltaNet
    layers must be of the chunked form; the activation buffers grow with it."""
    import dataclasses
    import layer_sliced_quantized_amd as slq
    import synth
    sh = synth.HYBRID_5120

    def ws(**kw):
        cfg = slq.make_config(sh, synth.Q4_0, 0, 4, max_seq=1024, max_verify=4, **kw)
        return slq.lib().slice_workspace_bytes(ctypes.byref(cfg))

    assert ws(max_prefill=64) > ws(max_prefill=16) > ws() > 0
    assert ws(max_prefill=65) == 0 and ws(max_prefill=-1) == 0
    q35 = synth.HYBRID_5120_Q35
    cfg = slq.make_config(q35, synth.Q4_0, 0, 4, max_seq=1024, max_verify=4, max_prefill=32)
    assert slq.lib().slice_workspace_bytes(ctypes.byref(cfg)) == 0
    cfg = slq.make_config(q35, synth.Q4_0, 3, 4, max_seq=1024, max_verify=4, max_prefill=32)   # attention only
    assert slq.lib().slice_workspace_bytes(ctypes.byref(cfg)) > 0


def test_build_refuses_scratch_in_kernels_with_counted_waits():
    """The build parses the compiler's resource-usage remarks and names every
    batched-product kernel that uses scratch (host logic only)."""
    from layer_sliced_quantized_amd import build
    text = ("x.hip:1:1: remark: Function Name: _ZN3slq11k_gemm_diagILi2EEEvv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark: Function Name: _ZN3slq12k_gemm_denseILi8EEEvv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark: Function Name: _ZN3slq6k_gemvILi2EEEvv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.scratch_users(text, "k_gemm_") == [("_ZN3slq12k_gemm_denseILi8EEEvv", 16)]
