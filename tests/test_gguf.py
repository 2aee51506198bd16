"""GGUF container: the reader against a file assembled byte by byte from the
published layout (independently of the writer), writer/reader round trips of
a slice's tensors, and the rejection of malformed files.  CPU only."""
import struct

import dataclasses

import numpy as np
import pytest

import synth
from layer_sliced_quantized_amd import gguf


def _s(text: str) -> bytes:
    b = text.encode("utf-8")
    return struct.pack("<Q", len(b)) + b


def _hand_made(path, align=64):
    """Two tensors and four metadata entries, laid out by hand:
    'v' F32 [3] at data offset 0, 'w' Q4_0 2 x 32 (two 18-byte blocks) at the
    next multiple of the alignment."""
    meta = (
        _s("general.architecture") + struct.pack("<I", 8) + _s("tiny") +
        _s("tiny.count") + struct.pack("<II", 4, 7) +
        _s("tiny.list") + struct.pack("<IIQ", 9, 5, 3) + struct.pack("<iii", 1, -2, 3) +
        _s("general.alignment") + struct.pack("<II", 4, align))
    infos = (
        _s("v") + struct.pack("<I", 1) + struct.pack("<Q", 3) + struct.pack("<IQ", 0, 0) +
        _s("w") + struct.pack("<I", 2) + struct.pack("<QQ", 32, 2) + struct.pack("<IQ", 2, align))
    head = b"GGUF" + struct.pack("<IQQ", 3, 2, 4) + meta + infos
    head += b"\0" * (-len(head) % align)
    vdata = struct.pack("<fff", 1.5, -2.0, 3.0)
    # block 0: d = 1.0 (0x3C00), codes 0..15; block 1: d = -0.5 (0xB800), codes 0xFF
    w = struct.pack("<H", 0x3C00) + bytes(range(16)) + struct.pack("<H", 0xB800) + b"\xff" * 16
    data = vdata + b"\0" * (align - len(vdata)) + w
    with open(path, "wb") as fh:
        fh.write(head + data)
    return w


def test_reader_on_hand_made_file(tmp_path):
    p = tmp_path / "hand.gguf"
    w = _hand_made(p)
    g = gguf.GGUFFile(str(p))
    assert g.version == 3
    assert g.metadata == {"general.architecture": "tiny", "tiny.count": 7, "tiny.list": [1, -2, 3],
                          "general.alignment": 64}
    assert g.alignment == 64 and g.data_start % 64 == 0
    assert g.tensors["v"].dims == (3,) and g.tensors["v"].ttype == gguf.T_F32
    assert g.tensors["w"].dims == (32, 2) and g.tensors["w"].shape == (2, 32)
    assert g.tensors["w"].offset == 64 and g.tensors["w"].nbytes == 36
    np.testing.assert_array_equal(g.array("v"), np.array([1.5, -2.0, 3.0], dtype=np.float32))
    assert bytes(g.raw("w")) == w
    assert g.array("w").shape == (2, 18)


def test_sizes_of_the_block_formats():
    assert gguf.tensor_nbytes(gguf.T_Q4_0, (5120, 17408)) == 17408 * 160 * 18
    assert gguf.tensor_nbytes(gguf.T_Q8_0, (5120, 17408)) == 17408 * 160 * 34
    assert gguf.tensor_nbytes(gguf.T_F16, (7, 3)) == 42
    with pytest.raises(gguf.GGUFError):
        gguf.tensor_nbytes(gguf.T_Q4_0, (48, 2))      # rows of 48 are not whole blocks
    with pytest.raises(gguf.GGUFError):
        gguf.tensor_nbytes(3, (32,))                   # a type the slice does not take


SHAPE = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)


def gguf_tensors(shape, tensors, qtype):
    """The slice's tensors under the default GGUF names, as write_gguf takes them."""
    qt = gguf.T_Q4_0 if qtype == synth.Q4_0 else gguf.T_Q8_0
    out = {}
    for l, d in tensors.items():
        mats = synth.matrix_shapes(shape, l)
        for name, arr in d.items():
            key = gguf.DEFAULT_NAMES[name].format(l=l)
            if name in mats:
                rows, cols = mats[name]
                out[key] = (qt, (cols, rows), arr.tobytes())
            else:
                out[key] = np.asarray(arr, dtype=np.float32)
    return out


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
@pytest.mark.parametrize("align", [32, 256])
def test_round_trip_of_slice_tensors(tmp_path, qtype, align):
    tensors = {l: synth.layer_tensors(SHAPE, qtype, 3, 91, l) for l in range(4)}
    p = tmp_path / "slice.gguf"
    gguf.write_gguf(str(p), {"general.architecture": "tiny_hybrid"}, gguf_tensors(SHAPE, tensors, qtype), alignment=align)
    g = gguf.GGUFFile(str(p))
    assert g.alignment == align
    for l in range(4):
        back = gguf.slice_tensors(g, l)
        assert set(back) == set(tensors[l])
        for name, arr in tensors[l].items():
            assert np.asarray(back[name]).tobytes() == np.asarray(arr).tobytes(), (l, name)


def test_malformed_files_are_rejected(tmp_path):
    p = tmp_path / "hand.gguf"
    _hand_made(p)
    good = p.read_bytes()
    bad = tmp_path / "bad.gguf"
    bad.write_bytes(b"GGUG" + good[4:])
    with pytest.raises(gguf.GGUFError):
        gguf.GGUFFile(str(bad))
    # w's offset 64 -> 65: not a multiple of the alignment
    raw = bytearray(good)
    k = raw.index(_s("w"))
    off_pos = k + len(_s("w")) + 4 + 16 + 4
    raw[off_pos:off_pos + 8] = struct.pack("<Q", 65)
    bad.write_bytes(bytes(raw))
    with pytest.raises(gguf.GGUFError):
        gguf.GGUFFile(str(bad))
    # the data section cut short
    bad.write_bytes(good[:-10])
    with pytest.raises(gguf.GGUFError):
        gguf.GGUFFile(str(bad))


def test_metadata_of_every_value_type_round_trips(tmp_path):
    # one key per GGUF value type (0..12 except the array marker), plus arrays
    # of strings and of floats, and an empty array
    meta = {
        "u8": (200, gguf.V_U8), "i8": (-100, gguf.V_I8), "u16": (60000, gguf.V_U16), "i16": (-30000, gguf.V_I16),
        "u32": (4000000000, gguf.V_U32), "i32": (-2000000000, gguf.V_I32), "f32": (1.5, gguf.V_F32),
        "bool": (True, gguf.V_BOOL), "str": ("Grüße", gguf.V_STR), "u64": (2 ** 63 + 5, gguf.V_U64),
        "i64": (-(2 ** 62), gguf.V_I64), "f64": (0.1, gguf.V_F64),
        "names": (["a", "bc", ""], gguf.V_STR), "scales": ([0.5, -2.0, 3.25], gguf.V_F32), "none": ([], gguf.V_I32),
    }
    path = tmp_path / "meta.gguf"
    gguf.write_gguf(str(path), meta, {})
    g = gguf.GGUFFile(str(path))
    assert g.tensors == {}
    for k, (v, _) in meta.items():
        got = g.metadata[k]
        if isinstance(v, list):
            assert list(got) == v, k
        else:
            assert got == v, k


# --------------------------------------- files checked against a slice config

_LIB = __import__("os").path.join(__import__("os").path.dirname(__import__("os").path.dirname(
    __import__("os").path.abspath(__file__))), "layer_sliced_quantized_amd", "libslq.so")
needs_lib = pytest.mark.skipif(not __import__("os").path.exists(_LIB), reason="libslq.so not built")


def _cfg(qtype=synth.Q4_0):
    import layer_sliced_quantized_amd as slq
    return slq.make_config(SHAPE, qtype, 0, 4, max_seq=256, max_verify=4, io_fp32=True)


@needs_lib
@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_well_formed_file_passes_the_config_check(tmp_path, qtype):
    tensors = {l: synth.layer_tensors(SHAPE, qtype, 0, 93, l) for l in range(4)}
    p = tmp_path / "ok.gguf"
    gguf.write_gguf(str(p), {}, gguf_tensors(SHAPE, tensors, qtype))
    todo = gguf.check_against_config(gguf.GGUFFile(str(p)), _cfg(qtype))
    assert len(todo) == sum(len(d) for d in tensors.values())


def _mutated_file(tmp_path, key, value):
    tensors = {l: synth.layer_tensors(SHAPE, synth.Q4_0, 0, 93, l) for l in range(4)}
    t = gguf_tensors(SHAPE, tensors, synth.Q4_0)
    t[key] = value
    p = tmp_path / "bad.gguf"
    gguf.write_gguf(str(p), {}, t)
    return gguf.GGUFFile(str(p))


@needs_lib
def test_misshaped_or_misformatted_tensors_are_refused(tmp_path):
    """A real file with other head counts, an F16 or Q8_0 matrix where the
    slice holds Q4_0, or a vector of the wrong length is refused by the host
    check, before any byte reaches the GPU (no GPU is used here)."""
    cases = {
        # 3 DeltaNet heads' worth of q rows (192) where the slice has 2 heads (128)
        "blk.0.dn_q.weight": (gguf.T_Q4_0, (128, 192), bytes(192 * 4 * 18)),
        # the right shape in F16
        "blk.0.dn_k.weight": (gguf.T_F16, (128, 128), bytes(128 * 128 * 2)),
        # the right shape in another block format
        "blk.3.attn_q.weight": (gguf.T_Q8_0, (128, 256), bytes(256 * 4 * 34)),
        # the FFN down projection stored transposed (256 x 128 instead of 128 x 256)
        "blk.1.ffn_down.weight": (gguf.T_Q4_0, (128, 256), bytes(256 * 4 * 18)),
        # a norm vector of the wrong length
        "blk.2.attn_norm.weight": np.ones(64, np.float32),
    }
    for key, val in cases.items():
        g = _mutated_file(tmp_path, key, val)
        with pytest.raises(gguf.GGUFError) as e:
            gguf.check_against_config(g, _cfg())
        assert key in str(e.value)


@needs_lib
def test_tensor_info_and_overrides_are_host_only():
    import layer_sliced_quantized_amd as slq
    cfg = _cfg()
    assert slq.tensor_info(cfg, 0, "dn_q") == {"rows": 128, "cols": 128, "kind": 2, "src_bytes": 128 * 4 * 18}
    assert slq.tensor_info(cfg, 3, "wo") == {"rows": 128, "cols": 256, "kind": 2, "src_bytes": 128 * 8 * 18}
    assert slq.tensor_info(cfg, 1, "w_down")["cols"] == 256
    assert slq.tensor_info(cfg, 3, "q_norm") == {"rows": 64, "cols": 1, "kind": 0, "src_bytes": 256}
    with pytest.raises(slq.SliceError):
        slq.tensor_info(cfg, 3, "dn_q")          # an attention layer has no DeltaNet tensors
    with pytest.raises(slq.SliceError):
        slq.tensor_info(cfg, 4, "attn_norm")     # outside the layer range
    with pytest.raises(slq.SliceError):
        slq.tensor_info(cfg, 0, "embed")         # no embedding in this slice
    slq.debug_override("KS_F1", 3)
    slq.debug_override("KS_F1", -1)
    with pytest.raises(slq.SliceError):
        slq.debug_override("KS_NOPE", 1)
    with slq.overrides(MFMA_MIN_T=2, EAGER=1):
        pass


SHAPE_Q35 = dataclasses.replace(SHAPE, name="tiny_hybrid_q35_128", dn_heads=4, dn_variant=1, dn_k_heads=2, dn_conv=4)


@needs_lib
def test_q35_file_round_trip_and_config_check(tmp_path):
    """A qwen3_5-form slice's tensors (conv taps, A_log, dt_bias, gated-norm
    weights and the narrower q/k projections) survive a GGUF round trip and
    pass the shape check; the plain form's config refuses them."""
    import layer_sliced_quantized_amd as slq
    tensors = {l: synth.layer_tensors(SHAPE_Q35, synth.Q4_0, 0, 97, l) for l in range(4)}
    assert {"dn_conv", "dn_alog", "dn_dtb", "dn_norm"} <= set(tensors[0])
    p = tmp_path / "q35.gguf"
    gguf.write_gguf(str(p), {}, gguf_tensors(SHAPE_Q35, tensors, synth.Q4_0))
    g = gguf.GGUFFile(str(p))
    for l in range(4):
        back = gguf.slice_tensors(g, l)
        for name, arr in tensors[l].items():
            np.testing.assert_array_equal(np.asarray(back[name]).reshape(-1).view(np.uint8),
                                          np.asarray(arr).reshape(-1).view(np.uint8))
    cfg = slq.make_config(SHAPE_Q35, synth.Q4_0, 0, 4, max_seq=256, max_verify=4, io_fp32=True)
    assert len(gguf.check_against_config(g, cfg)) == sum(len(d) for d in tensors.values())
    with pytest.raises(gguf.GGUFError):
        gguf.check_against_config(g, _cfg())



def draft_head_gguf_tensors(base, T, M, G, qtype):
    """A draft head's tensors under the "mtp." names (its layer T, its own
    tensors M) and the model's embedding and untied head (G), as write_gguf
    takes them."""
    qt = gguf.T_Q4_0 if qtype == synth.Q4_0 else gguf.T_Q8_0
    sh = synth.mtp_shape(base)
    H = sh.hidden
    mats = synth.matrix_shapes(sh, 0)
    out = {}
    for name, arr in T.items():
        key = gguf.MTP_NAMES[name]
        out[key] = (qt, tuple(reversed(mats[name])), arr.tobytes()) if name in mats else np.asarray(arr, np.float32)
    out["mtp.fc.weight"] = (qt, (2 * H, H), M["mtp_fc"].tobytes())
    out["mtp.norm_e.weight"] = M["mtp_norm_e"]
    out["mtp.norm_h.weight"] = M["mtp_norm_h"]
    out["mtp.output_norm.weight"] = M["mtp_out_norm"]
    out["token_embd.weight"] = (qt, (H, base.vocab), G["embed"].tobytes())
    out["output.weight"] = (qt, (H, base.vocab), G["head"].tobytes())
    return out


def test_draft_head_file_names_and_config_check(tmp_path):
    """A draft head stored under "mtp." beside a model: its layer, input
    projection, norms and final norm, with the model's embedding and head;
    the draft head's configuration takes exactly those, a plain stage of the
    model none of them."""
    import dataclasses
    import layer_sliced_quantized_amd as slq
    base = dataclasses.replace(SHAPE, vocab=64, tied_head=False)
    sh = synth.mtp_shape(base)
    T = synth.layer_tensors(sh, synth.Q4_0, 0, synth.WL_MTP, 0)
    M = synth.mtp_tensors(sh, synth.Q4_0, 0)
    G = synth.global_tensors(base, synth.Q4_0, 0, 91)
    p = tmp_path / "draft.gguf"
    gguf.write_gguf(str(p), {}, draft_head_gguf_tensors(base, T, M, G, synth.Q4_0))
    g = gguf.GGUFFile(str(p))
    # the arrays read back are the ones written
    np.testing.assert_array_equal(g.array("mtp.fc.weight").reshape(-1), M["mtp_fc"].reshape(-1))
    np.testing.assert_array_equal(g.array("mtp.norm_h.weight"), M["mtp_norm_h"])
    cfg = slq.make_config(sh, synth.Q4_0, 0, 1, max_seq=64, max_verify=1, has_embed=True, has_head=True,
                          has_mtp=True)
    todo = gguf.check_against_config(g, cfg, gguf.MTP_NAMES)
    assert {o for o, _, _ in todo} == set(T) | {"mtp_fc", "mtp_norm_e", "mtp_norm_h", "out_norm", "embed", "head"}
    assert all(l == 0 for _, l, _ in todo)
    # a plain stage reading the same file with the model's names loads nothing of the draft head
    plain = slq.make_config(base, synth.Q4_0, 0, 4, has_embed=True, has_head=True)
    assert {k for _, _, k in gguf.check_against_config(g, plain)} == {"token_embd.weight", "output.weight"}
    # the draft head's names refused by a slice that is not a draft head
    nomtp = slq.make_config(sh, synth.Q4_0, 0, 1, max_seq=64, max_verify=1, has_embed=True, has_head=True)
    assert not {o for o, _, _ in gguf.check_against_config(g, nomtp, gguf.MTP_NAMES)} & {"mtp_fc", "mtp_norm_e", "mtp_norm_h"}

