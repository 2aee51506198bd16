"""GGUF container: the reader against a file assembled byte by byte from the
published layout (independently of the writer), writer/reader round trips of
a slice's tensors, and the rejection of malformed files.  CPU only."""
import struct

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
