"""GGUF container: read (memory-mapped), write, and load into a slice.

The pages ship their weights as GGUF files with Q4_0 / Q8_0 blocks (SwarmLLM
README, model table; its engine parses GGUF in ``gguf.js``).  This module
implements the container as published with ggml, version 3, little-endian:

* header: magic ``GGUF``, uint32 version, uint64 tensor count, uint64
  metadata count;
* metadata entries: key (uint64 byte length + UTF-8 bytes), uint32 value type,
  value.  Value types: 0 u8, 1 i8, 2 u16, 3 i16, 4 u32, 5 i32, 6 f32, 7 bool,
  8 string, 9 array (uint32 element type, uint64 count, elements), 10 u64,
  11 i64, 12 f64;
* tensor infos: name (string), uint32 dimension count, uint64 dims (dims[0]
  varies fastest, so a rows x cols matrix is (cols, rows)), uint32 tensor
  type, uint64 offset into the data section;
* data section: starts at the first multiple of ``general.alignment``
  (default 32) after the tensor infos; every offset is a multiple of it.

Tensor types used by the slice: 0 F32, 1 F16, 2 Q4_0 (18 bytes per 32
weights), 8 Q8_0 (34 bytes per 32 weights).  Quantised tensors are handed to
the slice as their raw GGUF blocks, which ``slice_set_tensor`` repacks once.

Host-side only: nothing here runs on the decode path.
"""
from __future__ import annotations

import dataclasses
import struct

import numpy as np

MAGIC = b"GGUF"
VERSION = 3
DEFAULT_ALIGNMENT = 32

T_F32, T_F16, T_Q4_0, T_Q8_0 = 0, 1, 2, 8
_BLOCK = {T_Q4_0: (32, 18), T_Q8_0: (32, 34)}   # (weights, bytes) per block
_ELEM = {T_F32: 4, T_F16: 2}

V_U8, V_I8, V_U16, V_I16, V_U32, V_I32, V_F32, V_BOOL, V_STR, V_ARR, V_U64, V_I64, V_F64 = range(13)
_SCALAR = {V_U8: "<B", V_I8: "<b", V_U16: "<H", V_I16: "<h", V_U32: "<I", V_I32: "<i", V_F32: "<f",
           V_BOOL: "<?", V_U64: "<Q", V_I64: "<q", V_F64: "<d"}


class GGUFError(ValueError):
    pass


def tensor_nbytes(ttype: int, dims) -> int:
    n = 1
    for d in dims:
        n *= int(d)
    if ttype in _ELEM:
        return n * _ELEM[ttype]
    if ttype in _BLOCK:
        per, nb = _BLOCK[ttype]
        if int(dims[0]) % per:
            raise GGUFError(f"row length {dims[0]} is not a multiple of {per}")
        return n // per * nb
    raise GGUFError(f"tensor type {ttype} is not supported (F32, F16, Q4_0, Q8_0)")


@dataclasses.dataclass
class TensorInfo:
    name: str
    dims: tuple          # GGUF order: dims[0] fastest
    ttype: int
    offset: int          # from the start of the data section
    nbytes: int

    @property
    def shape(self) -> tuple:
        """NumPy order (slowest first): (rows, cols) for a matrix."""
        return tuple(reversed(self.dims))


class _Cursor:
    def __init__(self, buf):
        self.buf = buf
        self.pos = 0

    def take(self, n: int) -> bytes:
        if self.pos + n > len(self.buf):
            raise GGUFError("file ends inside the header or tensor infos")
        b = bytes(self.buf[self.pos:self.pos + n])
        self.pos += n
        return b

    def unpack(self, fmt: str):
        return struct.unpack(fmt, self.take(struct.calcsize(fmt)))[0]

    def string(self) -> str:
        n = self.unpack("<Q")
        return self.take(n).decode("utf-8")

    def value(self, vtype: int):
        if vtype in _SCALAR:
            return self.unpack(_SCALAR[vtype])
        if vtype == V_STR:
            return self.string()
        if vtype == V_ARR:
            etype = self.unpack("<I")
            count = self.unpack("<Q")
            return [self.value(etype) for _ in range(count)]
        raise GGUFError(f"unknown metadata value type {vtype}")


class GGUFFile:
    """A parsed GGUF file; tensor data stay in a memory map of the file."""

    def __init__(self, path: str):
        self.path = path
        # copy-on-write: views are writable (as torch.from_numpy wants) and the
        # file is never modified
        self._map = np.memmap(path, dtype=np.uint8, mode="c")
        cur = _Cursor(self._map)
        if cur.take(4) != MAGIC:
            raise GGUFError(f"{path}: not a GGUF file (magic)")
        self.version = cur.unpack("<I")
        if self.version not in (2, 3):
            raise GGUFError(f"{path}: GGUF version {self.version} is not supported")
        n_tensors = cur.unpack("<Q")
        n_kv = cur.unpack("<Q")
        self.metadata: dict = {}
        for _ in range(n_kv):
            key = cur.string()
            self.metadata[key] = cur.value(cur.unpack("<I"))
        self.alignment = int(self.metadata.get("general.alignment", DEFAULT_ALIGNMENT))
        if self.alignment <= 0 or self.alignment & (self.alignment - 1):
            raise GGUFError(f"{path}: alignment {self.alignment} is not a power of two")
        self.tensors: dict[str, TensorInfo] = {}
        for _ in range(n_tensors):
            name = cur.string()
            nd = cur.unpack("<I")
            dims = tuple(cur.unpack("<Q") for _ in range(nd))
            ttype = cur.unpack("<I")
            off = cur.unpack("<Q")
            if off % self.alignment:
                raise GGUFError(f"{path}: tensor {name} offset {off} is not aligned")
            self.tensors[name] = TensorInfo(name, dims, ttype, off, tensor_nbytes(ttype, dims))
        self.data_start = -(-cur.pos // self.alignment) * self.alignment
        for t in self.tensors.values():
            if self.data_start + t.offset + t.nbytes > len(self._map):
                raise GGUFError(f"{path}: tensor {t.name} runs past the end of the file")

    def raw(self, name: str) -> np.ndarray:
        """The tensor's bytes as stored (uint8, memory-mapped)."""
        t = self.tensors[name]
        a = self.data_start + t.offset
        return self._map[a:a + t.nbytes]

    def array(self, name: str) -> np.ndarray:
        """F32 / F16 tensors as float32 in NumPy order; quantised tensors as their
        raw blocks [rows][cols / 32 * block bytes]."""
        t = self.tensors[name]
        r = self.raw(name)
        if t.ttype == T_F32:
            return np.asarray(r).view("<f4").reshape(t.shape)
        if t.ttype == T_F16:
            return np.asarray(r).view("<f2").astype(np.float32).reshape(t.shape)
        rows = int(np.prod(t.shape[:-1])) if len(t.shape) > 1 else 1
        return np.asarray(r).reshape(rows, -1)


def _pack_value(v, vtype: int) -> bytes:
    if vtype in _SCALAR:
        return struct.pack(_SCALAR[vtype], v)
    if vtype == V_STR:
        b = v.encode("utf-8")
        return struct.pack("<Q", len(b)) + b
    raise GGUFError(f"cannot write value type {vtype}")


def _guess_type(v):
    if isinstance(v, bool):
        return V_BOOL
    if isinstance(v, int):
        return V_U32 if 0 <= v < 2**32 else V_I64
    if isinstance(v, float):
        return V_F32
    if isinstance(v, str):
        return V_STR
    raise GGUFError(f"cannot infer a GGUF type for {v!r}")


def write_gguf(path: str, metadata: dict, tensors: dict, alignment: int = DEFAULT_ALIGNMENT) -> None:
    """Write a GGUF v3 file.  metadata: {key: value or (value, vtype)}; lists
    are written as arrays of their first element's type.  tensors: {name:
    (ttype, dims, bytes-like)} with dims in GGUF order, or a float32 array
    (written as F32)."""
    meta = dict(metadata)
    if alignment != DEFAULT_ALIGNMENT:
        meta["general.alignment"] = (alignment, V_U32)
    out = bytearray()
    out += MAGIC + struct.pack("<IQQ", VERSION, len(tensors), len(meta))
    for key, v in meta.items():
        kb = key.encode("utf-8")
        out += struct.pack("<Q", len(kb)) + kb
        vtype = v[1] if isinstance(v, tuple) else None
        v = v[0] if isinstance(v, tuple) else v
        if isinstance(v, list):
            et = vtype if vtype is not None else _guess_type(v[0])
            out += struct.pack("<IIQ", V_ARR, et, len(v))
            for e in v:
                out += _pack_value(e, et)
        else:
            vtype = vtype if vtype is not None else _guess_type(v)
            out += struct.pack("<I", vtype) + _pack_value(v, vtype)
    blobs = []
    off = 0
    for name, spec in tensors.items():
        if isinstance(spec, np.ndarray):
            a = np.ascontiguousarray(spec, dtype="<f4")
            spec = (T_F32, tuple(reversed(a.shape)), a.tobytes())
        ttype, dims, data = spec
        data = bytes(data)
        if len(data) != tensor_nbytes(ttype, dims):
            raise GGUFError(f"tensor {name}: {len(data)} bytes for dims {dims} type {ttype}")
        nb = name.encode("utf-8")
        out += struct.pack("<Q", len(nb)) + nb + struct.pack("<I", len(dims))
        out += b"".join(struct.pack("<Q", int(d)) for d in dims)
        out += struct.pack("<IQ", ttype, off)
        blobs.append((off, data))
        off = -(-(off + len(data)) // alignment) * alignment
    out += b"\0" * (-len(out) % alignment)
    start = len(out)
    out += b"\0" * off
    for o, data in blobs:
        out[start + o:start + o + len(data)] = data
    with open(path, "wb") as fh:
        fh.write(out)


# The slice's tensor names -> GGUF tensor names ({l}: layer index).  The
# Llama-style tensors follow the names llama.cpp gives them; the hybrid's
# DeltaNet projections and attention gate have no name on the pages, and the
# names below are this library's own.  Pass another map for other files.
DEFAULT_NAMES = {
    "attn_norm": "blk.{l}.attn_norm.weight",
    "ffn_norm": "blk.{l}.ffn_norm.weight",
    "wq": "blk.{l}.attn_q.weight",
    "wk": "blk.{l}.attn_k.weight",
    "wv": "blk.{l}.attn_v.weight",
    "wo": "blk.{l}.attn_output.weight",
    "wg": "blk.{l}.attn_gate.weight",
    "q_norm": "blk.{l}.attn_q_norm.weight",
    "k_norm": "blk.{l}.attn_k_norm.weight",
    "dn_q": "blk.{l}.dn_q.weight",
    "dn_k": "blk.{l}.dn_k.weight",
    "dn_v": "blk.{l}.dn_v.weight",
    "dn_a": "blk.{l}.dn_a.weight",
    "dn_b": "blk.{l}.dn_b.weight",
    "dn_z": "blk.{l}.dn_z.weight",
    "dn_out": "blk.{l}.dn_out.weight",
    "dn_conv": "blk.{l}.dn_conv.weight",
    "dn_alog": "blk.{l}.dn_a_log",
    "dn_dtb": "blk.{l}.dn_dt_bias",
    "dn_norm": "blk.{l}.dn_norm.weight",
    "w_gate": "blk.{l}.ffn_gate.weight",
    "w_up": "blk.{l}.ffn_up.weight",
    "w_down": "blk.{l}.ffn_down.weight",
    "embed": "token_embd.weight",
    "head": "output.weight",
    "out_norm": "output_norm.weight",
}
_GLOBAL = ("embed", "head", "out_norm", "mtp_fc", "mtp_norm_e", "mtp_norm_h")
_MTP = ("mtp_fc", "mtp_norm_e", "mtp_norm_h")

# A draft head (a slice with has_mtp: one layer plus its input projection and
# norms) stored in the same file under "mtp.": its layer's tensors take the
# layer names above with "mtp." for "blk.{l}.", its final norm is
# "mtp.output_norm.weight", and it shares the model's embedding and head.
# These names are this library's own, like the hybrid's above.
MTP_NAMES = {
    **{k: v.replace("blk.{l}.", "mtp.") for k, v in DEFAULT_NAMES.items() if v.startswith("blk.{l}.")},
    "mtp_fc": "mtp.fc.weight",
    "mtp_norm_e": "mtp.norm_e.weight",
    "mtp_norm_h": "mtp.norm_h.weight",
    "out_norm": "mtp.output_norm.weight",
    "embed": "token_embd.weight",
    "head": "output.weight",
}


def slice_tensors(g: GGUFFile, layer: int, names: dict = DEFAULT_NAMES) -> dict:
    """{slice name: array} of one layer's tensors present in the file."""
    out = {}
    for ours, theirs in names.items():
        if ours in _GLOBAL:
            continue
        key = theirs.format(l=layer)
        if key in g.tensors:
            out[ours] = g.array(key)
    return out


def check_against_config(g: GGUFFile, cfg, names: dict = DEFAULT_NAMES) -> list:
    """Check every tensor the file holds for cfg's layer range (and its
    embedding / head / output norm when the slice has them) against the shape
    and format the slice expects (slice_tensor_info, host only).  Returns the
    [(slice name, layer, GGUF name)] that would be loaded; raises GGUFError on
    the first mismatch, before anything touches the GPU."""
    from . import tensor_info, SliceError
    todo = []
    for ours in _GLOBAL:
        key = names.get(ours)
        if not key or key not in g.tensors:
            continue
        if ours == "embed" and not (cfg.has_embed or (cfg.has_head and cfg.tied_head)):
            continue
        if ours in ("head", "out_norm") and not cfg.has_head:
            continue
        if ours in _MTP and not cfg.has_mtp:
            continue
        todo.append((ours, 0, key))
    for layer in range(cfg.layer_begin, cfg.layer_end):
        for ours, theirs in names.items():
            key = theirs.format(l=layer)
            if ours not in _GLOBAL and key in g.tensors:
                todo.append((ours, layer, key))
    for ours, layer, key in todo:
        info = g.tensors[key]
        try:
            want = tensor_info(cfg, layer, ours)
        except SliceError as e:
            raise GGUFError(f"{key}: not part of this slice ({e})") from None
        if want["kind"] == 0:
            ok = info.ttype == T_F32 and tuple(int(d) for d in info.dims) == (want["rows"],)
            what = f"F32 vector of {want['rows']}"
        else:
            ok = info.ttype == want["kind"] and tuple(int(d) for d in info.dims) == (want["cols"], want["rows"])
            what = f"type {want['kind']} matrix of {want['rows']} x {want['cols']}"
        if not ok:
            raise GGUFError(f"{key}: type {info.ttype} with dims {tuple(info.dims)}; the slice needs a {what}")
        if tensor_nbytes(info.ttype, info.dims) != want["src_bytes"]:
            raise GGUFError(f"{key}: {tensor_nbytes(info.ttype, info.dims)} bytes, the slice needs {want['src_bytes']}")
    return todo


def load_into_slice(s, g: GGUFFile, names: dict = DEFAULT_NAMES) -> int:
    """Stream the file's tensors for s's layer range (and its embedding / head
    when the slice has them) into the slice.  Every tensor is checked against
    the slice's configuration first (check_against_config); a file with a
    tensor of another shape or format is refused before any upload.  Returns
    the number of tensors loaded."""
    todo = check_against_config(g, s.cfg, names)
    glob = {o: g.array(k) for o, _, k in todo if o in _GLOBAL}
    n = 0
    for layer in range(s.cfg.layer_begin, s.cfg.layer_end):
        d = {o: g.array(k) for o, l, k in todo if l == layer and o not in _GLOBAL}
        s.load_numpy({layer: d})
        n += len(d)
    if glob:
        s.load_numpy({}, glob)
        n += len(glob)
    return n
