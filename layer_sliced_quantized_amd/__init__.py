"""Layer-sliced, block-quantised single-token decode on AMD MI355X (gfx950).

Python front end of libslq (include/slice.h).  The functions and the Slice
class marshal arguments for the C ABI; the work itself runs in libslq's HIP
kernels on the caller's current torch stream.  Without the built library every
call raises.
"""
from __future__ import annotations

import contextlib
import ctypes

import numpy as np
import torch

from ._native import (Q4_0, Q8_0, TENSOR_IDS, AttnDesc, SliceConfig, SliceError, check, lib)  # noqa: F401

__all__ = ["Q4_0", "Q8_0", "SliceConfig", "SliceError", "Slice", "make_config", "tensor_info",
           "packed_bytes", "repack", "dequant", "gemv", "gemv_workspace_bytes", "debug_override",
           "overrides", "read_probe", "dn_step", "dn_state_to_lib", "dn_state_from_lib", "AttnDecoder", "lib"]


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(arr, device="cuda") -> torch.Tensor:
    """numpy array -> contiguous device tensor with the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


# ------------------------------------------------------------ kernel level

def packed_bytes(qtype: int, rows: int, cols: int) -> int:
    return int(lib().slq_packed_bytes(qtype, rows, cols))


def repack(qtype: int, raw: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    """GGUF blocks (uint8 device tensor) -> packed device layout."""
    n = packed_bytes(qtype, rows, cols)
    if n == 0:
        raise SliceError(-2, "bad qtype or shape")
    out = torch.empty(n, dtype=torch.uint8, device=raw.device)
    check(lib().slq_repack(qtype, _ptr(raw), rows, cols, _ptr(out), _stream(stream)))
    return out


def dequant(qtype: int, packed: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    out = torch.empty((rows, cols), dtype=torch.float32, device=packed.device)
    check(lib().slq_dequant(qtype, _ptr(packed), rows, cols, _ptr(out), _stream(stream)))
    return out


def gemv_workspace_bytes(qtype: int, rows: int, cols: int, batch: int) -> int:
    return int(lib().slq_gemv_workspace_bytes(qtype, rows, cols, batch))


def gemv(qtype: int, packed: torch.Tensor, rows: int, cols: int, x: torch.Tensor,
         out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = W x for x fp32 [batch, cols] (batch <= 16) -> y fp32 [batch, rows]."""
    x2 = x.reshape(-1, cols)
    b = x2.shape[0]
    if out is None:
        out = torch.empty((b, rows), dtype=torch.float32, device=x.device)
    need = gemv_workspace_bytes(qtype, rows, cols, b)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=x.device)
    check(lib().slq_gemv(qtype, _ptr(packed), rows, cols, b, _ptr(x2), _ptr(out), _ptr(ws), ws.numel(),
                         _stream(stream)))
    return out


def debug_override(name: str, value: int) -> None:
    """Set a launch-shape override (value < 0 removes it); see slq_debug_override."""
    check(lib().slq_debug_override(name.encode(), int(value)))


@contextlib.contextmanager
def overrides(**kw):
    """Launch-shape overrides for the duration of a with-block, e.g.
    ``with overrides(MFMA_MIN_T=2, KS_GEMV=3): ...``; removed afterwards."""
    for k, v in kw.items():
        debug_override(k, v)
    try:
        yield
    finally:
        for k in kw:
            debug_override(k, -1)


READ_PROBE_GRID = 16384    # SLQ_READ_PROBE_GRID: most workgroups of slq_read_probe


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One streaming read of buf's bytes (slq_read_probe); sink: >= 4 * READ_PROBE_GRID int32."""
    check(lib().slq_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


# ------------------------------------------------- mixers on caller buffers

def dn_state_to_lib(S: torch.Tensor, stream=None) -> torch.Tensor:
    """Canonical fp32 [heads][dv][dk] state (device) -> the library's layout."""
    heads, dv, dk = S.shape
    S = S.contiguous()
    out = torch.empty_like(S)
    check(lib().slq_dn_state_layout(heads, dk, dv, _ptr(S), _ptr(out), 1, _stream(stream)))
    return out


def dn_state_from_lib(S_lib: torch.Tensor, heads: int, dk: int, dv: int, stream=None) -> torch.Tensor:
    out = torch.empty((heads, dv, dk), dtype=torch.float32, device=S_lib.device)
    check(lib().slq_dn_state_layout(heads, dk, dv, _ptr(out), _ptr(S_lib), 0, _stream(stream)))
    return out


def dn_step(heads: int, dk: int, dv: int, inp: torch.Tensor, state_lib: torch.Tensor,
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """T Gated DeltaNet tokens (slq_dn_step): inp fp32 [T][q|k|v|a|b|z], state in the
    library's layout, updated in place.  Returns out fp32 [T][heads*dv]."""
    T = inp.shape[0]
    if out is None:
        out = torch.empty((T, heads * dv), dtype=torch.float32, device=inp.device)
    check(lib().slq_dn_step(heads, dk, dv, T, _ptr(inp), _ptr(state_lib), _ptr(out), _stream(stream)))
    return out


class AttnDecoder:
    """Decode attention on caller buffers (slq_attn_decode): the descriptor,
    the workspace (RoPE table, partials) and fp16 K/V caches in the library's
    layout, all device memory from torch."""

    def __init__(self, q_heads, kv_heads, head_dim, rope_dims, rope_theta, qk_norm, has_gate, eps, max_seq,
                 q_norm=None, k_norm=None, t_max=16, device="cuda", stream=None):
        self.device = torch.device(device)
        self.q_norm = None if q_norm is None else torch.as_tensor(q_norm, dtype=torch.float32).to(self.device)
        self.k_norm = None if k_norm is None else torch.as_tensor(k_norm, dtype=torch.float32).to(self.device)
        d = AttnDesc()
        d.q_heads, d.kv_heads, d.head_dim, d.rope_dims = q_heads, kv_heads, head_dim, rope_dims
        d.rope_theta, d.qk_norm, d.has_gate, d.eps, d.max_seq = float(rope_theta), int(qk_norm), int(has_gate), \
            float(eps), max_seq
        d.q_norm_dev = self.q_norm.data_ptr() if self.q_norm is not None else None
        d.k_norm_dev = self.k_norm.data_ptr() if self.k_norm is not None else None
        self.desc = d
        n = int(lib().slq_attn_workspace_bytes(ctypes.byref(d), t_max))
        if n == 0:
            check(-2)
        self.ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        check(lib().slq_attn_prepare(ctypes.byref(d), _ptr(self.ws), n, _stream(stream)))
        shape = (kv_heads * max_seq * head_dim,)
        self.kc = torch.zeros(shape, dtype=torch.int16, device=self.device)
        self.vc = torch.zeros(shape, dtype=torch.int16, device=self.device)

    def set_kv(self, K: torch.Tensor, V: torch.Tensor, stream=None):
        """Rows [0, n) from canonical fp16 [kv_heads][n][head_dim]."""
        K = K.to(self.device).contiguous().view(torch.int16)
        V = V.to(self.device).contiguous().view(torch.int16)
        d = self.desc
        check(lib().slq_kv_layout(d.kv_heads, d.max_seq, d.head_dim, K.shape[1], _ptr(K), _ptr(V), _ptr(self.kc),
                                  _ptr(self.vc), 1, _stream(stream)))

    def get_kv(self, rows: int, stream=None):
        d = self.desc
        K = torch.empty((d.kv_heads, rows, d.head_dim), dtype=torch.float16, device=self.device)
        V = torch.empty_like(K)
        check(lib().slq_kv_layout(d.kv_heads, d.max_seq, d.head_dim, rows, _ptr(K), _ptr(V), _ptr(self.kc),
                                  _ptr(self.vc), 0, _stream(stream)))
        return K, V

    def decode(self, inp: torch.Tensor, pos: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """inp fp32 [T][q|g|k|v] at positions pos..pos+T-1 -> out fp32 [T][q_heads*head_dim]."""
        T = inp.shape[0]
        d = self.desc
        if out is None:
            out = torch.empty((T, d.q_heads * d.head_dim), dtype=torch.float32, device=self.device)
        check(lib().slq_attn_decode(ctypes.byref(d), T, pos, _ptr(inp), _ptr(self.kc), _ptr(self.vc), _ptr(out),
                                    _ptr(self.ws), self.ws.numel(), _stream(stream)))
        return out


# ------------------------------------------------------------------- slice

def make_config(shape, qtype: int, begin: int, end: int, *, max_seq: int = 1024, max_verify: int = 16,
                io_fp32: bool = False, has_embed: bool = False, has_head: bool = False,
                has_mtp: bool = False, max_prefill: int = 0) -> SliceConfig:
    """Build a slice_config from any object with the model-shape attributes."""
    c = SliceConfig()
    c.hidden = shape.hidden
    c.n_layers = shape.n_layers
    c.layer_begin, c.layer_end = begin, end
    c.attn_period = shape.attn_period
    c.dn_heads, c.dn_dk, c.dn_dv = shape.dn_heads, shape.dn_dk, shape.dn_dv
    c.q_heads, c.kv_heads, c.head_dim = shape.q_heads, shape.kv_heads, shape.head_dim
    c.rope_dims = shape.rope_dims
    c.rope_theta = float(shape.rope_theta)
    c.qk_norm = int(bool(shape.qk_norm))
    c.attn_gate = int(bool(shape.attn_gate))
    c.eps = float(shape.eps)
    c.dn_a_scale, c.dn_a_bias = float(shape.dn_a_scale), float(shape.dn_a_bias)
    c.dn_b_scale, c.dn_z_scale = float(shape.dn_b_scale), float(shape.dn_z_scale)
    c.ffn = shape.ffn
    c.vocab = shape.vocab
    c.has_embed, c.has_head = int(has_embed), int(has_head)
    c.tied_head = int(bool(shape.tied_head))
    c.max_seq, c.max_verify = max_seq, max_verify
    c.qtype = qtype
    c.io_fp32 = int(io_fp32)
    c.dn_variant = int(getattr(shape, "dn_variant", 0))
    c.dn_k_heads = int(getattr(shape, "dn_k_heads", 0))
    c.dn_conv = int(getattr(shape, "dn_conv", 0))
    c.has_mtp = int(has_mtp)
    c.max_prefill = int(max_prefill)
    return c


def tensor_info(cfg: SliceConfig, layer: int, name: str) -> dict:
    """Expected source of one tensor (host only): {"rows", "cols", "kind",
    "src_bytes"}; kind is the GGUF type of a quantised matrix or 0 for an fp32
    vector.  Raises SliceError if the slice does not hold the tensor."""
    r, c, k, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_size_t()
    check(lib().slice_tensor_info(ctypes.byref(cfg), layer, TENSOR_IDS[name], ctypes.byref(r), ctypes.byref(c),
                                  ctypes.byref(k), ctypes.byref(n)))
    return {"rows": r.value, "cols": c.value, "kind": k.value, "src_bytes": n.value}


class Slice:
    """A loaded layer slice: caller-owned weights and workspace on the GPU."""

    def __init__(self, cfg: SliceConfig, device: str = "cuda", stream=None):
        self.cfg = cfg
        self.device = torch.device(device)
        wb = int(lib().slice_weights_bytes(ctypes.byref(cfg)))
        sb = int(lib().slice_workspace_bytes(ctypes.byref(cfg)))
        if wb == 0 or sb == 0:
            check(-1)
        self.weights = torch.empty(wb, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(sb, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(lib().slice_load(ctypes.byref(cfg), _ptr(self.weights), _ptr(self.workspace), _stream(stream),
                               ctypes.byref(h)))
        self.handle = h
        self.io_dtype = torch.float32 if cfg.io_fp32 else torch.float16

    # ---- weights
    def set_tensor(self, layer: int, name: str, t: torch.Tensor, stream=None):
        t = t.contiguous()
        check(lib().slice_set_tensor(self.handle, layer, TENSOR_IDS[name], _ptr(t), t.numel() * t.element_size(),
                                     _stream(stream)))

    def load_numpy(self, tensors: dict, glob: dict | None = None, stream=None):
        """tensors: {layer: {name: np.ndarray}} (GGUF blocks or fp32 vectors); glob: embedding etc."""
        for layer, d in tensors.items():
            if not (self.cfg.layer_begin <= layer < self.cfg.layer_end):
                continue
            for name, arr in d.items():
                t = _dev(arr, self.device)
                self.set_tensor(layer, name, t, stream)
                torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
                del t
        for name, arr in (glob or {}).items():
            if name == "embed" and not (self.cfg.has_embed or (self.cfg.has_head and self.cfg.tied_head)):
                continue
            if name in ("head", "out_norm") and not self.cfg.has_head:
                continue
            if name.startswith("mtp_") and not self.cfg.has_mtp:
                continue
            self.set_tensor(0, name, _dev(arr, self.device), stream)
        torch.cuda.synchronize()

    # ---- state
    def reset(self, kv_len: int, stream=None):
        check(lib().slice_reset(self.handle, kv_len, _stream(stream)))

    def set_state(self, layer: int, S: torch.Tensor, stream=None):
        S = S.to(device=self.device, dtype=torch.float32).contiguous()
        check(lib().slice_dbg_set_state(self.handle, layer, _ptr(S), _stream(stream)))
        torch.cuda.synchronize()

    def get_state(self, layer: int, stream=None) -> torch.Tensor:
        c = self.cfg
        out = torch.empty((c.dn_heads, c.dn_dv, c.dn_dk), dtype=torch.float32, device=self.device)
        check(lib().slice_dbg_get_state(self.handle, layer, _ptr(out), _stream(stream)))
        return out

    def conv_dim(self) -> int:
        c = self.cfg
        return 2 * (c.dn_k_heads or c.dn_heads) * c.dn_dk + c.dn_heads * c.dn_dv

    def set_conv_state(self, layer: int, C: torch.Tensor, stream=None):
        """Conv inputs of a qwen3_5-form DeltaNet layer, fp32 [conv_dim][dn_conv - 1]."""
        C = C.to(device=self.device, dtype=torch.float32).contiguous()
        check(lib().slice_dbg_set_conv(self.handle, layer, _ptr(C), _stream(stream)))
        torch.cuda.synchronize()

    def get_conv_state(self, layer: int, stream=None) -> torch.Tensor:
        out = torch.empty((self.conv_dim(), self.cfg.dn_conv - 1), dtype=torch.float32, device=self.device)
        check(lib().slice_dbg_get_conv(self.handle, layer, _ptr(out), _stream(stream)))
        return out

    def set_kv(self, layer: int, K: torch.Tensor, V: torch.Tensor, stream=None):
        K = K.to(self.device).contiguous().view(torch.int16)
        V = V.to(self.device).contiguous().view(torch.int16)
        check(lib().slice_dbg_set_kv(self.handle, layer, _ptr(K), _ptr(V), K.shape[1], _stream(stream)))
        torch.cuda.synchronize()

    def get_kv(self, layer: int, rows: int, stream=None):
        c = self.cfg
        K = torch.empty((c.kv_heads, rows, c.head_dim), dtype=torch.float16, device=self.device)
        V = torch.empty_like(K)
        check(lib().slice_dbg_get_kv(self.handle, layer, _ptr(K), _ptr(V), rows, _stream(stream)))
        return K, V

    def get_hidden(self, k: int = 1, stream=None) -> torch.Tensor:
        """fp32 residual stream of the last step (before the boundary conversion)."""
        out = torch.empty((k, self.cfg.hidden), dtype=torch.float32, device=self.device)
        check(lib().slice_dbg_get_hidden(self.handle, _ptr(out), k, _stream(stream)))
        return out

    # ---- steps
    def decode(self, h_in: torch.Tensor, h_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        if h_out is None:
            h_out = torch.empty(self.cfg.hidden, dtype=self.io_dtype, device=self.device)
        check(lib().slice_decode(self.handle, _ptr(h_in), _ptr(h_out), _stream(stream)))
        return h_out

    OP_NAMES = ["entry", "dn_in", "deltanet", "dn_out", "att_in", "attention", "att_out", "ffn_in", "ffn_out",
                "exit", "chain"]

    def decode_profiled(self, h_in: torch.Tensor, h_out: torch.Tensor | None = None, stream=None):
        """One decode step, op by op, with a HIP event at every op boundary.
        Returns (h_out, [(op_name, ms), ...])."""
        if h_out is None:
            h_out = torch.empty(self.cfg.hidden, dtype=self.io_dtype, device=self.device)
        cap = 16 * (self.cfg.layer_end - self.cfg.layer_begin) + 8
        kinds = (ctypes.c_int * cap)()
        ms = (ctypes.c_float * cap)()
        n = lib().slice_decode_profiled(self.handle, _ptr(h_in), _ptr(h_out), kinds, ms, cap, _stream(stream))
        if n < 0:
            check(n)
        return h_out, [(self.OP_NAMES[kinds[i]], float(ms[i])) for i in range(n)]

    def run_gemv_op(self, op_name: str, stream=None):
        """Launch one GEMV op kind for every layer, back to back (timing aid)."""
        check(lib().slice_run_gemv_op(self.handle, self.OP_NAMES.index(op_name), _stream(stream)))

    def verify(self, h_in: torch.Tensor, h_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        k = h_in.shape[0]
        if h_out is None:
            h_out = torch.empty((k, self.cfg.hidden), dtype=self.io_dtype, device=self.device)
        check(lib().slice_verify(self.handle, k, _ptr(h_in), _ptr(h_out), _stream(stream)))
        return h_out

    def prefill(self, h_in: torch.Tensor, h_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """k prompt tokens in one pass (chunked DeltaNet); the position moves by k."""
        k = h_in.shape[0]
        if h_out is None:
            h_out = torch.empty((k, self.cfg.hidden), dtype=self.io_dtype, device=self.device)
        check(lib().slice_prefill(self.handle, k, _ptr(h_in), _ptr(h_out), _stream(stream)))
        return h_out

    def commit(self, accepted: int, stream=None):
        check(lib().slice_commit(self.handle, accepted, _stream(stream)))

    def embed(self, tok: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty(self.cfg.hidden, dtype=self.io_dtype, device=self.device)
        check(lib().slice_embed(self.handle, _ptr(tok), _ptr(out), _stream(stream)))
        return out

    def head_argmax(self, h: torch.Tensor, logits: torch.Tensor | None = None, tok: torch.Tensor | None = None,
                    stream=None):
        if tok is None:
            tok = torch.empty(1, dtype=torch.int32, device=self.device)
        check(lib().slice_head_argmax(self.handle, _ptr(h), _ptr(tok), _ptr(logits), _stream(stream)))
        return tok

    def mtp_input(self, tok: torch.Tensor, h: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
        """Draft head's layer input from the sampled token (int32 on the device)
        and the hidden state it was sampled from (boundary dtype)."""
        if out is None:
            out = torch.empty(self.cfg.hidden, dtype=self.io_dtype, device=self.device)
        check(lib().slice_mtp_input(self.handle, _ptr(tok), _ptr(h), _ptr(out), _stream(stream)))
        return out

    def sync_check(self, stream=None):
        """Wait for the stream; raise SliceError if a bounded wait inside a
        chained decode kernel gave up since the last reset."""
        check(lib().slice_sync_check(self.handle, _stream(stream)))

    @property
    def position(self) -> int:
        return int(lib().slice_position(self.handle))

    def free(self):
        if getattr(self, "handle", None):
            lib().slice_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
