"""Seeded synthetic inputs for the layer-slice decode path.

This module only draws random numbers and lays them out in the storage formats
that the model files use (GGUF Q4_0 / Q8_0 blocks, fp16 boundary vectors, fp32
DeltaNet states, fp16 KV rows).  It holds none of the method's arithmetic: no
dequantisation, no matrix products, no normalisation.  Both the CPU oracle and
the HIP library are fed from here; neither is imported by this file.

Every tensor comes from its own stream,
``PCG64(SeedSequence(seed, spawn_key=(workload, layer, tensor)))``, so any
single tensor can be regenerated without drawing the others.

Storage formats (GGUF block layouts, which the SwarmLLM README names as its
weight format, "GGUF Q4_0", and ChatTorrent as "q8"):

* Q4_0 block, 18 bytes per 32 weights: little-endian fp16 scale ``d``, then 16
  code bytes; byte ``j`` holds weight ``j`` in its low nibble and weight
  ``j + 16`` in its high nibble.
* Q8_0 block, 34 bytes per 32 weights: little-endian fp16 scale ``d``, then 32
  signed code bytes, weight ``j`` in byte ``j``.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

QK = 32                      # weights per quantisation block
Q4_0 = 2                     # GGUF tensor-type ids
Q8_0 = 8
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}

# workload ids used in the stream keys
WL_TINY_LLAMA = 0
WL_GEMV = 1
WL_DELTANET = 2
WL_ATTENTION = 3
WL_SLICE = 4
WL_MTP = 5                   # the draft head's own layer and tensors

# tensor ids used in the stream keys (stable; never renumber)
TENSOR_IDS = {
    "attn_norm": 0, "ffn_norm": 1,
    "dn_q": 10, "dn_k": 11, "dn_v": 12, "dn_a": 13, "dn_b": 14, "dn_z": 15, "dn_out": 16,
    "wq": 20, "wg": 21, "wk": 22, "wv": 23, "wo": 24, "q_norm": 25, "k_norm": 26,
    "w_gate": 30, "w_up": 31, "w_down": 32,
    "embed": 40, "head": 41, "out_norm": 42,
    # activations / state / cache
    "hidden": 50, "dn_state": 51, "kv_k": 52, "kv_v": 53, "gemv_x": 54,
    "accept": 55, "token": 56,
    # qwen3_5 form of the DeltaNet layers: conv taps, decay parameters, gated-norm weights, conv state
    "dn_conv": 17, "dn_alog": 18, "dn_dtb": 19, "dn_norm": 28, "dn_conv_state": 57,
    # the draft head: input projection [H][2H], the norms of its two inputs, its final norm
    "mtp_fc": 43, "mtp_norm_e": 44, "mtp_norm_h": 45, "mtp_out_norm": 46,
}


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shapes and scalar constants of a decoder slice (no arithmetic here)."""
    name: str
    hidden: int
    n_layers: int
    attn_period: int          # 0: every layer is attention; P: layer l is attention iff l % P == P - 1
    dn_heads: int = 0
    dn_dk: int = 0
    dn_dv: int = 0
    q_heads: int = 0
    kv_heads: int = 0
    head_dim: int = 0
    rope_dims: int = 0
    rope_theta: float = 10000.0
    qk_norm: bool = False
    attn_gate: bool = False
    eps: float = 1e-6
    ffn: int = 0              # 0: the layer has no FFN sublayer
    vocab: int = 0
    tied_head: bool = False
    # affine maps from the DeltaNet a/b/z projections to gate pre-activations
    dn_a_scale: float = 0.125
    dn_a_bias: float = 2.0
    dn_b_scale: float = 0.25
    dn_z_scale: float = 0.25
    # qwen3_5 form of the DeltaNet layers (dn_variant = 1): a short causal
    # conv of width dn_conv over q|k|v then SiLU, dn_k_heads query/key heads
    # shared by the dn_heads value heads, q scaled by 1/sqrt(dk), decay
    # exp(-exp(A_log) softplus(a + dt_bias)), output through a gated RMSNorm
    dn_variant: int = 0
    dn_k_heads: int = 0       # 0: dn_heads
    dn_conv: int = 0

    @property
    def k_heads(self) -> int:
        return self.dn_k_heads or self.dn_heads

    @property
    def conv_dim(self) -> int:
        """Channels of the short conv: q | k | v."""
        return 2 * self.k_heads * self.dn_dk + self.dn_heads * self.dn_dv

    def is_attention(self, layer: int) -> bool:
        if self.attn_period == 0:
            return True
        return layer % self.attn_period == self.attn_period - 1


# Tiny Llama-style model: 30 layers, hidden 576, 9/3 heads of 64, SwiGLU 1536,
# vocab 4096 with a tied head, RMSNorm eps 1e-5, full RoPE theta 1e4.
TINY_LLAMA = ModelShape(
    name="tiny_llama_30x576", hidden=576, n_layers=30, attn_period=0,
    q_heads=9, kv_heads=3, head_dim=64, rope_dims=64, rope_theta=1e4,
    qk_norm=False, attn_gate=False, eps=1e-5, ffn=1536, vocab=4096, tied_head=True)

# Hybrid Gated-DeltaNet + gated-attention model at hidden 5120: 3 DeltaNet
# layers then 1 attention layer, repeated; 32 DeltaNet heads of 128; 24/4
# attention heads of 256 with QK-norm, partial RoPE (64 dims, theta 1e7) and a
# sigmoid output gate; SwiGLU 17408; RMSNorm eps 1e-6.
HYBRID_5120 = ModelShape(
    name="hybrid_5120", hidden=5120, n_layers=64, attn_period=4,
    dn_heads=32, dn_dk=128, dn_dv=128,
    q_heads=24, kv_heads=4, head_dim=256, rope_dims=64, rope_theta=1e7,
    qk_norm=True, attn_gate=True, eps=1e-6, ffn=17408, vocab=248320, tied_head=False)

# The same hybrid with DeltaNet layers in the qwen3_5 form: 16 query/key heads
# shared by the 32 value heads, a width-4 causal conv, gated RMSNorm output.
HYBRID_5120_Q35 = dataclasses.replace(HYBRID_5120, name="hybrid_5120_q35", dn_variant=1, dn_k_heads=16, dn_conv=4)

# Matrix shapes of the standalone GEMV sweep (rows x cols).
GEMV_SHAPES = [(5120, 5120), (17408, 5120), (5120, 17408), (12288, 5120), (248320, 5120)]


def stream(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


def quant_blocks(rng: np.random.Generator, qtype: int, rows: int, cols: int, centered: bool = False) -> np.ndarray:
    """Random GGUF blocks, returned as uint8 [rows, cols // 32 * block_bytes].

    Scales: uniform [0.002, 0.02] drawn in fp64 and rounded to fp16 (RNE).
    Q4_0 codes: uniform bytes, i.e. every nibble uniform on 0..15 (weights
    q - 8 of mean -0.5); with centered, every nibble uniform on 1..15
    (weights of mean 0, so deep slices keep their residual stream in range).
    Q8_0 codes: uniform on -127..127 inclusive.
    """
    if cols % QK:
        raise ValueError("cols must be a multiple of 32")
    nb = cols // QK
    d = rng.uniform(0.002, 0.02, size=(rows, nb)).astype(np.float16)
    bb = BLOCK_BYTES[qtype]
    out = np.empty((rows, nb, bb), dtype=np.uint8)
    out[:, :, 0:2] = d.view(np.uint8).reshape(rows, nb, 2)
    if qtype == Q4_0 and centered:
        lo = rng.integers(1, 16, size=(rows, nb, 16), dtype=np.uint8)
        hi = rng.integers(1, 16, size=(rows, nb, 16), dtype=np.uint8)
        out[:, :, 2:] = lo | (hi << 4)
    elif qtype == Q4_0:
        out[:, :, 2:] = rng.integers(0, 256, size=(rows, nb, 16), dtype=np.uint8)
    elif qtype == Q8_0:
        out[:, :, 2:] = rng.integers(-127, 128, size=(rows, nb, 32), dtype=np.int8).view(np.uint8)
    else:
        raise ValueError(f"unknown qtype {qtype}")
    return out.reshape(rows, nb * bb)


def matrix_shapes(shape: ModelShape, layer: int) -> dict:
    """(rows, cols) of every quantised matrix of one layer."""
    H = shape.hidden
    m = {}
    if shape.is_attention(layer):
        nq = shape.q_heads * shape.head_dim
        nkv = shape.kv_heads * shape.head_dim
        m["wq"] = (nq, H)
        if shape.attn_gate:
            m["wg"] = (nq, H)
        m["wk"] = (nkv, H)
        m["wv"] = (nkv, H)
        m["wo"] = (H, nq)
    else:
        nk = shape.k_heads * shape.dn_dk
        nv = shape.dn_heads * shape.dn_dv
        m["dn_q"] = (nk, H)
        m["dn_k"] = (nk, H)
        m["dn_v"] = (nv, H)
        m["dn_a"] = (shape.dn_heads, H)
        m["dn_b"] = (shape.dn_heads, H)
        m["dn_z"] = (nv, H)
        m["dn_out"] = (H, nv)
    if shape.ffn:
        m["w_gate"] = (shape.ffn, H)
        m["w_up"] = (shape.ffn, H)
        m["w_down"] = (H, shape.ffn)
    return m


def vector_shapes(shape: ModelShape, layer: int) -> dict:
    """Lengths of the fp32 vectors of one layer: norm weights (all ones), and in
    the qwen3_5 DeltaNet form the conv taps ([conv_dim][dn_conv]), A_log and
    dt_bias per value head and the gated-norm weights (dn_extra_tensors)."""
    v = {"attn_norm": shape.hidden}
    if shape.dn_variant and not shape.is_attention(layer):
        v["dn_conv"] = shape.conv_dim * shape.dn_conv
        v["dn_alog"] = shape.dn_heads
        v["dn_dtb"] = shape.dn_heads
        v["dn_norm"] = shape.dn_dv
    if shape.ffn:
        v["ffn_norm"] = shape.hidden
    if shape.is_attention(layer) and shape.qk_norm:
        v["q_norm"] = shape.head_dim
        v["k_norm"] = shape.head_dim
    return v


def layer_tensors(shape: ModelShape, qtype: int, seed: int, workload: int, layer: int,
                  threads: int = 1, centered: bool = False) -> dict:
    """All tensors of one layer: raw GGUF blocks for matrices, fp32 ones for norm weights."""
    out = {name: np.ones(n, dtype=np.float32) for name, n in vector_shapes(shape, layer).items()}
    if shape.dn_variant and not shape.is_attention(layer):
        out.update(dn_extra_tensors(shape, seed, workload, layer))
    mats = matrix_shapes(shape, layer)

    def gen(item):
        name, (r, c) = item
        return name, quant_blocks(stream(seed, workload, layer, TENSOR_IDS[name]), qtype, r, c, centered)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            out.update(dict(ex.map(gen, mats.items())))
    else:
        out.update(dict(map(gen, mats.items())))
    return out


def dn_extra_tensors(shape: ModelShape, seed: int, workload: int, layer: int) -> dict:
    """fp32 parameters of a qwen3_5-form DeltaNet layer, drawn like a fresh
    model's: conv taps U[-0.5, 0.5] ([conv_dim][dn_conv], tap dn_conv-1 on
    the current input); A = U[1, 16] stored as A_log = log(A); dt =
    exp(U[log 0.001, log 0.1]) stored as dt_bias = dt + log(1 - exp(-dt)) (the
    value whose softplus is dt); gated-norm weights 1 + 0.1 N(0,1)."""
    r = stream(seed, workload, layer, TENSOR_IDS["dn_conv"])
    conv = r.uniform(-0.5, 0.5, size=shape.conv_dim * shape.dn_conv)
    r = stream(seed, workload, layer, TENSOR_IDS["dn_alog"])
    alog = np.log(r.uniform(1.0, 16.0, size=shape.dn_heads))
    r = stream(seed, workload, layer, TENSOR_IDS["dn_dtb"])
    dt = np.exp(r.uniform(np.log(0.001), np.log(0.1), size=shape.dn_heads))
    dtb = dt + np.log(-np.expm1(-dt))
    r = stream(seed, workload, layer, TENSOR_IDS["dn_norm"])
    norm = 1.0 + 0.1 * r.standard_normal(shape.dn_dv)
    return {"dn_conv": conv.astype(np.float32), "dn_alog": alog.astype(np.float32),
            "dn_dtb": dtb.astype(np.float32), "dn_norm": norm.astype(np.float32)}


def dn_conv_state0(seed: int, workload: int, layer: int, conv_dim: int, width: int) -> np.ndarray:
    """Prior conv inputs of a qwen3_5-form DeltaNet layer: N(0,1) fp32,
    [conv_dim][width - 1], oldest first."""
    rng = stream(seed, workload, layer, TENSOR_IDS["dn_conv_state"])
    return rng.standard_normal((conv_dim, width - 1)).astype(np.float32)


def global_tensors(shape: ModelShape, qtype: int, seed: int, workload: int) -> dict:
    """Embedding table, output norm and (untied) head."""
    out = {}
    if shape.vocab:
        out["embed"] = quant_blocks(stream(seed, workload, 0, TENSOR_IDS["embed"]), qtype,
                                    shape.vocab, shape.hidden)
        out["out_norm"] = np.ones(shape.hidden, dtype=np.float32)
        if not shape.tied_head:
            out["head"] = quant_blocks(stream(seed, workload, 0, TENSOR_IDS["head"]), qtype,
                                       shape.vocab, shape.hidden)
    return out


def mtp_shape(shape: ModelShape) -> ModelShape:
    """The draft head's stage: one layer of the model's full-attention kind."""
    return dataclasses.replace(shape, name=shape.name + "_mtp", n_layers=1, attn_period=0)


def mtp_tensors(shape: ModelShape, qtype: int, seed: int, workload: int = WL_MTP) -> dict:
    """The draft head's own tensors besides its layer: the input projection
    mtp_fc [H][2H] (GGUF blocks as quant_blocks), and fp32 weights 1 + 0.25
    N(0,1) of the embedding-side and hidden-side input norms and of its final
    norm (unequal, so that a swap of the two inputs shows)."""
    H = shape.hidden
    out = {"mtp_fc": quant_blocks(stream(seed, workload, 0, TENSOR_IDS["mtp_fc"]), qtype, H, 2 * H)}
    for name in ("mtp_norm_e", "mtp_norm_h", "mtp_out_norm"):
        r = stream(seed, workload, 0, TENSOR_IDS[name])
        out[name] = (1.0 + 0.25 * r.standard_normal(H)).astype(np.float32)
    return out


def hidden_inputs(seed: int, workload: int, n: int, hidden: int, step0: int = 0) -> np.ndarray:
    """n boundary vectors, N(0,1) rounded to fp16 (RNE): [n, hidden] float16."""
    out = np.empty((n, hidden), dtype=np.float16)
    for i in range(n):
        out[i] = stream(seed, workload, step0 + i, TENSOR_IDS["hidden"]).standard_normal(hidden).astype(np.float16)
    return out


def dn_state0(seed: int, workload: int, layer: int, heads: int, dv: int, dk: int) -> np.ndarray:
    """Initial DeltaNet state, N(0, 0.02) (std 0.02) in fp32, [heads, dv, dk]."""
    rng = stream(seed, workload, layer, TENSOR_IDS["dn_state"])
    return (rng.standard_normal((heads, dv, dk)) * 0.02).astype(np.float32)


def kv_prefill(seed: int, workload: int, layer: int, kv_heads: int, length: int, head_dim: int):
    """Prior KV rows, N(0,1) in fp16: (K, V), each [kv_heads, length, head_dim]."""
    k = stream(seed, workload, layer, TENSOR_IDS["kv_k"]).standard_normal((kv_heads, length, head_dim))
    v = stream(seed, workload, layer, TENSOR_IDS["kv_v"]).standard_normal((kv_heads, length, head_dim))
    return k.astype(np.float16), v.astype(np.float16)


def gemv_x(seed: int, batch: int, cols: int, tag: int = 0) -> np.ndarray:
    """GEMV right-hand sides, N(0,1) in fp32: [batch, cols]."""
    return stream(seed, WL_GEMV, tag, TENSOR_IDS["gemv_x"]).standard_normal((batch, cols)).astype(np.float32)


def tiny_llama_token(seed: int = 0) -> int:
    """Input token of the tiny-Llama step: np.random.default_rng(seed).integers(0, 4096)."""
    return int(np.random.default_rng(seed).integers(0, 4096))


def accept_pattern(seed: int, rounds: int, k: int) -> np.ndarray:
    """Number of accepted draft tokens per verify round, uniform on 0..k."""
    return stream(seed, WL_SLICE, 0, TENSOR_IDS["accept"]).integers(0, k + 1, size=rounds)


def dn_kernel_inputs(seed: int, T: int, heads: int, dk: int, dv: int, step0: int = 0) -> np.ndarray:
    """Inputs of the DeltaNet kernel on its own, fp32 [T][q|k|v|a|b|z] (heads
    x dk, heads x dk, heads x dv, heads, heads, heads x dv): q, k, v ~ N(0,1);
    decay pre-activation a ~ N(2, 0.5); write strength b ~ N(0,1); output
    gate z ~ N(0,1) (second parameters are standard deviations)."""
    out = np.empty((T, 2 * heads * dk + 2 * heads * dv + 2 * heads), dtype=np.float32)
    for t in range(T):
        r = stream(seed, WL_DELTANET, 1000 + step0 + t, TENSOR_IDS["hidden"])
        q = r.standard_normal(heads * dk)
        k = r.standard_normal(heads * dk)
        v = r.standard_normal(heads * dv)
        a = r.normal(2.0, 0.5, heads)
        b = r.standard_normal(heads)
        z = r.standard_normal(heads * dv)
        out[t] = np.concatenate([q, k, v, a, b, z]).astype(np.float32)
    return out


def attn_kernel_inputs(seed: int, T: int, q_heads: int, kv_heads: int, head_dim: int, gate: bool,
                       step0: int = 0) -> np.ndarray:
    """Inputs of the attention kernel on its own, fp32 [T][q|g|k|v], every
    entry N(0,1)."""
    n = (2 if gate else 1) * q_heads * head_dim + 2 * kv_heads * head_dim
    out = np.empty((T, n), dtype=np.float32)
    for t in range(T):
        out[t] = stream(seed, WL_ATTENTION, 1000 + step0 + t, TENSOR_IDS["hidden"]).standard_normal(n)
    return out
