"""CPU oracle, model part: one decode step of a contiguous slice of layers.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the library never imports or calls it.

Plain, slow, obviously correct: numpy in fp64 for every activation inside a
step; the persistent tensors keep the precision the model stores them in (the
DeltaNet state in fp32, the KV cache in fp16, the boundary vector in fp16 or
fp32).  Matrix-vector products go through qref.gemv (C, fp64 sums).

What the pages fix, by page and section:
  * Slicing: a stage runs a contiguous range of layers, takes a hidden state in
    and hands one out; the first stage owns the embedding, the last the head
    and sampling, every stage keeps its own cache ("Unstable Legion: the
    peer-to-peer ChatGPT", sections "Splitting the workload" and "The runtime:
    legion-stage-runtime").  One token's hidden state at 5,120 x f16 crosses a
    boundary (SwarmLLM README, pipeline diagram and bench paragraph).
  * Block kinds: Llama-style blocks (RMSNorm, GQA, RoPE, SwiGLU, tied head),
    and the qwen3_5 hybrid, whose linear-attention layers are Gated DeltaNet
    and whose remaining layers are full attention with RoPE on part of each
    head, per-head norms of q and k, and a sigmoid gate on the output
    (ChatTorrent README, "What it can run").
  * Verify: drafts are checked in one batched pass and the recurrent state is
    rolled back exactly; the speculative stream equals the plain one (SwarmLLM
    README, feature list and architecture paragraph).  Here verify(k) is
    defined as k plain decode steps and commit(j) as the state after j of them.

Readings where the pages are silent (each listed in the design notes):
  pre-norm residual blocks h += Mixer(RMSNorm(h)), h += FFN(RMSNorm(h));
  DeltaNet gates alpha = sigmoid(c_a a + b_a), beta = sigmoid(c_b b),
  gate = sigmoid(c_z z) from per-token projections a, b, z;
  q, k of DeltaNet divided by sqrt(sum of squares + 1e-6);
  QK-norm before RoPE; RoPE rotates pairs (i, i + rope_dims/2);
  the new K/V row is rounded to fp16 before it is attended;
  attention scale 1/sqrt(head_dim); head h reads KV head h // (q_heads/kv_heads).

The draft head (mtp_input, DraftHead): the pages say only that a draft head
guesses the token after the one just sampled, on the last stage, and that the
engine follows llama.cpp's graph for this model family (SwarmLLM README,
pipeline diagram and credits), so its form is read from the published
multi-token-prediction module of that family -- the embedding of the sampled
token and the hidden state it was sampled from (before the final norm), each
RMS-normalised with weights of its own, concatenated embedding first,
projected back to the hidden width, then one decoder layer of the
full-attention kind with its own KV cache, the head's own final norm and the
shared LM head; further drafts feed the draft and the layer's output back in.

The qwen3_5 form of the DeltaNet layers (deltanet_q35, selected by the
shape's dn_variant): the pages name the layer kind only, so its details are
read from the published form of the Gated DeltaNet mixer -- a depthwise causal
conv (width dn_conv) over q|k|v then SiLU, its state the last dn_conv - 1
inputs (rolled back with the recurrent state); value head h shares query/key
head h // (heads / k_heads); q and k L2-normalised, q scaled by 1/sqrt(d_k);
alpha = exp(-exp(A_log) softplus(c_a a + dt_bias)), beta = sigmoid(c_b b);
the head output through rmsnorm(o) * w * silu(c_z z).  Parity with a real
checkpoint is unpinned (no weights or reference outputs exist here); the
functions are pinned by closed forms in the tests.
"""
from __future__ import annotations

import numpy as np

from . import qref


# ----------------------------------------------------------------- primitives

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x_i / sqrt(mean_j x_j^2 + eps) * w_i (Llama-style RMSNorm)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x) + eps) * np.asarray(w, dtype=np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def softplus(z):
    """log(1 + e^z), computed as logaddexp(0, z) so large z does not overflow."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def l2normalize(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x) + eps)


def rope(x: np.ndarray, pos: int, rope_dims: int, theta: float) -> np.ndarray:
    """Rotary embedding on the first rope_dims entries of one head vector.

    Pairs (i, i + rope_dims/2) for i < rope_dims/2 are rotated by the angle
    pos * theta^(-2i/rope_dims), taken in fp64; the remaining entries pass
    through unchanged.
    """
    x = np.array(x, dtype=np.float64)
    half = rope_dims // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / rope_dims)
    c, s = np.cos(ang), np.sin(ang)
    a = x[:half].copy()
    b = x[half:rope_dims].copy()
    x[:half] = a * c - b * s
    x[half:rope_dims] = b * c + a * s
    return x


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query head over rows K[0..n), V[0..n).

    K, V: [n, head_dim] (fp16 cache rows); the max is subtracted before exp.
    """
    Kd = K.astype(np.float64)
    Vd = V.astype(np.float64)
    s = (Kd @ np.asarray(q, dtype=np.float64)) * scale
    s = s - np.max(s)
    p = np.exp(s)
    p = p / np.sum(p)
    return p @ Vd


def deltanet_update(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    alpha: float, beta: float):
    """One Gated DeltaNet step on one head.

    S: [d_v, d_k] state, q/k already normalised.  Returns (S_new, o) with
        S_new = alpha * S (I - beta k k^T) + beta v k^T,   o = S_new q,
    both in fp64 (the caller stores S_new in fp32).
    """
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    dk = k.shape[0]
    S_new = alpha * (S @ (np.eye(dk) - beta * np.outer(k, k))) + beta * np.outer(v, k)
    return S_new, S_new @ np.asarray(q, dtype=np.float64)


# ------------------------------------------------------- mixers, one token

def deltanet_heads(S: np.ndarray, q, k, v, alpha, beta, gate, dk: int, dv: int) -> np.ndarray:
    """One token of the Gated DeltaNet mixer over all heads.

    S: [heads, d_v, d_k] fp32, updated in place (each head's new state is
    rounded to fp32, as it is stored between tokens).  q, k: [heads * d_k];
    v, gate: [heads * d_v]; alpha, beta: [heads] (decay and write strength,
    already passed through their sigmoids).  Head h uses the h-th slice of q,
    k and v; q and k are L2-normalised per head.  Returns the gated output
    o * gate, [heads * d_v] in fp64.
    """
    heads = S.shape[0]
    o = np.empty(heads * dv)
    for hh in range(heads):
        qh = l2normalize(q[hh * dk:(hh + 1) * dk])
        kh = l2normalize(k[hh * dk:(hh + 1) * dk])
        vh = v[hh * dv:(hh + 1) * dv]
        S_new, o[hh * dv:(hh + 1) * dv] = deltanet_update(S[hh], qh, kh, vh, alpha[hh], beta[hh])
        S[hh] = S_new.astype(np.float32)
    return o * np.asarray(gate, dtype=np.float64)


def deltanet_token(S: np.ndarray, row: np.ndarray, dk: int, dv: int) -> np.ndarray:
    """The DeltaNet mixer fed its pre-activations directly: row = [q | k | v |
    a | b | z] (heads*d_k, heads*d_k, heads*d_v, heads, heads, heads*d_v) with
    alpha = sigmoid(a), beta = sigmoid(b), gate = sigmoid(z).  Updates S in
    place and returns the gated output."""
    heads = S.shape[0]
    row = np.asarray(row, dtype=np.float64)
    o = 0
    q = row[o:o + heads * dk]; o += heads * dk
    k = row[o:o + heads * dk]; o += heads * dk
    v = row[o:o + heads * dv]; o += heads * dv
    a = row[o:o + heads]; o += heads
    b = row[o:o + heads]; o += heads
    z = row[o:o + heads * dv]
    return deltanet_heads(S, q, k, v, sigmoid(a), sigmoid(b), sigmoid(z), dk, dv)


def conv_silu(state: np.ndarray, x: np.ndarray, w: np.ndarray):
    """Depthwise causal convolution of one token, then SiLU.

    state: [C][K-1] the channels' previous K-1 inputs, oldest first; x: [C]
    this token's inputs; w: [C][K] taps, tap K-1 applied to x.  Returns
    (silu(sum_j w[c][j] window[c][j]) in fp64, the new state [C][K-1]: the
    window without its oldest input, stored in fp32).
    """
    win = np.concatenate([np.asarray(state, dtype=np.float64), np.asarray(x, dtype=np.float64)[:, None]], axis=1)
    y = np.sum(win * np.asarray(w, dtype=np.float64), axis=1)
    return silu(y), win[:, 1:].astype(np.float32)


def gated_rmsnorm(o: np.ndarray, z: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of one head's output, weighted, times silu of the gate input."""
    return rmsnorm(o, w, eps) * silu(z)


def deltanet_heads_q35(S: np.ndarray, q, k, v, alpha, beta, z, norm_w, eps: float, dk: int, dv: int,
                       k_heads: int) -> np.ndarray:
    """One token of the qwen3_5-form Gated DeltaNet mixer over all value heads.

    S: [heads, d_v, d_k] fp32, updated in place.  q, k: [k_heads * d_k]
    (after the conv); v, z: [heads * d_v]; alpha, beta: [heads].  Value head h
    reads query/key head h // (heads / k_heads); q and k are L2-normalised per
    head and q is then scaled by 1/sqrt(d_k).  The update is the same rank-one
    rule as deltanet_update; the head's output o goes through
    rmsnorm(o) * norm_w * silu(z_h).  Returns [heads * d_v] in fp64.
    """
    heads = S.shape[0]
    ratio = heads // k_heads
    out = np.empty(heads * dv)
    for hh in range(heads):
        kh = hh // ratio
        qh = l2normalize(q[kh * dk:(kh + 1) * dk]) / np.sqrt(dk)
        kk = l2normalize(k[kh * dk:(kh + 1) * dk])
        vh = v[hh * dv:(hh + 1) * dv]
        S_new, o = deltanet_update(S[hh], qh, kk, vh, alpha[hh], beta[hh])
        S[hh] = S_new.astype(np.float32)
        out[hh * dv:(hh + 1) * dv] = gated_rmsnorm(o, z[hh * dv:(hh + 1) * dv], norm_w, eps)
    return out


def attention_heads(s, q, g, k, v, K: np.ndarray, V: np.ndarray, p: int, q_norm=None, k_norm=None) -> np.ndarray:
    """One token of (gated) grouped-query attention at position p.

    s: the attention geometry (head_dim, q_heads, kv_heads, rope_dims,
    rope_theta, qk_norm, attn_gate, eps).  q, g: [q_heads * head_dim] (g only
    with the gate); k, v: [kv_heads * head_dim]; q_norm, k_norm: [head_dim]
    QK-norm weights.  The token's key (QK-norm, then RoPE at p) and value are
    rounded to fp16 into row p of the caches K, V [kv_heads, rows, head_dim];
    query head i (QK-norm, RoPE at p) attends to rows 0..p of KV head
    i // (q_heads / kv_heads) with scale 1/sqrt(head_dim).  Returns the heads'
    outputs, times sigmoid(g) with the gate, [q_heads * head_dim] in fp64.
    """
    hd, nq, nkv = s.head_dim, s.q_heads, s.kv_heads
    grp = nq // nkv
    q = np.asarray(q, dtype=np.float64).reshape(nq, hd)
    k = np.asarray(k, dtype=np.float64).reshape(nkv, hd)
    v = np.asarray(v, dtype=np.float64).reshape(nkv, hd)
    for j in range(nkv):
        kj = rmsnorm(k[j], k_norm, s.eps) if s.qk_norm else k[j]
        K[j, p] = rope(kj, p, s.rope_dims, s.rope_theta).astype(np.float16)
        V[j, p] = v[j].astype(np.float16)
    scale = 1.0 / np.sqrt(hd)
    o = np.empty((nq, hd))
    for i in range(nq):
        qi = rmsnorm(q[i], q_norm, s.eps) if s.qk_norm else q[i]
        qi = rope(qi, p, s.rope_dims, s.rope_theta)
        j = i // grp
        o[i] = attend(qi, K[j, :p + 1], V[j, :p + 1], scale)
    u = o.reshape(-1)
    if s.attn_gate:
        u = u * sigmoid(g)
    return u


# --------------------------------------------------------------------- slice

class SliceOracle:
    """Reference for a slice [begin, end) of a decoder described by synth.ModelShape.

    tensors: {layer: {name: array}} in the layouts synth.layer_tensors returns;
    glob: synth.global_tensors output (only for the first/last stage helpers).
    """

    def __init__(self, shape, qtype: int, begin: int, end: int, tensors: dict,
                 glob: dict | None = None, max_seq: int = 1024, io_fp32: bool = False):
        self.s = shape
        self.qtype = qtype
        self.begin, self.end = begin, end
        self.W = tensors
        self.G = glob or {}
        self.max_seq = max_seq
        self.io_fp32 = io_fp32
        self.pos = 0
        self.kv = {}
        self.dn = {}
        self.conv = {}
        for l in range(begin, end):
            if shape.is_attention(l):
                shp = (shape.kv_heads, max_seq, shape.head_dim)
                self.kv[l] = (np.zeros(shp, np.float16), np.zeros(shp, np.float16))
            else:
                self.dn[l] = np.zeros((shape.dn_heads, shape.dn_dv, shape.dn_dk), np.float32)
                if shape.dn_variant:
                    self.conv[l] = np.zeros((shape.conv_dim, shape.dn_conv - 1), np.float32)
        self._pending = None

    # ---- state setters (the synthetic prior context)
    def reset(self, pos: int):
        self.pos = int(pos)
        self._pending = None

    def set_kv(self, layer: int, K: np.ndarray, V: np.ndarray):
        n = K.shape[1]
        self.kv[layer][0][:, :n] = K
        self.kv[layer][1][:, :n] = V

    def set_state(self, layer: int, S: np.ndarray):
        self.dn[layer][...] = S.astype(np.float32)

    def set_conv_state(self, layer: int, C: np.ndarray):
        self.conv[layer][...] = C.astype(np.float32)

    # ---- matrix helper
    def _mv(self, layer, name, x):
        raw = self.W[layer][name]
        rows = raw.shape[0]
        cols = np.asarray(x).shape[-1]
        return qref.gemv(self.qtype, raw, rows, cols, x)

    # ---- sublayers
    def deltanet(self, l: int, h: np.ndarray) -> np.ndarray:
        s, W = self.s, self.W[l]
        if s.dn_variant:
            return self.deltanet_q35(l, h)
        x = rmsnorm(h, W["attn_norm"], s.eps)
        q = self._mv(l, "dn_q", x)
        k = self._mv(l, "dn_k", x)
        v = self._mv(l, "dn_v", x)
        a = self._mv(l, "dn_a", x)
        b = self._mv(l, "dn_b", x)
        z = self._mv(l, "dn_z", x)
        alpha = sigmoid(np.float64(np.float32(s.dn_a_scale)) * a + np.float64(np.float32(s.dn_a_bias)))
        beta = sigmoid(np.float64(np.float32(s.dn_b_scale)) * b)
        gate = sigmoid(np.float64(np.float32(s.dn_z_scale)) * z)
        u = deltanet_heads(self.dn[l], q, k, v, alpha, beta, gate, s.dn_dk, s.dn_dv)
        return h + self._mv(l, "dn_out", u)

    def deltanet_q35(self, l: int, h: np.ndarray) -> np.ndarray:
        """The qwen3_5 form: the conv + SiLU on q|k|v with its state, the
        decay alpha = exp(-exp(A_log) softplus(c_a a + dt_bias)), beta =
        sigmoid(c_b b), gate input c_z z for the gated RMSNorm."""
        s, W = self.s, self.W[l]
        x = rmsnorm(h, W["attn_norm"], s.eps)
        q = self._mv(l, "dn_q", x)
        k = self._mv(l, "dn_k", x)
        v = self._mv(l, "dn_v", x)
        a = self._mv(l, "dn_a", x)
        b = self._mv(l, "dn_b", x)
        z = self._mv(l, "dn_z", x)
        nk = s.k_heads * s.dn_dk
        taps = np.asarray(W["dn_conv"], dtype=np.float64).reshape(s.conv_dim, s.dn_conv)
        qkv, self.conv[l][...] = conv_silu(self.conv[l], np.concatenate([q, k, v]), taps)
        q, k, v = qkv[:nk], qkv[nk:2 * nk], qkv[2 * nk:]
        a_log = np.asarray(W["dn_alog"], dtype=np.float64)
        dt_bias = np.asarray(W["dn_dtb"], dtype=np.float64)
        alpha = np.exp(-np.exp(a_log) * softplus(np.float64(np.float32(s.dn_a_scale)) * a + dt_bias))
        beta = sigmoid(np.float64(np.float32(s.dn_b_scale)) * b)
        zg = np.float64(np.float32(s.dn_z_scale)) * z
        u = deltanet_heads_q35(self.dn[l], q, k, v, alpha, beta, zg, W["dn_norm"], s.eps, s.dn_dk, s.dn_dv,
                               s.k_heads)
        return h + self._mv(l, "dn_out", u)

    def attention(self, l: int, h: np.ndarray) -> np.ndarray:
        s, W = self.s, self.W[l]
        hd, nq, nkv = s.head_dim, s.q_heads, s.kv_heads
        x = rmsnorm(h, W["attn_norm"], s.eps)
        q = self._mv(l, "wq", x).reshape(nq, hd)
        g = self._mv(l, "wg", x) if s.attn_gate else None
        k = self._mv(l, "wk", x).reshape(nkv, hd)
        v = self._mv(l, "wv", x).reshape(nkv, hd)
        K, V = self.kv[l]
        u = attention_heads(s, q, g, k, v, K, V, self.pos, W.get("q_norm"), W.get("k_norm"))
        return h + self._mv(l, "wo", u)

    def ffn(self, l: int, h: np.ndarray) -> np.ndarray:
        s, W = self.s, self.W[l]
        x = rmsnorm(h, W["ffn_norm"], s.eps)
        m = silu(self._mv(l, "w_gate", x)) * self._mv(l, "w_up", x)
        return h + self._mv(l, "w_down", m)

    # ---- one plain decode step of the whole slice
    def _step(self, h: np.ndarray) -> np.ndarray:
        h = np.asarray(h, dtype=np.float64)
        for l in range(self.begin, self.end):
            h = self.attention(l, h) if self.s.is_attention(l) else self.deltanet(l, h)
            if self.s.ffn:
                h = self.ffn(l, h)
        self.pos += 1
        return h

    def _round_out(self, h):
        return h.astype(np.float32) if self.io_fp32 else h.astype(np.float16)

    def decode(self, hid_in: np.ndarray, raw: bool = False):
        """hid_in: boundary vector [H] (fp16 or fp32).  Returns the boundary
        vector out (rounded to the boundary dtype) or, with raw=True, fp64."""
        if self._pending is not None:
            raise RuntimeError("decode while a verify is uncommitted")
        h = self._step(np.asarray(hid_in).astype(np.float64))
        return h if raw else self._round_out(h)

    def verify(self, hid_in: np.ndarray, raw: bool = False):
        """k plain steps on hid_in[0..k), keeping the state after each for commit()."""
        if self._pending is not None:
            raise RuntimeError("verify while a verify is uncommitted")
        p0 = self.pos

        def snapshot():
            return ({l: S.copy() for l, S in self.dn.items()}, {l: C.copy() for l, C in self.conv.items()})

        saved = [snapshot()]
        outs = []
        for t in range(hid_in.shape[0]):
            outs.append(self._step(np.asarray(hid_in[t]).astype(np.float64)))
            saved.append(snapshot())
        self._pending = (p0, saved)
        outs = np.stack(outs)
        return outs if raw else self._round_out(outs)

    def commit(self, accepted: int):
        p0, saved = self._pending
        if not 0 <= accepted < len(saved):
            raise ValueError("accepted out of range")
        for l in self.dn:
            self.dn[l][...] = saved[accepted][0][l]
        for l in self.conv:
            self.conv[l][...] = saved[accepted][1][l]
        self.pos = p0 + accepted
        self._pending = None

    # ---- first / last stage helpers
    def embed(self, token: int) -> np.ndarray:
        E = self.G["embed"]
        bb = E.shape[1] // (self.s.hidden // 32)
        row = E[token:token + 1]
        assert row.shape[1] == bb * self.s.hidden // 32
        return qref.dequant(self.qtype, row, 1, self.s.hidden)[0]

    def head_logits(self, h: np.ndarray) -> np.ndarray:
        x = rmsnorm(np.asarray(h, dtype=np.float64), self.G["out_norm"], self.s.eps)
        E = self.G["embed"] if self.s.tied_head else self.G["head"]
        return qref.gemv(self.qtype, E, self.s.vocab, self.s.hidden, x)

    @staticmethod
    def argmax(logits: np.ndarray) -> int:
        """Greedy choice; the lowest index wins an exact tie."""
        return int(np.argmax(logits))


# ------------------------------------------------------------- draft head

def mtp_input(qtype: int, E: np.ndarray, token: int, h: np.ndarray, w_e, w_h, fc: np.ndarray,
              hidden: int, eps: float) -> np.ndarray:
    """Input of the draft head's layer: fc [H][2H] times the concatenation of
    RMSNorm(embedding row `token`; w_e) and RMSNorm(h; w_h), embedding first.
    E: the embedding table's raw blocks [vocab][H/32 blocks]; h: the hidden
    state the token was sampled from."""
    if not 0 <= token < E.shape[0]:
        raise ValueError("token outside the vocabulary")
    e = qref.dequant(qtype, E[token:token + 1], 1, hidden)[0]
    c = np.concatenate([rmsnorm(e, w_e, eps), rmsnorm(np.asarray(h, dtype=np.float64), w_h, eps)])
    return qref.gemv(qtype, fc, hidden, 2 * hidden, c)


class DraftHead:
    """The draft head as a stage of its own: one full-attention decoder layer
    (layer 0 of `shape`, which must be an attention layer) with its own KV
    cache and position, mtp_input in front of it, and behind it its final
    norm (glob["out_norm"]) and the shared LM head (glob["embed"] / ["head"]).
    mtp: {"mtp_fc", "mtp_norm_e", "mtp_norm_h"}.  Boundary vectors (the input
    h, the layer's input and output) are in the boundary dtype."""

    def __init__(self, shape, qtype: int, layer: dict, mtp: dict, glob: dict, max_seq: int = 1024,
                 io_fp32: bool = False):
        if not shape.is_attention(0):
            raise ValueError("the draft head's layer is an attention layer")
        self.s = shape
        self.qtype = qtype
        self.mtp = mtp
        self.stage = SliceOracle(shape, qtype, 0, 1, {0: layer}, glob=glob, max_seq=max_seq, io_fp32=io_fp32)

    def reset(self, pos: int):
        self.stage.reset(pos)

    def set_kv(self, K: np.ndarray, V: np.ndarray):
        self.stage.set_kv(0, K, V)

    @property
    def pos(self) -> int:
        return self.stage.pos

    def input(self, token: int, h: np.ndarray) -> np.ndarray:
        """The layer's input, rounded to the boundary dtype."""
        x = mtp_input(self.qtype, self.stage.G["embed"], token, h, self.mtp["mtp_norm_e"], self.mtp["mtp_norm_h"],
                      self.mtp["mtp_fc"], self.s.hidden, self.s.eps)
        return self.stage._round_out(x)

    def draft(self, token: int, h: np.ndarray):
        """One draft at the head's position (which then advances): (draft
        token, the layer's output in the boundary dtype, its logits)."""
        out = self.stage.decode(self.input(token, h))
        logits = self.stage.head_logits(out)
        return SliceOracle.argmax(logits), out, logits
