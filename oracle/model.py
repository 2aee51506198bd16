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
  * Block kinds: Llama-style blocks (RMSNorm, GQA, RoPE, SwiGLU, tied head)
    and the qwen3_5 hybrid, Gated DeltaNet layers mixed with full-attention
    layers that have partial RoPE, QK-norm and an output gate (ChatTorrent
    README, "What it can run").
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
        for l in range(begin, end):
            if shape.is_attention(l):
                shp = (shape.kv_heads, max_seq, shape.head_dim)
                self.kv[l] = (np.zeros(shp, np.float16), np.zeros(shp, np.float16))
            else:
                self.dn[l] = np.zeros((shape.dn_heads, shape.dn_dv, shape.dn_dk), np.float32)
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

    # ---- matrix helper
    def _mv(self, layer, name, x):
        raw = self.W[layer][name]
        rows = raw.shape[0]
        cols = np.asarray(x).shape[-1]
        return qref.gemv(self.qtype, raw, rows, cols, x)

    # ---- sublayers
    def deltanet(self, l: int, h: np.ndarray) -> np.ndarray:
        s, W = self.s, self.W[l]
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
        dk, dv = s.dn_dk, s.dn_dv
        o = np.empty(s.dn_heads * dv)
        S = self.dn[l]
        for hh in range(s.dn_heads):
            qh = l2normalize(q[hh * dk:(hh + 1) * dk])
            kh = l2normalize(k[hh * dk:(hh + 1) * dk])
            vh = v[hh * dv:(hh + 1) * dv]
            S_new, o[hh * dv:(hh + 1) * dv] = deltanet_update(S[hh], qh, kh, vh, alpha[hh], beta[hh])
            S[hh] = S_new.astype(np.float32)
        return h + self._mv(l, "dn_out", o * gate)

    def attention(self, l: int, h: np.ndarray) -> np.ndarray:
        s, W = self.s, self.W[l]
        hd, nq, nkv = s.head_dim, s.q_heads, s.kv_heads
        grp = nq // nkv
        x = rmsnorm(h, W["attn_norm"], s.eps)
        q = self._mv(l, "wq", x).reshape(nq, hd)
        g = self._mv(l, "wg", x) if s.attn_gate else None
        k = self._mv(l, "wk", x).reshape(nkv, hd)
        v = self._mv(l, "wv", x).reshape(nkv, hd)
        p = self.pos
        K, V = self.kv[l]
        for j in range(nkv):
            kj = rmsnorm(k[j], W["k_norm"], s.eps) if s.qk_norm else k[j]
            K[j, p] = rope(kj, p, s.rope_dims, s.rope_theta).astype(np.float16)
            V[j, p] = v[j].astype(np.float16)
        scale = 1.0 / np.sqrt(hd)
        o = np.empty((nq, hd))
        for i in range(nq):
            qi = rmsnorm(q[i], W["q_norm"], s.eps) if s.qk_norm else q[i]
            qi = rope(qi, p, s.rope_dims, s.rope_theta)
            j = i // grp
            o[i] = attend(qi, K[j, :p + 1], V[j, :p + 1], scale)
        u = o.reshape(-1)
        if s.attn_gate:
            u = u * sigmoid(g)
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
        saved = [{l: S.copy() for l, S in self.dn.items()}]
        outs = []
        for t in range(hid_in.shape[0]):
            outs.append(self._step(np.asarray(hid_in[t]).astype(np.float64)))
            saved.append({l: S.copy() for l, S in self.dn.items()})
        self._pending = (p0, saved)
        outs = np.stack(outs)
        return outs if raw else self._round_out(outs)

    def commit(self, accepted: int):
        p0, saved = self._pending
        if not 0 <= accepted < len(saved):
            raise ValueError("accepted out of range")
        for l in self.dn:
            self.dn[l][...] = saved[accepted][l]
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
