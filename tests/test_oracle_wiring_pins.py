"""Closed-form pins of the oracle's sublayer wiring (CPU only).

The primitives (RMSNorm, RoPE, softmax attention, the DeltaNet update, the
block decoders) are pinned elsewhere; these tests pin how a layer wires them:
which projection feeds which input, the attention scale, QK-norm and RoPE of
the query at the current position, the per-head slicing of the DeltaNet
projections and the affine maps of its decay, write strength and output gate.

Every weight matrix here is "one-hot": a Q4_0 row is zero except for one code
(nibble 9 or 7, i.e. +-1 times the row's fp16 scale), so each projection
output is a known multiple of one entry of the normalised input.  The input
h is a +-1 pattern, whose RMSNorm is h / sqrt(1 + eps) in closed form.  The
expected outputs below are written out case by case from the layer
definitions (ChatTorrent README, "What it can run": Llama-style blocks with
SwiGLU, the hybrid's gated attention with QK-norm and partial RoPE, Gated
DeltaNet), not by calling the oracle's layer code.

Each pin is then re-run against deliberately broken copies of the oracle (a
mistake planted in its source text): swapped gate/up, a dropped attention
scale, RoPE of q one position off, a dropped q-norm, swapped q/k projections,
wrong decay / write-strength / gate coefficients, a wrong head slice.  Every
mutant must fail at least one pin.
"""
import dataclasses
import inspect
import math
import textwrap

import numpy as np
import pytest

import oracle
import synth
from oracle import model as omodel
from oracle import qref

# the small hybrid of the other oracle pins: hidden 64, 2 DeltaNet heads of
# 32, 4 query / 2 KV heads of 32 with 16 rotated dims, SwiGLU 96
TINY = synth.ModelShape(
    name="tiny_hybrid", hidden=64, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=32, dn_dv=32, q_heads=4, kv_heads=2, head_dim=32, rope_dims=16,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=96, vocab=0)
EPS = TINY.eps
S_NORM = 1.0 / math.sqrt(1.0 + EPS)      # RMSNorm of a +-1 vector (weights 1)


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def onehot_q4(rows: int, cols: int, entries: dict) -> np.ndarray:
    """Q4_0 blocks of a rows x cols matrix that is zero except
    W[r, c] = sgn * d for every r -> (c, d, sgn) in entries (d exact in fp16)."""
    nb = cols // 32
    blk = np.zeros((rows, nb, 18), np.uint8)
    blk[:, :, 2:] = 0x88                      # every nibble 8: weight 0
    for r, (c, d, sgn) in entries.items():
        b, e = divmod(c, 32)
        blk[r, b, 0:2] = np.array([d], np.float16).view(np.uint8)
        byte, nib = 2 + e % 16, 8 + sgn
        if e < 16:
            blk[r, b, byte] = (blk[r, b, byte] & 0xF0) | nib
        else:
            blk[r, b, byte] = (blk[r, b, byte] & 0x0F) | (nib << 4)
    return blk.reshape(rows, nb * 18)


def test_onehot_blocks_decode_to_the_intended_matrix():
    ent = {0: (5, 0.5, 1), 3: (17, 1.5, -1), 4: (40, 0.25, 1), 6: (63, 2.0, -1)}
    W = qref.dequant(synth.Q4_0, onehot_q4(8, 64, ent), 8, 64)
    ref = np.zeros((8, 64))
    for r, (c, d, sgn) in ent.items():
        ref[r, c] = sgn * d
    np.testing.assert_array_equal(W, ref)


def _pm1(seed, n):
    return np.where(np.random.default_rng(seed).random(n) < 0.5, -1.0, 1.0).astype(np.float32)


def _zero_all(T, layer, names):
    """Set the named matrices of one layer's tensors to zero (scale 0 everywhere)."""
    shapes = synth.matrix_shapes(TINY, layer)
    for n in names:
        T[n] = onehot_q4(*shapes[n], {})


def _layer(l):
    return synth.layer_tensors(TINY, synth.Q4_0, 0, 91, l)


# ------------------------------------------------------------------ FFN

def pin_ffn():
    """Layer 1 (DeltaNet) with a zero mixer, which leaves h unchanged, and a
    one-hot SwiGLU: m_i = silu(gate_i) * up_i, h += W_down m."""
    T = _layer(1)
    _zero_all(T, 1, ["dn_q", "dn_k", "dn_v", "dn_a", "dn_b", "dn_z", "dn_out"])
    F, H = TINY.ffn, TINY.hidden
    T["w_gate"] = onehot_q4(F, H, {0: (2, 1.5, 1), 1: (3, 0.5, -1), 7: (9, 2.0, 1)})
    T["w_up"] = onehot_q4(F, H, {0: (4, 0.25, 1), 1: (5, 2.0, 1), 7: (10, 1.0, -1)})
    T["w_down"] = onehot_q4(H, F, {0: (0, 1.0, 1), 1: (1, 0.5, 1), 2: (2, 1.0, 1), 9: (7, 0.75, -1)})
    orc = oracle.SliceOracle(TINY, synth.Q4_0, 1, 2, {1: T}, max_seq=16, io_fp32=True)
    orc.set_state(1, synth.dn_state0(0, 91, 1, 2, 32, 32))
    orc.reset(3)
    h = _pm1(1, H)
    out = orc.decode(h, raw=True)
    x = S_NORM * h.astype(np.float64)

    def silu_times(g, u):
        return g * sig(g) * u

    m0 = silu_times(1.5 * x[2], 0.25 * x[4])
    m1 = silu_times(-0.5 * x[3], 2.0 * x[5])
    m7 = silu_times(2.0 * x[9], -1.0 * x[10])
    exp = h.astype(np.float64).copy()
    exp[0] += 1.0 * m0
    exp[1] += 0.5 * m1
    exp[2] += 1.0 * 0.0        # gate row 2 is zero, so m_2 = silu(0) * 0 = 0
    exp[9] += -0.75 * m7
    np.testing.assert_allclose(out, exp, rtol=1e-12, atol=1e-15)


def test_ffn_closed_form():
    pin_ffn()


# ------------------------------------------------------------- attention

def pin_attention():
    """Layer 3 (attention), one prior cache row, decode at position p = 1.

    Query head 0 is one-hot at dimension 0 (q_raw = 0.5 x[5]); QK-norm over
    its 32 entries makes it qn = q_raw / sqrt(q_raw^2 / 32 + eps); RoPE at
    p = 1 rotates the pair (0, 8) by 1 rad (frequency theta^0).  The prior key
    row of KV head 0 holds 1.5 at dimension 0 and 1.0 at dimension 8, so its
    score is qn (1.5 cos 1 + 1.0 sin 1) / sqrt(32); the new row's key and value
    are 0 (W_k = W_v = 0), score 0.  Head 0 thus weights the prior value row by
    sigmoid(s0).  Head 1 (q = 0) weights both rows 1/2; heads 2, 3 read KV head
    1 likewise.  W_g = 0 gives the gate sigmoid(0) = 1/2; h += W_o u."""
    T = _layer(3)
    nq, H, hd = TINY.q_heads * TINY.head_dim, TINY.hidden, TINY.head_dim
    T["wq"] = onehot_q4(nq, H, {0: (5, 0.5, 1)})
    _zero_all(T, 3, ["wg", "wk", "wv", "w_gate", "w_up", "w_down"])
    orc = oracle.SliceOracle(TINY, synth.Q4_0, 3, 4, {3: T}, max_seq=16, io_fp32=True)
    K = np.zeros((2, 1, hd), np.float16)
    K[0, 0, 0], K[0, 0, 8] = 1.5, 1.0
    K[1, 0, 3] = -2.0
    V = np.random.default_rng(2).standard_normal((2, 1, hd)).astype(np.float16)
    orc.set_kv(3, K, V)
    orc.reset(1)
    h = _pm1(3, H)
    out = orc.decode(h, raw=True)
    x = S_NORM * h.astype(np.float64)
    q_raw = 0.5 * x[5]
    qn = q_raw / math.sqrt(q_raw * q_raw / hd + EPS)
    s0 = qn * (1.5 * math.cos(1.0) + 1.0 * math.sin(1.0)) / math.sqrt(hd)
    w0 = sig(s0)                     # softmax over [s0, 0]
    V0, V1 = V[0, 0].astype(np.float64), V[1, 0].astype(np.float64)
    o = np.concatenate([w0 * V0, 0.5 * V0, 0.5 * V1, 0.5 * V1])
    u = 0.5 * o
    Wo = qref.dequant(synth.Q4_0, T["wo"], H, nq)
    np.testing.assert_allclose(out, h.astype(np.float64) + Wo @ u, rtol=1e-10, atol=1e-12)
    # the new cache row: k = v = 0 after norm and RoPE
    assert np.all(orc.kv[3][0][:, 1] == 0) and np.all(orc.kv[3][1][:, 1] == 0)


def pin_attention_key():
    """The key side: k of KV head 1 one-hot at dimension 1 (k_raw = -0.75 x[7]),
    v one-hot at dimension 30.  The cache row written at p = 5 is
    fp16(RoPE_5(k-norm(k))) and fp16(v): dimension 1 pairs with 9 and turns by
    5 theta^(-1/8) rad.  Query head 2 (which reads KV head 1) is one-hot at
    dimension 1 too, so its score against the new row is qn kn / sqrt(32)
    whatever the angle, and against the 5 zero prior rows 0."""
    T = _layer(3)
    nq, nkv, H, hd = TINY.q_heads * TINY.head_dim, TINY.kv_heads * TINY.head_dim, TINY.hidden, TINY.head_dim
    T["wq"] = onehot_q4(nq, H, {2 * hd + 1: (11, 1.0, 1)})
    T["wk"] = onehot_q4(nkv, H, {hd + 1: (7, 0.75, -1)})
    T["wv"] = onehot_q4(nkv, H, {hd + 30: (12, 2.0, 1)})
    _zero_all(T, 3, ["wg", "w_gate", "w_up", "w_down"])
    orc = oracle.SliceOracle(TINY, synth.Q4_0, 3, 4, {3: T}, max_seq=16, io_fp32=True)
    z = np.zeros((2, 5, hd), np.float16)
    orc.set_kv(3, z, z)
    orc.reset(5)
    h = _pm1(4, H)
    out = orc.decode(h, raw=True)
    x = S_NORM * h.astype(np.float64)
    k_raw = -0.75 * x[7]
    kn = k_raw / math.sqrt(k_raw * k_raw / hd + EPS)
    ang = 5.0 * 1e7 ** (-2.0 / 16)
    krow = np.zeros(hd)
    krow[1], krow[9] = kn * math.cos(ang), kn * math.sin(ang)
    np.testing.assert_array_equal(orc.kv[3][0][1, 5], krow.astype(np.float16))
    vrow = np.zeros(hd)
    vrow[30] = 2.0 * x[12]
    np.testing.assert_array_equal(orc.kv[3][1][1, 5], vrow.astype(np.float16))
    assert np.all(orc.kv[3][0][0, 5] == 0)
    q_raw = 1.0 * x[11]
    qn = q_raw / math.sqrt(q_raw * q_raw / hd + EPS)
    # the rotated query: pair (1, 9) of R(5) qn e_1
    qrot = np.zeros(hd)
    qrot[1], qrot[9] = qn * math.cos(ang), qn * math.sin(ang)
    kc = orc.kv[3][0][1, 5].astype(np.float64)
    s_new = float(qrot @ kc) / math.sqrt(hd)
    w_new = math.exp(s_new) / (math.exp(s_new) + 5.0)
    vc = orc.kv[3][1][1, 5].astype(np.float64)
    o = np.zeros((4, hd))
    o[2] = w_new * vc
    o[3] = vc / 6.0                 # head 3: q = 0, six equal scores
    u = 0.5 * o.reshape(-1)
    Wo = qref.dequant(synth.Q4_0, T["wo"], H, nq)
    np.testing.assert_allclose(out, h.astype(np.float64) + Wo @ u, rtol=1e-10, atol=1e-12)


def test_attention_query_side_closed_form():
    pin_attention()


def test_attention_key_side_closed_form():
    pin_attention_key()


# -------------------------------------------------------------- DeltaNet

def pin_deltanet():
    """Layer 0 (DeltaNet), two heads of 32.

    Head 0: q and k one-hot at the same key dimension 3, v non-zero at value
    dimensions 5 and 6, decay input a = 2 x[30], write strength b = 1.5 x[31].
    Head 1: q at key dimension 10, k at 20, v at dimension 2, a = 0, b = x[32].
    With kh = kappa e_j (kappa = k / sqrt(k^2 + 1e-6)) the update
    S' = alpha S (I - beta kh kh^T) + beta v kh^T scales every column by alpha
    and replaces column j by alpha (1 - beta kappa^2) S[:, j] + beta kappa v;
    o = rho S'[:, j_q].  alpha = sigmoid(0.125 a + 2), beta = sigmoid(0.25 b);
    the output is gated by sigmoid(0.25 z) (z one-hot at two rows, else 0)."""
    T = _layer(0)
    H, nk = TINY.hidden, TINY.dn_heads * TINY.dn_dk
    T["dn_q"] = onehot_q4(nk, H, {3: (7, 0.25, 1), 32 + 10: (11, 0.5, -1)})
    T["dn_k"] = onehot_q4(nk, H, {3: (13, 0.5, 1), 32 + 20: (17, 0.75, 1)})
    T["dn_v"] = onehot_q4(nk, H, {5: (21, 1.0, 1), 6: (22, 0.5, -1), 32 + 2: (23, 0.25, 1)})
    T["dn_a"] = onehot_q4(2, H, {0: (30, 2.0, 1)})
    T["dn_b"] = onehot_q4(2, H, {0: (31, 1.5, 1), 1: (32, 1.0, -1)})
    T["dn_z"] = onehot_q4(nk, H, {3: (33, 2.0, 1), 32 + 10: (34, 1.0, 1)})
    _zero_all(T, 0, ["w_gate", "w_up", "w_down"])
    orc = oracle.SliceOracle(TINY, synth.Q4_0, 0, 1, {0: T}, max_seq=16, io_fp32=True)
    S0 = synth.dn_state0(0, 91, 0, 2, 32, 32) * 10
    orc.set_state(0, S0)
    orc.reset(4)
    h = _pm1(5, H)
    out = orc.decode(h, raw=True)
    x = S_NORM * h.astype(np.float64)
    S = S0.astype(np.float64)

    def unit(a):
        return a / math.sqrt(a * a + 1e-6)

    alpha = [sig(0.125 * (2.0 * x[30]) + 2.0), sig(2.0)]
    beta = [sig(0.25 * (1.5 * x[31])), sig(0.25 * (-1.0 * x[32]))]
    kappa = [unit(0.5 * x[13]), unit(0.75 * x[17])]
    rho = [unit(0.25 * x[7]), unit(-0.5 * x[11])]
    jk, jq = [3, 20], [3, 10]
    v = np.zeros((2, 32))
    v[0, 5], v[0, 6], v[1, 2] = 1.0 * x[21], -0.5 * x[22], 0.25 * x[23]
    Sn = np.empty_like(S)
    o = np.empty((2, 32))
    for hh in range(2):
        Sn[hh] = alpha[hh] * S[hh]
        Sn[hh][:, jk[hh]] = alpha[hh] * (1 - beta[hh] * kappa[hh] ** 2) * S[hh][:, jk[hh]] \
            + beta[hh] * kappa[hh] * v[hh]
        o[hh] = rho[hh] * Sn[hh][:, jq[hh]]
    z = np.zeros(64)
    z[3], z[32 + 10] = 2.0 * x[33], 1.0 * x[34]
    u = o.reshape(-1) * np.array([sig(0.25 * zz) for zz in z])
    Wout = qref.dequant(synth.Q4_0, T["dn_out"], H, nk)
    np.testing.assert_allclose(orc.dn[0], Sn.astype(np.float32), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(out, h.astype(np.float64) + Wout @ u, rtol=1e-10, atol=1e-12)


def test_deltanet_wiring_closed_form():
    pin_deltanet()


# ------------------------------------------------------- planted mistakes

# (method of SliceOracle, text in its source, replacement): each is a
# plausible wiring mistake that one of the pins above must catch.
def pin_deltanet_token():
    """The DeltaNet mixer fed its pre-activations as one row [q|k|v|a|b|z],
    three heads of d_k = 4, d_v = 3, each with q = c_q e_{jq} and k = c_k e_{jk}
    at distinct dimensions (jq != jk): after L2 normalisation kh = kappa e_jk
    and qh = rho e_jq, so S' = alpha S (I - beta kh kh^T) + beta v kh^T keeps
    column jq at alpha S[:, jq] and o = rho alpha S[:, jq]; column jk becomes
    alpha (1 - beta kappa^2) S[:, jk] + beta kappa v.  alpha = sigmoid(a),
    beta = sigmoid(b), and the output is o * sigmoid(z)."""
    heads, dk, dv = 3, 4, 3
    jq, jk = [0, 2, 3], [1, 0, 2]
    cq, ck = [2.0, -0.5, 1.25], [0.75, 3.0, -1.5]
    a, b = [0.5, -1.0, 2.5], [1.0, -0.25, 0.0]
    v = np.array([[1.0, -2.0, 0.5], [0.25, 0.0, -1.0], [3.0, 1.5, -0.75]])
    z = np.array([[0.1, -0.2, 0.3], [1.0, 0.0, -1.0], [2.0, -2.0, 0.5]])
    q = np.zeros((heads, dk))
    k = np.zeros((heads, dk))
    for h in range(heads):
        q[h, jq[h]], k[h, jk[h]] = cq[h], ck[h]
    row = np.concatenate([q.ravel(), k.ravel(), v.ravel(), a, b, z.ravel()])
    S0 = synth.dn_state0(0, 93, 0, heads, dv, dk) * 10
    S = S0.copy()
    out = omodel.deltanet_token(S, row, dk, dv)
    for h in range(heads):
        def unit(c):
            return c / math.sqrt(c * c + 1e-6)
        al, be = sig(a[h]), sig(b[h])
        kap, rho = unit(ck[h]), unit(cq[h])
        S0h = S0[h].astype(np.float64)
        col_q = al * S0h[:, jq[h]]
        col_k = al * (1 - be * kap * kap) * S0h[:, jk[h]] + be * kap * v[h]
        want_o = rho * col_q * np.array([sig(t) for t in z[h]])
        np.testing.assert_allclose(out[h * dv:(h + 1) * dv], want_o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[h][:, jq[h]], col_q.astype(np.float32), rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(S[h][:, jk[h]], col_k.astype(np.float32), rtol=1e-6, atol=1e-7)
        for j in range(dk):
            if j not in (jq[h], jk[h]):
                np.testing.assert_allclose(S[h][:, j], (al * S0h[:, j]).astype(np.float32), rtol=1e-6, atol=1e-7)


def test_deltanet_token_closed_form():
    pin_deltanet_token()


# ------------------------------------------------ qwen3_5-form DeltaNet

def silu_(z):
    return z / (1.0 + math.exp(-z))


def pin_conv_silu():
    """Two channels, width 4: window = state (oldest first) then the input,
    tap 3 on the input.  Channel 0: taps (0.5, -1, 2, 0.25) over (1, 2, 3, 5)
    give 0.5 - 2 + 6 + 1.25 = 5.75; channel 1: taps (1, 0, 0, 0) pick the
    oldest input, -1.  The new state drops the oldest input."""
    state = np.array([[1.0, 2.0, 3.0], [-1.0, 0.0, 4.0]], np.float32)
    x = np.array([5.0, -2.0])
    w = np.array([[0.5, -1.0, 2.0, 0.25], [1.0, 0.0, 0.0, 0.0]])
    y, st = omodel.conv_silu(state, x, w)
    np.testing.assert_allclose(y, [silu_(5.75), silu_(-1.0)], rtol=1e-15)
    np.testing.assert_array_equal(st, np.array([[2.0, 3.0, 5.0], [0.0, 4.0, -2.0]], np.float32))


def pin_gated_rmsnorm():
    """o = (3, 4): mean square 12.5; weights (1, 2); gate inputs (0, 1):
    silu(0) = 0 silences the first entry, the second is 4 / sqrt(12.5 + eps)
    * 2 * silu(1)."""
    out = omodel.gated_rmsnorm(np.array([3.0, 4.0]), np.array([0.0, 1.0]), np.array([1.0, 2.0]), 1e-6)
    np.testing.assert_allclose(out, [0.0, 4.0 / math.sqrt(12.5 + 1e-6) * 2.0 * silu_(1.0)], rtol=1e-14, atol=1e-300)


def pin_deltanet_heads_q35():
    """Four value heads of d_v = 3 sharing two query/key heads of d_k = 4
    (heads 0, 1 read key head 0; heads 2, 3 key head 1).  Key head m has
    q = c_q e_{jq} and k = c_k e_{jk} (jq != jk), so qh = rho e_jq / 2
    (rho = c_q / sqrt(c_q^2 + 1e-6), 1/sqrt(d_k) = 1/2) and kh = kappa e_jk.
    Column jq of S' is alpha S[:, jq], so o = (rho / 2) alpha S[:, jq]; the
    head's output is rmsnorm(o) * w * silu(z_h)."""
    heads, kheads, dk, dv = 4, 2, 4, 3
    jq, jk = [0, 3], [2, 1]
    cq, ck = [2.0, -0.5], [0.75, 3.0]
    q = np.zeros(kheads * dk)
    k = np.zeros(kheads * dk)
    for m in range(kheads):
        q[m * dk + jq[m]], k[m * dk + jk[m]] = cq[m], ck[m]
    v = np.arange(heads * dv, dtype=np.float64) * 0.25 - 1.0
    z = np.linspace(-1.5, 2.0, heads * dv)
    alpha = np.array([0.9, 0.5, 0.25, 0.75])
    beta = np.array([0.1, 0.6, 0.3, 0.8])
    w = np.array([1.0, 0.5, 2.0])
    S0 = synth.dn_state0(0, 94, 0, heads, dv, dk) * 10
    S = S0.copy()
    out = omodel.deltanet_heads_q35(S, q, k, v, alpha, beta, z, w, 1e-6, dk, dv, kheads)
    for h in range(heads):
        m = h // 2
        rho = cq[m] / math.sqrt(cq[m] ** 2 + 1e-6)
        o = (rho / 2.0) * alpha[h] * S0[h][:, jq[m]].astype(np.float64)
        ms = np.mean(o * o)
        want = o / math.sqrt(ms + 1e-6) * w * np.array([silu_(zz) for zz in z[h * dv:(h + 1) * dv]])
        np.testing.assert_allclose(out[h * dv:(h + 1) * dv], want, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(S[h][:, jq[m]], (alpha[h] * S0[h][:, jq[m]].astype(np.float64)).astype(np.float32),
                                   rtol=1e-6)


TINY_Q35 = synth.ModelShape(
    name="tiny_hybrid_q35", hidden=64, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=32, dn_dv=32, q_heads=4, kv_heads=2, head_dim=32, rope_dims=16,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=96, vocab=0,
    dn_variant=1, dn_k_heads=1, dn_conv=4)


def pin_deltanet_q35_layer():
    """Layer 0 of a qwen3_5-form slice: two value heads of 32 sharing one
    query/key head, conv taps (0, 0, 0, 1) on every channel (the conv passes
    the current input; then SiLU) from a zero conv state.  q is one-hot at key
    dimension 3 (0.5 x[7]), k at 10 (0.75 x[11]); head 0's v at 5 (x[21]),
    head 1's at 2 (-0.5 x[23]); a = 2 x[30] and -x[31], b = 1.5 x[32] and
    x[33]; every gate row is +-0.5 times one input entry.  alpha = exp(-exp(A_log)
    softplus(0.125 a + dt_bias)), beta = sigmoid(0.25 b); column 3 of S' is
    alpha S[:, 3], so o = alpha rho / sqrt(32) S[:, 3] with rho = unit(silu(0.5 x[7]));
    column 10 becomes alpha (1 - beta kappa^2) S[:, 10] + beta kappa silu(v)
    (kappa = unit(silu(0.75 x[11]))).  The new conv state's last column holds
    the pre-conv q | k | v."""
    sh = TINY_Q35
    T = synth.layer_tensors(sh, synth.Q4_0, 0, 95, 0)
    H, nk, nv = sh.hidden, sh.k_heads * sh.dn_dk, sh.dn_heads * sh.dn_dv
    T["dn_q"] = onehot_q4(nk, H, {3: (7, 0.5, 1)})
    T["dn_k"] = onehot_q4(nk, H, {10: (11, 0.75, 1)})
    T["dn_v"] = onehot_q4(nv, H, {5: (21, 1.0, 1), 32 + 2: (23, 0.5, -1)})
    T["dn_a"] = onehot_q4(2, H, {0: (30, 2.0, 1), 1: (31, 1.0, -1)})
    T["dn_b"] = onehot_q4(2, H, {0: (32, 1.5, 1), 1: (33, 1.0, 1)})
    zrows = {r: ((r * 7) % 64, 0.5, 1 if r % 2 == 0 else -1) for r in range(nv)}
    T["dn_z"] = onehot_q4(nv, H, zrows)
    taps = np.zeros((sh.conv_dim, 4), np.float32)
    taps[:, 3] = 1.0
    T["dn_conv"] = taps.reshape(-1)
    shapes = synth.matrix_shapes(sh, 0)
    for n in ("w_gate", "w_up", "w_down"):
        T[n] = onehot_q4(*shapes[n], {})
    orc = oracle.SliceOracle(sh, synth.Q4_0, 0, 1, {0: T}, max_seq=16, io_fp32=True)
    S0 = synth.dn_state0(0, 95, 0, 2, 32, 32) * 10
    orc.set_state(0, S0)
    orc.reset(2)
    h = _pm1(6, H)
    out = orc.decode(h, raw=True)
    x = S_NORM * h.astype(np.float64)

    def unit(c):
        return c / math.sqrt(c * c + 1e-6)

    def softplus(t):
        return math.log1p(math.exp(t))

    alog, dtb, wn = (T[n].astype(np.float64) for n in ("dn_alog", "dn_dtb", "dn_norm"))
    a = [2.0 * x[30], -1.0 * x[31]]
    b = [1.5 * x[32], 1.0 * x[33]]
    alpha = [math.exp(-math.exp(alog[hh]) * softplus(0.125 * a[hh] + dtb[hh])) for hh in range(2)]
    beta = [sig(0.25 * b[hh]) for hh in range(2)]
    rho = unit(silu_(0.5 * x[7]))
    kappa = unit(silu_(0.75 * x[11]))
    vv = np.zeros((2, 32))
    vv[0, 5], vv[1, 2] = silu_(1.0 * x[21]), silu_(-0.5 * x[23])
    S = S0.astype(np.float64)
    u = np.empty(nv)
    for hh in range(2):
        Sn = alpha[hh] * S[hh]
        Sn[:, 10] = alpha[hh] * (1 - beta[hh] * kappa ** 2) * S[hh][:, 10] + beta[hh] * kappa * vv[hh]
        np.testing.assert_allclose(orc.dn[0][hh], Sn.astype(np.float32), rtol=1e-6, atol=1e-9)
        o = rho / math.sqrt(32.0) * Sn[:, 3]
        zg = np.array([0.25 * zrows[r][2] * 0.5 * x[zrows[r][0]] for r in range(hh * 32, hh * 32 + 32)])
        u[hh * 32:(hh + 1) * 32] = o / math.sqrt(np.mean(o * o) + 1e-6) * wn * np.array([silu_(t) for t in zg])
    Wout = qref.dequant(synth.Q4_0, T["dn_out"], H, nv)
    np.testing.assert_allclose(out, h.astype(np.float64) + Wout @ u, rtol=1e-9, atol=1e-12)
    pre = np.zeros(sh.conv_dim)
    pre[3], pre[nk + 10] = 0.5 * x[7], 0.75 * x[11]
    pre[2 * nk + 5], pre[2 * nk + 32 + 2] = 1.0 * x[21], -0.5 * x[23]
    np.testing.assert_allclose(orc.conv[0][:, 2], pre.astype(np.float32), rtol=1e-6, atol=1e-12)
    assert not orc.conv[0][:, :2].any()


def test_conv_silu_closed_form():
    pin_conv_silu()


def test_gated_rmsnorm_closed_form():
    pin_gated_rmsnorm()


def test_deltanet_heads_q35_closed_form():
    pin_deltanet_heads_q35()


def test_deltanet_q35_layer_closed_form():
    pin_deltanet_q35_layer()


# ------------------------------------------------------------ draft head

def _const_rows_q4(values: list, cols: int) -> np.ndarray:
    """Q4_0 rows whose every weight is the given (code, scale): value (code - 8) * scale."""
    nb = cols // 32
    blk = np.zeros((len(values), nb, 18), np.uint8)
    for r, (code, d) in enumerate(values):
        blk[r, :, 0:2] = np.array([d], np.float16).view(np.uint8)
        blk[r, :, 2:] = code | (code << 4)
    return blk.reshape(len(values), nb * 18)


def pin_mtp_input():
    """The draft head's input projection on one-hot rows of fc: each output is a
    known multiple of one entry of [RMSNorm(e; w_e), RMSNorm(h; w_h)].  The
    embedding rows are constant (value v, so RMSNorm gives v / sqrt(v^2 + eps)
    times w_e) and h is a +-3 pattern (RMSNorm h / sqrt(9 + eps) times w_h)."""
    H = 64
    rows = [(9, 0.5), (5, 0.25), (12, 2.0), (8, 1.0)]          # values 0.5, -0.75, 8, 0
    E = _const_rows_q4(rows, H)
    h = 3.0 * _pm1(7, H).astype(np.float64)
    w_e = (1.0 + np.arange(H) / 64.0).astype(np.float32)
    w_h = (2.0 - np.arange(H) / 128.0).astype(np.float32)
    ent = {0: (3, 1.0, 1), 1: (H + 5, 0.5, -1), 2: (H - 1, 2.0, 1), 3: (2 * H - 1, 0.25, 1), 6: (H, 1.5, -1)}
    fc = onehot_q4(H, 2 * H, ent)
    for tok, (code, d) in enumerate(rows):
        v = (code - 8) * d
        ne = v / math.sqrt(v * v + EPS)
        nh = h / math.sqrt(9.0 + EPS)
        c = np.concatenate([ne * w_e.astype(np.float64), nh * w_h.astype(np.float64)])
        exp = np.zeros(H)
        for r, (col, dd, sgn) in ent.items():
            exp[r] = sgn * dd * c[col]
        got = omodel.mtp_input(synth.Q4_0, E, tok, h, w_e, w_h, fc, H, EPS)
        np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-15)


def test_mtp_input_closed_form():
    pin_mtp_input()


def test_mtp_input_rejects_a_token_outside_the_vocabulary():
    E = _const_rows_q4([(9, 0.5)], 64)
    with pytest.raises(ValueError):
        omodel.mtp_input(synth.Q4_0, E, 1, np.ones(64), np.ones(64), np.ones(64), onehot_q4(64, 128, {}), 64, EPS)


def test_draft_head_through_an_identity_layer():
    """With every matrix of the draft head's layer zero the layer leaves its
    input unchanged, so a draft is argmax(W_head RMSNorm(x; out_norm)) of the
    rounded projection x, computed here from the dequantised matrices with
    numpy products."""
    sh = synth.mtp_shape(dataclasses.replace(TINY, vocab=48, tied_head=False))
    T = synth.layer_tensors(sh, synth.Q4_0, 0, synth.WL_MTP, 0)
    _zero_all_shape(T, sh, 0)
    M = synth.mtp_tensors(sh, synth.Q4_0, 3)
    G = synth.global_tensors(sh, synth.Q4_0, 3, 0)
    G["out_norm"] = M["mtp_out_norm"]
    dh = oracle.DraftHead(sh, synth.Q4_0, T, M, G, max_seq=16, io_fp32=False)
    dh.reset(2)
    H = sh.hidden
    h = synth.hidden_inputs(3, 0, 1, H)[0]
    Ed = qref.dequant(synth.Q4_0, G["embed"], sh.vocab, H)
    Fd = qref.dequant(synth.Q4_0, M["mtp_fc"], H, 2 * H)
    Hd = qref.dequant(synth.Q4_0, G["head"], sh.vocab, H)

    def rms(v, w):
        return v / np.sqrt(np.mean(v * v) + EPS) * w.astype(np.float64)

    for tok in (0, 17, 47):
        x = Fd @ np.concatenate([rms(Ed[tok], M["mtp_norm_e"]), rms(h.astype(np.float64), M["mtp_norm_h"])])
        xr = x.astype(np.float16)
        logits = Hd @ rms(xr.astype(np.float64), M["mtp_out_norm"])
        d, out, lg = dh.draft(tok, h)
        np.testing.assert_array_equal(out, xr)
        np.testing.assert_allclose(lg, logits, rtol=1e-9, atol=1e-12)
        assert d == int(np.argmax(logits))
    assert dh.pos == 5


def _zero_all_shape(T, shape, layer):
    for n, (r, c) in synth.matrix_shapes(shape, layer).items():
        T[n] = onehot_q4(r, c, {})


MUTANTS = {
    "ffn_gate_up_swapped": ("SliceOracle.ffn", 'silu(self._mv(l, "w_gate", x)) * self._mv(l, "w_up", x)',
                            'silu(self._mv(l, "w_up", x)) * self._mv(l, "w_gate", x)'),
    "attn_scale_dropped": ("attention_heads", "scale = 1.0 / np.sqrt(hd)", "scale = 1.0"),
    "attn_scale_head_count": ("attention_heads", "scale = 1.0 / np.sqrt(hd)", "scale = 1.0 / np.sqrt(nq)"),
    "attn_q_rope_next_pos": ("attention_heads", "qi = rope(qi, p, ", "qi = rope(qi, p + 1, "),
    "attn_q_rope_prev_pos": ("attention_heads", "qi = rope(qi, p, ", "qi = rope(qi, p - 1, "),
    "attn_q_norm_dropped": ("attention_heads", "qi = rmsnorm(q[i], q_norm, s.eps) if s.qk_norm else q[i]",
                            "qi = q[i]"),
    "attn_k_rope_dropped": ("attention_heads", "rope(kj, p, s.rope_dims, s.rope_theta)", "kj"),
    "attn_head_map_mod": ("attention_heads", "j = i // grp", "j = i % nkv"),
    "attn_gate_dropped": ("attention_heads", "u = u * sigmoid(g)", "u = u"),
    "dn_q_k_swapped": ("SliceOracle.deltanet", 'q = self._mv(l, "dn_q", x)\n    k = self._mv(l, "dn_k", x)',
                       'k = self._mv(l, "dn_q", x)\n    q = self._mv(l, "dn_k", x)'),
    "dn_beta_coeff": ("SliceOracle.deltanet", "np.float32(s.dn_b_scale)", "np.float32(s.dn_a_scale)"),
    "dn_gate_coeff": ("SliceOracle.deltanet", "np.float32(s.dn_z_scale)", "np.float32(s.dn_a_scale)"),
    "dn_gate_dropped": ("deltanet_heads", "return o * np.asarray(gate, dtype=np.float64)", "return o"),
    "dn_alpha_bias": ("SliceOracle.deltanet", "+ np.float64(np.float32(s.dn_a_bias))", ""),
    "dn_head_slice": ("deltanet_heads", "kh = l2normalize(k[hh * dk:(hh + 1) * dk])", "kh = l2normalize(k[0:dk])"),
    "dn_token_a_b_swapped": ("deltanet_token", "sigmoid(a), sigmoid(b)", "sigmoid(b), sigmoid(a)"),
    "dn_token_q_k_swapped": ("deltanet_token", "deltanet_heads(S, q, k, v,", "deltanet_heads(S, k, q, v,"),
    "dn_token_z_offset": ("deltanet_token", "z = row[o:o + heads * dv]", "z = row[o - heads:o - heads + heads * dv]"),
    "q35_conv_taps_reversed": ("conv_silu", "y = np.sum(win * np.asarray(w, dtype=np.float64), axis=1)",
                               "y = np.sum(win * np.asarray(w, dtype=np.float64)[:, ::-1], axis=1)"),
    "q35_conv_state_not_shifted": ("conv_silu", "win[:, 1:].astype(np.float32)", "win[:, :-1].astype(np.float32)"),
    "q35_q_scale_dropped": ("deltanet_heads_q35", "l2normalize(q[kh * dk:(kh + 1) * dk]) / np.sqrt(dk)",
                            "l2normalize(q[kh * dk:(kh + 1) * dk])"),
    "q35_head_share_mod": ("deltanet_heads_q35", "kh = hh // ratio", "kh = hh % k_heads"),
    "q35_gate_sigmoid": ("gated_rmsnorm", "* silu(z)", "* sigmoid(z)"),
    "q35_norm_weight_dropped": ("gated_rmsnorm", "rmsnorm(o, w, eps)", "rmsnorm(o, np.ones_like(w), eps)"),
    "q35_softplus_dropped": ("SliceOracle.deltanet_q35", "softplus(np.float64(np.float32(s.dn_a_scale)) * a + dt_bias)",
                             "(np.float64(np.float32(s.dn_a_scale)) * a + dt_bias)"),
    "q35_alog_not_exp": ("SliceOracle.deltanet_q35", "-np.exp(a_log)", "-a_log"),
    "q35_qkv_order": ("SliceOracle.deltanet_q35", "np.concatenate([q, k, v])", "np.concatenate([k, q, v])"),
    "q35_beta_coeff": ("SliceOracle.deltanet_q35", "sigmoid(np.float64(np.float32(s.dn_b_scale)) * b)",
                       "sigmoid(np.float64(np.float32(s.dn_a_scale)) * b)"),
    "q35_gate_coeff": ("SliceOracle.deltanet_q35", "zg = np.float64(np.float32(s.dn_z_scale)) * z", "zg = z"),
    "dn_v_for_k": ("deltanet_heads", "vh = v[hh * dv:(hh + 1) * dv]", "vh = k[hh * dv:(hh + 1) * dv]"),
    "mtp_inputs_swapped": ("mtp_input", "np.concatenate([rmsnorm(e, w_e, eps), rmsnorm(np.asarray(h, dtype=np.float64), w_h, eps)])",
                           "np.concatenate([rmsnorm(np.asarray(h, dtype=np.float64), w_h, eps), rmsnorm(e, w_e, eps)])"),
    "mtp_norm_weights_swapped": ("mtp_input", "rmsnorm(e, w_e, eps), rmsnorm(np.asarray(h, dtype=np.float64), w_h, eps)",
                                 "rmsnorm(e, w_h, eps), rmsnorm(np.asarray(h, dtype=np.float64), w_e, eps)"),
    "mtp_embed_norm_dropped": ("mtp_input", "rmsnorm(e, w_e, eps)", "e * np.asarray(w_e, dtype=np.float64)"),
    "mtp_hidden_norm_dropped": ("mtp_input", "rmsnorm(np.asarray(h, dtype=np.float64), w_h, eps)",
                                "np.asarray(h, dtype=np.float64) * np.asarray(w_h, dtype=np.float64)"),
    "mtp_next_token_row": ("mtp_input", "E[token:token + 1]", "E[token + 1:token + 2]"),
}

PINS = [pin_ffn, pin_attention, pin_attention_key, pin_deltanet, pin_deltanet_token, pin_conv_silu,
        pin_gated_rmsnorm, pin_deltanet_heads_q35, pin_deltanet_q35_layer, pin_mtp_input]


def _mutant(where: str, old: str, new: str):
    """(owner, name, function) with the planted mistake; owner is the class or
    the oracle module the function lives in."""
    owner, _, name = where.rpartition(".")
    owner = getattr(omodel, owner) if owner else omodel
    src = textwrap.dedent(inspect.getsource(getattr(owner, name)))
    assert old in src, f"planted mistake no longer matches the oracle source: {old!r}"
    g = dict(vars(omodel))
    exec(compile(src.replace(old, new, 1), f"<mutant {where}>", "exec"), g)
    return owner, name, g[name]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    owner, fn, mutant = _mutant(*MUTANTS[name])
    monkeypatch.setattr(owner, fn, mutant)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin fails when the oracle has the mistake {name}"


def test_q35_commit_restores_conv_state():
    """verify(3) then commit(1) leaves the states (recurrent and conv) of one
    plain decode step, and the next steps agree."""
    sh = TINY_Q35
    tensors = {l: synth.layer_tensors(sh, synth.Q4_0, 0, 96, l) for l in range(4)}
    orcs = [oracle.SliceOracle(sh, synth.Q4_0, 0, 4, tensors, max_seq=32, io_fp32=True) for _ in range(2)]
    for orc in orcs:
        for l in range(3):
            orc.set_state(l, synth.dn_state0(0, 96, l, sh.dn_heads, sh.dn_dv, sh.dn_dk))
            orc.set_conv_state(l, synth.dn_conv_state0(0, 96, l, sh.conv_dim, sh.dn_conv))
        orc.reset(5)
    H = synth.hidden_inputs(0, 96, 6, sh.hidden).astype(np.float32)
    a, b = orcs
    a.verify(H[0:3], raw=True)
    a.commit(1)
    b.decode(H[0], raw=True)
    for l in range(3):
        np.testing.assert_array_equal(a.dn[l], b.dn[l])
        np.testing.assert_array_equal(a.conv[l], b.conv[l])
        assert not np.array_equal(a.conv[l], synth.dn_conv_state0(0, 96, l, sh.conv_dim, sh.dn_conv))
    for t in range(3, 6):
        np.testing.assert_array_equal(a.decode(H[t], raw=True), b.decode(H[t], raw=True))
