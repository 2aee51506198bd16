"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes part of the oracle against the format definitions (hand-decoded
golden blocks), numpy's own fp16 decoder, brute force on tiny shapes, closed
forms or invariants of the mathematics, chosen so that a dropped term, a wrong
sign, a wrong index or a transposed operand fails at least one of them.
"""
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import qref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_blocks():
    out = []
    cur = {}
    with open(os.path.join(GOLDEN, "quant_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "type":
                cur = {"type": {"Q4_0": synth.Q4_0, "Q8_0": synth.Q8_0}[rest.strip()]}
            elif key == "bytes":
                cur["bytes"] = np.array([int(b, 16) for b in rest.split()], dtype=np.uint8)
            elif key == "values":
                cur["values"] = np.array([float(v) for v in rest.split()])
                out.append(cur)
    return out


def test_golden_blocks_decode_exactly():
    blocks = _read_blocks()
    assert len(blocks) == 7
    for b in blocks:
        assert b["bytes"].size == synth.BLOCK_BYTES[b["type"]]
        got = qref.dequant(b["type"], b["bytes"][None, :], 1, 32)[0]
        np.testing.assert_array_equal(got, b["values"])


def test_half_decode_matches_numpy_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    # one Q8_0 block per pattern, code 1 in slot 0: the decoded weight is d itself
    blk = np.zeros((65536, 34), dtype=np.uint8)
    blk[:, 0:2] = bits.view(np.uint8).reshape(-1, 2)
    blk[:, 2] = 1
    got = qref.dequant(synth.Q8_0, blk, 65536, 32)[:, 0]
    np.testing.assert_array_equal(got[finite], ref[finite])
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.all(got[np.isinf(ref)] == ref[np.isinf(ref)])


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_generator_distributions(qtype):
    raw = synth.quant_blocks(synth.stream(0, 99, 0, 0), qtype, 256, 1024)
    bb = synth.BLOCK_BYTES[qtype]
    blk = raw.reshape(256, 32, bb)
    d = blk[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    assert d.min() >= np.float16(0.002) and d.max() <= np.float16(0.02)
    if qtype == synth.Q4_0:
        nib = np.concatenate([blk[:, :, 2:] & 15, blk[:, :, 2:] >> 4])
        assert nib.min() == 0 and nib.max() == 15
    else:
        q = blk[:, :, 2:].view(np.int8)
        assert q.min() == -127 and q.max() == 127


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_gemv_unit_vectors_give_columns_exactly(qtype):
    rows, cols = 64, 96
    raw = synth.quant_blocks(synth.stream(1, 99, 1, qtype), qtype, rows, cols)
    W = qref.dequant(qtype, raw, rows, cols)
    for j in (0, 1, 15, 16, 17, 31, 32, 63, 64, 95):
        e = np.zeros(cols)
        e[j] = 1.0
        np.testing.assert_array_equal(qref.gemv(qtype, raw, rows, cols, e), W[:, j])


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_gemv_matches_dense_product(qtype):
    rows, cols = 80, 160
    raw = synth.quant_blocks(synth.stream(2, 99, 2, qtype), qtype, rows, cols)
    W = qref.dequant(qtype, raw, rows, cols)
    x = synth.gemv_x(3, 5, cols).astype(np.float64)
    y = qref.gemv(qtype, raw, rows, cols, x)
    np.testing.assert_allclose(y, x @ W.T, rtol=1e-12, atol=1e-12)
    # one right-hand side at a time gives the same sums bit for bit
    for t in range(5):
        np.testing.assert_array_equal(qref.gemv(qtype, raw, rows, cols, x[t]), y[t])


def test_gemv_rejects_bad_shapes():
    raw = np.zeros((4, 18), np.uint8)
    with pytest.raises(ValueError):
        qref.gemv(synth.Q4_0, raw, 4, 33, np.zeros(33))


# ------------------------------------------------------------------ RMSNorm etc.

def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (0.5, -3.0, 1e-3):
        y = oracle.rmsnorm(np.full(8, c), np.ones(8), eps)
        np.testing.assert_allclose(y, c / np.sqrt(c * c + eps), rtol=1e-15)
    x = np.arange(1.0, 9.0)
    w = np.linspace(0.5, 2.0, 8)
    ms = np.mean(x * x)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, 0.0), x * w / np.sqrt(ms), rtol=1e-15)
    # scale invariance when eps is negligible
    np.testing.assert_allclose(oracle.rmsnorm(1000 * x, w, 1e-12), oracle.rmsnorm(x, w, 1e-12), rtol=1e-12)


def test_sigmoid_silu_values():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.sigmoid(np.log(3.0)), 0.75, rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.log(3.0)), 0.75 * np.log(3.0), rtol=1e-15)
    assert oracle.silu(-40.0) < 0 and abs(oracle.silu(-40.0)) < 1e-15


def test_l2normalize():
    v = np.array([3.0, 4.0])
    np.testing.assert_allclose(oracle.l2normalize(v, 0.0), [0.6, 0.8], rtol=1e-15)
    assert abs(np.linalg.norm(oracle.l2normalize(np.arange(1.0, 129.0))) - 1) < 1e-9


# ------------------------------------------------------------------------ RoPE

def _rope_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "rope.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "case":
                cur = dict(kv.split("=") for kv in rest.split())
            elif key == "x":
                cur["x"] = np.array([float(v) for v in rest.split()])
            elif key == "y":
                cur["y"] = np.array([float(v) for v in rest.split()])
                cases.append(cur)
    return cases


def test_rope_golden():
    cases = _rope_cases()
    assert len(cases) == 2
    for c in cases:
        y = oracle.rope(c["x"], int(c["pos"]), int(c["rope_dims"]), float(c["theta"]))
        np.testing.assert_allclose(y, c["y"], rtol=1e-14, atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(256)
    np.testing.assert_array_equal(oracle.rope(x, 0, 64, 1e7), x)          # position 0: identity
    y = oracle.rope(x, 12345, 64, 1e7)
    np.testing.assert_array_equal(y[64:], x[64:])                          # partial: tail untouched
    h = 32
    np.testing.assert_allclose(y[:h] ** 2 + y[h:64] ** 2, x[:h] ** 2 + x[h:64] ** 2, rtol=1e-12)
    # relative position: <R(p)q, R(p')k> depends only on p - p'
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = oracle.rope(q, 10, 64, 1e4) @ oracle.rope(k, 7, 64, 1e4)
    b = oracle.rope(q, 103, 64, 1e4) @ oracle.rope(k, 100, 64, 1e4)
    np.testing.assert_allclose(a, b, rtol=1e-10)


# ------------------------------------------------------------------- attention

def test_attend_single_row_is_value_row():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((1, 16)).astype(np.float16)
    V = rng.standard_normal((1, 16)).astype(np.float16)
    o = oracle.attend(rng.standard_normal(16), K, V, 0.25)
    np.testing.assert_array_equal(o, V[0].astype(np.float64))


def test_attend_equal_keys_average_values():
    rng = np.random.default_rng(7)
    K = np.tile(rng.standard_normal((1, 16)), (5, 1)).astype(np.float16)
    V = rng.standard_normal((5, 16)).astype(np.float16)
    o = oracle.attend(rng.standard_normal(16), K, V, 0.25)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), rtol=1e-12, atol=1e-15)


def test_attend_dominant_key_and_weights():
    # two keys, scores s0 = 0, s1 = ln 3 -> weights 1/4, 3/4
    K = np.array([[0.0, 0.0], [1.0, 0.0]], np.float16)
    V = np.array([[4.0, 0.0], [0.0, 8.0]], np.float16)
    o = oracle.attend(np.array([np.log(3.0), 5.0]), K, V, 1.0)
    np.testing.assert_allclose(o, [1.0, 6.0], rtol=1e-12)
    # row order does not matter
    o2 = oracle.attend(np.array([np.log(3.0), 5.0]), K[::-1].copy(), V[::-1].copy(), 1.0)
    np.testing.assert_allclose(o, o2, rtol=1e-14)


# -------------------------------------------------------------------- DeltaNet

def _dn_inputs(seed, d=8):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((d, d)) * 0.1
    q = oracle.l2normalize(rng.standard_normal(d))
    k = oracle.l2normalize(rng.standard_normal(d))
    v = rng.standard_normal(d)
    return S, q, k, v


def test_deltanet_alpha1_beta0_leaves_state():
    S, q, k, v = _dn_inputs(8)
    S32 = S.astype(np.float32)
    S_new, o = oracle.deltanet_update(S32, q, k, v, 1.0, 0.0)
    np.testing.assert_array_equal(S_new.astype(np.float32), S32)
    np.testing.assert_allclose(o, S32.astype(np.float64) @ q, rtol=1e-14)


def test_deltanet_beta0_decays():
    S, q, k, v = _dn_inputs(9)
    S_new, _ = oracle.deltanet_update(S, q, k, v, 0.7, 0.0)
    np.testing.assert_allclose(S_new, 0.7 * S, rtol=1e-14)


def test_deltanet_key_direction_identities():
    S, q, k, v = _dn_inputs(10)
    alpha, beta = 0.83, 0.37
    S_new, o = oracle.deltanet_update(S, q, k, v, alpha, beta)
    # along the key: S'k = alpha (1 - beta) S k + beta v   (|k| = 1 up to the 1e-6 eps)
    kk = k @ k
    np.testing.assert_allclose(S_new @ k, alpha * (1 - beta * kk) * (S @ k) + beta * kk * v, rtol=1e-12)
    # orthogonal to the key: S'u = alpha S u
    u = np.random.default_rng(11).standard_normal(k.size)
    u -= (u @ k) / kk * k
    np.testing.assert_allclose(S_new @ u, alpha * (S @ u), rtol=1e-10, atol=1e-14)
    # alpha = beta = 1 writes v along k exactly
    S1, _ = oracle.deltanet_update(S, q, k, v, 1.0, 1.0)
    np.testing.assert_allclose(S1 @ k, (1 - kk) * (S @ k) + kk * v, rtol=1e-12)
    # output reads the updated state
    np.testing.assert_allclose(o, S_new @ q, rtol=1e-15)
    # rectangular state: rows index v, columns index k
    rng = np.random.default_rng(12)
    Sr = rng.standard_normal((3, 5))
    kr = oracle.l2normalize(rng.standard_normal(5))
    vr = rng.standard_normal(3)
    Sn, _ = oracle.deltanet_update(Sr, kr, kr, vr, 1.0, 1.0)
    np.testing.assert_allclose(Sn @ kr, (1 - kr @ kr) * (Sr @ kr) + (kr @ kr) * vr, rtol=1e-12)


# --------------------------------------------------------------- slice wiring

TINY_HYBRID = synth.ModelShape(
    name="tiny_hybrid", hidden=64, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=32, dn_dv=32, q_heads=4, kv_heads=2, head_dim=32, rope_dims=16,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=96, vocab=0)


def _tiny_slice(begin=0, end=4, io_fp32=True, seed=0):
    sh = TINY_HYBRID
    T = {l: synth.layer_tensors(sh, synth.Q4_0, seed, 90, l) for l in range(sh.n_layers)}
    orc = oracle.SliceOracle(sh, synth.Q4_0, begin, end, T, max_seq=64, io_fp32=io_fp32)
    for l in range(begin, end):
        if sh.is_attention(l):
            K, V = synth.kv_prefill(seed, 90, l, sh.kv_heads, 8, sh.head_dim)
            orc.set_kv(l, K, V)
        else:
            orc.set_state(l, synth.dn_state0(seed, 90, l, sh.dn_heads, sh.dn_dv, sh.dn_dk))
    orc.reset(8)
    return orc, T


def test_zero_weights_leave_residual_and_decay_state():
    sh = TINY_HYBRID
    orc, T = _tiny_slice(0, 1)
    for name, raw in T[0].items():
        if name.startswith("dn_") or name.startswith("w_"):
            blk = raw.reshape(raw.shape[0], -1, 18)
            blk[:, :, 0:2] = 0          # scale 0 -> every weight 0
    S0 = orc.dn[0].copy()
    h = synth.hidden_inputs(0, 90, 1, sh.hidden)[0].astype(np.float32)
    out = orc.decode(h, raw=True)
    np.testing.assert_array_equal(out, h.astype(np.float64))
    # k = 0 -> S' = alpha S with alpha = sigmoid(bias_a) = sigmoid(2)
    np.testing.assert_allclose(orc.dn[0], (oracle.sigmoid(2.0) * S0.astype(np.float64)).astype(np.float32),
                               rtol=1e-6)


def test_verify_commit_equals_plain_steps():
    sh = TINY_HYBRID
    H = synth.hidden_inputs(1, 90, 4, sh.hidden).astype(np.float32)
    a, _ = _tiny_slice()
    plain = [a.decode(H[t], raw=True) for t in range(4)]
    for j in range(5):
        b, _ = _tiny_slice()
        out = b.verify(H, raw=True)
        np.testing.assert_array_equal(out, np.stack(plain))
        b.commit(j)
        assert b.pos == 8 + j
        c, _ = _tiny_slice()
        for t in range(j):
            c.decode(H[t])
        for l in c.dn:
            np.testing.assert_array_equal(b.dn[l], c.dn[l])
        # continuing after commit equals a run that never saw the rejected inputs
        np.testing.assert_array_equal(b.decode(H[0], raw=True), c.decode(H[0], raw=True))


def test_slice_composition_fp32_boundary():
    sh = TINY_HYBRID
    H = synth.hidden_inputs(2, 90, 1, sh.hidden)[0]
    whole, _ = _tiny_slice(0, 4)
    first, _ = _tiny_slice(0, 2)
    second, _ = _tiny_slice(2, 4)
    np.testing.assert_array_equal(whole.decode(H, raw=True), second.decode(first.decode(H, raw=True), raw=True))


def _zero_scale(raw, bb=18):
    blk = raw.reshape(raw.shape[0], -1, bb)
    blk[:, :, 0:2] = 0


def test_attention_layer_closed_form():
    # Layer 3 is attention.  With W_k, W_v, W_g and the FFN zeroed, and all prior
    # keys zero, every score is 0 and softmax is uniform over the L prior rows
    # plus the new row (whose value is 0).  Prior values of KV head g are the
    # constant row c_g, so head h sees (L/(L+1)) c_{h // group}; the gate is
    # sigmoid(0) = 1/2; the residual adds W_o u.  A wrong head mapping (h % group),
    # a missing new row, a missing gate or a missing residual fails this.
    sh = TINY_HYBRID
    orc, T = _tiny_slice(3, 4)
    W = T[3]
    for name in ("wk", "wv", "wg", "w_gate", "w_up", "w_down"):
        _zero_scale(W[name])
    L = 8
    c = np.stack([np.linspace(-1, 1, 32), np.linspace(2, -3, 32)]).astype(np.float16)
    K = np.zeros((2, L, 32), np.float16)
    V = np.repeat(c[:, None, :], L, axis=1)
    orc.set_kv(3, K, V)
    orc.reset(L)
    h = synth.hidden_inputs(3, 90, 1, sh.hidden)[0].astype(np.float32)
    out = orc.decode(h, raw=True)
    grp = sh.q_heads // sh.kv_heads
    u = np.concatenate([0.5 * L / (L + 1) * c[i // grp].astype(np.float64) for i in range(sh.q_heads)])
    Wo = qref.dequant(synth.Q4_0, W["wo"], sh.hidden, sh.q_heads * sh.head_dim)
    np.testing.assert_allclose(out, h.astype(np.float64) + Wo @ u, rtol=1e-12, atol=1e-12)
    # the new row was written to the cache, rounded to fp16 (k = 0 after QK-norm)
    assert np.all(orc.kv[3][0][:, L] == 0) and np.all(orc.kv[3][1][:, L] == 0)


def test_centered_q4_codes_have_zero_mean_weights():
    """The centred Q4_0 draw: nibbles 1..15 only, so weights (q - 8) d are
    symmetric about 0; the default draw keeps nibble 0 (mean -0.5)."""
    import synth
    raw = synth.quant_blocks(synth.stream(0, 1, 2, 3), synth.Q4_0, 64, 256, centered=True).reshape(64, 8, 18)
    nib = np.concatenate([raw[:, :, 2:] & 15, raw[:, :, 2:] >> 4]).ravel()
    assert nib.min() == 1 and nib.max() == 15
    assert abs(nib.astype(np.float64).mean() - 8.0) < 0.05
    plain = synth.quant_blocks(synth.stream(0, 1, 2, 3), synth.Q4_0, 64, 256).reshape(64, 8, 18)
    assert (np.concatenate([plain[:, :, 2:] & 15, plain[:, :, 2:] >> 4]) == 0).any()
