"""The mixers on caller buffers, through the C ABI: slq_dn_step (Gated
DeltaNet, T tokens) and slq_attn_decode (gated GQA over an fp16 cache),
against the oracle's per-token mixers on the same seeded inputs."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import TOL, rel_err
from oracle import model as omodel

pytestmark = pytest.mark.gpu

MIX_TOL = 1e-4    # DeltaNet: fp32 kernel against fp64, max relative error (RMS floor)
# Attention writes each new key to the fp16 cache: the kernel rounds an fp32
# value, the oracle an fp64 one, and near a tie the two round one unit apart
# (2^-11 relative).  Such a key moves its score by up to |q_i| 2^-11 |k_i| /
# sqrt(head_dim) and, over few rows, the output by a few 1e-4; the bound is the
# slice tolerance for fp16-cached attention.
ATTN_TOL = TOL


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _dn_oracle(S0, rows, dk, dv):
    S = S0.copy()
    outs = np.stack([omodel.deltanet_token(S, r, dk, dv) for r in rows])
    return outs, S


@pytest.mark.parametrize("heads,dk,dv,T", [(32, 128, 128, 1), (32, 128, 128, 16), (2, 64, 64, 5),
                                           (3, 32, 96, 7), (4, 96, 32, 16), (1, 128, 256, 3)])
def test_dn_step_against_oracle(heads, dk, dv, T):
    import layer_sliced_quantized_amd as slq
    rows = synth.dn_kernel_inputs(0, T, heads, dk, dv, step0=heads + dk + dv)
    S0 = synth.dn_state0(0, synth.WL_DELTANET, 7, heads, dv, dk) * 20
    St = slq.dn_state_to_lib(_t(S0))
    out = slq.dn_step(heads, dk, dv, _t(rows), St).cpu().numpy()
    S = slq.dn_state_from_lib(St, heads, dk, dv).cpu().numpy()
    want, S_want = _dn_oracle(S0, rows, dk, dv)
    for t in range(T):
        assert rel_err(out[t], want[t]) <= MIX_TOL, t
    assert rel_err(S, S_want) <= MIX_TOL


def test_dn_tokens_in_one_call_equal_one_at_a_time():
    """Sixteen tokens in one call and the same tokens one call each: the same
    bits for every output and for the final state."""
    import layer_sliced_quantized_amd as slq
    heads, dk, dv = 32, 128, 128
    rows = _t(synth.dn_kernel_inputs(1, 16, heads, dk, dv))
    S0 = _t(synth.dn_state0(1, synth.WL_DELTANET, 0, heads, dv, dk))
    Sa, Sb = slq.dn_state_to_lib(S0), slq.dn_state_to_lib(S0)
    out_a = slq.dn_step(heads, dk, dv, rows, Sa)
    out_b = torch.cat([slq.dn_step(heads, dk, dv, rows[t:t + 1].contiguous(), Sb) for t in range(16)])
    assert torch.equal(out_a, out_b)
    assert torch.equal(Sa, Sb)


def test_dn_state_layout_round_trip():
    import layer_sliced_quantized_amd as slq
    S0 = _t(synth.dn_state0(2, synth.WL_DELTANET, 0, 5, 64, 96))
    lib_form = slq.dn_state_to_lib(S0)
    assert torch.equal(slq.dn_state_from_lib(lib_form, 5, 96, 64), S0)


def test_dn_identity_step_leaves_state_bits():
    """a = +inf, b = -inf: alpha = 1 and beta = 0, so S' = S exactly and the
    output is S q^ gated; the state keeps its bits over several tokens."""
    import layer_sliced_quantized_amd as slq
    heads, dk, dv, T = 32, 128, 128, 4
    rows = synth.dn_kernel_inputs(3, T, heads, dk, dv)
    o_a = 2 * heads * dk + heads * dv
    rows[:, o_a:o_a + heads] = np.inf
    rows[:, o_a + heads:o_a + 2 * heads] = -np.inf
    S0 = synth.dn_state0(3, synth.WL_DELTANET, 0, heads, dv, dk) * 20
    St = slq.dn_state_to_lib(_t(S0))
    out = slq.dn_step(heads, dk, dv, _t(rows), St).cpu().numpy()
    np.testing.assert_array_equal(slq.dn_state_from_lib(St, heads, dk, dv).cpu().numpy(), S0)
    want, S_want = _dn_oracle(S0, rows, dk, dv)
    np.testing.assert_array_equal(S_want, S0)
    assert rel_err(out, want) <= MIX_TOL


# ------------------------------------------------------------------ attention

GEOM = synth.HYBRID_5120          # 24 query heads, 4 KV heads of 256, RoPE on 64, QK-norm, gate


def _decoder(shape, max_seq, t_max=16, seed=0):
    import layer_sliced_quantized_amd as slq
    rng = synth.stream(seed, synth.WL_ATTENTION, 99, synth.TENSOR_IDS["q_norm"])
    qn = (1.0 + 0.25 * rng.standard_normal(shape.head_dim)).astype(np.float32) if shape.qk_norm else None
    kn = (1.0 + 0.25 * rng.standard_normal(shape.head_dim)).astype(np.float32) if shape.qk_norm else None
    dec = slq.AttnDecoder(shape.q_heads, shape.kv_heads, shape.head_dim, shape.rope_dims, shape.rope_theta,
                          shape.qk_norm, shape.attn_gate, shape.eps, max_seq, qn, kn, t_max=t_max)
    return dec, qn, kn


def _attn_oracle(shape, rows, K, V, pos, qn, kn):
    hd, nq, nkv = shape.head_dim, shape.q_heads, shape.kv_heads
    outs = []
    for t, r in enumerate(rows):
        r = r.astype(np.float64)
        o = 0
        q = r[o:o + nq * hd]; o += nq * hd
        g = None
        if shape.attn_gate:
            g = r[o:o + nq * hd]; o += nq * hd
        k = r[o:o + nkv * hd]; o += nkv * hd
        v = r[o:o + nkv * hd]
        outs.append(omodel.attention_heads(shape, q, g, k, v, K, V, pos + t, qn, kn))
    return np.stack(outs)


def _attn_case(shape, L, T, seed, max_seq=None, check_rows=True):
    max_seq = max_seq or ((L + T + 63) // 64) * 64
    dec, qn, kn = _decoder(shape, max_seq, seed=seed)
    K = np.zeros((shape.kv_heads, max_seq, shape.head_dim), np.float16)
    V = np.zeros_like(K)
    if L:
        K[:, :L], V[:, :L] = synth.kv_prefill(seed, synth.WL_ATTENTION, 0, shape.kv_heads, L, shape.head_dim)
        dec.set_kv(torch.from_numpy(K[:, :L]), torch.from_numpy(V[:, :L]))
    rows = synth.attn_kernel_inputs(seed, T, shape.q_heads, shape.kv_heads, shape.head_dim, shape.attn_gate,
                                    step0=L)
    out = dec.decode(_t(rows), L).cpu().numpy()
    want = _attn_oracle(shape, rows, K, V, L, qn, kn)
    for t in range(T):
        assert rel_err(out[t], want[t]) <= ATTN_TOL, (L, t)
    if check_rows:
        Kg, Vg = dec.get_kv(L + T)
        np.testing.assert_array_equal(Vg.cpu().numpy(), V[:, :L + T])
        # new keys: the same fp16 value or one unit in the last place apart
        kd = np.abs(Kg.cpu().numpy()[:, L:].astype(np.float64) - K[:, L:L + T].astype(np.float64))
        ulp = np.spacing(np.abs(K[:, L:L + T]).astype(np.float16)).astype(np.float64)
        assert np.all(kd <= ulp)
        np.testing.assert_array_equal(Kg.cpu().numpy()[:, :L], K[:, :L])
    return dec, out


@pytest.mark.parametrize("L", [512, 4096])
@pytest.mark.parametrize("T", [1, 16])
def test_attn_decode_against_oracle(L, T):
    _attn_case(GEOM, L, T, seed=L + T)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 16])
def test_attn_decode_long_context(T):
    _attn_case(GEOM, 32768, T, seed=5 + T)


@pytest.mark.parametrize("shape", [
    dataclasses.replace(GEOM, qk_norm=False, attn_gate=False, rope_dims=256, rope_theta=1e4),
    dataclasses.replace(synth.TINY_LLAMA),
    dataclasses.replace(GEOM, q_heads=8, kv_heads=8, head_dim=128, rope_dims=128),
    dataclasses.replace(GEOM, q_heads=16, kv_heads=2, head_dim=64, rope_dims=32),
], ids=["plain_gqa_256", "tiny_llama", "mha_128", "gqa_64"])
@pytest.mark.parametrize("L", [0, 63, 200])
def test_attn_decode_geometries(shape, L):
    _attn_case(shape, L, 3, seed=L + shape.head_dim)


def test_attn_first_position_returns_v():
    """At position 0 the only cached row is the token's own: the softmax
    weight is exactly 1 and the output is v rounded to fp16, every bit."""
    shape = dataclasses.replace(GEOM, attn_gate=False)
    dec, _, _ = _decoder(shape, 64)
    rows = synth.attn_kernel_inputs(11, 1, shape.q_heads, shape.kv_heads, shape.head_dim, False)
    out = dec.decode(_t(rows), 0).cpu().numpy()[0].reshape(shape.q_heads, shape.head_dim)
    v = rows[0, (shape.q_heads + shape.kv_heads) * shape.head_dim:].reshape(shape.kv_heads, shape.head_dim)
    grp = shape.q_heads // shape.kv_heads
    for i in range(shape.q_heads):
        np.testing.assert_array_equal(out[i], v[i // grp].astype(np.float16).astype(np.float32))


@pytest.mark.parametrize("L", [1000, 5000, 9000])
def test_attn_tokens_in_one_call_equal_one_at_a_time(L):
    """Sixteen tokens in one call (a verify pass) and one call per token (decode)
    give the same bits, and leave the same cache rows.  From 5000 cached rows a
    decode call takes all six query heads of a KV head per workgroup (and at
    9000 two chunks per workgroup), the verify pass two heads and one chunk:
    each chunk's partial is the same computation either way."""
    a, out_a = _attn_case(GEOM, L, 16, seed=21, check_rows=False)
    b, _, _ = _decoder(GEOM, a.desc.max_seq, seed=21)
    K, V = synth.kv_prefill(21, synth.WL_ATTENTION, 0, GEOM.kv_heads, L, GEOM.head_dim)
    b.set_kv(torch.from_numpy(K), torch.from_numpy(V))
    rows = synth.attn_kernel_inputs(21, 16, GEOM.q_heads, GEOM.kv_heads, GEOM.head_dim, True, step0=L)
    out_b = np.stack([b.decode(_t(rows[t:t + 1]), L + t).cpu().numpy()[0] for t in range(16)])
    np.testing.assert_array_equal(out_a, out_b)
    for x, y in zip(a.get_kv(L + 16), b.get_kv(L + 16)):
        assert torch.equal(x, y)


def test_attn_last_positions():
    """Tokens that fill the cache to its last row."""
    L, T = 4096 - 16, 16
    _attn_case(GEOM, L, T, seed=31, max_seq=4096)


def test_kv_layout_round_trip():
    dec, _, _ = _decoder(GEOM, 320)
    K, V = synth.kv_prefill(41, synth.WL_ATTENTION, 0, GEOM.kv_heads, 300, GEOM.head_dim)
    dec.set_kv(torch.from_numpy(K), torch.from_numpy(V))
    Kg, Vg = dec.get_kv(300)
    np.testing.assert_array_equal(Kg.cpu().numpy(), K)
    np.testing.assert_array_equal(Vg.cpu().numpy(), V)
