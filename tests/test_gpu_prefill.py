"""GPU parity of prompt ingestion (slice_prefill): k tokens in one pass, the
DeltaNet layers in the chunked form, against k plain steps of the CPU oracle.

Hidden states, DeltaNet states and the new KV rows: max relative error <= 2e-3
against the fp64 oracle; the position moves by k and decoding carries on from
the prefilled state."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import make_pair, inputs, rel_err, TOL

import layer_sliced_quantized_amd as slq

pytestmark = pytest.mark.gpu

TINY_H = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)
WL = 93


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check_prefill(shape, qtype, k, prefill, *, workload=WL, max_seq=512, layers=4, max_prefill=0):
    s, orc, _, _ = make_pair(shape, qtype, 0, layers, workload=workload, prefill=prefill, max_seq=max_seq,
                             max_prefill=max_prefill)
    H = inputs(shape, k + 1, workload=workload)
    out = s.prefill(_t(H[:k])).cpu().numpy()
    for t in range(k):
        ref = orc.decode(H[t], raw=True)
        assert np.isfinite(out[t]).all(), t
        assert rel_err(out[t], ref) <= TOL, t
    assert s.position == orc.pos == prefill + k
    for l in range(layers):
        if shape.is_attention(l):
            K, V = s.get_kv(l, prefill + k)
            Ko, Vo = orc.kv[l]
            np.testing.assert_array_equal(K.cpu().numpy()[:, :prefill], Ko[:, :prefill])
            assert rel_err(K.cpu().numpy()[:, prefill:prefill + k], Ko[:, prefill:prefill + k]) <= TOL
            assert rel_err(V.cpu().numpy()[:, prefill:prefill + k], Vo[:, prefill:prefill + k]) <= TOL
        else:
            assert rel_err(s.get_state(l).cpu().numpy(), orc.dn[l]) <= TOL, l
    # decoding carries on from the prefilled state and position
    nxt = s.decode(_t(H[k])).cpu().numpy()
    assert rel_err(nxt, orc.decode(H[k], raw=True)) <= TOL


@pytest.mark.parametrize("k", [1, 2, 5, 9, 16])
def test_tiny_hybrid_prefill(k):
    _check_prefill(TINY_H, synth.Q4_0, k, 300)


@pytest.mark.parametrize("prefill", [0, 250])
def test_tiny_hybrid_prefill_16_from_empty_and_across_chunk(prefill):
    _check_prefill(TINY_H, synth.Q4_0, 16, prefill)


def test_tiny_hybrid_q8_prefill():
    _check_prefill(TINY_H, synth.Q8_0, 16, 100)


@pytest.mark.parametrize("a_bias", [-40.0, 40.0])
def test_prefill_with_vanishing_and_unit_decay(a_bias):
    # alpha ~ 4e-18: the decay products of a 16-token chunk underflow fp32;
    # alpha = 1 in fp32: no decay at all
    shape = dataclasses.replace(TINY_H, name=f"tiny_hybrid_a{a_bias:+.0f}", dn_a_bias=a_bias)
    _check_prefill(shape, synth.Q4_0, 16, 300, layers=3)


def test_prefill_after_verify_and_errors():
    s, orc, _, _ = make_pair(TINY_H, synth.Q4_0, 0, 4, workload=WL, prefill=300, max_seq=320, max_verify=16)
    H = inputs(TINY_H, 24, workload=WL)
    s.verify(_t(H[:4]))
    with pytest.raises(slq.SliceError):
        s.prefill(_t(H[4:8]))            # a verify is pending
    s.commit(2)
    orc.decode(H[0], raw=True)
    orc.decode(H[1], raw=True)
    with pytest.raises(slq.SliceError):
        s.prefill(_t(np.zeros((17, TINY_H.hidden), np.float32)))   # k > max_verify
    out = s.prefill(_t(H[2:18])).cpu().numpy()
    for t in range(16):
        assert rel_err(out[t], orc.decode(H[2 + t], raw=True)) <= TOL, t
    assert s.position == 318
    with pytest.raises(slq.SliceError):
        s.prefill(_t(H[18:21]))          # positions would pass max_seq
    assert s.position == 318


DN_LAYER = dataclasses.replace(synth.HYBRID_5120, name="deltanet_layer_5120", ffn=0)


@pytest.mark.timeout(300)
def test_deltanet_layer_5120_prefill_16():
    s, orc, _, _ = make_pair(DN_LAYER, synth.Q4_0, 0, 1, workload=synth.WL_DELTANET, max_seq=64)
    H = inputs(DN_LAYER, 17, workload=synth.WL_DELTANET)
    s.decode(_t(H[0]))
    orc.decode(H[0], raw=True)
    out = s.prefill(_t(H[1:])).cpu().numpy()
    for t in range(16):
        assert rel_err(out[t], orc.decode(H[1 + t], raw=True)) <= TOL, t
    assert rel_err(s.get_state(0).cpu().numpy(), orc.dn[0]) <= TOL


@pytest.mark.parametrize("dk,dv", [(32, 64), (96, 32)])
def test_prefill_other_key_widths(dk, dv):
    # d_k = 32 and 96: one and three state entries per lane to finalise
    shape = dataclasses.replace(TINY_H, name=f"tiny_hybrid_dk{dk}", dn_dk=dk, dn_dv=dv)
    _check_prefill(shape, synth.Q4_0, 16, 300, layers=3)
    _check_prefill(shape, synth.Q4_0, 7, 300, layers=3)


def test_tiny_llama_prefill():
    """A slice without DeltaNet layers: the pass is products and attention only."""
    sh = synth.TINY_LLAMA
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 6, workload=synth.WL_TINY_LLAMA, prefill=128, max_seq=256)
    H = inputs(sh, 13, workload=synth.WL_TINY_LLAMA)
    out = s.prefill(_t(H[:12])).cpu().numpy()
    for t in range(12):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    assert s.position == 140
    assert rel_err(s.decode(_t(H[12])).cpu().numpy(), orc.decode(H[12], raw=True)) <= TOL


@pytest.mark.timeout(900)
def test_hybrid_64_layer_q4_prefill_16():
    """The prompt pass the benchmark times: 64-layer Q4_0 hybrid slice, 512
    prior KV rows, 16 fp16 inputs in one slice_prefill; every token's fp32
    residual stream against 16 plain steps of the oracle, then one decode."""
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 64, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=16, io_fp32=False, threads=16)
    H = inputs(sh, 17, workload=synth.WL_SLICE, io_fp32=False, step0=200)
    s.prefill(_t(H[:16]))
    out = s.get_hidden(16).cpu().numpy()
    for t in range(16):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    assert s.position == 528
    s.decode(_t(H[16]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[16], raw=True)) <= TOL


# ---------------------------------------------- passes of more than 16 tokens

@pytest.mark.parametrize("k", [17, 32, 33, 48, 64])
def test_tiny_hybrid_wide_prefill(k):
    """17..64 tokens in one pass: the products take every token at once in
    token groups of 16 (the last group ragged), the mixers run in sub-passes
    of 16; from position 300 the pass crosses the attention's 32-row chunks."""
    _check_prefill(TINY_H, synth.Q4_0, k, 300, max_prefill=64)


def test_tiny_hybrid_wide_prefill_from_empty_q8():
    _check_prefill(TINY_H, synth.Q8_0, 40, 0, max_prefill=48)


def test_wide_prefill_limits():
    s, orc, _, _ = make_pair(TINY_H, synth.Q4_0, 0, 4, workload=WL, prefill=100, max_seq=256, max_verify=4,
                             max_prefill=32)
    H = inputs(TINY_H, 40, workload=WL)
    with pytest.raises(slq.SliceError):
        s.prefill(_t(H[:33]))            # more than max_prefill
    with pytest.raises(slq.SliceError):
        s.verify(_t(H[:5]))              # verify stays within max_verify
    out = s.prefill(_t(H[:32])).cpu().numpy()
    for t in range(32):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    # a 4-token verify and commit after the wide pass
    Y = s.verify(_t(H[32:36])).cpu().numpy()
    ref = orc.verify(H[32:36], raw=True)
    for t in range(4):
        assert rel_err(Y[t], ref[t]) <= TOL, t
    s.commit(3)
    orc.commit(3)
    assert s.position == orc.pos == 135
    assert rel_err(s.decode(_t(H[36])).cpu().numpy(), orc.decode(H[36], raw=True)) <= TOL


def test_tiny_llama_wide_prefill():
    sh = synth.TINY_LLAMA
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 6, workload=synth.WL_TINY_LLAMA, prefill=128, max_seq=256,
                             max_prefill=64)
    H = inputs(sh, 41, workload=synth.WL_TINY_LLAMA)
    out = s.prefill(_t(H[:40])).cpu().numpy()
    for t in range(40):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    assert s.position == 168
    assert rel_err(s.decode(_t(H[40])).cpu().numpy(), orc.decode(H[40], raw=True)) <= TOL


@pytest.mark.timeout(300)
def test_deltanet_layer_5120_prefill_64():
    s, orc, _, _ = make_pair(DN_LAYER, synth.Q4_0, 0, 1, workload=synth.WL_DELTANET, max_seq=128, max_prefill=64)
    H = inputs(DN_LAYER, 65, workload=synth.WL_DELTANET)
    s.decode(_t(H[0]))
    orc.decode(H[0], raw=True)
    out = s.prefill(_t(H[1:])).cpu().numpy()
    for t in range(64):
        assert rel_err(out[t], orc.decode(H[1 + t], raw=True)) <= TOL, t
    assert rel_err(s.get_state(0).cpu().numpy(), orc.dn[0]) <= TOL


ATT_LAYER = dataclasses.replace(synth.HYBRID_5120, name="attention_layer_5120", ffn=0)
FFN_DN_LAYER = dataclasses.replace(synth.HYBRID_5120, name="deltanet_ffn_layer_5120")


@pytest.mark.timeout(300)
def test_attention_layer_5120_prefill_64():
    s, orc, _, _ = make_pair(ATT_LAYER, synth.Q4_0, 3, 4, workload=synth.WL_ATTENTION, prefill=512, max_seq=640,
                             max_prefill=64)
    H = inputs(ATT_LAYER, 64, workload=synth.WL_ATTENTION, step0=512)
    out = s.prefill(_t(H)).cpu().numpy()
    for t in range(64):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    K, V = s.get_kv(3, 576)
    assert rel_err(K.cpu().numpy()[:, 512:], orc.kv[3][0][:, 512:576]) <= TOL
    assert rel_err(V.cpu().numpy()[:, 512:], orc.kv[3][1][:, 512:576]) <= TOL


@pytest.mark.timeout(300)
def test_deltanet_and_ffn_layer_5120_prefill_48():
    """A whole hidden-5120 layer (DeltaNet, SwiGLU 17408): every product of the
    pass with three token groups (the fourth past the last token)."""
    s, orc, _, _ = make_pair(FFN_DN_LAYER, synth.Q4_0, 0, 1, workload=synth.WL_DELTANET, max_seq=128,
                             max_prefill=64, centered=True)
    H = inputs(FFN_DN_LAYER, 48, workload=synth.WL_DELTANET)
    out = s.prefill(_t(H)).cpu().numpy()
    for t in range(48):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t


@pytest.mark.timeout(600)
def test_hybrid_8_layer_prefill_64():
    """The benchmark's 64-token pass on the first 8 layers of the hidden-5120
    hybrid (6 DeltaNet, 2 attention, SwiGLU 17408; 512 prior KV rows, fp16
    inputs): every token's fp32 residual stream against 64 plain oracle
    steps, then one decode."""
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 8, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=16, io_fp32=False, threads=16, max_prefill=64)
    H = inputs(sh, 65, workload=synth.WL_SLICE, io_fp32=False, step0=400)
    s.prefill(_t(H[:64]))
    out = s.get_hidden(64).cpu().numpy()
    for t in range(64):
        assert rel_err(out[t], orc.decode(H[t], raw=True)) <= TOL, t
    assert s.position == 576
    s.decode(_t(H[64]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[64], raw=True)) <= TOL

