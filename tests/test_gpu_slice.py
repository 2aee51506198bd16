"""GPU parity of whole slices (decode, verify, commit) against the CPU oracle.

Every call goes through the C ABI.  Hidden states: max relative error <= 2e-3
against the fp64 oracle.  Rollback, speculative-vs-plain and slice composition
are checked bit for bit on the GPU itself.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import make_pair, inputs, rel_err, TOL

import layer_sliced_quantized_amd as slq

pytestmark = pytest.mark.gpu

# Small hybrid: every kernel of the 5120-wide model at toy width; the KV prefix
# spans several 64-row attention chunks and ends inside one.
TINY_H = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)
WL = 90


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _tiny(begin=0, end=4, **kw):
    kw.setdefault("prefill", 300)
    kw.setdefault("max_seq", 512)
    return make_pair(TINY_H, synth.Q4_0, begin, end, workload=WL, **kw)


def test_tiny_hybrid_decode_states_and_cache():
    s, orc, _, _ = _tiny()
    H = inputs(TINY_H, 3, workload=WL)
    for t in range(3):
        out = s.decode(_t(H[t])).cpu().numpy()
        ref = orc.decode(H[t], raw=True)
        assert rel_err(out, ref) <= TOL, t
    assert s.position == orc.pos == 303
    for l in (0, 1, 2):
        assert rel_err(s.get_state(l).cpu().numpy(), orc.dn[l]) <= TOL
    K, V = s.get_kv(3, 303)
    Ko, Vo = orc.kv[3]
    np.testing.assert_array_equal(K.cpu().numpy()[:, :300], Ko[:, :300])
    assert rel_err(K.cpu().numpy()[:, 300:303], Ko[:, 300:303]) <= TOL
    assert rel_err(V.cpu().numpy()[:, 300:303], Vo[:, 300:303]) <= TOL


@pytest.mark.parametrize("mfma_min", ["2", "17"])
@pytest.mark.parametrize("accepted", [0, 1, 2, 3, 4])
def test_tiny_hybrid_verify_commit(accepted, mfma_min, ovr):
    """Verify 4 drafts through the int8-MFMA products (2) or the per-token
    integer dot products (17), commit, continue."""
    ovr(MFMA_MIN_T=mfma_min)
    H = inputs(TINY_H, 5, workload=WL, step0=10)
    s, orc, _, _ = _tiny()
    out = s.verify(_t(H[:4])).cpu().numpy()
    ref = orc.verify(H[:4], raw=True)
    for t in range(4):
        assert rel_err(out[t], ref[t]) <= TOL, t
    s.commit(accepted)
    orc.commit(accepted)
    assert s.position == orc.pos == 300 + accepted
    # the same inputs through plain decode steps give the same bits
    p, _, _, _ = _tiny(with_oracle=False)
    plain = [p.decode(_t(H[t])).cpu().numpy() for t in range(accepted)]
    for t in range(accepted):
        np.testing.assert_array_equal(plain[t], out[t])
    for l in (0, 1, 2):
        np.testing.assert_array_equal(s.get_state(l).cpu().numpy(), p.get_state(l).cpu().numpy())
        assert rel_err(s.get_state(l).cpu().numpy(), orc.dn[l]) <= TOL
    # continuing after the commit: as if the rejected inputs never came
    nxt = s.decode(_t(H[4])).cpu().numpy()
    np.testing.assert_array_equal(nxt, p.decode(_t(H[4])).cpu().numpy())
    assert rel_err(nxt, orc.decode(H[4], raw=True)) <= TOL


@pytest.mark.parametrize("k", [2, 3, 16])
def test_tiny_hybrid_q8_verify_equals_plain(k):
    """Q8_0 weights: a verify pass of k tokens (int8 MFMA products) gives the
    bits of k plain decode steps, and stays within tolerance of the oracle."""
    H = inputs(TINY_H, k, workload=WL, step0=40)
    s, orc, _, _ = make_pair(TINY_H, synth.Q8_0, 0, 4, workload=WL, prefill=300, max_seq=512, max_verify=16)
    out = s.verify(_t(H)).cpu().numpy()
    ref = orc.verify(H, raw=True)
    for t in range(k):
        assert rel_err(out[t], ref[t]) <= TOL, t
    p, _, _, _ = make_pair(TINY_H, synth.Q8_0, 0, 4, workload=WL, prefill=300, max_seq=512, max_verify=16,
                           with_oracle=False)
    for t in range(k):
        np.testing.assert_array_equal(p.decode(_t(H[t])).cpu().numpy(), out[t])
    s.commit(k)
    for l in (0, 1, 2):
        np.testing.assert_array_equal(s.get_state(l).cpu().numpy(), p.get_state(l).cpu().numpy())


@pytest.mark.parametrize("prefill", [31, 250, 255])
def test_tiny_hybrid_verify_across_chunk_boundary(prefill):
    """A 16-token pass whose positions cross a 32-row attention chunk boundary
    (its K/V rows land in two chunks, and each chunk sees a different first
    token): the bits of 16 plain decode steps, within tolerance of the oracle,
    and the same K/V rows after commit."""
    k = 16
    H = inputs(TINY_H, k, workload=WL, step0=60)
    s, orc, _, _ = make_pair(TINY_H, synth.Q4_0, 0, 4, workload=WL, prefill=prefill, max_seq=512, max_verify=16)
    out = s.verify(_t(H)).cpu().numpy()
    ref = orc.verify(H, raw=True)
    for t in range(k):
        assert rel_err(out[t], ref[t]) <= TOL, t
    p, _, _, _ = make_pair(TINY_H, synth.Q4_0, 0, 4, workload=WL, prefill=prefill, max_seq=512, max_verify=16,
                           with_oracle=False)
    for t in range(k):
        np.testing.assert_array_equal(p.decode(_t(H[t])).cpu().numpy(), out[t])
    s.commit(k)
    K1, V1 = s.get_kv(3, prefill + k)
    K2, V2 = p.get_kv(3, prefill + k)
    np.testing.assert_array_equal(K1.cpu().numpy(), K2.cpu().numpy())
    np.testing.assert_array_equal(V1.cpu().numpy(), V2.cpu().numpy())


def test_commit_zero_restores_state_exactly():
    s, _, _, _ = _tiny(with_oracle=False)
    before = [s.get_state(l).cpu().numpy() for l in (0, 1, 2)]
    s.verify(_t(inputs(TINY_H, 3, workload=WL)))
    s.commit(0)
    for l, b in zip((0, 1, 2), before):
        np.testing.assert_array_equal(s.get_state(l).cpu().numpy(), b)
    assert s.position == 300


def test_slice_composition_fp32_boundary_bitwise():
    H = inputs(TINY_H, 2, workload=WL, step0=20)
    whole, _, _, _ = _tiny(0, 4, with_oracle=False)
    a, _, _, _ = _tiny(0, 2, with_oracle=False)
    b, _, _, _ = _tiny(2, 4, with_oracle=False)
    for t in range(2):
        w = whole.decode(_t(H[t])).cpu().numpy()
        ab = b.decode(a.decode(_t(H[t]))).cpu().numpy()
        np.testing.assert_array_equal(w, ab)


def test_repeat_runs_bitwise_equal():
    H = inputs(TINY_H, 2, workload=WL, step0=30)
    outs = []
    for _ in range(2):
        s, _, _, _ = _tiny(with_oracle=False)
        outs.append([s.decode(_t(H[t])).cpu().numpy() for t in range(2)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_error_states():
    s, _, _, _ = _tiny(with_oracle=False, max_seq=320, max_verify=4)
    h = _t(inputs(TINY_H, 4, workload=WL))
    with pytest.raises(slq.SliceError) as e:
        s.commit(0)
    assert e.value.code == -4
    with pytest.raises(slq.SliceError) as e:
        s.verify(torch.zeros((5, 128), device="cuda"))
    assert e.value.code == -3
    s.verify(h[:2])
    with pytest.raises(slq.SliceError) as e:
        s.decode(h[0])
    assert e.value.code == -4
    with pytest.raises(slq.SliceError) as e:
        s.commit(3)
    assert e.value.code == -3
    s.commit(2)
    s.reset(319)
    s.decode(h[0])
    with pytest.raises(slq.SliceError) as e:
        s.decode(h[1])
    assert e.value.code == -3


def test_fp16_boundary():
    s, orc, _, _ = _tiny(io_fp32=False)
    H = inputs(TINY_H, 2, workload=WL, io_fp32=False)
    for t in range(2):
        out = s.decode(_t(H[t])).cpu().numpy()
        assert out.dtype == np.float16
        ref = orc.decode(H[t])
        assert rel_err(out, ref) <= TOL


# ------------------------------------------------------------ tiny Llama step

def test_tiny_llama_token():
    """Embedding row of the seeded token, 30 Llama layers over a 128-row KV
    prefix, final norm, tied head, greedy argmax."""
    sh = synth.TINY_LLAMA
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 30, workload=synth.WL_TINY_LLAMA, prefill=128, max_seq=256,
                             has_embed=True, has_head=True)
    tok = synth.tiny_llama_token(0)
    h0 = s.embed(torch.tensor([tok], dtype=torch.int32, device="cuda"))
    h0_ref = orc.embed(tok)
    np.testing.assert_array_equal(h0.cpu().numpy().astype(np.float64), h0_ref)   # exact dequant
    h1 = s.decode(h0)
    h1_ref = orc.decode(h0_ref, raw=True)
    assert rel_err(h1.cpu().numpy(), h1_ref) <= TOL
    logits = torch.empty(sh.vocab, dtype=torch.float32, device="cuda")
    t_gpu = int(s.head_argmax(h1, logits=logits).item())
    lg = logits.cpu().numpy()
    # the whole chain against the oracle's own chain
    assert rel_err(lg, orc.head_logits(h1_ref)) <= TOL
    # the head alone: fp64 logits from the GPU's own hidden state, so that only
    # the head product differs; the token must then be exact whenever the
    # top-two margin exceeds the observed logit error (here by a wide margin)
    lg_own = orc.head_logits(h1.cpu().numpy().astype(np.float64))
    assert rel_err(lg, lg_own) <= 1e-5
    err = float(np.max(np.abs(lg - lg_own)))
    top = np.sort(lg_own)[::-1]
    assert top[0] - top[1] > 4 * err, (top[0] - top[1], err)
    assert t_gpu == orc.argmax(lg_own)


# ---------------------------------------------- full-width layers (5120 hidden)

DN_LAYER = dataclasses.replace(synth.HYBRID_5120, name="deltanet_layer_5120", ffn=0)


@pytest.mark.timeout(300)
def test_deltanet_layer_5120_token_then_16_chunk():
    s, orc, _, _ = make_pair(DN_LAYER, synth.Q4_0, 0, 1, workload=synth.WL_DELTANET, max_seq=64)
    H = inputs(DN_LAYER, 17, workload=synth.WL_DELTANET)
    out0 = s.decode(_t(H[0])).cpu().numpy()
    assert rel_err(out0, orc.decode(H[0], raw=True)) <= TOL
    S1 = s.get_state(0).cpu().numpy()
    assert rel_err(S1, orc.dn[0]) <= TOL
    out = s.verify(_t(H[1:])).cpu().numpy()
    ref = orc.verify(H[1:], raw=True)
    for t in range(16):
        assert rel_err(out[t], ref[t]) <= TOL, t
    s.commit(16)
    orc.commit(16)
    assert rel_err(s.get_state(0).cpu().numpy(), orc.dn[0]) <= TOL


ATT_LAYER = dataclasses.replace(synth.HYBRID_5120, name="attention_layer_5120", ffn=0)


@pytest.mark.parametrize("L", [512, 4096, 32768])
@pytest.mark.timeout(300)
def test_attention_layer_5120_decode_and_verify(L):
    s, orc, _, _ = make_pair(ATT_LAYER, synth.Q4_0, 3, 4, workload=synth.WL_ATTENTION, prefill=L,
                             max_seq=L + 64)
    H = inputs(ATT_LAYER, 17, workload=synth.WL_ATTENTION, step0=L)
    out0 = s.decode(_t(H[0])).cpu().numpy()
    assert rel_err(out0, orc.decode(H[0], raw=True)) <= TOL
    out = s.verify(_t(H[1:])).cpu().numpy()
    ref = orc.verify(H[1:], raw=True)
    for t in range(16):
        assert rel_err(out[t], ref[t]) <= TOL, t
    s.commit(16)
    orc.commit(16)
    K, V = s.get_kv(3, L + 17)
    assert rel_err(K.cpu().numpy()[:, L:], orc.kv[3][0][:, L:L + 17]) <= TOL
    assert rel_err(V.cpu().numpy()[:, L:], orc.kv[3][1][:, L:L + 17]) <= TOL


@pytest.mark.timeout(300)
def test_attention_short_context_in_long_cache():
    """A cache of more than 64 chunks launches the eight-wave combine; at 512
    rows the merge still takes the one-wave branch while the other waves wait
    at the barrier and leave."""
    s, orc, _, _ = make_pair(ATT_LAYER, synth.Q4_0, 3, 4, workload=synth.WL_ATTENTION, prefill=512,
                             max_seq=4160)
    H = inputs(ATT_LAYER, 17, workload=synth.WL_ATTENTION, step0=512)
    out0 = s.decode(_t(H[0])).cpu().numpy()
    assert rel_err(out0, orc.decode(H[0], raw=True)) <= TOL
    out = s.verify(_t(H[1:])).cpu().numpy()
    ref = orc.verify(H[1:], raw=True)
    for t in range(16):
        assert rel_err(out[t], ref[t]) <= TOL, t


# ------------------------------------------------------ the 64-layer slice

@pytest.mark.timeout(900)
def test_hybrid_64_layer_q4_slice():
    """64-layer Q4_0 hybrid slice: decode two tokens, verify 4 drafts, commit
    the seeded number of accepted drafts, decode once more.  fp16 inputs as a
    middle stage receives them; the outputs are compared on the fp32 residual
    stream, because with these synthetic weights |h| grows past the fp16 range
    within two layers (every fp16 output entry saturates)."""
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q4_0, 0, 64, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=4, io_fp32=False, threads=16)
    H = inputs(sh, 7, workload=synth.WL_SLICE, io_fp32=False)
    for t in range(2):
        s.decode(_t(H[t]))
        assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[t], raw=True)) <= TOL, t
    s.verify(_t(H[2:6]))
    out = s.get_hidden(4).cpu().numpy()
    ref = orc.verify(H[2:6], raw=True)
    for t in range(4):
        assert rel_err(out[t], ref[t]) <= TOL, t
    j = int(synth.accept_pattern(0, 1, 4)[0])
    s.commit(j)
    orc.commit(j)
    s.decode(_t(H[6]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[6], raw=True)) <= TOL


@pytest.mark.timeout(600)
def test_hybrid_q8_slice_8_layers():
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q8_0, 0, 8, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=4, io_fp32=False, threads=16)
    H = inputs(sh, 5, workload=synth.WL_SLICE, io_fp32=False, step0=100)
    s.decode(_t(H[0]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[0], raw=True)) <= TOL
    s.verify(_t(H[1:5]))
    out = s.get_hidden(4).cpu().numpy()
    ref = orc.verify(H[1:5], raw=True)
    for t in range(4):
        assert rel_err(out[t], ref[t]) <= TOL, t


@pytest.mark.timeout(900)
def test_hybrid_64_layer_q8_slice():
    """The Q8_0 slice the benchmark times: all 64 layers (25.3 GB of Q8_0
    weights), decode, a 4-token verify, a commit and one more decode, on the
    fp32 residual stream against the oracle."""
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q8_0, 0, 64, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=4, io_fp32=False, threads=16)
    H = inputs(sh, 6, workload=synth.WL_SLICE, io_fp32=False, step0=300)
    s.decode(_t(H[0]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[0], raw=True)) <= TOL
    s.verify(_t(H[1:5]))
    out = s.get_hidden(4).cpu().numpy()
    ref = orc.verify(H[1:5], raw=True)
    for t in range(4):
        assert rel_err(out[t], ref[t]) <= TOL, t
    s.commit(2)
    orc.commit(2)
    s.decode(_t(H[5]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[5], raw=True)) <= TOL


DEEP = synth.ModelShape(
    name="deep_hybrid_128", hidden=128, n_layers=64, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)


def test_deep_slice_in_range_through_the_fp16_boundary():
    """64 layers whose weights have mean 0 (centred Q4_0 codes), so the
    residual stream stays in fp16 range and every layer sees an input that
    is not dominated by one direction: the fp16 outputs of decode steps and a
    verify pass match the oracle, and |h| stays far below the fp16 limit.
    (Random Q8_0 codes span +-127 and make rows ~10x larger, so the stream
    leaves fp16 range whatever their mean; Q8_0 is covered elsewhere.)"""
    s, orc, _, _ = make_pair(DEEP, synth.Q4_0, 0, 64, workload=120, prefill=24, max_seq=128, max_verify=4,
                             io_fp32=False, centered=True)
    H = inputs(DEEP, 8, workload=120, io_fp32=False)
    for t in range(4):
        got = s.decode(torch.from_numpy(H[t]).cuda()).cpu().numpy().astype(np.float64)
        want = orc.decode(H[t], raw=True)
        assert np.max(np.abs(want)) < 1e3
        assert rel_err(got, want) <= TOL, t
    got = s.verify(torch.from_numpy(H[4:8]).cuda()).cpu().numpy().astype(np.float64)
    want = orc.verify(H[4:8], raw=True)
    for t in range(4):
        assert rel_err(got[t], want[t]) <= TOL, t
    s.sync_check()
