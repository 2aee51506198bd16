"""The qwen3_5 form of the Gated DeltaNet layers on the GPU, through the C ABI.

A shape flag selects the form the pages' qwen3_5 hybrid names (ChatTorrent
README, "What it can run"): a causal conv over q|k|v then SiLU, with its
state kept beside the recurrent state; value heads sharing query/key heads;
q scaled by 1/sqrt(d_k); the exp/softplus decay; a gated RMSNorm on each
head's output.  Checked against the oracle's deltanet_q35 on the same
seeded inputs (outputs, recurrent and conv states), and bit for bit between
verify + commit and plain decode steps, and between prompt passes and
decode steps.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import TOL, inputs, make_pair, rel_err

pytestmark = pytest.mark.gpu

TINY_Q35 = synth.ModelShape(
    name="tiny_hybrid_q35_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=4, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0,
    dn_variant=1, dn_k_heads=2, dn_conv=4)

STATE_TOL = 1e-4


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check_states(s, orc, shape, layers):
    for l in layers:
        assert rel_err(s.get_state(l).cpu().numpy(), orc.dn[l]) <= STATE_TOL, l
        assert rel_err(s.get_conv_state(l).cpu().numpy(), orc.conv[l]) <= STATE_TOL, l


def _decode_vs_oracle(shape, qtype, layers, steps, workload, **kw):
    s, orc, _, _ = make_pair(shape, qtype, 0, layers, workload=workload, **kw)
    dn_layers = [l for l in range(layers) if not shape.is_attention(l)]
    H = inputs(shape, steps, workload=workload, step0=3)
    for t in range(steps):
        s.decode(_t(H[t]))
        want = orc.decode(H[t], raw=True)
        assert rel_err(s.get_hidden().cpu().numpy()[0], want) <= TOL, t
    _check_states(s, orc, shape, dn_layers)
    s.sync_check()
    return s, orc


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_q35_decode_against_oracle(qtype):
    _decode_vs_oracle(TINY_Q35, qtype, 4, 6, 110, prefill=20, max_seq=128, max_verify=4)


@pytest.mark.parametrize("geom", [
    dict(dn_dk=128, dn_dv=64, dn_heads=4, dn_k_heads=4, dn_conv=3),
    dict(dn_dk=32, dn_dv=32, dn_heads=8, dn_k_heads=2, dn_conv=2),
    dict(dn_dk=96, dn_dv=128, dn_heads=2, dn_k_heads=1, dn_conv=4),
], ids=["dk128_dv64_conv3", "dk32_dv32_conv2", "dk96_dv128_conv4"])
def test_q35_geometries(geom):
    shape = dataclasses.replace(TINY_Q35, name="tiny_q35_geom", **geom)
    _decode_vs_oracle(shape, synth.Q4_0, 3, 5, 111, prefill=8, max_seq=64, max_verify=4)


@pytest.mark.timeout(600)
def test_q35_hybrid_5120_layers():
    """Layers 0..3 of the hidden-5120 hybrid in the qwen3_5 form (3 DeltaNet
    layers of 32 value / 16 key heads, one attention layer)."""
    _decode_vs_oracle(synth.HYBRID_5120_Q35, synth.Q4_0, 4, 3, synth.WL_SLICE, prefill=512, max_seq=576,
                      max_verify=4, io_fp32=True, threads=16)


def test_q35_verify_commit_equals_decode():
    """verify(k) + commit(j) leaves the bits of j plain decode steps: outputs,
    recurrent states and conv states; then both continue identically."""
    kw = dict(workload=112, prefill=10, max_seq=128, max_verify=4, with_oracle=False)
    a, _, _, _ = make_pair(TINY_Q35, synth.Q4_0, 0, 4, **kw)
    b, _, _, _ = make_pair(TINY_Q35, synth.Q4_0, 0, 4, **kw)
    H = inputs(TINY_Q35, 20, workload=112, step0=1)
    i = 0
    for k, j in ((4, 2), (3, 0), (4, 4), (2, 1)):
        ver = a.verify(_t(H[i:i + k])).cpu().numpy()
        a.commit(j)
        dec = [b.decode(_t(H[i + t])).cpu().numpy() for t in range(j)]
        if j:
            np.testing.assert_array_equal(ver[:j], np.stack(dec))
        i += k
        # the rejected inputs never reached b; a rolled them back
    for l in (0, 1, 2):
        assert torch.equal(a.get_state(l), b.get_state(l)), l
        assert torch.equal(a.get_conv_state(l), b.get_conv_state(l)), l
    for t in range(3):
        x = _t(H[16 + t])
        assert torch.equal(a.decode(x), b.decode(x))


def test_q35_prefill_equals_decode():
    """A prompt pass of k tokens (a verify whose tokens are all kept) leaves
    the bits of k decode steps."""
    kw = dict(workload=113, prefill=4, max_seq=128, max_verify=8, with_oracle=False)
    a, _, _, _ = make_pair(TINY_Q35, synth.Q8_0, 0, 4, **kw)
    b, _, _, _ = make_pair(TINY_Q35, synth.Q8_0, 0, 4, **kw)
    H = inputs(TINY_Q35, 16, workload=113)
    outs = a.prefill(_t(H[:8])).cpu().numpy()
    dec = np.stack([b.decode(_t(H[t])).cpu().numpy() for t in range(8)])
    np.testing.assert_array_equal(outs, dec)
    assert a.position == b.position
    for l in (0, 1, 2):
        assert torch.equal(a.get_state(l), b.get_state(l))
        assert torch.equal(a.get_conv_state(l), b.get_conv_state(l))


def test_q35_chain_equals_separate_kernels(ovr):
    kw = dict(workload=114, prefill=12, max_seq=128, max_verify=4, with_oracle=False)
    a, _, _, _ = make_pair(TINY_Q35, synth.Q4_0, 0, 4, **kw)
    ovr(CHAIN=0)
    b, _, _, _ = make_pair(TINY_Q35, synth.Q4_0, 0, 4, **kw)
    H = inputs(TINY_Q35, 5, workload=114)
    for t in range(5):
        x = _t(H[t])
        assert torch.equal(a.decode(x), b.decode(x)), t
    a.sync_check()


def test_q35_conv_state_round_trip():
    s, _, _, _ = make_pair(TINY_Q35, synth.Q4_0, 0, 4, workload=115, prefill=2, max_seq=64, max_verify=2,
                           with_oracle=False)
    C = synth.dn_conv_state0(1, 115, 0, TINY_Q35.conv_dim, TINY_Q35.dn_conv)
    s.set_conv_state(0, torch.from_numpy(C))
    np.testing.assert_array_equal(s.get_conv_state(0).cpu().numpy(), C)
