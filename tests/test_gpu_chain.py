"""Chained decode products against separate kernels, through the C ABI.

Decode runs each layer's DeltaNet update (in DeltaNet layers) and the products
after its mixer (mixer output, gate/up + SwiGLU, down, the next layer's input
projections) in kernels whose workgroups wait for the phase before theirs; one
launch runs the phases of consecutive layers up to the next attention layer.  With the same launch shapes
as the separate GEMV kernels, the results must be the same bits; they are
also checked against the CPU oracle, and slice_sync_check must report no
wait that gave up.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from helpers import TOL, inputs, make_pair, rel_err

pytestmark = pytest.mark.gpu

TINY_H = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _pair(shape, qtype, begin, end, ovr, chain, **kw):
    ovr(CHAIN=int(chain))
    s, orc, _, _ = make_pair(shape, qtype, begin, end, **kw)
    ovr(CHAIN=1)
    return s, orc


def _compare(shape, qtype, begin, end, ovr, steps, workload, layers_dn, layer_attn=None, **kw):
    a, orc = _pair(shape, qtype, begin, end, ovr, True, workload=workload, **kw)
    b, _ = _pair(shape, qtype, begin, end, ovr, False, workload=workload, with_oracle=False, **kw)
    H = inputs(shape, steps, workload=workload, step0=50, io_fp32=kw.get("io_fp32", True))
    for t in range(steps):
        x = _t(H[t])
        ya = a.decode(x).cpu().numpy()
        yb = b.decode(x).cpu().numpy()
        np.testing.assert_array_equal(ya, yb)
        assert rel_err(a.get_hidden().cpu().numpy()[0], orc.decode(H[t], raw=True)) <= TOL, t
    a.sync_check()
    b.sync_check()
    for l in layers_dn:
        np.testing.assert_array_equal(a.get_state(l).cpu().numpy(), b.get_state(l).cpu().numpy())
    if layer_attn is not None:
        n = a.position
        Ka, Va = a.get_kv(layer_attn, n)
        Kb, Vb = b.get_kv(layer_attn, n)
        np.testing.assert_array_equal(Ka.cpu().numpy(), Kb.cpu().numpy())
        np.testing.assert_array_equal(Va.cpu().numpy(), Vb.cpu().numpy())


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_chain_equals_separate_kernels_tiny_hybrid(qtype, ovr):
    _compare(TINY_H, qtype, 0, 4, ovr, 5, 95, [0, 1, 2], 3, prefill=40, max_seq=128, max_verify=4)


def test_chain_equals_separate_kernels_tiny_llama(ovr):
    _compare(synth.TINY_LLAMA, synth.Q4_0, 0, 30, ovr, 3, synth.WL_TINY_LLAMA, [], 0, prefill=128, max_seq=256,
             max_verify=4)


def test_chain_without_ffn(ovr):
    sh = dataclasses.replace(TINY_H, name="tiny_hybrid_noffn", ffn=0)
    _compare(sh, synth.Q4_0, 0, 4, ovr, 4, 96, [0, 1, 2], 3, prefill=10, max_seq=128, max_verify=4)


@pytest.mark.timeout(600)
def test_chain_equals_separate_kernels_hybrid_5120(ovr):
    """Layers 0..7 of the hidden-5120 hybrid (6 DeltaNet, 2 attention), at the
    launch shapes of the benchmark: the same bits as separate kernels."""
    _compare(synth.HYBRID_5120, synth.Q4_0, 0, 8, ovr, 3, synth.WL_SLICE, [0, 1, 2, 4], 3, prefill=512,
             max_seq=1024, max_verify=4, io_fp32=False, threads=16)


def test_chain_with_verify_and_graph_replays(ovr):
    """Chained decode steps between verify passes (separate kernels) and
    commits: decode outputs equal the verify pass's bits for the same inputs,
    over many graph replays (the chains' counters advance every step)."""
    H = inputs(TINY_H, 24, workload=97)
    a, _ = _pair(TINY_H, synth.Q4_0, 0, 4, ovr, True, workload=97, prefill=20, max_seq=256, max_verify=4,
                 with_oracle=False)
    b, _ = _pair(TINY_H, synth.Q4_0, 0, 4, ovr, True, workload=97, prefill=20, max_seq=256, max_verify=4,
                 with_oracle=False)
    for r in range(5):
        k = 4
        xs = _t(H[4 * r:4 * r + k])
        ver = a.verify(xs).cpu().numpy()
        a.commit(k)
        dec = np.stack([b.decode(xs[t]).cpu().numpy() for t in range(k)])
        np.testing.assert_array_equal(ver, dec)
    a.sync_check()
    b.sync_check()
    # a run of decode steps long after: still the same bits as the other slice
    for t in range(20, 24):
        x = _t(H[t])
        np.testing.assert_array_equal(a.decode(x).cpu().numpy(), b.decode(x).cpu().numpy())
    b.sync_check()


@pytest.mark.parametrize("extra", [{"CHAIN_DN": 0}, {"CHAIN_ATT": 0}, {"CHAIN_G1": 0}, {"CHAIN_MAX": 5},
                                   {"CHAIN_MAX": 2}, {"CHAIN_MAX": 1}],
                         ids=["deltanet_own_kernel", "attention_merge_own_kernel", "first_input_own_kernel",
                              "one_layer_per_launch", "two_phases_per_launch", "one_phase_per_launch"])
def test_chain_variants_equal_separate_kernels(extra, ovr):
    """The DeltaNet update, the attention merge or the first layer's input
    projections as kernels of their own, one layer's phases per launch, or a
    layer's phases spread over several launches: the same bits as separate
    kernels, states and caches included.  (By default the first launch starts
    with the first layer's input projections and runs all three DeltaNet
    layers, each update waiting for the input projections before it, and the
    attention layer's launch starts with its merge.)"""
    ovr(**extra)
    _compare(TINY_H, synth.Q4_0, 0, 4, ovr, 4, 99, [0, 1, 2], 3, prefill=20, max_seq=128, max_verify=4)


@pytest.mark.timeout(300)
def test_chained_attention_merge_at_its_limit(ovr):
    """A cache of 64 chunks (2048 rows), the most the chained merge takes,
    with the position in its last chunk: the same bits as separate kernels,
    and so for a cache one chunk past the limit (the merge as its own
    kernel)."""
    for max_seq in (2048, 2112):
        _compare(TINY_H, synth.Q4_0, 0, 4, ovr, 3, 98, [0, 1, 2], 3, prefill=max_seq - 8, max_seq=max_seq,
                 max_verify=4)
