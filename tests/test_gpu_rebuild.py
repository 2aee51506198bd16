"""Rebuilding a stage from its input history.

A stage that is lost mid-sequence is rebuilt from the same weights and prior
context by replaying the inputs it accepted (ChatTorrent README, "How it
works": a replacement stage rebuilds its cache from the token history).  The
rebuilt slice must hold the same bits as the one that ran: DeltaNet states,
KV rows below the position, the position itself, and the next outputs.  The
original mixes decode steps with verify passes and partial commits; the
rebuild replays only the accepted inputs as plain decode steps, which is what
a commit is defined to equal.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import inputs, make_pair

pytestmark = pytest.mark.gpu

TINY_H = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)

# (op, k, accepted): decode steps, and verify passes of k inputs with `accepted` kept
SCRIPT = [("decode", 1, 1), ("decode", 1, 1), ("verify", 4, 2), ("decode", 1, 1), ("verify", 3, 0),
          ("verify", 4, 4), ("decode", 1, 1), ("verify", 2, 1), ("decode", 1, 1)]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(shape, qtype, workload, layers, prefill):
    max_seq = (prefill + 128 + 63) // 64 * 64
    a, _, _, _ = make_pair(shape, qtype, 0, layers, workload=workload, prefill=prefill, max_seq=max_seq, max_verify=4,
                           with_oracle=False)
    H = inputs(shape, 64, workload=workload, step0=7)
    log, i = [], 0
    for op, k, acc in SCRIPT:
        if op == "decode":
            a.decode(_t(H[i]))
            log.append(H[i])
            i += 1
        else:
            a.verify(_t(H[i:i + k]))
            a.commit(acc)
            log.extend(H[i:i + acc])
            i += k          # rejected inputs are gone from the history
    a.sync_check()
    # the stage is lost here; a new one replays the accepted history
    b, _, _, _ = make_pair(shape, qtype, 0, layers, workload=workload, prefill=prefill, max_seq=max_seq, max_verify=4,
                           with_oracle=False)
    for x in log:
        b.decode(_t(x))
    b.sync_check()
    assert a.position == b.position == prefill + len(log)
    for l in range(layers):
        if shape.is_attention(l):
            for x, y in zip(a.get_kv(l, a.position), b.get_kv(l, b.position)):
                assert torch.equal(x, y), l
        else:
            assert torch.equal(a.get_state(l), b.get_state(l)), l
    # and the two carry on identically, by decode and by verify
    for t in range(3):
        x = _t(H[40 + t])
        assert torch.equal(a.decode(x), b.decode(x))
    xs = _t(H[50:54])
    assert torch.equal(a.verify(xs), b.verify(xs))


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_rebuild_from_accepted_history_hybrid(qtype):
    _run(TINY_H, qtype, 98, 4, 30)


def test_rebuild_from_accepted_history_llama():
    _run(synth.TINY_LLAMA, synth.Q4_0, synth.WL_TINY_LLAMA, 6, 100)


@pytest.mark.timeout(600)
def test_rebuild_hybrid_5120():
    """Four layers of the hidden-5120 hybrid (three DeltaNet, one attention)."""
    _run(synth.HYBRID_5120, synth.Q4_0, synth.WL_SLICE, 4, 512)
