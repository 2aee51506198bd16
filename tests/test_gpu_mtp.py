"""The draft head (multi-token prediction) on the GPU against the oracle, and
the speculative loop driven by its drafts.

The last stage samples a token and its draft head predicts the token that
follows it (SwarmLLM README, pipeline diagram); drafts are checked in one
batched pass and the speculative stream equals the plain one (feature list,
benchmark table).  The head's form is the oracle's reading (oracle.model.mtp_input,
DraftHead): the input projection of the normalised embedding and hidden
state, one full-attention layer with its own cache, its own final norm, the
model's LM head.  Its weights are synthetic, so its drafts are poor guesses;
the loop must still give the plain stream bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import layer_sliced_quantized_amd as slq
import oracle
import synth
from helpers import TOL, make_pair, rel_err

pytestmark = pytest.mark.gpu

# the hybrid of the speculative-loop test, with an untied head
TINY_LM = synth.ModelShape(
    name="tiny_hybrid_lm_untied", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=1024, tied_head=False)
# the hidden-5120 hybrid with a small vocabulary (the layer is full size)
WIDE_LM = dataclasses.replace(synth.HYBRID_5120, name="hybrid_5120_vocab2048", vocab=2048)
WL_MAIN = 97


def make_draft_head(base, qtype, *, seed=0, prefill=0, max_seq=256, io_fp32=False, glob=None, with_layer=True):
    """(GPU Slice, oracle DraftHead) of the draft head of model `base`, whose
    embedding and head tables (glob) it shares."""
    sh = synth.mtp_shape(base)
    T = synth.layer_tensors(sh, qtype, seed, synth.WL_MTP, 0, threads=8) if with_layer else {}
    M = synth.mtp_tensors(sh, qtype, seed)
    G = dict(glob if glob is not None else synth.global_tensors(base, qtype, seed, WL_MAIN))
    G["out_norm"] = M["mtp_out_norm"]
    cfg = slq.make_config(sh, qtype, 0, 1, max_seq=max_seq, max_verify=1, io_fp32=io_fp32, has_embed=True,
                          has_head=True, has_mtp=True)
    s = slq.Slice(cfg)
    s.load_numpy({0: T} if with_layer else {}, {**G, **{k: M[k] for k in ("mtp_fc", "mtp_norm_e", "mtp_norm_h")}})
    dh = oracle.DraftHead(sh, qtype, T, M, G, max_seq=max_seq, io_fp32=io_fp32)
    if prefill:
        K, V = synth.kv_prefill(seed, synth.WL_MTP, 0, sh.kv_heads, prefill, sh.head_dim)
        s.set_kv(0, torch.from_numpy(K), torch.from_numpy(V))
        dh.set_kv(K, V)
    s.reset(prefill)
    dh.reset(prefill)
    torch.cuda.synchronize()
    return s, dh, sh


def _tok(t):
    return torch.tensor([t], dtype=torch.int32, device="cuda")


def _h(sh, n, io_fp32, step0=0):
    h = synth.hidden_inputs(5, synth.WL_MTP, n, sh.hidden, step0=step0)
    return h.astype(np.float32) if io_fp32 else h


@pytest.mark.parametrize("base,qtype,io_fp32", [(TINY_LM, synth.Q4_0, True), (TINY_LM, synth.Q8_0, False),
                                               (WIDE_LM, synth.Q4_0, False), (WIDE_LM, synth.Q8_0, True)],
                         ids=["tiny-q4-fp32", "tiny-q8-fp16", "5120-q4-fp16", "5120-q8-fp32"])
@pytest.mark.timeout(300)
def test_mtp_input_matches_the_oracle(base, qtype, io_fp32):
    """The input projection (embedding row and hidden state, each normalised,
    through the 2H-wide product): tokens at both ends of the table, and ids
    outside it, which read row 0."""
    s, dh, sh = make_draft_head(base, qtype, io_fp32=io_fp32, with_layer=False)
    H = _h(sh, 5, io_fp32)
    V = sh.vocab
    for i, (tok, ref_tok) in enumerate([(0, 0), (V - 1, V - 1), (777 % V, 777 % V), (-5, 0), (V + 7, 0)]):
        got = s.mtp_input(_tok(tok), torch.from_numpy(H[i]).cuda()).cpu().numpy()
        ref = oracle.mtp_input(qtype, dh.stage.G["embed"], ref_tok, H[i], dh.mtp["mtp_norm_e"],
                               dh.mtp["mtp_norm_h"], dh.mtp["mtp_fc"], sh.hidden, sh.eps)
        assert got.dtype == (np.float32 if io_fp32 else np.float16)
        assert rel_err(got, ref) <= TOL, (tok, rel_err(got, ref))
    assert s.position == 0   # the input touches no position


@pytest.mark.parametrize("base,prefill,io_fp32", [(TINY_LM, 64, False), (WIDE_LM, 512, True)], ids=["tiny", "5120"])
@pytest.mark.timeout(300)
def test_draft_chain_matches_the_oracle(base, prefill, io_fp32):
    """Four drafts in a row, each fed the previous draft and the layer's
    output: every step's input, layer output and logits against the oracle
    driven by the same inputs; each draft token exact wherever the top-two
    margin of the logits exceeds the head product's error.  (At hidden 5120
    the synthetic weights, of mean -0.5 d, take the layer's output past the
    fp16 range, so that case keeps its vectors in fp32, as a host stage can.)"""
    s, dh, sh = make_draft_head(base, synth.Q4_0, prefill=prefill, max_seq=prefill + 64, io_fp32=io_fp32)
    h = _h(sh, 1, io_fp32)[0]
    tok = 3
    logits = torch.empty(sh.vocab, dtype=torch.float32, device="cuda")
    for step in range(4):
        x = s.mtp_input(_tok(tok), torch.from_numpy(h).cuda())
        x_np = x.cpu().numpy()
        assert rel_err(x_np, oracle.mtp_input(synth.Q4_0, dh.stage.G["embed"], tok, h, dh.mtp["mtp_norm_e"],
                                              dh.mtp["mtp_norm_h"], dh.mtp["mtp_fc"], sh.hidden, sh.eps)) <= TOL
        y = s.decode(x)
        y_np = y.cpu().numpy()
        y_ref = dh.stage.decode(x_np, raw=True)          # the oracle's layer on the same input
        assert rel_err(y_np, y_ref) <= TOL, (step, rel_err(y_np, y_ref))
        d = int(s.head_argmax(y, logits=logits).item())
        lg = logits.cpu().numpy()
        lg_own = dh.stage.head_logits(y_np.astype(np.float64))
        assert rel_err(lg, lg_own) <= 1e-5
        err = float(np.max(np.abs(lg - lg_own)))
        top = np.sort(lg_own)[::-1]
        if top[0] - top[1] > 4 * err:
            assert d == int(np.argmax(lg_own)), step
        else:
            assert lg_own[d] >= top[0] - 4 * err, step
        tok, h = d, y_np
    assert s.position == prefill + 4 and dh.pos == prefill + 4


@pytest.mark.timeout(300)
def test_speculative_loop_with_the_draft_head_equals_plain():
    """Greedy generation on a whole tiny hybrid (embedding, untied head) with
    K-1 drafts per round from the draft head: each round verifies the last
    token and the drafts, keeps the drafts up to the first miss, commits, and
    rolls the draft head's position back to match.  Tokens and every kept
    hidden output equal the plain run's bit for bit."""
    N, K = 32, 4
    sh = TINY_LM

    def main():
        s, _, _, glob = make_pair(sh, synth.Q4_0, 0, sh.n_layers, workload=WL_MAIN, prefill=128, max_seq=512,
                                  max_verify=K, io_fp32=False, has_embed=True, has_head=True, with_oracle=False)
        return s, glob

    s, glob = main()
    plain, plain_h = [], []
    tok = 11
    for _ in range(N + K):
        y = s.decode(s.embed(_tok(tok)))
        plain_h.append(y.cpu().numpy())
        tok = int(s.head_argmax(y).item())
        plain.append(tok)

    s, glob = main()
    mtp, _, _ = make_draft_head(sh, synth.Q4_0, glob=glob, prefill=128, max_seq=512)
    # the first token comes from a plain step; the draft head starts at its position
    y = s.decode(s.embed(_tok(11)))
    cur = int(s.head_argmax(y).item())
    out, out_h = [cur], [y.cpu().numpy()]
    mtp.reset(s.position - 1)
    X = torch.empty((K, sh.hidden), dtype=s.io_dtype, device="cuda")
    accepted = []
    while len(out) < N:
        P = s.position
        drafts, t, hh = [], cur, y
        for _ in range(K - 1):
            hh = mtp.decode(mtp.mtp_input(_tok(t), hh))
            t = int(mtp.head_argmax(hh).item())
            drafts.append(t)
        for i, t in enumerate([cur] + drafts):
            s.embed(_tok(t), out=X[i])
        Y = s.verify(X)
        a = [int(s.head_argmax(Y[i]).item()) for i in range(K)]
        m = 0
        while m < K - 1 and drafts[m] == a[m]:
            m += 1
        s.commit(m + 1)
        out.extend(a[:m + 1])
        out_h.extend(Y[:m + 1].cpu().numpy())
        cur, y = a[m], Y[m].clone()
        mtp.reset(P + m)
        accepted.append(m)
    assert out[:N] == plain[:N]
    for i in range(N):
        np.testing.assert_array_equal(out_h[i], plain_h[i])
    assert s.position == 128 + len(out)
    assert mtp.position == s.position - 1
    mtp.sync_check()
    s.sync_check()


def test_draft_head_rejects_a_plain_slice():
    s, _, _, _ = make_pair(TINY_LM, synth.Q4_0, 0, 1, workload=WL_MAIN, max_seq=64, with_oracle=False,
                           has_embed=True)
    with pytest.raises(slq.SliceError):
        s.mtp_input(_tok(0), torch.zeros(TINY_LM.hidden, dtype=torch.float32, device="cuda"))
