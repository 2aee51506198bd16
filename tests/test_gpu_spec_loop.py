"""Greedy generation with speculative drafts gives exactly the plain greedy
token stream (the pages report the same output for plain and speculative
decoding; SwarmLLM README, benchmark table).  A whole small model (a tiny
Llama, and a tiny hybrid whose DeltaNet layers roll back by state slot; each
with embedding and tied head) runs as one slice.  The drafts are the plain
stream with seeded corruptions, so rounds both accept and reject: each round
feeds the last token and K-1 drafts through slice_verify, keeps the drafts up
to the first one that differs from the model's own argmax, and commits the
inputs that produced kept tokens.  The tokens and every kept position's hidden
output must equal the plain run's exactly."""
import numpy as np
import pytest
import torch

import synth
from helpers import make_pair

pytestmark = pytest.mark.gpu

N = 40    # tokens generated
K = 4     # inputs per verify round: the last token and K-1 drafts


# the hybrid layer mix (DeltaNet layers roll back by state slot) with a small
# vocabulary and a tied head
TINY_HYBRID_LM = synth.ModelShape(
    name="tiny_hybrid_lm", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=1024, tied_head=True)

MODELS = {"tiny_llama": (synth.TINY_LLAMA, synth.WL_TINY_LLAMA), "tiny_hybrid": (TINY_HYBRID_LM, 95)}


def _model(name):
    sh, wl = MODELS[name]
    s, _, _, _ = make_pair(sh, synth.Q4_0, 0, sh.n_layers, workload=wl, prefill=128,
                           max_seq=512, max_verify=K, has_embed=True, has_head=True, with_oracle=False)
    return s, sh


def _tok(t):
    return torch.tensor([t], dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("model", list(MODELS))
def test_speculative_stream_equals_plain_stream(model):
    s, sh = _model(model)
    vocab = sh.vocab
    tok0 = synth.tiny_llama_token(0) % vocab

    plain, plain_h = [], []
    tok = tok0
    for _ in range(N + K):
        y = s.decode(s.embed(_tok(tok)))
        plain_h.append(y.cpu().numpy())
        tok = int(s.head_argmax(y).item())
        plain.append(tok)
    assert s.position == 128 + N + K

    s, _ = _model(model)
    rng = np.random.default_rng(5)
    out, out_h, cur = [], [], tok0
    accepted_counts = []
    X = torch.empty((K, sh.hidden), dtype=s.io_dtype, device="cuda")
    while len(out) < N:
        L = len(out)
        drafts = [plain[L + i] if rng.random() > 0.3 else (plain[L + i] + 1) % vocab for i in range(K - 1)]
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
        cur = a[m]
        accepted_counts.append(m)
    assert out[:N] == plain[:N]
    # every kept position's hidden output is the plain step's, bit for bit (the
    # synthetic weights can make the greedy stream repeat one token; the hidden
    # states still differ from position to position)
    for i in range(N):
        np.testing.assert_array_equal(out_h[i], plain_h[i])
    assert s.position == 128 + len(out)
    assert min(accepted_counts) < K - 1 and max(accepted_counts) > 0, accepted_counts
