"""A slice loaded from a GGUF file decodes with the bits of a slice loaded from
the same tensors directly, and within tolerance of the oracle; a file whose
blocks are not in the slice's format is refused."""
import numpy as np
import pytest
import torch

import synth
import layer_sliced_quantized_amd as slq
from layer_sliced_quantized_amd import gguf
from helpers import TOL, inputs, make_pair, rel_err
from test_gguf import SHAPE, gguf_tensors

pytestmark = pytest.mark.gpu

WL = 92


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_slice_from_gguf_decodes_like_direct_load(tmp_path, qtype):
    prefill = 40
    s_ref, orc, tensors, _ = make_pair(SHAPE, qtype, 0, 4, workload=WL, prefill=prefill, max_seq=256, max_verify=4)
    path = tmp_path / "tiny.gguf"
    gguf.write_gguf(str(path), {"general.architecture": "tiny_hybrid"}, gguf_tensors(SHAPE, tensors, qtype))
    g = gguf.GGUFFile(str(path))
    s = slq.Slice(slq.make_config(SHAPE, qtype, 0, 4, max_seq=256, max_verify=4, io_fp32=True))
    assert gguf.load_into_slice(s, g) == sum(len(d) for d in tensors.values())
    # the prior context make_pair gives the reference slice
    for l in range(4):
        if SHAPE.is_attention(l):
            K, V = synth.kv_prefill(0, WL, l, SHAPE.kv_heads, prefill, SHAPE.head_dim)
            s.set_kv(l, torch.from_numpy(K), torch.from_numpy(V))
        else:
            s.set_state(l, torch.from_numpy(synth.dn_state0(0, WL, l, SHAPE.dn_heads, SHAPE.dn_dv, SHAPE.dn_dk)))
    s.reset(prefill)
    H = inputs(SHAPE, 3, workload=WL)
    for t in range(3):
        x = torch.from_numpy(H[t]).cuda()
        a = s.decode(x).cpu().numpy()
        np.testing.assert_array_equal(a, s_ref.decode(x).cpu().numpy())
        assert rel_err(a, orc.decode(H[t], raw=True)) <= TOL, t


def test_gguf_in_another_block_format_is_refused(tmp_path):
    tensors = {l: synth.layer_tensors(SHAPE, synth.Q8_0, 0, WL, l) for l in range(4)}
    path = tmp_path / "q8.gguf"
    gguf.write_gguf(str(path), {}, gguf_tensors(SHAPE, tensors, synth.Q8_0))
    s = slq.Slice(slq.make_config(SHAPE, synth.Q4_0, 0, 4, max_seq=256, max_verify=4, io_fp32=True))
    with pytest.raises(gguf.GGUFError):
        gguf.load_into_slice(s, gguf.GGUFFile(str(path)))


def test_draft_head_from_gguf_drafts_like_direct_load(tmp_path):
    """A draft head read from its "mtp." tensors in a file gives the input
    projection, layer output and logits of one loaded from the same arrays
    directly, bit for bit, over three chained drafts."""
    from test_gguf import draft_head_gguf_tensors
    from test_gpu_mtp import TINY_LM, WL_MAIN, make_draft_head
    base, qt = TINY_LM, synth.Q4_0
    ref, _, sh = make_draft_head(base, qt, max_seq=64)
    T = synth.layer_tensors(sh, qt, 0, synth.WL_MTP, 0, threads=8)
    M = synth.mtp_tensors(sh, qt, 0)
    G = synth.global_tensors(base, qt, 0, WL_MAIN)
    path = tmp_path / "draft.gguf"
    gguf.write_gguf(str(path), {}, draft_head_gguf_tensors(base, T, M, G, qt))
    s = slq.Slice(slq.make_config(sh, qt, 0, 1, max_seq=64, max_verify=1, has_embed=True, has_head=True,
                                  has_mtp=True))
    assert gguf.load_into_slice(s, gguf.GGUFFile(str(path)), gguf.MTP_NAMES) == len(T) + 6
    s.reset(0)
    tok = torch.tensor([5], dtype=torch.int32, device="cuda")
    h = torch.from_numpy(synth.hidden_inputs(5, synth.WL_MTP, 1, sh.hidden)[0]).cuda()
    la = torch.empty(sh.vocab, dtype=torch.float32, device="cuda")
    lb = torch.empty_like(la)
    for _ in range(3):
        xa, xb = s.mtp_input(tok, h), ref.mtp_input(tok, h)
        np.testing.assert_array_equal(xa.cpu().numpy(), xb.cpu().numpy())
        ya, yb = s.decode(xa), ref.decode(xb)
        np.testing.assert_array_equal(ya.cpu().numpy(), yb.cpu().numpy())
        da, db = s.head_argmax(ya, logits=la), ref.head_argmax(yb, logits=lb)
        np.testing.assert_array_equal(la.cpu().numpy(), lb.cpu().numpy())
        assert int(da.item()) == int(db.item())
        tok, h = da.reshape(1).to(torch.int32), ya
