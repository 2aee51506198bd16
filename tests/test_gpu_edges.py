"""GPU edge cases against the CPU oracle, through the C ABI.

* Hand-decoded GGUF blocks (negative and subnormal fp16 scales, the Q8_0 code
  -128 that the seeded generator never draws) placed among random blocks:
  dequantisation bit-exact, products within 1e-5.
* Activation blocks at the ends of the range: tiny and subnormal entries, an
  all-zero block, and a block holding inf or NaN (the products must not turn
  it into finite garbage).
* The 248320-row LM head of the hybrid driven through slice_head_argmax on a
  slice that holds no layers, only the last stage's head.
* Decode at position 0, where attention sees only the row it appends.
* The 64-layer Q8_0 hybrid slice that the benchmark also times.
"""
import os

import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import qref
from helpers import TOL, inputs, make_pair, rel_err

import layer_sliced_quantized_amd as slq

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_blocks.txt")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _golden(qtype):
    out = []
    cur = None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(None, 1)
        if key == "type":
            cur = {"Q4_0": synth.Q4_0, "Q8_0": synth.Q8_0}[rest.strip()]
        elif key == "bytes" and cur == qtype:
            out.append(np.array([int(b, 16) for b in rest.split()], dtype=np.uint8))
    return out


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_golden_blocks_dequant_and_gemv(qtype):
    rows, cols = 200, 32 * 19
    bb = synth.BLOCK_BYTES[qtype]
    raw = synth.quant_blocks(synth.stream(31, synth.WL_GEMV, 300, qtype), qtype, rows, cols)
    blk = raw.reshape(rows, cols // 32, bb)
    gold = _golden(qtype)
    assert len(gold) >= 2
    rng = np.random.default_rng(qtype)
    # every golden block in many places: first/last row and block, ragged tile
    for i in range(400):
        r = int(rng.integers(0, rows)) if i > 3 else (0, rows - 1, 63, 64)[i]
        b = int(rng.integers(0, cols // 32)) if i > 3 else (0, cols // 32 - 1, 16, 18)[i]
        blk[r, b] = gold[i % len(gold)]
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    got = slq.dequant(qtype, packed, rows, cols).cpu().numpy()
    ref = qref.dequant(qtype, raw, rows, cols)
    np.testing.assert_array_equal(got.astype(np.float64), ref)
    for batch in (1, 5):
        x = synth.gemv_x(32, batch, cols, tag=qtype)
        y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
        yr = qref.gemv(qtype, raw, rows, cols, x.astype(np.float64))
        for t in range(batch):
            assert rel_err(y[t], yr[t]) <= 1e-5, (batch, t)


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
@pytest.mark.parametrize("batch", [1, 4])
def test_activation_blocks_at_range_ends(qtype, batch):
    rows, cols = 128, 32 * 12
    raw = synth.quant_blocks(synth.stream(33, synth.WL_GEMV, 301, qtype), qtype, rows, cols)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    x = synth.gemv_x(34, batch, cols, tag=qtype).astype(np.float32)
    x[:, 0:32] *= 1e-30                     # tiny block
    x[:, 64:96] = 0.0                       # zero block
    x[:, 96:128] = np.float32(1e-40) * np.sign(x[:, 96:128])   # subnormal entries
    x[:, 200] = 0.0
    y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    yr = qref.gemv(qtype, raw, rows, cols, x.astype(np.float64))
    assert np.all(np.isfinite(y))
    for t in range(batch):
        assert rel_err(y[t], yr[t]) <= 1e-5, t
    # every block tiny: the result is tiny but still accurate
    xt = (synth.gemv_x(35, batch, cols, tag=qtype) * 1e-30).astype(np.float32)
    yt = slq.gemv(qtype, packed, rows, cols, _dev(xt)).cpu().numpy()
    yrt = qref.gemv(qtype, raw, rows, cols, xt.astype(np.float64))
    for t in range(batch):
        assert rel_err(yt[t], yrt[t]) <= 1e-5, t
    # a non-finite entry poisons every output, as in the exact sums
    for bad in (np.inf, -np.inf, np.nan):
        xb = x.copy()
        xb[:, 170] = bad
        yb = slq.gemv(qtype, packed, rows, cols, _dev(xb)).cpu().numpy()
        ybr = qref.gemv(qtype, raw, rows, cols, xb.astype(np.float64))
        assert np.all(~np.isfinite(ybr))
        assert np.all(np.isnan(yb)), bad


@pytest.mark.timeout(300)
def test_lm_head_248320_through_head_argmax():
    """Last stage of the hybrid: final RMSNorm, the 248320 x 5120 Q4_0 head,
    greedy argmax.  The logits must match the fp64 oracle within 1e-5 and the
    token exactly, with a margin well above the observed logit error."""
    sh = synth.HYBRID_5120
    raw = synth.quant_blocks(synth.stream(0, synth.WL_SLICE, 0, synth.TENSOR_IDS["head"]), synth.Q4_0,
                             sh.vocab, sh.hidden)
    glob = {"head": raw, "out_norm": np.ones(sh.hidden, np.float32)}
    cfg = slq.make_config(sh, synth.Q4_0, sh.n_layers, sh.n_layers, max_seq=64, max_verify=1, io_fp32=True,
                          has_head=True)
    s = slq.Slice(cfg)
    s.load_numpy({}, glob)
    orc = oracle.SliceOracle(sh, synth.Q4_0, sh.n_layers, sh.n_layers, {}, glob, max_seq=64, io_fp32=True)
    for seed in (0, 1):
        h = inputs(sh, 1, workload=synth.WL_SLICE, seed=seed, step0=900)[0] * 3.0
        logits = torch.empty(sh.vocab, dtype=torch.float32, device="cuda")
        tok = int(s.head_argmax(_dev(h), logits=logits).item())
        lg = logits.cpu().numpy()
        ref = orc.head_logits(h)
        assert rel_err(lg, ref) <= 1e-5
        err = float(np.max(np.abs(lg - ref)))
        top = np.sort(ref)[::-1]
        assert top[0] - top[1] > 4 * err, (top[0] - top[1], err)
        assert tok == orc.argmax(ref) == int(np.argmax(lg))
    del s
    torch.cuda.empty_cache()


TINY_H = synth.ModelShape(
    name="tiny_hybrid_128", hidden=128, n_layers=4, attn_period=4,
    dn_heads=2, dn_dk=64, dn_dv=64, q_heads=4, kv_heads=2, head_dim=64, rope_dims=32,
    rope_theta=1e7, qk_norm=True, attn_gate=True, eps=1e-6, ffn=256, vocab=0)


@pytest.mark.parametrize("qtype", [synth.Q4_0, synth.Q8_0])
def test_decode_at_position_zero(qtype):
    """An empty cache: the first token's attention sees only the row it
    appends, then the next steps see 2 and 3 rows."""
    s, orc, _, _ = make_pair(TINY_H, qtype, 0, 4, workload=94, prefill=0, max_seq=64, max_verify=4)
    H = inputs(TINY_H, 3, workload=94)
    for t in range(3):
        out = s.decode(_dev(H[t])).cpu().numpy()
        assert rel_err(out, orc.decode(H[t], raw=True)) <= TOL, t
    K, V = s.get_kv(3, 3)
    assert rel_err(K.cpu().numpy(), orc.kv[3][0][:, :3]) <= TOL
    assert rel_err(V.cpu().numpy(), orc.kv[3][1][:, :3]) <= TOL


@pytest.mark.timeout(1200)
def test_hybrid_64_layer_q8_slice():
    """The 64-layer Q8_0 hybrid slice (25.3 GB of weights): decode, a 4-draft
    verify, commit of the seeded accepted count, decode again; compared on the
    fp32 residual stream (with these synthetic weights |h| passes the fp16
    range within two layers)."""
    sh = synth.HYBRID_5120
    s, orc, _, _ = make_pair(sh, synth.Q8_0, 0, 64, workload=synth.WL_SLICE, prefill=512, max_seq=1024,
                             max_verify=4, io_fp32=False, threads=16)
    H = inputs(sh, 6, workload=synth.WL_SLICE, io_fp32=False, step0=200)
    s.decode(_dev(H[0]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[0], raw=True)) <= TOL
    s.verify(_dev(H[1:5]))
    out = s.get_hidden(4).cpu().numpy()
    ref = orc.verify(H[1:5], raw=True)
    for t in range(4):
        assert rel_err(out[t], ref[t]) <= TOL, t
    j = int(synth.accept_pattern(1, 1, 4)[0])
    s.commit(j)
    orc.commit(j)
    s.decode(_dev(H[5]))
    assert rel_err(s.get_hidden().cpu().numpy()[0], orc.decode(H[5], raw=True)) <= TOL
    del s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n16", [1, 16 * 256 * 4096 + 12345, 16 * 256 * 16384 + 777])
def test_read_probe_reads_every_word_once(n16):
    """The XOR of the probe's per-wave folds equals the XOR of every 32-bit
    word of the buffer: each word was read exactly once (the sixteen-load
    loop and the tail; grids of one workgroup, below the cap and at it)."""
    import layer_sliced_quantized_amd as slq
    words = synth.stream(0, synth.WL_GEMV, 300, n16).integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(4 * slq.READ_PROBE_GRID, dtype=torch.int32, device="cuda")
    slq.read_probe(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
