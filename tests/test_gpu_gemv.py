"""GPU parity of the Q4_0 / Q8_0 decode and GEMV kernels against the CPU oracle.

Called through the C ABI (slq_repack, slq_dequant, slq_gemv).  Decode must be
bit-exact (every (q-8)*d and q*d is exact in fp32); products must be within
max relative error 2e-3 of the fp64 oracle (they land near 1e-6).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import qref
from helpers import rel_err, TOL

import layer_sliced_quantized_amd as slq

pytestmark = pytest.mark.gpu

QTYPES = [synth.Q4_0, synth.Q8_0]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _raw(qtype, rows, cols, tag):
    return synth.quant_blocks(synth.stream(11, synth.WL_GEMV, tag, rows % 1000, cols % 1000), qtype, rows, cols)


# several tiles, ragged row groups (rows % 64) and a ragged last tile (blocks % 8)
SMALL = [(64, 256), (200, 32 * 19), (1000, 32 * 37), (37, 32 * 3), (5120, 512)]


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("rows,cols", SMALL)
def test_dequant_bit_exact(qtype, rows, cols):
    raw = _raw(qtype, rows, cols, 1)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    got = slq.dequant(qtype, packed, rows, cols).cpu().numpy()
    ref = qref.dequant(qtype, raw, rows, cols)
    np.testing.assert_array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("rows,cols", SMALL)
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_gemv_parity_small(qtype, rows, cols, batch):
    raw = _raw(qtype, rows, cols, 2)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    x = synth.gemv_x(5, batch, cols, tag=rows)
    y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    ref = qref.gemv(qtype, raw, rows, cols, x.astype(np.float64))
    for t in range(batch):
        e = rel_err(y[t], ref[t])
        assert e <= TOL, (t, e)
        assert e <= 1e-5, (t, e)     # integer block dots: expected ~1e-7


@pytest.mark.parametrize("qtype", QTYPES)
def test_gemv_batch_equals_single_bitwise(qtype):
    rows, cols = 1000, 32 * 37
    raw = _raw(qtype, rows, cols, 3)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    x = synth.gemv_x(6, 16, cols)
    y16 = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    for t in (0, 7, 15):
        y1 = slq.gemv(qtype, packed, rows, cols, _dev(x[t:t + 1])).cpu().numpy()
        np.testing.assert_array_equal(y1[0], y16[t])


# (split-K workgroups, waves per workgroup) of the standalone GEMV, forced
# through the plan overrides; batched calls (int8 MFMA) must reproduce the
# single-token GEMV bit for bit under every split
SPLITS = [(1, 1), (1, 8), (3, 2), (16, 1), (2, 8), (5, 3)]


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("ks,w", SPLITS)
@pytest.mark.parametrize("rows,cols", [(200, 32 * 19), (1000, 32 * 37), (64, 32 * 130)])
def test_gemm_batch_equals_single_bitwise(qtype, ks, w, rows, cols, ovr):
    ovr(MFMA_MIN_T="2")      # every batched call on the matrix cores
    ovr(KS_GEMV=ks)
    ovr(W_GEMV=w)
    raw = _raw(qtype, rows, cols, 9)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    x = synth.gemv_x(12, 16, cols, tag=ks * 10 + w)
    x[3] = 0.0                      # an all-zero token
    x[5, 64:96] = 0.0               # an all-zero block inside a token
    x[9, ::5] *= 1e3                # wide range inside blocks
    y1 = np.stack([slq.gemv(qtype, packed, rows, cols, _dev(x[t:t + 1])).cpu().numpy()[0] for t in range(16)])
    assert np.all(y1[3] == 0)
    for batch in (2, 5, 11, 16):
        yb = slq.gemv(qtype, packed, rows, cols, _dev(x[:batch])).cpu().numpy()
        np.testing.assert_array_equal(yb, y1[:batch])
    ref = qref.gemv(qtype, raw, rows, cols, x.astype(np.float64))
    for t in range(16):
        assert rel_err(y1[t], ref[t]) <= 1e-5, t


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("batch,min_t", [(1, "0"), (5, "17"), (5, "2"), (16, "2")])
def test_split_tickets_reset_on_reuse(qtype, batch, min_t, ovr):
    """The split that takes a row group's last ticket resets it: one workspace
    reused for different inputs gives each call the result of a fresh
    workspace, and its tickets end at zero.  (min_t 17 keeps a 5-token call on
    the per-row GEMV, 2 sends it to the MFMA products.)"""
    ks, w = 5, 2
    ovr(KS_GEMV=ks)
    ovr(W_GEMV=w)
    ovr(MFMA_MIN_T=min_t)
    rows, cols = 1000, 32 * 37
    raw = _raw(qtype, rows, cols, 14)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    xa = synth.gemv_x(21, batch, cols)
    xb = synth.gemv_x(22, batch, cols)
    fresh_a = slq.gemv(qtype, packed, rows, cols, _dev(xa)).cpu().numpy()
    fresh_b = slq.gemv(qtype, packed, rows, cols, _dev(xb)).cpu().numpy()
    ws = torch.zeros(slq.gemv_workspace_bytes(qtype, rows, cols, batch), dtype=torch.uint8, device="cuda")
    for x, ref in ((xa, fresh_a), (xb, fresh_b), (xa, fresh_a)):
        y = slq.gemv(qtype, packed, rows, cols, _dev(x), ws=ws).cpu().numpy()
        np.testing.assert_array_equal(y, ref)
    # the workspace ends with the 16 row groups' tickets (one 256-byte line)
    assert int(torch.count_nonzero(ws[-256:])) == 0


@pytest.mark.parametrize("qtype", QTYPES)
def test_gemm_single_token_through_mfma(qtype, ovr):
    """With the MFMA path forced for one token the result equals the GEMV's."""
    rows, cols = 1000, 32 * 37
    raw = _raw(qtype, rows, cols, 10)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    x = synth.gemv_x(13, 1, cols)
    y_gemv = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    ovr(MFMA_MIN_T="1")
    y_mfma = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    np.testing.assert_array_equal(y_gemv, y_mfma)


@pytest.mark.parametrize("qtype", QTYPES)
def test_gemv_many_blocks(qtype):
    """4000 activation blocks: the largest entry of a block sits on the
    quantiser's range limit, which must not overflow the digits."""
    rows, cols = 64, 32 * 4000
    raw = _raw(qtype, rows, cols, 5)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    for tag in range(3):
        x = synth.gemv_x(8, 2, cols, tag=tag)
        y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
        ref = qref.gemv(qtype, raw, rows, cols, x.astype(np.float64))
        for t in range(2):
            assert rel_err(y[t], ref[t]) <= 1e-5


@pytest.mark.parametrize("qtype", QTYPES)
def test_gemv_edge_inputs(qtype):
    rows, cols = 128, 32 * 10
    raw = _raw(qtype, rows, cols, 4)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    W = qref.dequant(qtype, raw, rows, cols)
    # zero input -> exactly zero
    y = slq.gemv(qtype, packed, rows, cols, torch.zeros((1, cols), device="cuda")).cpu().numpy()
    assert np.all(y == 0)
    # unit vector -> one column
    for j in (0, 17, 31, 32, 319):
        x = np.zeros((1, cols), np.float32)
        x[0, j] = 1.0
        y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
        assert rel_err(y[0], W[:, j]) <= 1e-6
    # wide dynamic range inside a block
    x = synth.gemv_x(7, 1, cols)
    x[0, ::7] *= 1e4
    x[0, 1::11] *= 1e-4
    y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    assert rel_err(y[0], W @ x[0].astype(np.float64)) <= TOL
    # determinism: same call, same bits
    y2 = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
    np.testing.assert_array_equal(y, y2)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("rows,cols", synth.GEMV_SHAPES)
@pytest.mark.timeout(300)
def test_gemv_full_shapes_sampled_rows(qtype, rows, cols):
    """The GEMV sweep shapes at full size, batch 1 and 16; 96 sampled rows against the oracle."""
    raw = synth.quant_blocks(synth.stream(0, synth.WL_GEMV, 100, rows, cols), qtype, rows, cols)
    packed = slq.repack(qtype, _dev(raw), rows, cols)
    rng = np.random.default_rng(rows + cols)
    sample = np.sort(np.concatenate([[0, rows - 1], rng.choice(rows, 94, replace=False)]))
    for batch in (1, 16):
        x = synth.gemv_x(0, batch, cols, tag=batch)
        y = slq.gemv(qtype, packed, rows, cols, _dev(x)).cpu().numpy()
        ref = qref.gemv(qtype, raw[sample], len(sample), cols, x.astype(np.float64))
        for t in range(batch):
            assert rel_err(y[t, sample], ref[t]) <= TOL
    del packed
    torch.cuda.empty_cache()
