"""Host logic of bench.py (no GPU): the one-GPU contract and the rule that
the PMC traffic figure is reported only for the kernel sources it was
measured on."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_withheld_when_the_sources_differ(monkeypatch):
    monkeypatch.setattr(bench, "chain_source_hash", lambda: "0" * 64)
    assert bench.profiled_traffic() is None


def _chain_weight_bytes(shape):
    """Packed Q4_0 bytes of every matrix the chained launches read: all of the
    slice's matrices except layer 0's mixer input projections (which run before
    the first chain)."""
    import synth
    total = 0
    for l in range(shape.n_layers):
        for name, (r, c) in synth.matrix_shapes(shape, l).items():
            if l == 0 and name in ("dn_q", "dn_k", "dn_v", "dn_a", "dn_b", "dn_z", "wq", "wg", "wk", "wv"):
                continue
            total += r * c // 32 * 18
    return total


def test_chain_bytes_cover_the_slice_weights():
    import synth
    sh = synth.HYBRID_5120
    w = _chain_weight_bytes(sh)
    b = bench.chain_step_bytes(sh, synth.Q4_0, deltanet=False)
    # 255 products over the step, each with its fp32 input and output vectors (< 200 KB each)
    assert w < b < w + 255 * 200_000
    # with the DeltaNet updates inside: the 48 layers' fp32 states (2 MB) read and written, plus their inputs
    state = 48 * 2 * 32 * 128 * 128 * 4
    assert b + state < bench.chain_step_bytes(sh, synth.Q4_0) < b + state + 48 * 100_000


def test_traffic_of_the_committed_profile():
    import synth
    t = bench.profiled_traffic()
    if t is None:
        pytest.skip("the chained-products kernel sources changed after its PMC traffic was taken")
    text = open(bench.TRAFFIC_PROFILE).read()
    launches = int(re.search(r"launches_per_step: (\d+)", text).group(1))
    m = re.search(r"first_input_projections_chained: (\d)", text)
    alg = bench.chain_step_bytes(synth.HYBRID_5120, synth.Q4_0, deltanet="DeltaNet" in text,
                                 first_g1=bool(m and m.group(1) == "1")) / launches
    # measured HBM bytes per launch against the algorithmic bytes: no re-read of weights
    assert 0.99 * alg <= t <= 1.05 * alg
