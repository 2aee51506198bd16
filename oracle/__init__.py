"""CPU oracle for the layer-slice decode path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or build anything here.  The
library in ``layer_sliced_quantized_amd`` never does, and shares no code with it:
the only common module is ``synth`` (seeded input generators, no arithmetic of
the method).

Pins (tests/test_oracle_pins.py, run on the CPU): hand-decoded golden blocks,
numpy's own fp16 decoding, brute force on tiny shapes, closed forms and
invariants of RMSNorm, RoPE, attention and the DeltaNet update.  Parity
unpinned: fidelity to a real trained checkpoint (no weights or golden outputs
exist for it).
"""
from . import qref  # noqa: F401
from .model import SliceOracle, DraftHead, mtp_input, rmsnorm, sigmoid, silu, l2normalize, rope, attend, deltanet_update  # noqa: F401
