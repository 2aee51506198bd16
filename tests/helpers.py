"""Shared set-up for the GPU parity tests: one seeded input set feeds both the
HIP slice (through the C ABI) and the CPU oracle."""
from __future__ import annotations

import numpy as np

import synth


def rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, RMS(ref)) (RMS floor keeps near-zero entries meaningful)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


TOL = 2e-3   # max relative error on hidden states (fp32 accumulation)


def make_pair(shape, qtype, begin, end, *, workload, seed=0, max_seq=1024, max_verify=16, io_fp32=True,
              prefill=0, has_embed=False, has_head=False, threads=8, with_oracle=True, centered=False,
              max_prefill=0):
    """Build (gpu Slice, SliceOracle, tensors) with identical weights, states and KV prefix."""
    import torch
    import layer_sliced_quantized_amd as slq
    from oracle import SliceOracle

    tensors = {l: synth.layer_tensors(shape, qtype, seed, workload, l, threads=threads, centered=centered)
               for l in range(begin, end)}
    glob = synth.global_tensors(shape, qtype, seed, workload) if (has_embed or has_head) else {}
    cfg = slq.make_config(shape, qtype, begin, end, max_seq=max_seq, max_verify=max_verify, io_fp32=io_fp32,
                          has_embed=has_embed, has_head=has_head, max_prefill=max_prefill)
    s = slq.Slice(cfg)
    s.load_numpy(tensors, glob)
    orc = SliceOracle(shape, qtype, begin, end, tensors, glob, max_seq=max_seq, io_fp32=io_fp32) if with_oracle else None
    for l in range(begin, end):
        if shape.is_attention(l):
            if prefill:
                K, V = synth.kv_prefill(seed, workload, l, shape.kv_heads, prefill, shape.head_dim)
                s.set_kv(l, torch.from_numpy(K), torch.from_numpy(V))
                if orc:
                    orc.set_kv(l, K, V)
        else:
            S0 = synth.dn_state0(seed, workload, l, shape.dn_heads, shape.dn_dv, shape.dn_dk)
            s.set_state(l, torch.from_numpy(S0))
            if orc:
                orc.set_state(l, S0)
            if getattr(shape, "dn_variant", 0):
                C0 = synth.dn_conv_state0(seed, workload, l, shape.conv_dim, shape.dn_conv)
                s.set_conv_state(l, torch.from_numpy(C0))
                if orc:
                    orc.set_conv_state(l, C0)
    s.reset(prefill)
    if orc:
        orc.reset(prefill)
    torch.cuda.synchronize()
    return s, orc, tensors, glob


def inputs(shape, n, *, workload, seed=0, step0=0, io_fp32=True):
    h = synth.hidden_inputs(seed, workload, n, shape.hidden, step0=step0)
    return h.astype(np.float32) if io_fp32 else h
