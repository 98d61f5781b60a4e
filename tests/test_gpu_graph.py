"""Multi-step decode graphs, as bench.py times them: n consecutive decode
steps captured in one HIP graph that first restores the layers' staging
rings.  Every replay, with eager work and synchronisations between replays,
must reproduce bit for bit the eager run of the same steps from the same
state: every step's outputs (copied out inside the graph) and the caches.
The CSA steps cross two entry completions, the HCA steps (128 of them) one.
"""
import dataclasses

import pytest
import torch

from compressed_sparse_amd import path, synth

pytestmark = pytest.mark.gpu

CASES = {
    "csa_fp8": (path.CsaLayer, dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=2, tokens=8192), 8),
    "csa_mxfp4": (path.CsaLayer, dataclasses.replace(synth.PAIR_CSA_DECODE_B4_1M, batch=2, tokens=8192), 8),
    "hca": (path.HcaLayer, dataclasses.replace(synth.HCA_DECODE_B16_1M, batch=2, tokens=65536), 128),
}


def cache_tensors(lay):
    return [t for c in lay.caches() for t in (c.nope, c.scale, c.rope, c.ring) if t is not None]


@pytest.mark.parametrize("case", list(CASES))
def test_multistep_decode_graph_replays_match_eager(case):
    cls, w, n = CASES[case]
    lay = cls(w, w.batch, w.tokens // w.m + n + 2)
    lay.prefill_context(w.tokens)
    out = lay.alloc_decode_outputs()
    xs = lay.decode_input_steps([[w.tokens + i] * w.batch for i in range(n)])
    hist = [{k: torch.empty_like(v) for k, v in out.items()} for _ in range(n)]

    def step(i):
        lay.decode_step(xs[i], out)
        for k, v in out.items():
            hist[i][k].copy_(v)

    dg = path.DecodeGraph([lay], step, n)   # runs the steps eagerly once, then captures
    torch.cuda.synchronize()
    ref_hist = [{k: v.clone() for k, v in h.items()} for h in hist]
    ref_cache = [t.clone() for t in cache_tensors(lay)]
    for r in range(3):
        for h in hist:  # eager work between replays
            for v in h.values():
                v.zero_()
        torch.cuda.synchronize()
        dg.replay()
        torch.cuda.synchronize()
        for i in range(n):
            for k in out:
                assert torch.equal(hist[i][k], ref_hist[i][k]), f"replay {r}, step {i}: {k} differs"
        for j, (t, rt) in enumerate(zip(cache_tensors(lay), ref_cache)):
            assert torch.equal(t, rt), f"replay {r}: cache tensor {j} differs"
