"""Decode steps captured in a HIP graph (how bench.py times them) give the
eager result on every replay, with eager work and synchronisations between
the replays.  The step is idempotent at a fixed position (the compressor
rewrites the same ring slot and entry), so every replay must reproduce the
eager outputs bit for bit."""
import dataclasses

import pytest
import torch

from compressed_sparse_amd import path, synth

pytestmark = pytest.mark.gpu

CASES = {
    "csa_fp8": (path.CsaLayer, dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=2, tokens=8192)),
    "csa_mxfp4": (path.CsaLayer, dataclasses.replace(synth.PAIR_CSA_DECODE_B4_1M, batch=2, tokens=8192)),
    "hca": (path.HcaLayer, dataclasses.replace(synth.HCA_DECODE_B16_1M, batch=2, tokens=65536)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_decode_graph_replays_match_eager(case):
    cls, w = CASES[case]
    lay = cls(w, w.batch, w.tokens // w.m + 2)
    lay.prefill_context(w.tokens)
    out = lay.alloc_decode_outputs()
    x = lay.decode_inputs([w.tokens] * w.batch)
    lay.decode_step(x, out)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lay.decode_step(x, out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.decode_step(x, out)
    for r in range(3):
        for v in out.values():
            v.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, ref[k]), f"replay {r}: {k} differs"
