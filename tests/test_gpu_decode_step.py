"""The fused CSA decode step (csa_decode_step) gives the same bits as the
four separate decode calls: two layers with the same inputs, one stepped by
the fused entry point and one by the separate ones, over steps that cross
entry completions; outputs and every cache tensor compared after each step."""
import dataclasses

import pytest
import torch

from compressed_sparse_amd import path, synth

pytestmark = pytest.mark.gpu

CASES = {
    "fp8_keys": dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=3, tokens=16384),
    "mxfp4_keys": dataclasses.replace(synth.PAIR_CSA_DECODE_B4_1M, batch=3, tokens=16384),
}


def tensors(lay):
    return [t for c in lay.caches() for t in (c.nope, c.scale, c.rope, c.ring) if t is not None]


@pytest.mark.parametrize("case", list(CASES))
def test_fused_decode_step_equals_separate_calls(case):
    w = CASES[case]
    cap = w.tokens // w.m + 8
    fused = path.CsaLayer(w, w.batch, cap)
    apart = path.CsaLayer(w, w.batch, cap)
    for lay in (fused, apart):
        lay.prefill_context(w.tokens)
    of, oa = fused.alloc_decode_outputs(), apart.alloc_decode_outputs()
    xs = fused.decode_input_steps([[w.tokens + i] * w.batch for i in range(6)])  # entry completed at step 3
    for i, x in enumerate(xs):
        sf = torch.zeros((w.batch, cap), dtype=torch.float32, device="cuda")
        sa = torch.zeros_like(sf)
        fused.decode_step(x, of, sf)
        apart.decode_step_separate(x, oa, sa)
        torch.cuda.synchronize()
        for k in of:
            assert torch.equal(of[k], oa[k]), f"step {i}: {k} differs"
        assert torch.equal(sf, sa), f"step {i}: scores differ"
        for j, (a, b) in enumerate(zip(tensors(fused), tensors(apart))):
            assert torch.equal(a, b), f"step {i}: cache tensor {j} differs"
