"""A sequence's decode results do not depend on the batch around it: the
same seeded sequence decoded alone, inside a batch of 4 and inside a batch of
32 (at different slots, next to other sequences) gives bitwise-equal top-k
lists, outputs and log-sum-exps.  The split of a sequence's entries over
work items depends on its own entry count only.  ("百万令牌的智慧觉醒" page,
§ on the infrastructure: batch-invariant, deterministic kernels.)"""
import dataclasses

import pytest
import torch

from compressed_sparse_amd import path, synth

pytestmark = pytest.mark.gpu

SEQ = 5


def batches(B_max):
    """(batch size, slot of SEQ, the batch's sequence ids)."""
    out = [(1, 0, [SEQ])]
    for B, slot in ((4, 2), (B_max, 17)):
        ids = [100 + i for i in range(B)]
        ids[slot] = SEQ
        out.append((B, slot, ids))
    return out


CASES = {
    "csa_fp8": (path.CsaLayer, dataclasses.replace(synth.CSA_DECODE_B32_128K, tokens=32768)),
    "csa_mxfp4": (path.CsaLayer, dataclasses.replace(synth.PAIR_CSA_DECODE_B4_1M, tokens=32768)),
    "hca": (path.HcaLayer, dataclasses.replace(synth.HCA_DECODE_B16_1M, tokens=131072)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_decode_is_batch_invariant(case):
    cls, w = CASES[case]
    cap = w.tokens // w.m + 4    # the same descriptor for every batch
    got = []
    for B, slot, ids in batches(32):
        print(f"{case}: B={B} slot {slot}", flush=True)
        lay = cls(w, B, cap, seq_ids=ids)
        lay.prefill_context(w.tokens)
        out = lay.alloc_decode_outputs()
        # CSA: four steps, the last completes entry tokens/4
        for s in range(4 if w.m == 4 else 1):
            x = lay.decode_inputs([w.tokens + s] * B)
            lay.decode_step(x, out)
        torch.cuda.synchronize()
        got.append({k: v[slot].clone() for k, v in out.items()})
        del lay, out
        torch.cuda.empty_cache()
    for g in got[1:]:
        for k in got[0]:
            assert torch.equal(g[k], got[0][k]), f"{case}: {k} differs between batch sizes"
