"""moba_gate_topk_noalloc: the gate with the library's fixed scratch instead of a
workspace, for callers that cannot allocate (MI355X only).

Two calls in a row, the second on a smaller input, must each equal
moba_gate_topk with a workspace bit for bit (indices and scores): the same
kernels run on scratch that keeps the previous call's contents.  A shape whose
workspace exceeds the fixed scratch is rejected before anything is enqueued.
"""

import numpy as np
import pytest
import torch

from csa_inputs import tiny_block_workload
from parity import upload, poisoned

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import context_sparse_attention_amd as csa


def _both(w):
    d = upload(w)
    shape = (w.n_q, w.hq, w.topk + 1)
    ref_idx, ref_score = csa.moba_gate_topk(d["q"], d["k"], d["layout"], w.block_size, w.topk,
                                            return_score=True)
    idx = poisoned(shape, torch.int32)
    score = poisoned(shape, torch.float32)
    csa.moba_gate_topk_noalloc(d["q"], d["k"], d["layout"], w.block_size, w.topk, idx, score)
    torch.cuda.synchronize()
    return ref_idx.cpu(), ref_score.cpu(), idx.cpu(), score.cpu()


def test_noalloc_gate_matches_workspace_gate_on_two_calls():
    big = tiny_block_workload(seed=51, layout="all", lengths=(3000, 1100, 900), hq=8, hkv=2,
                              d=128, block=64, topk=4, dtype="bf16")
    small = tiny_block_workload(seed=52, layout="zigzag", lengths=(1024,), cp=2, rank=1,
                                hq=4, hkv=2, d=64, block=64, topk=2, dtype="bf16")
    for w in (big, small):
        print("[case] noalloc gate", w.q.shape, w.k.shape, flush=True)
        ref_idx, ref_score, idx, score = _both(w)
        assert torch.equal(idx, ref_idx)
        assert torch.equal(score.view(torch.int32), ref_score.view(torch.int32))
        assert (idx >= -1).all()


def test_noalloc_gate_rejects_shapes_beyond_its_scratch():
    # one-token blocks: 4096 blocks x 8 heads x 128 dims of means, beyond 16 MiB
    w = tiny_block_workload(seed=53, layout="contiguous", cp=4, rank=3, lengths=(4096,), hq=8,
                            hkv=8, d=128, block=1, topk=2, dtype="bf16")
    d = upload(w)
    need = csa.lib.moba_gate_topk_workspace_size(d["layout"].c, w.hkv, w.dqk, w.block_size)
    assert need > csa.GATE_SCRATCH_BYTES
    idx = poisoned((w.n_q, w.hq, w.topk + 1), torch.int32)
    with pytest.raises(csa.CsaError) as e:
        csa.moba_gate_topk_noalloc(d["q"], d["k"], d["layout"], w.block_size, w.topk, idx)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (idx.cpu() == -7777).all()  # nothing was enqueued
