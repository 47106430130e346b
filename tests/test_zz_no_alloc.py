"""The LM head + confidence without a workspace argument (library-owned scratch)
against the call that takes a workspace: same kernels, so top ids, probabilities and
logits must be bitwise equal. Two calls in a row, the second with a smaller input, so
the scratch array is reused with stale partials from the first call in it."""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import synth
from tests.gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _both(h, w, fused, logits_in=None):
    status_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    status_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    if logits_in is None:
        la, ia, pa = mars.mars_lmhead_confidence(h, w, fused=fused, status=status_a)
        lb, ib, pb = mars.mars_lmhead_confidence_noalloc(h, w, fused=fused, status=status_b)
    else:
        la, ia, pa = mars.mars_lmhead_confidence(None, None, logits_in, status=status_a)
        lb, ib, pb = mars.mars_lmhead_confidence_noalloc(None, None, logits_in, status=status_b)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib)
    assert torch.equal(pa.view(torch.int32), pb.view(torch.int32))
    if la is not None and logits_in is None:
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
    assert int(status_a.item()) == int(status_b.item()) == 0


@pytest.mark.parametrize("fused", [True, False])
def test_noalloc_lmhead_matches_the_workspace_call_twice(fused):
    # first call: 256 rows x 152064-entry vocabulary (the 7B decode step's LM head)
    say(f"[noalloc] fused={fused}: N=256 D=3584 V=152064, then N=40 D=256 V=5000")
    h, w = synth.lmhead_inputs(1004, 256, 3584, 152064)
    _both(to_dev(h), to_dev(w), fused)
    # second call, smaller: the scratch still holds the first call's partials
    h2, w2 = synth.lmhead_inputs(1005, 40, 256, 5000)
    _both(to_dev(h2), to_dev(w2), fused)


def test_noalloc_confidence_alone_twice():
    say("[noalloc] confidence of given logits: 2048 x 152064, then 16 x 1000")
    pool = synth.PeakedLogitsPool(1005, 2048, 152064, taus=(0.9, 0.6))
    _both(None, None, False, logits_in=to_dev(pool.logits(0)))
    _both(None, None, False, logits_in=to_dev(synth.normal_logits(1001, 16, 1000, 3.0)))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # 4096 rows x 152064 fused needs 4096 x 476 x 16 B > 16 MiB: refused on the host,
    # nothing enqueued (the weights are never read)
    N, D, V = 4096, 64, 152064
    h = torch.zeros((N, D), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((V, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mars.MarsError) as e:
        mars.mars_lmhead_confidence_noalloc(h, w, fused=True)
    assert e.value.code == -6
