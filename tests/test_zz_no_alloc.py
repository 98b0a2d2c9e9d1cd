"""The no-allocation entry point (dspark_confidence_logits_noalloc, through the
C ABI) against the entry point it varies (dspark_confidence_logits with a
caller workspace): the same kernels on the same inputs, so the outputs must be
bitwise equal; both are also checked against the oracle's confidence head.

Two calls in a row on one GPU, the second with fewer rows, share the
library's scratch array; the largest problem that fits the scratch, and one
that does not (DSPARK_ERR_SCRATCH), are covered too.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_draft_dspark_amd import (DSparkError, confidence_logits,
                                                   confidence_logits_noalloc)
from tests.gpu_common import normwise, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
SCRATCH = 16 << 20


def _problem(R, Hd, r, Vt, dtype, seed, masked, with_markov):
    g = torch.Generator().manual_seed(seed)
    dt = DT[dtype]
    h = (torch.randn(R, Hd, generator=g, dtype=torch.float64)).to(dt)
    W1 = (torch.randn(Vt, r, generator=g, dtype=torch.float64) * 0.5).to(dt)
    prev = torch.randint(0, Vt, (R,), generator=g, dtype=torch.int32)
    Wc = (torch.randn(1, Hd + (r if with_markov else 0), generator=g,
                      dtype=torch.float64) * 0.02).to(dt)
    bc = (torch.randn(1, generator=g, dtype=torch.float64) * 0.5).to(dt)
    valid = (torch.rand(R, generator=g) > 0.3).to(torch.uint8) if masked else None
    return h, W1, prev, Wc, bc, valid


def _run_pair(R, Hd, r, Vt, dtype, seed, masked, with_markov):
    h, W1, prev, Wc, bc, valid = _problem(R, Hd, r, Vt, dtype, seed, masked, with_markov)
    args = (h.to(DEV), Wc.to(DEV), bc.to(DEV), prev.to(DEV), W1.to(DEV),
            None if valid is None else valid.to(DEV))
    ref = confidence_logits(*args, with_markov=with_markov)
    got = confidence_logits_noalloc(*args, with_markov=with_markov)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "no-allocation output differs from the workspace entry point"
    v = np.ones(R, bool) if valid is None else valid.numpy().astype(bool)
    inp = oracle.Inputs(B=1, N=1, K=R, z=np.zeros((R, 8)), target_ids=np.zeros(R, np.int32),
                        eval_mask=v.astype(np.uint8), prev_ids=prev.numpy(),
                        W1=W1.double().numpy(), W2=np.zeros((8, r)), h_d=h.double().numpy(),
                        W_c=Wc.double().numpy(), b_c=bc.double().numpy(),
                        with_markov_conf=with_markov)
    o = oracle.confidence_head_logits(inp, v.astype(np.uint8))
    out = got.double().cpu().numpy()
    assert not np.any(out[~v])
    assert normwise(out, o) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_two_calls_second_smaller(dtype):
    say(f"[noalloc] {dtype}: 3000 rows, no mask, then 700 rows, masked")
    _run_pair(3000, 520, 64, 901, dtype, 1, False, True)
    _run_pair(700, 520, 64, 901, dtype, 2, True, True)


def test_noalloc_without_markov_features_and_largest_fit():
    say("[noalloc] hidden-only head; then the largest bf16 rank-256 problem the scratch holds")
    _run_pair(500, 264, 32, 300, "bf16", 3, True, False)
    rows = 32000  # 32000 x 256 x 2 bytes of embeddings + a ones mask fit 16 MiB
    _run_pair(rows, 64, 256, 5000, "bf16", 4, False, True)
    _run_pair(96, 64, 256, 5000, "bf16", 5, True, True)


def test_noalloc_rejects_problems_beyond_the_scratch():
    h, W1, prev, Wc, bc, _ = _problem(40000, 8, 256, 100, "bf16", 6, False, True)
    with pytest.raises(DSparkError, match="ERR_SCRATCH|scratch"):
        confidence_logits_noalloc(h.to(DEV), Wc.to(DEV), bc.to(DEV), prev.to(DEV), W1.to(DEV),
                                  None, with_markov=True)
