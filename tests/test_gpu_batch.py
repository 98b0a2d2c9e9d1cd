"""GPU parity of the batch construction (dspark_build_blocks, through the C
ABI) against oracle/batch.py: integer outputs, so bit-exact."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.batch import anchor_candidates, build_blocks as oracle_build_blocks
from speculative_decoding_draft_dspark_amd import build_blocks
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("B,L,N,K,seed", [(4, 300, 20, 7, 1), (1, 9, 5, 4, 2), (3, 1000, 64, 7, 3)])
def test_build_blocks_bit_exact(B, L, N, K, seed):
    rng = np.random.default_rng(seed)
    say(f"[batch] build_blocks B={B} L={L} N={N} K={K}")
    ids = rng.integers(0, 151936, (B, L), dtype=np.int32)
    lm = (rng.random((B, L)) > 0.12).astype(np.uint8)
    lm[:, : L // 10] = 0                      # a prompt region with no loss
    cand = anchor_candidates(lm)
    anchors = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        pool = np.flatnonzero(cand[b])
        anchors[b] = rng.choice(pool, N) if len(pool) else 0
    # invalid anchors: negative, last position, past the end, outside the mask
    anchors[0, 0] = -1
    anchors[0, 1 % N] = L - 1
    anchors[-1, -1] = L + 5
    anchors[-1, 0] = 0
    out = build_blocks(torch.from_numpy(ids).to(DEV), torch.from_numpy(lm).to(DEV),
                       torch.from_numpy(anchors).to(DEV), K, with_candidates=True)
    torch.cuda.synchronize()
    t, p, e, keep = oracle_build_blocks(ids, lm, anchors, K)
    assert np.array_equal(out["target_ids"].cpu().numpy(), t)
    assert np.array_equal(out["prev_ids"].cpu().numpy(), p)
    assert np.array_equal(out["eval_mask"].cpu().numpy(), e)
    assert np.array_equal(out["block_keep"].cpu().numpy(), keep)
    assert np.array_equal(out["anchor_ok"].cpu().numpy(), cand)
