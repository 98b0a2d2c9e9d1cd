"""FP64/integer CPU oracle of the DSpark batch construction (the step before
the loss): per sampled anchor, the block's labels, previous-token ids and
supervision mask.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: TorchSpec pull request #132, PR description (its list of the pieces
specific to DSpark: each slot is labelled by the token one past it and all
slots of a block are supervised; the eval mask is a running product, so it is
a prefix; the Markov head's previous-token input starts from the anchor; an
anchor is drawn only where both it and its first label are valid) and the
review thread on the label offsets (slot j is labelled by the offset j + 1
from the anchor).

Readings where the pages are silent:
  R22 "valid" for a position is the loss mask: an anchor a may be sampled
      when loss_mask[a] and loss_mask[a + 1] are both nonzero and a + 1 lies
      in the sequence; anchors come from the caller's sampler (random draws
      are inputs), an invalid or out-of-range anchor drops its block.
  R23 the previous-token id of slot j is the token at a + j (slot 0: the
      anchor itself, slot j > 0: slot j - 1's label); labels and previous
      tokens past the end of the sequence are id 0, the slot unsupervised.
  R24 the emitted eval mask is already the contiguous prefix (cumprod of the
      loss mask at the label positions); a dropped block emits zeros.
"""

from __future__ import annotations

import numpy as np


def anchor_candidates(loss_mask: np.ndarray) -> np.ndarray:
    """[B, L] uint8: 1 where an anchor may be sampled (R22)."""
    lm = np.asarray(loss_mask) != 0
    B, L = lm.shape
    ok = np.zeros((B, L), dtype=np.uint8)
    for b in range(B):
        for a in range(L - 1):
            ok[b, a] = 1 if (lm[b, a] and lm[b, a + 1]) else 0
    return ok


def build_blocks(input_ids: np.ndarray, loss_mask: np.ndarray, anchors: np.ndarray,
                 block_size: int):
    """Rows r = (b N + n) K + k of the loss for anchors [B, N].

    Returns (target_ids [R] int32, prev_ids [R] int32, eval_mask [R] uint8,
    block_keep [B N] uint8), written slot by slot from the definitions above.
    """
    ids = np.asarray(input_ids)
    lm = np.asarray(loss_mask) != 0
    anc = np.asarray(anchors)
    B, L = ids.shape
    N = anc.shape[1]
    K = block_size
    R = B * N * K
    target = np.zeros(R, dtype=np.int32)
    prev = np.zeros(R, dtype=np.int32)
    evalm = np.zeros(R, dtype=np.uint8)
    keep = np.zeros(B * N, dtype=np.uint8)
    for b in range(B):
        for n in range(N):
            a = int(anc[b, n])
            ok = 0 <= a and a + 1 < L and lm[b, a] and lm[b, a + 1]
            keep[b * N + n] = 1 if ok else 0
            if not ok:
                continue
            run = 1
            for k in range(K):
                r = (b * N + n) * K + k
                pos = a + k + 1                      # slot k predicts anchor + k + 1
                # previous token, starting from the anchor (0 past the end, R23)
                prev[r] = ids[b, a + k] if a + k < L else 0
                if pos < L:
                    target[r] = ids[b, pos]
                    run = run * (1 if lm[b, pos] else 0)
                else:
                    run = 0
                evalm[r] = run                       # contiguous supervised prefix
    return target, prev, evalm, keep
