"""FP64 CPU oracle of the loss split over the draft vocabulary (tensor
parallel), as the exchange-and-merge protocol of the vocabulary-sharded
heads.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: NeMo-RL design doc "DSpark Auxiliary Heads", "Tensor Parallelism": the
projection W2 is sharded over the vocabulary (axis 0) while W1 is
replicated, and where the embeddings enter the projection that is split
over the vocabulary, their contributions are summed over the tensor-parallel
ranks.  The loss over a
vocabulary split needs exactly these exchanges (the plain definitions of
log-sum-exp, L1 and the gradient, taken column range by column range):

  per shard g (columns [v0, v1)):  m_g = max_v z'_v,  l_g = sum_v e^(z'_v - m_g)
                                   (and the same for the teacher logits)
  merge:                           lse = M + log sum_g l_g e^(m_g - M),  M = max_g m_g
  per shard g, given the lse:      L1_g = sum_v |p_v - q_v|,  S_g = sum_v p_v sign(p_v - q_v),
                                   z'_y on the shard that owns the target y (else 0)
  merge:                           L1 = sum_g L1_g,  S = sum_g S_g,  CE = lse_z - sum_g z'_y,g
  per shard g, given S:            G_v for v in [v0, v1) (the target's -ce term on its
                                   owner only); dE_g = G_g W2_g, dW2_g = G_g^T e
  merge:                           dE = sum_g dE_g (+ the confidence term once).

Every function works on the rows of the loss's effective mask; masked rows
contribute nothing (m = -inf, l = 0).
"""

from __future__ import annotations

import numpy as np

from .dspark_oracle import (F64, Inputs, HParams, decay_weights, draft_logits_corrected,
                            effective_mask, markov_embedding, teacher_logits)


def _valid(inp: Inputs) -> np.ndarray:
    return np.nonzero(effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, inp.K))[0]


def _logits(inp: Inputs, rows: np.ndarray):
    e = markov_embedding(inp, rows)
    return e, draft_logits_corrected(inp, rows, e), teacher_logits(inp, rows)


def shard_stats(inp: Inputs, v0: int, v1: int) -> np.ndarray:
    """[R, 4]: (m_z, l_z, m_t, l_t) of the columns [v0, v1) per row."""
    out = np.zeros((inp.R, 4), dtype=F64)
    out[:, 0] = out[:, 2] = -np.inf
    rows = _valid(inp)
    if len(rows) == 0:
        return out
    _, zp, t = _logits(inp, rows)
    for k, x in ((0, zp[:, v0:v1]), (2, t[:, v0:v1])):
        m = np.max(x, axis=1)
        out[rows, k] = m
        out[rows, k + 1] = np.sum(np.exp(x - m[:, None]), axis=1)
    return out


def merge_stats(parts) -> np.ndarray:
    """[R, 2] (lse_z, lse_t) from the shards' [R, 4] statistics."""
    P = np.stack(parts)                                  # [G, R, 4]
    out = np.zeros((P.shape[1], 2), dtype=F64)
    for j, k in ((0, 0), (1, 2)):
        m = P[:, :, k]
        M = np.max(m, axis=0)
        fin = np.isfinite(M)
        Ms = np.where(fin, M, 0.0)
        s = np.sum(P[:, :, k + 1] * np.exp(np.where(np.isfinite(m), m - Ms[None, :], -np.inf)),
                   axis=0)
        out[:, j] = np.where(fin, Ms + np.log(np.where(fin, s, 1.0)), 0.0)
    return out


def shard_terms(inp: Inputs, v0: int, v1: int, lse: np.ndarray) -> np.ndarray:
    """[R, 3]: (L1_g, S_g, z'_y if the shard owns y else 0) given the merged lse."""
    out = np.zeros((inp.R, 3), dtype=F64)
    rows = _valid(inp)
    if len(rows) == 0:
        return out
    _, zp, t = _logits(inp, rows)
    p = np.exp(zp[:, v0:v1] - lse[rows, 0:1])
    q = np.exp(t[:, v0:v1] - lse[rows, 1:2])
    d = p - q
    out[rows, 0] = np.sum(np.abs(d), axis=1)
    out[rows, 1] = np.sum(p * np.sign(d), axis=1)
    y = inp.target_ids[rows].astype(np.int64)
    own = (y >= v0) & (y < v1)
    out[rows[own], 2] = zp[np.nonzero(own)[0], y[own]]
    return out


def shard_grad(inp: Inputs, hp: HParams, v0: int, v1: int, lse: np.ndarray, S: np.ndarray,
               grad_scale: float = 1.0):
    """dz[:, v0:v1] and this shard's dE_g [R, r] and dW2_g [v1 - v0, r] (no
    confidence term), given the merged lse and S."""
    R, K = inp.R, inp.K
    dec = decay_weights(K, hp.loss_decay_gamma)
    kpos = np.arange(R) % K
    dz = np.zeros((R, v1 - v0), dtype=F64)
    r = inp.W1.shape[1] if inp.has_markov else 0
    dE = np.zeros((R, r), dtype=F64)
    dW2 = np.zeros((v1 - v0, r), dtype=F64)
    rows = _valid(inp)
    if len(rows) == 0:
        return dz, dE, dW2
    e, zp, t = _logits(inp, rows)
    p = np.exp(zp[:, v0:v1] - lse[rows, 0:1])
    q = np.exp(t[:, v0:v1] - lse[rows, 1:2])
    s = np.sign(p - q)
    onehot = np.zeros_like(p)
    y = inp.target_ids[rows].astype(np.int64)
    own = (y >= v0) & (y < v1)
    onehot[np.nonzero(own)[0], y[own] - v0] = 1.0
    wr = dec[kpos[rows]]
    G = (F64(grad_scale) * wr)[:, None] * (hp.ce_alpha * (p - onehot) +
                                           hp.l1_alpha * p * (s - S[rows][:, None]))
    dz[rows] = G
    if r:
        dE[rows] = G @ inp.W2[v0:v1].astype(F64)
        dW2 = G.T @ e
    return dz, dE, dW2
