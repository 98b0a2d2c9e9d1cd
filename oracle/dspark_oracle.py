"""FP64 CPU oracle of the DSpark draft-training loss (forward, backward, report).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` call it.  It shares no code with the HIP path.

It is the plain, unchunked definition of what the method computes, written in
float64 with numpy.  Rows are independent (per the API page, splitting the
rows into chunks leaves the result unchanged), so rows are visited in groups
of ``row_chunk`` only to bound host memory; each row is the textbook formula.

Sources (the pages; cited by title and section):
  [API]   Megatron-Bridge API page ``bridge.training.post_training.dspark.loss``
          -- module docstring, ``DSparkForwardOutput``, ``_loss_weight_mask``,
          ``_chunk_terms``, ``_ce_and_l1_per_token``, ``dspark_loss``,
          ``_acceptance_report``.
  [PR5241] Megatron-Bridge pull request #5241 -- closing comment, "Tests" and
          "Merge note" sections of the PR body.
  [TS132] TorchSpec pull request #132 -- PR description (scope list, recipe)
          and "Testing".
  [HEADS] NeMo-RL design doc "DSpark Auxiliary Heads" -- "Inputs and Outputs",
          "Checkpoint Contract".

Readings where the pages are silent (each is repeated where it is used):
  R2  decay index k is the 0-based block slot.
  R3  effective mask m = block_keep * cumprod(eval != 0) over the block.
  R4  masked rows are selected away: CE = L1 = BCE = 0, accept = 1, c = 0.
  R5  every term pair has numerator sum(w * term) and denominator num_tokens.
  R6  the BCE label (accept) is detached.
  R7  confidence input is [draft_hidden ; markov_embedding], in that order.
  R8  tau per kept block = 1 + sum_k prod_{j<=k} (m_j * accept_j); the tau
      denominator is the number of kept blocks.
  R9  sign(0) = 0 in the L1 subgradient.
  R11 draft vocab may differ from target vocab; prev ids index W1 (target
      vocab), logits / L1 live in the draft vocab.
  R13 with no teacher only CE is allowed, and every row's L1 is zero.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F64 = np.float64


@dataclass
class Inputs:
    """Float arrays are float64 copies of the exact (already rounded) values."""
    B: int
    N: int
    K: int
    z: np.ndarray                              # [R, Vd] draft logits
    target_ids: np.ndarray                     # [R] teacher-forced next token
    eval_mask: np.ndarray                      # [R] nonzero = supervised
    block_keep: Optional[np.ndarray] = None    # [B*N] nonzero = kept; None = all
    prev_ids: Optional[np.ndarray] = None      # [R] ids into W1 rows
    W1: Optional[np.ndarray] = None            # [Vt, r]
    W2: Optional[np.ndarray] = None            # [Vd, r]
    H_t: Optional[np.ndarray] = None           # [R, H] target final hidden (post norm)
    LM: Optional[np.ndarray] = None            # [Vd, H] target lm_head rows
    aligned: Optional[np.ndarray] = None       # [R, Vd] teacher logits given directly
    h_d: Optional[np.ndarray] = None           # [R, Hd] confidence-head hidden input
    W_c: Optional[np.ndarray] = None           # [1, Hd (+ r)]
    b_c: Optional[np.ndarray] = None           # [1]
    with_markov_conf: bool = True

    @property
    def R(self) -> int:
        return self.B * self.N * self.K

    @property
    def has_markov(self) -> bool:
        return self.W1 is not None and self.W2 is not None and self.W1.shape[1] > 0

    @property
    def has_teacher(self) -> bool:
        return self.aligned is not None or (self.H_t is not None and self.LM is not None)

    @property
    def has_conf(self) -> bool:
        return self.h_d is not None and self.W_c is not None


@dataclass
class HParams:
    """Defaults of ``dspark_loss`` on the [API] page."""
    ce_alpha: float = 0.1
    l1_alpha: float = 0.9
    confidence_alpha: float = 1.0
    loss_decay_gamma: Optional[float] = 4.0


@dataclass
class Forward:
    m: np.ndarray            # [R] effective mask (int)
    w: np.ndarray            # [R] decay weight on valid rows, 0 elsewhere
    ce: np.ndarray           # [R]
    l1: np.ndarray           # [R] raw L1, no 1/2
    S: np.ndarray            # [R] sum_v p_v sign(p_v - q_v)
    accept: np.ndarray       # [R] clamp(1 - L1/2, 0, 1); 1 on masked rows
    conf_logit: np.ndarray   # [R] 0 on masked rows
    bce: np.ndarray          # [R]
    lse_z: np.ndarray        # [R]
    lse_t: np.ndarray        # [R]
    loss: float
    num_tokens: int
    pairs: dict = field(default_factory=dict)   # name -> (numerator, denominator)


@dataclass
class Grads:
    dz: np.ndarray
    dW1: Optional[np.ndarray]
    dW2: Optional[np.ndarray]
    dW_c: Optional[np.ndarray]
    db_c: Optional[np.ndarray]
    dh_d: Optional[np.ndarray]


# --------------------------------------------------------------------------- masks

def effective_mask(eval_mask, block_keep, B, N, K) -> np.ndarray:
    """Supervision mask of each slot: a contiguous, loss-enabled prefix.

    [API] ``DSparkForwardOutput.eval_mask``: the supervised slots of a block
    form a prefix (contiguous, inside the sequence, loss-enabled); [TS132]
    scope list: that prefix is built with a cumulative product.  Reading R3: the kept-anchor mask
    (``block_keep_mask``) multiplies the whole block; a float mask counts as
    supervised where it is nonzero ([API]: "Bool/float").
    """
    ev = (np.asarray(eval_mask).reshape(B, N, K) != 0).astype(np.int64)
    m = np.cumprod(ev, axis=2)
    if block_keep is not None:
        m = m * (np.asarray(block_keep).reshape(B, N, 1) != 0).astype(np.int64)
    return m.reshape(-1)


def decay_weights(K: int, gamma: Optional[float]) -> np.ndarray:
    """Per-slot weight exp(-k / gamma); gamma None (or <= 0) disables decay.

    [API] module docstring (slot k of a block carries the weight
    exp(-k / loss_decay_gamma)) and ``_loss_weight_mask``.  Reading R2: k is
    the 0-based slot; slot 0 predicts the token right after the anchor ([TS132]).
    """
    k = np.arange(K, dtype=F64)
    if gamma is None or gamma <= 0:
        return np.ones(K, dtype=F64)
    return np.exp(-k / F64(gamma))


# --------------------------------------------------------------------------- pieces

def markov_embedding(inp: Inputs, rows: np.ndarray) -> np.ndarray:
    """e_r = W1[prev_r]: the Markov head's previous-token embedding.

    [HEADS] "Inputs and Outputs" and "Checkpoint Contract": W1 is
    ``markov_w1.weight [target_vocab, rank]``, indexed by previous-token ids of
    the target vocabulary.  Only called for valid rows.
    """
    if not inp.has_markov:
        return np.zeros((len(rows), 0), dtype=F64)
    return inp.W1[inp.prev_ids[rows].astype(np.int64)].astype(F64)


def draft_logits_corrected(inp: Inputs, rows: np.ndarray, e: np.ndarray) -> np.ndarray:
    """z' = z + W2 e: base logits plus the low-rank previous-token bias.

    [HEADS] "Inputs and Outputs" (on a valid slot the head returns the base
    logits plus a low-rank bias computed from the previous token); [TS132] "Testing" (Markov bias ==
    W2(W1[prev])).  W2 is ``markov_w2.weight [draft_vocab, rank]``.
    """
    z = inp.z[rows].astype(F64)
    if inp.has_markov:
        z = z + e @ inp.W2.astype(F64).T
    return z


def teacher_logits(inp: Inputs, rows: np.ndarray) -> np.ndarray:
    """Target next-token logits: lm_head applied to the target's final hidden.

    [TS132] scope list (the L1 teacher is the target model's LM head on that
    model's last hidden state); [API] ``aligned_target_logits`` (the teacher may
    also be given directly).
    """
    if inp.aligned is not None:
        return inp.aligned[rows].astype(F64)
    return inp.H_t[rows].astype(F64) @ inp.LM.astype(F64).T


def log_softmax_rows(x: np.ndarray) -> np.ndarray:
    """Row-wise log-softmax, max-shifted (the textbook definition)."""
    mx = np.max(x, axis=1, keepdims=True)
    s = np.sum(np.exp(x - mx), axis=1, keepdims=True)
    return x - (mx + np.log(s))


def bce_with_logits(c: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Binary cross-entropy of logit c against label y in [0, 1].

    -[y log sigma(c) + (1-y) log(1 - sigma(c))] in its overflow-free form
    max(c, 0) - c y + log(1 + exp(-|c|)).
    """
    return np.maximum(c, 0.0) - c * y + np.log1p(np.exp(-np.abs(c)))


def sigmoid(c: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * c))


def confidence_logit(inp: Inputs, rows: np.ndarray, e: np.ndarray) -> np.ndarray:
    """One confidence logit per slot: proj([h ; e]) + bias.

    [HEADS] "Inputs and Outputs" (the head reads the hidden state, and with
    with_markov=True also the Markov embedding) and "Checkpoint Contract" (``proj.weight [1, hidden +
    markov_rank]``, ``proj.bias [1]``; ``[1, hidden]`` when with_markov=False).
    Reading R7: the concatenation order is [hidden ; embedding].
    """
    Wc = inp.W_c.astype(F64).reshape(-1)
    Hd = inp.h_d.shape[1]
    c = inp.h_d[rows].astype(F64) @ Wc[:Hd] + F64(inp.b_c.reshape(-1)[0])
    if inp.with_markov_conf and inp.has_markov:
        c = c + e @ Wc[Hd:]
    return c


# --------------------------------------------------------------------------- heads alone

def markov_head_logits(inp: Inputs, valid) -> np.ndarray:
    """The Markov head used on its own: corrected logits per slot.

    [HEADS] "Inputs and Outputs": the head adds the low-rank previous-token
    bias W2 W1[prev] to the base logits of the valid slots, and both auxiliary
    heads output zero for the slots that are not valid.  Reading R21: the
    whole row of an invalid slot is zero.  Without a Markov head (rank 0) a
    valid row is the base logits themselves.  Invalid rows are never read.
    """
    v = np.asarray(valid).reshape(-1) != 0
    out = np.zeros(inp.z.shape, dtype=F64)
    rows = np.nonzero(v)[0]
    if len(rows):
        out[rows] = draft_logits_corrected(inp, rows, markov_embedding(inp, rows))
    return out


def confidence_head_logits(inp: Inputs, valid) -> np.ndarray:
    """The confidence head used on its own: one logit per slot.

    [HEADS] "Inputs and Outputs" (input: the hidden state, with the Markov
    embedding appended when with_markov is set; zero on invalid slots) and
    "Checkpoint Contract" (``proj.weight`` [1, hidden (+ rank)], ``proj.bias``
    [1]).  Invalid rows are never read and give 0.
    """
    v = np.asarray(valid).reshape(-1) != 0
    out = np.zeros(inp.h_d.shape[0], dtype=F64)
    rows = np.nonzero(v)[0]
    if len(rows):
        e = markov_embedding(inp, rows) if (inp.with_markov_conf and inp.has_markov) else None
        out[rows] = confidence_logit(inp, rows, e)
    return out


# --------------------------------------------------------------------------- forward

def _row_terms(inp: Inputs, rows: np.ndarray):
    """Everything the loss needs for a set of valid rows (fp64)."""
    e = markov_embedding(inp, rows)
    zp = draft_logits_corrected(inp, rows, e)
    lz = log_softmax_rows(zp)                                  # [API] _chunk_terms: one log_softmax
    p = np.exp(lz)
    y = inp.target_ids[rows].astype(np.int64)
    ce = -lz[np.arange(len(rows)), y]                          # [API] module docstring: ce
    if inp.has_teacher:
        t = teacher_logits(inp, rows)
        lt = log_softmax_rows(t)
        q = np.exp(lt)
        d = p - q
        l1 = np.sum(np.abs(d), axis=1)                         # raw L1, no 1/2 ([API]; [PR5241])
        s = np.sign(d)                                         # R9: sign(0) = 0
        S = np.sum(p * s, axis=1)
        lse_t = (t - lt)[:, 0]
    else:                                                      # R13: L1 output is zeros
        q = None
        s = np.zeros_like(p)
        l1 = np.zeros(len(rows))
        S = np.zeros(len(rows))
        lse_t = np.zeros(len(rows))
    lse_z = (zp - lz)[:, 0]
    return dict(e=e, p=p, q=q, s=s, S=S, ce=ce, l1=l1, y=y, lse_z=lse_z, lse_t=lse_t)


def forward(inp: Inputs, hp: HParams, row_chunk: int = 64) -> Forward:
    """``dspark_loss`` of the [API] page, with the fused Markov / confidence heads.

    loss      = sum_r w_r (ce_alpha CE_r + l1_alpha L1_r + confidence_alpha BCE_r)
                ([API] module docstring: three terms, each weighted by position;
                defaults 0.1 / 0.9 / 1.0 from the ``dspark_loss`` signature)
    accept_r  = clamp(1 - L1_r / 2, 0, 1)  ([API] docstring; clamp from the
                [PR5241] merge note)
    BCE_r     = BCE(c_r, accept_r), label detached (R6)
    """
    R, K = inp.R, inp.K
    if not inp.has_teacher and (hp.l1_alpha != 0 or inp.has_conf):
        # [API] dspark_loss "Raises": L1 term or confidence head without a teacher.
        raise ValueError("L1 term or confidence head requested without a teacher")
    m = effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, K)
    dec = decay_weights(K, hp.loss_decay_gamma)
    kpos = np.arange(R) % K
    w = np.where(m != 0, dec[kpos], 0.0)

    ce = np.zeros(R); l1 = np.zeros(R); S = np.zeros(R)
    accept = np.ones(R); c = np.zeros(R); bce = np.zeros(R)
    lse_z = np.zeros(R); lse_t = np.zeros(R)
    valid = np.nonzero(m)[0]
    for i in range(0, len(valid), row_chunk):
        rows = valid[i:i + row_chunk]
        t = _row_terms(inp, rows)
        ce[rows] = t["ce"]; l1[rows] = t["l1"]; S[rows] = t["S"]
        lse_z[rows] = t["lse_z"]; lse_t[rows] = t["lse_t"]
        acc = np.clip(1.0 - 0.5 * t["l1"], 0.0, 1.0)
        accept[rows] = acc
        if inp.has_conf:
            cr = confidence_logit(inp, rows, t["e"])
            c[rows] = cr
            bce[rows] = bce_with_logits(cr, acc)

    num_tokens = int(m.sum())
    ce_num = float(np.sum(w * ce))
    l1_num = float(np.sum(w * l1))
    conf_num = float(np.sum(w * bce))
    loss = hp.ce_alpha * ce_num + hp.l1_alpha * l1_num + hp.confidence_alpha * conf_num
    acc_num, acc_den, tau_num, tau_den = accept_report(accept, m, inp.block_keep, inp.B, inp.N, K)
    pairs = {
        "dspark ce": (ce_num, num_tokens),
        "dspark l1": (l1_num, num_tokens),
        "dspark confidence": (conf_num, num_tokens),
        "dspark accept rate": (acc_num, acc_den),
        "dspark tau": (tau_num, tau_den),
    }
    return Forward(m=m, w=w, ce=ce, l1=l1, S=S, accept=accept, conf_logit=c, bce=bce,
                   lse_z=lse_z, lse_t=lse_t, loss=float(loss), num_tokens=num_tokens, pairs=pairs)


def accept_report(accept, eval_mask, block_keep, B, N, K):
    """Analytical acceptance diagnostics as [numerator, denominator] pairs.

    [API] ``_acceptance_report``: accept_rate is the probability that each
    slot's token is accepted; a draft token is kept only when all earlier
    tokens of its block are accepted, so per kept block tau counts the
    verified anchor plus the cumulative products of the acceptances along the
    block.  Reading R8: masked slots stop the product; the tau pair is summed
    over kept blocks and counts kept blocks.
    Returns (accept_num, accept_den, tau_num, tau_den).
    """
    m = effective_mask(eval_mask, block_keep, B, N, K).reshape(B, N, K)
    a = np.where(m != 0, np.asarray(accept, dtype=F64).reshape(B, N, K), 0.0)
    acc_num = float(np.sum(a))
    acc_den = int(m.sum())
    run = np.cumprod(a, axis=2)
    tau = 1.0 + np.sum(run, axis=2)                         # [B, N]
    keep = np.ones((B, N)) if block_keep is None else (np.asarray(block_keep).reshape(B, N) != 0)
    tau_num = float(np.sum(np.where(keep, tau, 0.0)))
    tau_den = int(np.sum(keep))
    return acc_num, acc_den, tau_num, tau_den


# --------------------------------------------------------------------------- backward

def _round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (round to nearest even), back in float64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def backward(inp: Inputs, hp: HParams, grad_scale: float = 1.0, row_chunk: int = 64,
             g_bf16: bool = False) -> Grads:
    """Gradient of ``loss`` (upstream gradient ``grad_scale``) by hand.

    dCE/dz'_u  = p_u - [u = y]
    dL1/dz'_u  = p_u (s_u - sum_v p_v s_v),  s = sign(p - q)   (q is detached:
                 [API] ``_ce_and_l1_per_token`` receives the teacher detached)
    dBCE/dc    = sigmoid(c) - accept  (label detached, R6)
    z' = z + W2 e, e = W1[prev], c = W_c [h ; e] + b_c  (chain rule).

    ``g_bf16``: the Markov weight products dE = G W2 and dW2 = G^T e take G
    rounded to bf16 (round to nearest even), as a bf16 autograd of the loss
    would when the logit gradient is stored in bf16 (reading R19); dz itself
    stays exact.
    """
    R, K = inp.R, inp.K
    m = effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, K)
    dec = decay_weights(K, hp.loss_decay_gamma)
    kpos = np.arange(R) % K
    g = F64(grad_scale)

    dz = np.zeros(inp.z.shape, dtype=F64)
    dW1 = np.zeros(inp.W1.shape, dtype=F64) if inp.has_markov else None
    dW2 = np.zeros(inp.W2.shape, dtype=F64) if inp.has_markov else None
    dW_c = np.zeros(inp.W_c.shape, dtype=F64) if inp.has_conf else None
    db_c = np.zeros(inp.b_c.shape, dtype=F64) if inp.has_conf else None
    dh_d = np.zeros(inp.h_d.shape, dtype=F64) if inp.has_conf else None
    Hd = inp.h_d.shape[1] if inp.has_conf else 0

    valid = np.nonzero(m)[0]
    for i in range(0, len(valid), row_chunk):
        rows = valid[i:i + row_chunk]
        t = _row_terms(inp, rows)
        wr = dec[kpos[rows]]
        p, s, S = t["p"], t["s"], t["S"]
        onehot = np.zeros_like(p)
        onehot[np.arange(len(rows)), t["y"]] = 1.0
        G = (g * wr)[:, None] * (hp.ce_alpha * (p - onehot) + hp.l1_alpha * p * (s - S[:, None]))
        dz[rows] = G
        dE = np.zeros_like(t["e"])
        if inp.has_markov:
            Gm = _round_bf16(G) if g_bf16 else G
            dE = Gm @ inp.W2.astype(F64)
            dW2 += Gm.T @ t["e"]
        if inp.has_conf:
            acc = np.clip(1.0 - 0.5 * t["l1"], 0.0, 1.0)
            cr = confidence_logit(inp, rows, t["e"])
            dc = g * wr * hp.confidence_alpha * (sigmoid(cr) - acc)
            Wc = inp.W_c.astype(F64).reshape(-1)
            hd = inp.h_d[rows].astype(F64)
            dW_c[0, :Hd] += dc @ hd
            db_c[0] += np.sum(dc)
            dh_d[rows] = dc[:, None] * Wc[None, :Hd]
            if inp.with_markov_conf and inp.has_markov:
                dW_c[0, Hd:] += dc @ t["e"]
                dE = dE + dc[:, None] * Wc[None, Hd:]
        if inp.has_markov:
            np.add.at(dW1, inp.prev_ids[rows].astype(np.int64), dE)
    return Grads(dz=dz, dW1=dW1, dW2=dW2, dW_c=dW_c, db_c=db_c, dh_d=dh_d)


# --------------------------------------------------------------------------- rows only

def forward_rows(inp: Inputs, hp: HParams, rows: np.ndarray) -> dict:
    """Per-row terms of ``forward`` for a subset of rows (rows are independent).

    Used to check outputs at sizes where the full oracle is too slow: each
    returned row equals the corresponding row of ``forward``.
    """
    R, K = inp.R, inp.K
    m = effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, K)
    dec = decay_weights(K, hp.loss_decay_gamma)
    rows = np.asarray(rows, dtype=np.int64)
    out = {k: np.zeros(len(rows)) for k in ("ce", "l1", "S", "bce", "conf_logit", "lse_z", "lse_t")}
    out["accept"] = np.ones(len(rows))
    out["w"] = np.where(m[rows] != 0, dec[rows % K], 0.0)
    out["m"] = m[rows]
    sel = np.nonzero(m[rows])[0]
    if len(sel):
        vr = rows[sel]
        t = _row_terms(inp, vr)
        for k in ("ce", "l1", "S", "lse_z", "lse_t"):
            out[k][sel] = t[k]
        acc = np.clip(1.0 - 0.5 * t["l1"], 0.0, 1.0)
        out["accept"][sel] = acc
        if inp.has_conf:
            cr = confidence_logit(inp, vr, t["e"])
            out["conf_logit"][sel] = cr
            out["bce"][sel] = bce_with_logits(cr, acc)
    return out


def grad_rows(inp: Inputs, hp: HParams, rows: np.ndarray, grad_scale: float = 1.0) -> np.ndarray:
    """dz of ``backward`` restricted to ``rows`` (row r of dz depends on row r only)."""
    R, K = inp.R, inp.K
    m = effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, K)
    dec = decay_weights(K, hp.loss_decay_gamma)
    rows = np.asarray(rows, dtype=np.int64)
    dz = np.zeros((len(rows), inp.z.shape[1]))
    sel = np.nonzero(m[rows])[0]
    if len(sel):
        vr = rows[sel]
        t = _row_terms(inp, vr)
        p, s, S = t["p"], t["s"], t["S"]
        onehot = np.zeros_like(p)
        onehot[np.arange(len(vr)), t["y"]] = 1.0
        wr = dec[vr % K]
        dz[sel] = (grad_scale * wr)[:, None] * (hp.ce_alpha * (p - onehot)
                                                + hp.l1_alpha * p * (s - S[:, None]))
    return dz
