"""Vocabulary-sharded (tensor-parallel) DSpark loss: thin binding of the
``dspark_shard_*`` entry points.

Each shard holds columns [v0, v0 + Vs) of the draft logits, teacher and W2
and shard-local target ids; the row partials it returns merge exactly into
the unsplit loss (the log-sum-exp of a softmax is the log-sum-exp of its
parts' log-sum-exps, and L1, S and z'_y are sums over columns).  Between the
steps the caller runs the collectives of its tensor-parallel group: gather the
[R, 2] log-sum-exp parts, sum the [R, 4] terms, sum the [R, r] embedding
gradients.  ``shard_loss`` runs every shard of a group in one process with
those collectives done by stacking and summing tensors.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional

import torch

from . import _capi as capi
from .loss import (DSparkBatch, FwdResult, HParams, _inputs, _ptr, _stream, make_shape)


class VocabShard:
    """One shard's workspace and the five steps of a sharded loss call."""

    def __init__(self, b: DSparkBatch, hp: HParams = HParams(),
                 grad_dtype: Optional[torch.dtype] = None):
        self.b, self.hp, self.grad_dtype = b, hp, grad_dtype
        self.sh = make_shape(b, grad_dtype, 0)
        n = capi.lib().dspark_workspace_size(C.byref(self.sh))
        if n == 0:
            raise capi.DSparkError("invalid shard shape")
        self.dev = b.draft_logits.device
        self.ws = torch.empty(n, dtype=torch.uint8, device=self.dev)
        self.flags = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self._inp = _inputs(b)
        self._hpc = hp.c()

    def _common(self):
        return (C.byref(self.sh), C.byref(self._hpc), C.byref(self._inp), _ptr(self.ws),
                self.ws.numel())

    def fwd_stats(self, stream=None) -> torch.Tensor:
        """[R, 2] fp32: this shard's log-sum-exp of z' and of T (-inf when unsupervised)."""
        out = torch.empty(self.b.R, 2, dtype=torch.float32, device=self.dev)
        st = capi.lib().dspark_shard_fwd_stats(*self._common(), _ptr(out), _ptr(self.flags),
                                               _stream(stream))
        capi.check(st, "dspark_shard_fwd_stats")
        return out

    def fwd_terms(self, lse: torch.Tensor, stream=None) -> torch.Tensor:
        """[R, 4] fp64 (L1, S, z'_y if owned, 1 if owned) of this shard, given the merged lse."""
        out = torch.empty(self.b.R, 4, dtype=torch.float64, device=self.dev)
        st = capi.lib().dspark_shard_fwd_terms(*self._common(), _ptr(lse), _ptr(out),
                                               _stream(stream))
        capi.check(st, "dspark_shard_fwd_terms")
        return out

    def fwd_finish(self, terms: torch.Tensor, row_outputs: bool = True, stream=None) -> FwdResult:
        dev, R = self.dev, self.b.R
        loss = torch.empty(1, dtype=torch.float64, device=dev)
        ntok = torch.empty(1, dtype=torch.int64, device=dev)
        pairs = torch.empty(5, 2, dtype=torch.float64, device=dev)
        acc = torch.empty(R, dtype=torch.float32, device=dev) if row_outputs else None
        rt = torch.empty(R, 4, dtype=torch.float32, device=dev) if row_outputs else None
        o = capi.FwdOutC(_ptr(loss), _ptr(ntok), _ptr(pairs), _ptr(acc), _ptr(rt),
                         _ptr(self.flags))
        st = capi.lib().dspark_shard_fwd_finish(*self._common(), _ptr(terms), C.byref(o),
                                                _stream(stream))
        capi.check(st, "dspark_shard_fwd_finish")
        return FwdResult(loss, ntok, pairs, acc, rt, self.flags, self.ws, self.grad_dtype, 0)

    def bwd(self, grad_scale: float = 1.0, stream=None) -> dict:
        """This shard's d_draft_logits, d_markov_w2 rows and G . W2 term of dE."""
        b, dev = self.b, self.dev
        gdt = self.grad_dtype or b.draft_logits.dtype
        out = {"d_draft_logits": torch.empty(b.draft_logits.shape, dtype=gdt, device=dev)}
        if b.markov_w1 is not None:
            out["d_markov_w2"] = torch.empty(b.markov_w2.shape, dtype=torch.float32, device=dev)
            out["d_embed"] = torch.empty(b.R, b.markov_w1.shape[1], dtype=torch.float32,
                                         device=dev)
        st = capi.lib().dspark_shard_bwd(*self._common(), float(grad_scale),
                                         _ptr(out["d_draft_logits"]), _ptr(out.get("d_markov_w2")),
                                         _ptr(out.get("d_embed")), _stream(stream))
        capi.check(st, "dspark_shard_bwd")
        return out

    def bwd_finish(self, d_embed: Optional[torch.Tensor], grad_scale: float = 1.0,
                   conf_hidden_grad: bool = False, stream=None) -> dict:
        """The replicated gradients (W1, confidence head) from the summed d_embed."""
        b, dev, f32 = self.b, self.dev, torch.float32
        out = {}
        if b.markov_w1 is not None:
            out["d_markov_w1"] = torch.empty(b.markov_w1.shape, dtype=f32, device=dev)
        if b.conf_hidden is not None:
            out["d_conf_w"] = torch.empty(b.conf_w.shape, dtype=f32, device=dev)
            out["d_conf_b"] = torch.empty(1, dtype=f32, device=dev)
            if conf_hidden_grad:
                out["d_conf_hidden"] = torch.empty(b.conf_hidden.shape, dtype=f32, device=dev)
        o = capi.BwdOutC(None, _ptr(out.get("d_markov_w1")), None, _ptr(out.get("d_conf_w")),
                         _ptr(out.get("d_conf_b")), _ptr(out.get("d_conf_hidden")))
        st = capi.lib().dspark_shard_bwd_finish(*self._common(), float(grad_scale),
                                                _ptr(d_embed), C.byref(o), _stream(stream))
        capi.check(st, "dspark_shard_bwd_finish")
        return out


def merge_lse(parts: torch.Tensor, stream=None) -> torch.Tensor:
    """[R, 2] log-sum-exp over the shards of parts [G, R, 2] (``dspark_shard_merge_lse``)."""
    G, R = parts.shape[0], parts.shape[1]
    out = torch.empty(R, 2, dtype=torch.float32, device=parts.device)
    st = capi.lib().dspark_shard_merge_lse(G, R, _ptr(parts.contiguous()), _ptr(out),
                                           _stream(stream))
    capi.check(st, "dspark_shard_merge_lse")
    return out


def shard_loss(shards: List[VocabShard], grad_scale: Optional[float] = 1.0,
               conf_hidden_grad: bool = False):
    """Forward (and backward unless grad_scale is None) of every shard of one
    group in this process; the collectives are a stack and sums on the device.
    Returns (FwdResult of shard 0, list of per-shard bwd dicts, replicated grads)."""
    lse = merge_lse(torch.stack([s.fwd_stats() for s in shards]))
    terms = torch.stack([s.fwd_terms(lse) for s in shards]).sum(0)
    fwd = [s.fwd_finish(terms) for s in shards][0]
    if grad_scale is None:
        return fwd, None, None
    per = [s.bwd(grad_scale) for s in shards]
    dE = torch.stack([p["d_embed"] for p in per]).sum(0) if "d_embed" in per[0] else None
    rep = shards[0].bwd_finish(dE, grad_scale, conf_hidden_grad)
    return fwd, per, rep
