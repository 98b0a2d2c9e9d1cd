"""Python binding of the DSpark loss library: the C-ABI calls under the same names.

PyTorch provides device memory and the current stream; every step of the
loss runs in the HIP kernels of libdspark.so.  The return values follow the
Megatron-Bridge API page ``bridge.training.post_training.dspark.loss``
(``dspark_loss`` return contract: an unnormalised loss numerator, the
supervised token count and a report of [numerator, denominator] pairs).
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import _capi as capi

REPORT_KEYS = ("dspark ce", "dspark l1", "dspark confidence", "dspark accept rate", "dspark tau")


@dataclass
class HParams:
    """``dspark_loss`` keyword arguments (defaults from the API page)."""
    ce_alpha: float = 0.1
    l1_alpha: float = 0.9
    confidence_alpha: float = 1.0
    loss_decay_gamma: Optional[float] = 4.0

    def c(self) -> capi.HParamsC:
        g = self.loss_decay_gamma
        return capi.HParamsC(self.ce_alpha, self.l1_alpha, self.confidence_alpha,
                             0.0 if g is None else float(g))


@dataclass
class DSparkBatch:
    """Device tensors of one loss call; rows are (b, n, k) with the vocab innermost.

    Shapes (R = B*N*K): draft_logits [R, Vd] (or [B, N, K, Vd]), target_ids [R],
    eval_mask [R], block_keep_mask [B*N] or None, prev_ids [R], markov_w1 [Vt, r],
    markov_w2 [Vd, r], target_hidden [R, H], lm_head [Vd, H],
    aligned_target_logits [R, Vd] or None, conf_hidden [R, Hd], conf_w [1, Hd (+ r)],
    conf_b [1].  Float tensors share one dtype (float32 or bfloat16).
    """
    B: int
    N: int
    K: int
    draft_logits: torch.Tensor
    target_ids: torch.Tensor
    eval_mask: torch.Tensor
    block_keep_mask: Optional[torch.Tensor] = None
    prev_ids: Optional[torch.Tensor] = None
    markov_w1: Optional[torch.Tensor] = None
    markov_w2: Optional[torch.Tensor] = None
    target_hidden: Optional[torch.Tensor] = None
    lm_head: Optional[torch.Tensor] = None
    aligned_target_logits: Optional[torch.Tensor] = None
    conf_hidden: Optional[torch.Tensor] = None
    conf_w: Optional[torch.Tensor] = None
    conf_b: Optional[torch.Tensor] = None
    with_markov_conf: bool = True

    @property
    def R(self) -> int:
        return self.B * self.N * self.K

    @classmethod
    def from_workload(cls, d: dict, teacher: str = "hidden", conf: bool = True) -> "DSparkBatch":
        """From a ``workloads.make_inputs`` dict (keys z, target_ids, ..., W_c, b_c)."""
        wl = d["workload"]
        kw = dict(B=wl.B, N=wl.N, K=wl.K, draft_logits=d["z"], target_ids=d["target_ids"],
                  eval_mask=d["eval_mask"], block_keep_mask=d.get("block_keep"),
                  prev_ids=d.get("prev_ids"), markov_w1=d.get("W1"), markov_w2=d.get("W2"),
                  with_markov_conf=bool(d.get("with_markov_conf", True)))
        if teacher == "hidden":
            kw.update(target_hidden=d["H_t"], lm_head=d["LM"])
        elif teacher == "aligned":
            kw.update(aligned_target_logits=d["aligned"])
        if conf and "h_d" in d:
            kw.update(conf_hidden=d["h_d"], conf_w=d["W_c"], conf_b=d["b_c"])
        return cls(**kw)


_DT = {torch.float32: capi.DSPARK_F32, torch.bfloat16: capi.DSPARK_BF16}


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise capi.DSparkError("DSpark tensors must be on the GPU")
    if not t.is_contiguous():
        raise capi.DSparkError("DSpark tensors must be contiguous")
    return t.data_ptr()


def make_shape(b: DSparkBatch, grad_dtype: Optional[torch.dtype] = None,
               options: int = 0) -> capi.Shape:
    z = b.draft_logits
    Vd = z.shape[-1]
    dt = _DT.get(z.dtype)
    if dt is None:
        raise capi.DSparkError(f"unsupported dtype {z.dtype}")
    r = 0 if b.markov_w1 is None else b.markov_w1.shape[1]
    Vt = 0 if b.markov_w1 is None else b.markov_w1.shape[0]
    H = b.lm_head.shape[1] if (b.lm_head is not None and b.target_hidden is not None) else 0
    Hd = 0 if b.conf_hidden is None else b.conf_hidden.shape[-1]
    gd = _DT[grad_dtype] if grad_dtype is not None else dt
    return capi.Shape(b.B, b.N, b.K, Vd, Vt, H, Hd, r, int(b.with_markov_conf and r > 0), dt, gd,
                      options)


def _inputs(b: DSparkBatch) -> capi.InputsC:
    return capi.InputsC(_ptr(b.draft_logits), _ptr(b.target_ids), _ptr(b.eval_mask),
                        _ptr(b.block_keep_mask), _ptr(b.prev_ids), _ptr(b.markov_w1),
                        _ptr(b.markov_w2), _ptr(b.target_hidden), _ptr(b.lm_head),
                        _ptr(b.aligned_target_logits), _ptr(b.conf_hidden), _ptr(b.conf_w),
                        _ptr(b.conf_b))


def _options(store_draft_logits: bool, deterministic: bool = False) -> int:
    return ((capi.OPT_STORE_DRAFT_LOGITS if store_draft_logits else 0)
            | (capi.OPT_DETERMINISTIC if deterministic else 0))


def dspark_workspace_size(b: DSparkBatch, grad_dtype: Optional[torch.dtype] = None,
                          store_draft_logits: bool = False, deterministic: bool = False) -> int:
    sh = make_shape(b, grad_dtype, _options(store_draft_logits, deterministic))
    n = capi.lib().dspark_workspace_size(C.byref(sh))
    if n == 0:
        raise capi.DSparkError("invalid shape for dspark_workspace_size")
    return int(n)


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclass
class FwdResult:
    loss: torch.Tensor           # [1] float64 (unnormalised numerator)
    num_tokens: torch.Tensor     # [1] int64
    pairs: torch.Tensor          # [5, 2] float64
    accept_rate: Optional[torch.Tensor]
    row_terms: Optional[torch.Tensor]   # [R, 4]: ce, l1, bce, confidence logit
    flags: torch.Tensor          # [1] int32 (uint32 bits)
    workspace: torch.Tensor = field(repr=False)
    grad_dtype: Optional[torch.dtype] = None
    options: int = 0

    def report(self) -> dict:
        return {k: self.pairs[i] for i, k in enumerate(REPORT_KEYS)}


def dspark_loss_fwd(b: DSparkBatch, hp: HParams = HParams(), *, workspace=None,
                    grad_dtype: Optional[torch.dtype] = None, row_outputs: bool = True,
                    store_draft_logits: bool = False, deterministic: bool = False,
                    stream=None) -> FwdResult:
    """Forward of the DSpark loss (``dspark_loss_fwd`` of the C ABI).

    ``store_draft_logits`` sets DSPARK_OPT_STORE_DRAFT_LOGITS (materialise the
    fp32 corrected draft logits instead of recomputing the Markov bias);
    ``deterministic`` sets DSPARK_OPT_DETERMINISTIC (the backward's d_markov_w1
    bitwise reproducible); both carry over to ``dspark_loss_bwd``."""
    dev = b.draft_logits.device
    opts = _options(store_draft_logits, deterministic)
    sh = make_shape(b, grad_dtype, opts)
    L = capi.lib()
    need = L.dspark_workspace_size(C.byref(sh))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    ntok = torch.empty(1, dtype=torch.int64, device=dev)
    pairs = torch.empty(5, 2, dtype=torch.float64, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.empty(b.R, dtype=torch.float32, device=dev) if row_outputs else None
    rt = torch.empty(b.R, 4, dtype=torch.float32, device=dev) if row_outputs else None
    out = capi.FwdOutC(_ptr(loss), _ptr(ntok), _ptr(pairs), _ptr(acc), _ptr(rt), _ptr(flags))
    inp = _inputs(b)
    hpc = hp.c()
    st = L.dspark_loss_fwd(C.byref(sh), C.byref(hpc), C.byref(inp), _ptr(workspace),
                           workspace.numel(), C.byref(out), _stream(stream))
    capi.check(st, "dspark_loss_fwd")
    return FwdResult(loss, ntok, pairs, acc, rt, flags, workspace, grad_dtype, opts)


def dspark_loss_bwd(b: DSparkBatch, hp: HParams, fwd: FwdResult, grad_scale: float = 1.0, *,
                    conf_hidden_grad: bool = False, stream=None, out: Optional[dict] = None) -> dict:
    """Backward (``dspark_loss_bwd``): gradients of grad_scale * loss, overwritten."""
    dev = b.draft_logits.device
    sh = make_shape(b, fwd.grad_dtype, fwd.options)
    gdt = fwd.grad_dtype or b.draft_logits.dtype
    f32 = torch.float32
    if out is None:
        out = {"d_draft_logits": torch.empty(b.draft_logits.shape, dtype=gdt, device=dev)}
        if b.markov_w1 is not None:
            out["d_markov_w1"] = torch.empty(b.markov_w1.shape, dtype=f32, device=dev)
            out["d_markov_w2"] = torch.empty(b.markov_w2.shape, dtype=f32, device=dev)
        if b.conf_hidden is not None:
            out["d_conf_w"] = torch.empty(b.conf_w.shape, dtype=f32, device=dev)
            out["d_conf_b"] = torch.empty(1, dtype=f32, device=dev)
            if conf_hidden_grad:
                out["d_conf_hidden"] = torch.empty(b.conf_hidden.shape, dtype=f32, device=dev)
    o = capi.BwdOutC(_ptr(out.get("d_draft_logits")), _ptr(out.get("d_markov_w1")),
                     _ptr(out.get("d_markov_w2")), _ptr(out.get("d_conf_w")),
                     _ptr(out.get("d_conf_b")), _ptr(out.get("d_conf_hidden")))
    inp = _inputs(b)
    hpc = hp.c()
    st = capi.lib().dspark_loss_bwd(C.byref(sh), C.byref(hpc), C.byref(inp), _ptr(fwd.workspace),
                                    fwd.workspace.numel(), float(grad_scale), C.byref(o),
                                    _stream(stream))
    capi.check(st, "dspark_loss_bwd")
    return out


def dspark_accept_report(accept_rate: torch.Tensor, eval_mask: torch.Tensor,
                         block_keep_mask: Optional[torch.Tensor], B: int, N: int, K: int,
                         stream=None) -> torch.Tensor:
    """``dspark_accept_report``: [accept_num, accept_den, tau_num, tau_den] (float64)."""
    out4 = torch.empty(4, dtype=torch.float64, device=accept_rate.device)
    st = capi.lib().dspark_accept_report(B, N, K, _ptr(accept_rate), _ptr(eval_mask),
                                         _ptr(block_keep_mask), _ptr(out4), _stream(stream))
    capi.check(st, "dspark_accept_report")
    return out4


def build_blocks(input_ids: torch.Tensor, loss_mask: torch.Tensor, anchors: torch.Tensor,
                 block_size: int, with_candidates: bool = False, stream=None) -> dict:
    """``dspark_build_blocks``: the loss rows of sampled anchors.

    input_ids [B, L] int32, loss_mask [B, L], anchors [B, N] int32 ->
    {"target_ids", "prev_ids" [B*N*K] int32, "eval_mask" [B*N*K] uint8,
    "block_keep" [B*N] uint8} (+ "anchor_ok" [B, L] uint8 when asked)."""
    B, L = input_ids.shape
    N = anchors.shape[1]
    R = B * N * block_size
    dev = input_ids.device
    ids = input_ids.to(torch.int32).contiguous()
    lm = _u8_mask(loss_mask).contiguous()
    anc = anchors.to(torch.int32).contiguous()
    out = {"target_ids": torch.empty(R, dtype=torch.int32, device=dev),
           "prev_ids": torch.empty(R, dtype=torch.int32, device=dev),
           "eval_mask": torch.empty(R, dtype=torch.uint8, device=dev),
           "block_keep": torch.empty(B * N, dtype=torch.uint8, device=dev)}
    if with_candidates:
        out["anchor_ok"] = torch.empty(B, L, dtype=torch.uint8, device=dev)
    st = capi.lib().dspark_build_blocks(B, L, N, block_size, _ptr(ids), _ptr(lm), _ptr(anc),
                                        _ptr(out["target_ids"]), _ptr(out["prev_ids"]),
                                        _ptr(out["eval_mask"]), _ptr(out["block_keep"]),
                                        _ptr(out.get("anchor_ok")), _stream(stream))
    capi.check(st, "dspark_build_blocks")
    return out


def _u8_mask(m: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if m is None:
        return None
    return m if m.dtype == torch.uint8 else m.to(torch.uint8)


def markov_logits(draft_logits: torch.Tensor, prev_ids: Optional[torch.Tensor] = None,
                  markov_w1: Optional[torch.Tensor] = None,
                  markov_w2: Optional[torch.Tensor] = None,
                  valid_mask: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``dspark_markov_logits``: the Markov head's corrected logits (fp32)
    z + W2 W1[prev] on valid slots, zero rows on the others; no head (W1
    None): z on valid slots."""
    z = draft_logits.reshape(-1, draft_logits.shape[-1])
    rows, V = z.shape
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    Vt = 0 if markov_w1 is None else markov_w1.shape[0]
    dt = _DT[z.dtype]
    mask = _u8_mask(None if valid_mask is None else valid_mask.reshape(-1))
    out = torch.empty(rows, V, dtype=torch.float32, device=z.device)
    nbytes = capi.lib().dspark_markov_logits_workspace_size(rows, V, r, dt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=z.device)
    pid = None if prev_ids is None else prev_ids.reshape(-1)
    st = capi.lib().dspark_markov_logits(rows, V, Vt, r, dt, _ptr(z), _ptr(pid), _ptr(mask),
                                         _ptr(markov_w1), _ptr(markov_w2), _ptr(out), _ptr(ws),
                                         nbytes, _stream(stream))
    capi.check(st, "dspark_markov_logits")
    return out.reshape(*draft_logits.shape[:-1], V)


def confidence_logits(draft_hidden: torch.Tensor, conf_w: torch.Tensor, conf_b: torch.Tensor,
                      prev_ids: Optional[torch.Tensor] = None,
                      markov_w1: Optional[torch.Tensor] = None,
                      valid_mask: Optional[torch.Tensor] = None,
                      with_markov: bool = False, stream=None) -> torch.Tensor:
    """``dspark_confidence_logits``: W_c . [h ; W1[prev]] + b per slot (fp32);
    the embedding is zero on invalid slots and left out unless with_markov."""
    h = draft_hidden.reshape(-1, draft_hidden.shape[-1])
    rows, Hd = h.shape
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    Vt = 0 if markov_w1 is None else markov_w1.shape[0]
    dt = _DT[h.dtype]
    mask = _u8_mask(None if valid_mask is None else valid_mask.reshape(-1))
    out = torch.empty(rows, dtype=torch.float32, device=h.device)
    nbytes = capi.lib().dspark_confidence_logits_workspace_size(rows, r, int(with_markov), dt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=h.device)
    pid = None if prev_ids is None else prev_ids.reshape(-1)
    st = capi.lib().dspark_confidence_logits(rows, Hd, Vt, r, int(with_markov), dt, _ptr(h),
                                             _ptr(pid), _ptr(mask), _ptr(markov_w1),
                                             _ptr(conf_w), _ptr(conf_b), _ptr(out), _ptr(ws),
                                             nbytes, _stream(stream))
    capi.check(st, "dspark_confidence_logits")
    return out.reshape(draft_hidden.shape[:-1])


def confidence_logits_noalloc(draft_hidden: torch.Tensor, conf_w: torch.Tensor,
                              conf_b: torch.Tensor, prev_ids: Optional[torch.Tensor] = None,
                              markov_w1: Optional[torch.Tensor] = None,
                              valid_mask: Optional[torch.Tensor] = None,
                              with_markov: bool = False, out: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """``dspark_confidence_logits_noalloc``: as ``confidence_logits``, with the
    library's per-GPU scratch array in place of a workspace (the library
    allocates nothing; pass ``out`` to allocate nothing here either)."""
    h = draft_hidden.reshape(-1, draft_hidden.shape[-1])
    rows, Hd = h.shape
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    Vt = 0 if markov_w1 is None else markov_w1.shape[0]
    dt = _DT[h.dtype]
    mask = _u8_mask(None if valid_mask is None else valid_mask.reshape(-1))
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=h.device)
    pid = None if prev_ids is None else prev_ids.reshape(-1)
    st = capi.lib().dspark_confidence_logits_noalloc(rows, Hd, Vt, r, int(with_markov), dt,
                                                     _ptr(h), _ptr(pid), _ptr(mask),
                                                     _ptr(markov_w1), _ptr(conf_w), _ptr(conf_b),
                                                     _ptr(out), _stream(stream))
    capi.check(st, "dspark_confidence_logits_noalloc")
    return out.reshape(draft_hidden.shape[:-1])


def dspark_loss(b: DSparkBatch, hp: HParams = HParams(), **kw):
    """The API page's 3-tuple: (loss numerator, num_tokens, {metric: [num, den]})."""
    f = dspark_loss_fwd(b, hp, **kw)
    return f.loss[0], f.num_tokens[0], f.report()
