"""Helpers for the GPU parity tests: run the HIP path and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import HParams as OHP
from speculative_decoding_draft_dspark_amd import (DSparkBatch, HParams, dspark_loss_bwd,
                                                   dspark_loss_fwd)

TOL = {"f32": 1e-4, "bf16": 2e-3}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(d: dict, hp: HParams, grad_scale: float = 1.0, teacher: str = "hidden",
            conf: bool = True, grad_dtype=None, bwd: bool = True, stored: bool = False):
    b = DSparkBatch.from_workload(d, teacher=teacher, conf=conf)
    f = dspark_loss_fwd(b, hp, grad_dtype=grad_dtype, store_draft_logits=stored)
    g = dspark_loss_bwd(b, hp, f, grad_scale, conf_hidden_grad=conf) if bwd else None
    torch.cuda.synchronize()
    return b, f, g


def ohp(hp: HParams) -> OHP:
    return OHP(hp.ce_alpha, hp.l1_alpha, hp.confidence_alpha, hp.loss_decay_gamma)


def rel(x, ref):
    x = float(x); ref = float(ref)
    return abs(x - ref) / max(abs(ref), 1e-30)


def normwise(x, ref):
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def assert_scalar(name, x, ref, tol):
    e = rel(x, ref)
    assert e <= tol, f"{name}: {x} vs {ref} (rel {e:.3e} > {tol})"


def assert_norm(name, x, ref, tol):
    e = normwise(x, ref)
    assert e <= tol, f"{name}: normwise rel err {e:.3e} > {tol}"


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def assert_grad(name, t: torch.Tensor, ref, tol):
    """A gradient tensor against the fp64 oracle, normwise.

    A gradient stored in bf16 carries two errors: the format's own rounding of
    the exact gradient, and what the kernels add.  The kernels' part is held to
    ``tol`` against the oracle rounded to bf16 the same way; the error against
    the fp64 oracle is held to ``tol`` too, except where the rounding alone
    exceeds it (a few dominant elements per row, the target columns, can put
    it near bf16's relative step of 2^-8), and then to that rounding + 10 %.
    """
    x = to_np(t)
    if t.dtype != torch.bfloat16:
        assert_norm(name, x, ref, tol)
        return
    ref = np.asarray(ref, dtype=np.float64)
    ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    e16, efmt, e64 = normwise(x, ref16), normwise(ref16, ref), normwise(x, ref)
    assert e16 <= tol, f"{name}: normwise rel err {e16:.3e} against bf16(oracle) > {tol}"
    bound = max(tol, 1.1 * efmt)
    assert e64 <= bound, (f"{name}: normwise rel err {e64:.3e} > {bound:.3e} (bf16 rounding of "
                          f"the exact gradient alone: {efmt:.3e})")


def compare_forward(f, fw_ref: oracle.Forward, tol, rows=None):
    """Scalars, pairs (denominators exact) and per-row terms against the oracle."""
    assert int(f.num_tokens.item()) == fw_ref.num_tokens
    assert_scalar("loss", f.loss.item(), fw_ref.loss, tol)
    pairs = f.pairs.cpu().numpy()
    for i, k in enumerate(("dspark ce", "dspark l1", "dspark confidence", "dspark accept rate",
                           "dspark tau")):
        num, den = fw_ref.pairs[k]
        assert pairs[i, 1] == den, f"{k} denominator {pairs[i, 1]} != {den}"
        if abs(num) > 0:
            assert_scalar(k, pairs[i, 0], num, tol)
        else:
            assert abs(pairs[i, 0]) <= 1e-30
    rt = to_np(f.row_terms)
    acc = to_np(f.accept_rate)
    for j, (k, ref) in enumerate((("ce", fw_ref.ce), ("l1", fw_ref.l1), ("bce", fw_ref.bce),
                                  ("conf", fw_ref.conf_logit))):
        if np.any(ref):
            assert_norm("row " + k, rt[:, j], ref, tol)
        else:
            assert not np.any(rt[:, j]), k
    assert_norm("accept_rate", acc, fw_ref.accept, tol)
