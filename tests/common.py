"""Helpers shared by the tests: oracle input construction and small problems."""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from oracle import Inputs, HParams
from workloads import Workload, make_inputs, to_numpy_f64


def oracle_inputs(inp: dict, teacher: str = "hidden", conf: bool = True) -> Inputs:
    """oracle.Inputs from a workloads input dict (float64 copies of the rounded values)."""
    wl = inp["workload"]
    n = to_numpy_f64(inp)
    kw = dict(B=wl.B, N=wl.N, K=wl.K, z=n["z"], target_ids=n["target_ids"],
              eval_mask=n["eval_mask"], block_keep=n.get("block_keep"),
              prev_ids=n.get("prev_ids"), W1=n.get("W1"), W2=n.get("W2"),
              with_markov_conf=bool(inp.get("with_markov_conf", True)))
    if teacher == "hidden":
        kw.update(H_t=n["H_t"], LM=n["LM"])
    elif teacher == "aligned":
        kw.update(aligned=n["aligned"])
    if conf and "h_d" in n:
        kw.update(h_d=n["h_d"], W_c=n["W_c"], b_c=n["b_c"])
    return Inputs(**kw)


def tiny_workload(V=32, H=16, r=8, B=1, N=3, K=7, seed=7, dtype="f32", Vt=None) -> Workload:
    return Workload(f"unit-v{V}", B=B, N=N, K=K, Vd=V, Vt=Vt or V, H=H, Hd=H, r=r,
                    dtype=dtype, seed=seed, recipe="tiny")


def tiny_inputs(V=32, H=16, r=8, B=1, N=3, K=7, seed=7, prefix=None, **kw) -> Inputs:
    """A small float64 problem with moderate logits (no sign ties in practice)."""
    wl = tiny_workload(V=V, H=H, r=r, B=B, N=N, K=K, seed=seed, Vt=kw.pop("Vt", None))
    d = make_inputs(wl, "cpu")
    if prefix is not None:
        d["eval_mask"] = torch.as_tensor(prefix, dtype=torch.uint8).reshape(-1)
    inp = oracle_inputs(d)
    # scale the random fields so that the distributions are neither flat nor saturated
    inp.W1 = inp.W1 * 20.0
    inp.W2 = inp.W2 * 20.0
    inp.LM = inp.LM * 0.3
    inp.W_c = inp.W_c * 20.0
    return inp


def clone_inputs(inp: Inputs, **changes) -> Inputs:
    fields = {f.name: getattr(inp, f.name) for f in dataclasses.fields(inp)}
    for k, v in fields.items():
        if isinstance(v, np.ndarray):
            fields[k] = v.copy()
    fields.update(changes)
    return Inputs(**fields)


DEFAULT_HP = HParams()
