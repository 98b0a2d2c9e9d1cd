"""Seeded synthetic tensors for the DSpark loss workloads.

Every tensor is drawn from ``torch.Generator(device).manual_seed(seed)`` in a
fixed order, in float32, then rounded to the workload dtype (round to nearest
even).  Both sides of every parity test consume the same rounded tensors.

Data synthesis only: where a workload asks for labels drawn from the teacher
distribution, or for draft logits close to the teacher logits, the teacher
field is formed with a plain library matmul and labels are drawn by the
Gumbel-max trick.  Nothing here computes any term of the loss.
"""

from __future__ import annotations

import dataclasses

import torch

from .configs import Workload

_ROW_CHUNK = 1024


def _dt(wl: Workload):
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


class _Draw:
    def __init__(self, wl: Workload, device):
        self.g = torch.Generator(device=device)
        self.g.manual_seed(wl.seed)
        self.device = device
        self.dt = _dt(wl)

    def normal(self, *shape, std=1.0, dtype=None):
        dtype = dtype or self.dt
        rows = shape[0]
        out = torch.empty(*shape, dtype=dtype, device=self.device)
        for r0 in range(0, rows, _ROW_CHUNK):
            r1 = min(rows, r0 + _ROW_CHUNK)
            x = torch.randn(r1 - r0, *shape[1:], generator=self.g, device=self.device,
                            dtype=torch.float32)
            out[r0:r1] = (x * std).to(dtype)
        return out

    def randint(self, lo, hi, shape):
        return torch.randint(lo, hi, shape, generator=self.g, device=self.device,
                             dtype=torch.int64)

    def uniform(self, shape):
        return torch.rand(shape, generator=self.g, device=self.device, dtype=torch.float32)


def _gumbel_labels(d: _Draw, H_t, LM, rows=None):
    """Labels y ~ Categorical(softmax(H_t LM^T)) by argmax(logits + Gumbel noise)."""
    R = H_t.shape[0]
    y = torch.empty(R, dtype=torch.int64, device=d.device)
    LMf = LM.float()
    for r0 in range(0, R, _ROW_CHUNK):
        r1 = min(R, r0 + _ROW_CHUNK)
        t = H_t[r0:r1].float() @ LMf.T
        u = d.uniform(t.shape).clamp_(1e-20, 1.0 - 1e-7)
        y[r0:r1] = torch.argmax(t - torch.log(-torch.log(u)), dim=1)
    return y


def _prefix_eval(B, N, K, lengths, device):
    k = torch.arange(K, device=device).view(1, K)
    return (k < lengths.view(-1, 1)).to(torch.uint8).reshape(B * N * K)


def make_inputs(wl: Workload, device="cpu", with_conf: bool = True) -> dict:
    """All inputs of one workload, on ``device``.

    Keys: z [R,Vd], target_ids [R] int32, eval_mask [R] u8, block_keep [B*N] u8,
    prev_ids [R] int32, W1 [Vt,r], W2 [Vd,r], H_t [R,H], LM [Vd,H], and when
    ``with_conf``: h_d [R,Hd], W_c [1,Hd+r], b_c [1].  Float tensors are in the
    workload dtype.
    """
    d = _Draw(wl, device)
    B, N, K, R = wl.B, wl.N, wl.K, wl.R
    Vd, Vt, H, Hd, r = wl.Vd, wl.Vt, wl.H, wl.Hd, wl.r
    out = {}
    keep = torch.ones(B * N, dtype=torch.uint8, device=device)
    ev = torch.ones(R, dtype=torch.uint8, device=device)

    if wl.recipe == "tiny":
        z = d.normal(R, Vd)
        H_t = d.normal(R, H)
        LM = d.normal(Vd, H)
        W1 = d.normal(Vt, r, std=0.02)
        W2 = d.normal(Vd, r, std=0.02)
        prev = d.randint(0, Vt, (R,))
        y = d.randint(0, Vd, (R,))
    elif wl.recipe == "small":
        z = d.normal(R, Vd, std=2.0)
        H_t = d.normal(R, H)
        LM = d.normal(Vd, H, std=0.02)
        W1 = d.normal(Vt, r, std=0.02)
        W2 = d.normal(Vd, r, std=0.02)
        prev = d.randint(0, Vt, (R,))
        y = d.randint(0, Vd, (R,))
        ev = _prefix_eval(B, N, K, d.randint(1, K + 1, (B * N,)), device)
    elif wl.recipe in ("qwen", "large"):
        H_t = d.normal(R, H)
        LM = d.normal(Vd, H, std=0.02)
        W1 = d.normal(Vt, r, std=0.02)
        W2 = d.normal(Vd, r, std=0.02)
        prev = d.randint(0, Vt, (R,))
        if wl.recipe == "qwen":
            z = d.normal(R, Vd, std=3.0)
            nblk = B * N
            ntrunc = int(round(0.1 * nblk))
            lengths = torch.full((nblk,), K, dtype=torch.int64, device=device)
            which = torch.randperm(nblk, generator=d.g, device=device)[:ntrunc]
            lengths[which] = d.randint(1, K, (ntrunc,))
            ev = _prefix_eval(B, N, K, lengths, device)
        else:
            # draft logits = teacher logits + N(0, 0.5) noise, rounded to bf16
            z = torch.empty(R, Vd, dtype=d.dt, device=device)
            LMf = LM.float()
            for r0 in range(0, R, _ROW_CHUNK):
                r1 = min(R, r0 + _ROW_CHUNK)
                t = H_t[r0:r1].float() @ LMf.T
                noise = torch.randn(t.shape, generator=d.g, device=device, dtype=torch.float32)
                z[r0:r1] = (t + 0.5 * noise).to(d.dt)
            del LMf
        y = _gumbel_labels(d, H_t, LM)
    elif wl.recipe == "edge":
        z, H_t, LM, W1, W2, prev, y, ev, keep = _edge(d, wl)
    else:
        raise ValueError(wl.recipe)

    out.update(z=z, target_ids=y.to(torch.int32), eval_mask=ev, block_keep=keep,
               prev_ids=prev.to(torch.int32), W1=W1, W2=W2, H_t=H_t, LM=LM)
    if with_conf:
        out["h_d"] = d.normal(R, Hd)
        out["W_c"] = d.normal(1, Hd + r, std=0.02)
        out["b_c"] = d.normal(1, std=0.02)
    out["with_markov_conf"] = True
    out["workload"] = wl
    return out


def _edge(d: _Draw, wl: Workload):
    """Edge-distribution workload: four block classes by block index n mod 4.

    (0) near-one-hot: z = N(0,1) + 30 e_jd, H_t = 18 LM[jt]; jd == jt in half
        of these blocks (L1 near 0), jd != jt in the other half (L1 near 2);
    (1) identical: H_t = 64 e_i and z = 64 LM[:, i], so z and the teacher
        logits are bitwise equal, prev id 0 (W1 row 0 is zero, no bias);
    (2) uniform: z = 0, prev 0; H_t = 0 in half (teacher uniform too),
        N(0,1) in the other half;
    (3) invalid: slots 3..6 unsupervised, block (b=0, n=3) not kept; their
        draft logits are NaN / +Inf and their ids are -1.
    """
    B, N, K, R = wl.B, wl.N, wl.K, wl.R
    Vd, Vt, H, r = wl.Vd, wl.Vt, wl.H, wl.r
    dev = d.device
    LM = d.normal(Vd, H, std=0.02)
    W1 = d.normal(Vt, r, std=0.02)
    W1[0].zero_()
    W2 = d.normal(Vd, r, std=0.02)
    z = d.normal(R, Vd, std=3.0)
    H_t = d.normal(R, H)
    prev = d.randint(1, Vt, (R,))
    ev = torch.ones(R, dtype=torch.uint8, device=dev)
    keep = torch.ones(B * N, dtype=torch.uint8, device=dev)
    blk = torch.arange(R, device=dev) // K
    n = blk % N
    b = blk // N
    cls = n % 4
    kk = torch.arange(R, device=dev) % K
    half = ((b + n // 4) % 2) == 0

    # (0) near-one-hot
    jd = d.randint(0, Vd, (R,))
    jt = d.randint(0, Vd, (R,))
    jt = torch.where(half, jd, jt)
    noise = d.normal(R, Vd, std=1.0)
    rows0 = torch.nonzero(cls == 0).flatten()
    z[rows0] = noise[rows0]
    z[rows0, jd[rows0]] = (noise[rows0, jd[rows0]].float() + 30.0).to(z.dtype)
    H_t[rows0] = (18.0 * LM[jt[rows0]].float()).to(H_t.dtype)
    del noise
    # (1) identical
    rows1 = torch.nonzero(cls == 1).flatten()
    col = d.randint(0, H, (R,))
    H_t[rows1] = 0
    H_t[rows1, col[rows1]] = 64.0
    z[rows1] = (64.0 * LM[:, col[rows1]].T.float()).to(z.dtype)
    prev[rows1] = 0
    # (2) uniform
    rows2 = torch.nonzero(cls == 2).flatten()
    z[rows2] = 0
    prev[rows2] = 0
    rows2z = torch.nonzero((cls == 2) & half).flatten()
    H_t[rows2z] = 0
    # (3) invalid slots
    bad = (cls == 3) & (kk >= 3)
    ev[bad] = 0
    keep[0 * N + 3] = 0
    dropped = (b == 0) & (n == 3)
    inval = bad | dropped
    rows3 = torch.nonzero(inval).flatten()
    fill = torch.where(kk[rows3] % 2 == 0, float("nan"), float("inf"))
    z[rows3] = fill.view(-1, 1).to(z.dtype)
    prev[inval] = -1

    y = _gumbel_labels(d, H_t, LM)
    y[inval] = -1
    return z, H_t, LM, W1, W2, prev, y, ev, keep


def subset_blocks(inp: dict, blocks) -> dict:
    """The inputs restricted to whole blocks ``blocks`` (flat b*N+n indices).

    Rows of different blocks are independent, so a subset of whole blocks is
    itself a valid input (batch 1, num_blocks = len(blocks)).
    """
    wl = inp["workload"]
    K = wl.K
    blocks = torch.as_tensor(blocks, dtype=torch.int64)
    rows = (blocks.view(-1, 1) * K + torch.arange(K).view(1, K)).reshape(-1)
    dev = inp["z"].device
    rows_d = rows.to(dev)
    blocks_d = blocks.to(dev)
    out = dict(inp)
    for k in ("z", "target_ids", "eval_mask", "prev_ids", "H_t", "h_d"):
        if k in inp:
            out[k] = inp[k][rows_d].contiguous()
    out["block_keep"] = inp["block_keep"][blocks_d].contiguous()
    out["workload"] = dataclasses.replace(wl, name=wl.name + f"-sub{len(blocks)}", B=1,
                                          N=len(blocks))
    return out


def to_numpy_f64(inp: dict) -> dict:
    """Host float64 / int64 numpy copies of every tensor in ``inp``."""
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            if v.is_floating_point():
                out[k] = v.detach().to("cpu", torch.float64).numpy()
            else:
                out[k] = v.detach().to("cpu", torch.int64).numpy()
        else:
            out[k] = v
    return out

