"""GPU parity of the standalone head ops (dspark_markov_logits,
dspark_confidence_logits, through the C ABI) against the oracle's head
functions: the Markov head's corrected logits z + W2 W1[prev] and the
confidence head's logit W_c . [h ; e] + b on valid slots, zero on invalid
ones (both heads return zero there).

The inputs are rounded to the op's dtype before both sides see them, so the
only differences are the kernels' fp32 accumulation orders: 1e-5 normwise,
and exact zeros on invalid slots.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_draft_dspark_amd import confidence_logits, markov_logits
from tests.common import oracle_inputs
from tests.gpu_common import normwise, run_gpu, say, to_np
from speculative_decoding_draft_dspark_amd import HParams
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
HEAD_TOL = 1e-5


def _rand(shape, std, dtype, g):
    return (torch.randn(shape, generator=g, dtype=torch.float64) * std).to(DT[dtype])


def _f64(t):
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("dtype,rank,masked,R", [
    ("bf16", 64, True, 200), ("bf16", 24, True, 200), ("f32", 32, True, 200),
    ("bf16", 0, True, 200), ("f32", 0, True, 200), ("bf16", 256, True, 600),
    ("bf16", 128, False, 200), ("bf16", 96, True, 200), ("bf16", 32, False, 300)])
def test_markov_logits_parity(dtype, rank, masked, R):
    # rows and vocabulary not multiples of the 256-row workgroups or the
    # 64-column slices (ragged tails); bf16 with rank 0, 32, 64, 128 or 256
    # takes the sweep engine's store pass, bf16 rank 96 the LDS-DMA projection
    # kernel, rank 24 and fp32 the generic one; without a mask every row is valid
    V, Vt = 1000, 777
    g = torch.Generator().manual_seed(11 + rank + R)
    say(f"[heads] markov logits {dtype} R={R} V={V} rank={rank} masked={masked}")
    z = _rand((R, V), 2.0, dtype, g)
    prev = torch.randint(0, Vt, (R,), generator=g, dtype=torch.int32)
    valid = ((torch.rand(R, generator=g) > 0.25) if masked else torch.ones(R, dtype=torch.bool)).to(torch.uint8)
    W1 = _rand((Vt, rank), 0.5, dtype, g) if rank else None
    W2 = _rand((V, rank), 0.5, dtype, g) if rank else None
    out = markov_logits(z.to(DEV), prev.to(DEV), None if W1 is None else W1.to(DEV),
                        None if W2 is None else W2.to(DEV), valid.to(DEV) if masked else None)
    got = to_np(out)
    inp = oracle.Inputs(B=1, N=1, K=R, z=_f64(z), target_ids=np.zeros(R, np.int32),
                        eval_mask=valid.numpy(), prev_ids=prev.numpy(),
                        W1=None if W1 is None else _f64(W1), W2=None if W2 is None else _f64(W2))
    v = valid.numpy().astype(bool)
    ref = oracle.markov_head_logits(inp, valid.numpy())  # zero rows on invalid slots
    err = normwise(got, ref)
    assert err <= HEAD_TOL, f"z' normwise rel err {err:.3e}"
    assert np.all(np.abs(got - ref) <= HEAD_TOL * (1.0 + np.abs(ref)))
    assert not np.any(got[~v])
    if rank == 0:
        assert np.array_equal(got[v], _f64(z)[v])


@pytest.mark.parametrize("dtype,with_markov,masked", [("bf16", True, True), ("bf16", False, True),
                                                      ("f32", True, False), ("f32", False, True)])
def test_confidence_logits_parity(dtype, with_markov, masked):
    R, Hd, r, Vt = 300, 520, 32, 901
    g = torch.Generator().manual_seed(5 + int(with_markov) + 2 * int(masked))
    say(f"[heads] confidence logits {dtype} markov={with_markov} masked={masked}")
    h = _rand((R, Hd), 1.0, dtype, g)
    W1 = _rand((Vt, r), 0.5, dtype, g)
    prev = torch.randint(0, Vt, (R,), generator=g, dtype=torch.int32)
    Wc = _rand((1, Hd + (r if with_markov else 0)), 0.02, dtype, g)
    bc = _rand((1,), 0.5, dtype, g)
    valid = (torch.rand(R, generator=g) > 0.3).to(torch.uint8) if masked else None
    out = confidence_logits(h.to(DEV), Wc.to(DEV), bc.to(DEV), prev.to(DEV), W1.to(DEV),
                            None if valid is None else valid.to(DEV), with_markov=with_markov)
    got = to_np(out)
    v = np.ones(R, bool) if valid is None else valid.numpy().astype(bool)
    inp = oracle.Inputs(B=1, N=1, K=R, z=np.zeros((R, 8)), target_ids=np.zeros(R, np.int32),
                        eval_mask=v.astype(np.uint8), prev_ids=prev.numpy(), W1=_f64(W1),
                        W2=np.zeros((8, r)), h_d=_f64(h), W_c=_f64(Wc), b_c=_f64(bc),
                        with_markov_conf=with_markov)
    ref = oracle.confidence_head_logits(inp, v.astype(np.uint8))  # 0 on invalid slots
    assert not np.any(got[~v])
    err = normwise(got, ref)
    assert err <= HEAD_TOL, f"conf logit normwise rel err {err:.3e}"
    assert np.all(np.abs(got - ref) <= 1e-4 * (1.0 + np.abs(ref)))


def test_confidence_head_matches_the_loss_logits():
    """With the loss's effective mask the head op returns the loss's own
    confidence logits bit for bit (one shared routine; 0 on masked slots)."""
    wl = get_workload(1)
    say(f"[heads] confidence head vs loss on {wl.name}")
    d = make_inputs(wl, DEV)
    b, f, _ = run_gpu(d, HParams(), 1.0, bwd=False)
    inp = oracle_inputs(d)
    m = oracle.effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, inp.K).astype(bool)
    mask = torch.from_numpy(m.astype(np.uint8)).to(DEV)
    c = confidence_logits(d["h_d"], d["W_c"], d["b_c"], d["prev_ids"], d["W1"], mask,
                          with_markov=bool(d.get("with_markov_conf", True)))
    terms = f.row_terms
    assert terms is not None
    assert np.array_equal(c.cpu().numpy(), terms[:, 3].cpu().numpy())


@pytest.mark.timeout(600)
def test_markov_logits_full_size_sampled_rows():
    """The Markov head op at the large-batch shapes (14336 rows, vocabulary
    151936, rank 256, bf16: every row tile and vocabulary range of the sweep
    grid) on sampled rows against the oracle, with a mask; invalid rows exactly
    zero everywhere."""
    wl = get_workload(3)
    R, V, Vt, r = wl.R, wl.Vd, wl.Vt, wl.r
    say(f"[heads] markov logits full size R={R} V={V} rank={r}")
    d = make_inputs(wl, DEV)
    g = torch.Generator().manual_seed(7)
    p = d["prev_ids"].cpu()
    # valid slots hold in-range previous tokens (the loss's masked rows may not)
    valid = ((torch.rand(R, generator=g) > 0.2) & (p >= 0) & (p < Vt)).to(torch.uint8)
    out = markov_logits(d["z"], d["prev_ids"], d["W1"], d["W2"], valid.to(DEV))
    torch.cuda.synchronize()
    v = valid.numpy().astype(bool)
    inval = torch.from_numpy(~v).to(DEV)
    assert not bool(out[inval].any().item())
    # first and last rows of the batch, both sides of each 256-row tile edge,
    # and random rows
    rows = sorted(set([0, 1, R - 1, R - 2, 255, 256, 4095, 4096, 8191, 8192]
                      + torch.randint(0, R, (22,), generator=g).tolist()))
    idx = torch.tensor(rows, dtype=torch.long)
    got = out[idx.to(DEV)].double().cpu().numpy()
    z = d["z"][idx.to(DEV)].double().cpu().numpy()
    prev = d["prev_ids"][idx.to(DEV)].cpu().numpy()
    inp = oracle.Inputs(B=1, N=1, K=len(rows), z=z, target_ids=np.zeros(len(rows), np.int32),
                        eval_mask=valid.numpy()[rows], prev_ids=prev,
                        W1=d["W1"].double().cpu().numpy(), W2=d["W2"].double().cpu().numpy())
    ref = oracle.markov_head_logits(inp, valid.numpy()[rows])
    err = normwise(got, ref)
    assert err <= HEAD_TOL, f"z' normwise rel err {err:.3e} on rows {rows}"
    assert np.all(np.abs(got - ref) <= HEAD_TOL * (1.0 + np.abs(ref)))
