"""GPU parity of the vocabulary-sharded loss (dspark_shard_*, through the C
ABI): the draft vocabulary split into G column ranges, every shard run on this
GPU with its own workspace, the exchanges done by stacking and summing.

Checked against (a) the oracle's per-shard protocol (oracle.shard: log-sum-exp
parts, (L1, S, z'_y) parts, per-shard dz, dE and dW2 rows) and (b) the oracle's
unsplit loss and gradients, at the bf16 tolerance 2e-3 (normwise for arrays,
exact token counts and denominators); and (c) against the unsplit GPU path,
which differs from the merged shards only by fp32 summation order: 1e-5 on the
forward terms, 1e-3 normwise on the gradients (a bf16 dz element may land one
rounding step apart).
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import shard as oshard
from speculative_decoding_draft_dspark_amd import DSparkBatch, HParams
from speculative_decoding_draft_dspark_amd.shard import VocabShard, merge_lse, shard_loss
from tests.common import oracle_inputs
from tests.gpu_common import (TOL, assert_grad, assert_norm, assert_scalar, compare_forward, ohp,
                              run_gpu, say, to_np)
from workloads import Workload, get_workload, make_inputs
from workloads.synth import subset_blocks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GS = 0.0125


def _cuts(V, widths):
    cuts = [0]
    for w in widths:
        cuts.append(cuts[-1] + w)
    assert cuts[-1] == V
    return list(zip(cuts[:-1], cuts[1:]))


def _shard_batch(b: DSparkBatch, v0: int, v1: int) -> DSparkBatch:
    """The shard's columns of the vocabulary-indexed inputs; shard-local target ids."""
    cols = lambda t: None if t is None else t[..., v0:v1].contiguous()
    rows = lambda t: None if t is None else t[v0:v1].contiguous()
    return dataclasses.replace(
        b, draft_logits=cols(b.draft_logits), target_ids=(b.target_ids - v0).contiguous(),
        markov_w2=rows(b.markov_w2), lm_head=rows(b.lm_head),
        aligned_target_logits=cols(b.aligned_target_logits))


def _run_shards(d, hp, spans, conf=True, teacher="hidden", grad_dtype=None):
    b = DSparkBatch.from_workload(d, teacher=teacher, conf=conf)
    shards = [VocabShard(_shard_batch(b, v0, v1), hp, grad_dtype) for v0, v1 in spans]
    fwd, per, rep = shard_loss(shards, GS, conf_hidden_grad=conf)
    torch.cuda.synchronize()
    return b, shards, fwd, per, rep


def _check(d, hp, spans, conf=True, teacher="hidden", grad_dtype=None):
    b, shards, fwd, per, rep = _run_shards(d, hp, spans, conf, teacher, grad_dtype)
    inp = oracle_inputs(d, teacher=teacher, conf=conf)
    tol = TOL["bf16"]
    # (a) the oracle's per-shard protocol
    stats = [oshard.shard_stats(inp, v0, v1) for v0, v1 in spans]
    lse_ref = oshard.merge_stats(stats)
    parts = torch.stack([s.fwd_stats() for s in shards])
    lse = merge_lse(parts)
    torch.cuda.synchronize()
    valid = np.isfinite(stats[0][:, 0])
    for g, st in enumerate(stats):
        got = to_np(parts[g])
        assert np.all(np.isneginf(got[~valid])), "unsupervised rows must give -inf"
        ref = st[valid][:, [0, 2]] + np.log(st[valid][:, [1, 3]])
        assert_norm(f"shard {g} lse parts", got[valid], ref, 1e-5)
    assert_norm("merged lse", to_np(lse)[valid], lse_ref[valid], 1e-5)
    terms_ref = [oshard.shard_terms(inp, v0, v1, lse_ref) for v0, v1 in spans]
    S_ref = np.sum([t[:, 1] for t in terms_ref], axis=0)  # the protocol's merged S
    for g, (v0, v1) in enumerate(spans):
        ref = terms_ref[g]
        got = to_np(shards[g].fwd_terms(lse))
        assert not np.any(got[~valid])
        y = inp.target_ids.astype(np.int64)
        owned = valid & (y >= v0) & (y < v1)
        assert np.array_equal(got[:, 3], owned.astype(np.float64)), "owner column"
        for j, k in enumerate(("L1_g", "S_g", "z'_y")):
            if np.any(ref[:, j]):
                assert_norm(f"shard {g} {k}", got[:, j], ref[:, j], tol)
            else:
                assert not np.any(got[:, j]), k
        dz_ref, dE_ref, dW2_ref = oshard.shard_grad(inp, ohp(hp), v0, v1, lse_ref, S_ref, GS)
        assert_grad(f"shard {g} dz", per[g]["d_draft_logits"], dz_ref, tol)
        if inp.has_markov:
            assert_norm(f"shard {g} dE", to_np(per[g]["d_embed"]), dE_ref, tol)
            assert_norm(f"shard {g} dW2", to_np(per[g]["d_markov_w2"]), dW2_ref, tol)
    # (b) the unsplit oracle
    fw = oracle.forward(inp, ohp(hp))
    compare_forward(fwd, fw, tol)
    gr = oracle.backward(inp, ohp(hp), grad_scale=GS)
    dz_t = torch.cat([p["d_draft_logits"] for p in per], dim=1)
    dz = to_np(dz_t)
    assert_grad("dz", dz_t, gr.dz, tol)
    if inp.has_markov:
        assert_norm("dW1", to_np(rep["d_markov_w1"]), gr.dW1, tol)
        dW2 = np.concatenate([to_np(p["d_markov_w2"]) for p in per], axis=0)
        assert_norm("dW2", dW2, gr.dW2, tol)
    if inp.has_conf:
        assert_norm("dW_c", to_np(rep["d_conf_w"]), gr.dW_c, tol)
        assert_scalar("db_c", rep["d_conf_b"].item(), gr.db_c[0], tol)
        assert_norm("dh_d", to_np(rep["d_conf_hidden"]), gr.dh_d, tol)
    # (c) the unsplit GPU path
    _, f1, g1 = run_gpu(d, hp, GS, conf=conf, teacher=teacher, grad_dtype=grad_dtype)
    assert int(f1.num_tokens.item()) == int(fwd.num_tokens.item())
    assert int(fwd.flags.item()) == int(f1.flags.item()) == 0
    assert_scalar("loss vs unsplit", fwd.loss.item(), f1.loss.item(), 1e-5)
    assert_norm("row terms vs unsplit", to_np(fwd.row_terms), to_np(f1.row_terms), 1e-5)
    assert_norm("dz vs unsplit", dz, to_np(g1["d_draft_logits"]), 1e-3)
    if inp.has_markov:
        assert_norm("dW1 vs unsplit", to_np(rep["d_markov_w1"]), to_np(g1["d_markov_w1"]), 1e-3)
        assert_norm("dW2 vs unsplit", dW2, to_np(g1["d_markov_w2"]), 1e-3)
    if inp.has_conf:
        assert_norm("dW_c vs unsplit", to_np(rep["d_conf_w"]), to_np(g1["d_conf_w"]), 1e-3)


@pytest.mark.parametrize("widths", [(8000, 8000, 8000, 8000), (7968, 16032, 8000)],
                         ids=["4-even", "3-uneven"])
def test_vocab_shards_match_oracle_and_unsplit(widths):
    wl = get_workload(1)
    say(f"[shard] {wl.name} widths={widths}")
    d = make_inputs(wl, DEV)
    _check(d, HParams(ce_alpha=0.3, l1_alpha=0.7, confidence_alpha=0.5), _cuts(wl.Vd, widths))


def test_vocab_shards_no_markov_head():
    wl = Workload("shard-nomarkov-v2048", B=1, N=32, K=7, Vd=2048, Vt=2048, H=64, Hd=64, r=8,
                  dtype="bf16", seed=77, recipe="tiny")
    say(f"[shard] {wl.name} no Markov head")
    d = make_inputs(wl, DEV)
    for k in ("prev_ids", "W1", "W2"):
        d.pop(k)
    d["with_markov_conf"] = False
    d["W_c"] = d["W_c"][:, :wl.Hd].contiguous()
    d["eval_mask"][7 * 3 + 2:7 * 4] = 0   # one truncated block
    d["block_keep"][5] = 0                # one dropped block
    _check(d, HParams(), _cuts(wl.Vd, (1024, 512, 512)))


@pytest.mark.parametrize("teacher,grad_dtype", [("aligned", None), ("hidden", torch.float32)],
                         ids=["aligned-teacher", "fp32-grads"])
def test_vocab_shards_teacher_and_grad_variants(teacher, grad_dtype):
    """Teacher logits given directly (sliced per shard), and fp32 dz (the Markov
    products then take G as bf16 hi + lo parts)."""
    wl = get_workload(1)
    say(f"[shard] {wl.name} teacher={teacher} grad_dtype={grad_dtype}")
    d = make_inputs(wl, DEV)
    if teacher == "aligned":
        d["aligned"] = (d["H_t"].float() @ d["LM"].float().T).to(torch.bfloat16).contiguous()
    _check(d, HParams(ce_alpha=0.2, l1_alpha=0.8, confidence_alpha=0.7), _cuts(wl.Vd, (16000, 16000)),
           teacher=teacher, grad_dtype=grad_dtype)


def test_vocab_shards_flag_a_target_no_shard_owns():
    """A supervised row whose global target id lies outside the vocabulary has
    no owner: the finish sets DSPARK_FLAG_TARGET_ID_RANGE, as the unsplit loss
    does for an out-of-range id."""
    wl = get_workload(1)
    say(f"[shard] {wl.name} unowned target")
    d = make_inputs(wl, DEV)
    spans = _cuts(wl.Vd, (16000, 16000))
    hp = HParams()
    _, _, fwd, _, _ = _run_shards(d, hp, spans)
    assert int(fwd.flags.item()) == 0
    m = oracle.effective_mask(d["eval_mask"].cpu().numpy(), d["block_keep"].cpu().numpy(),
                              wl.B, wl.N, wl.K)
    r = int(np.nonzero(m)[0][3])
    d["target_ids"][r] = wl.Vd + 5
    _, _, fwd, _, _ = _run_shards(d, hp, spans)
    assert int(fwd.flags.item()) & 1


@pytest.mark.timeout(900)
@pytest.mark.parametrize("G", [4, 8])
def test_vocab_shards_full_vocabulary(G):
    """G shards of the full 151936-column vocabulary on the Qwen3-8B-shaped
    rows (widths multiples of 32, the last shard the remainder, as one rank of
    a G-way tensor-parallel group would hold): the merged loss, row terms and
    gradients equal the unsplit GPU path, which the full-size oracle test
    checks; on a sample of blocks every shard's log-sum-exp parts,
    (L1, S, z'_y) parts, dz columns and dE rows match the oracle's per-shard
    protocol."""
    wl = get_workload(2)
    say(f"[shard] {wl.name} G={G} full vocabulary")
    d = make_inputs(wl, DEV)
    Vs = wl.Vd // G // 32 * 32
    spans = _cuts(wl.Vd, [Vs] * (G - 1) + [wl.Vd - Vs * (G - 1)])
    hp = HParams()
    b, shards, fwd, per, rep = _run_shards(d, hp, spans)
    # the unsplit GPU path
    _, f1, g1 = run_gpu(d, hp, GS)
    assert int(fwd.flags.item()) == int(f1.flags.item()) == 0
    assert int(f1.num_tokens.item()) == int(fwd.num_tokens.item())
    assert_scalar("loss vs unsplit", fwd.loss.item(), f1.loss.item(), 1e-5)
    assert_norm("row terms vs unsplit", to_np(fwd.row_terms), to_np(f1.row_terms), 1e-5)
    dz = torch.cat([p["d_draft_logits"] for p in per], dim=1)
    assert_norm("dz vs unsplit", to_np(dz), to_np(g1["d_draft_logits"]), 1e-3)
    dW2 = torch.cat([p["d_markov_w2"] for p in per], dim=0)
    assert_norm("dW2 vs unsplit", to_np(dW2), to_np(g1["d_markov_w2"]), 1e-3)
    assert_norm("dW1 vs unsplit", to_np(rep["d_markov_w1"]), to_np(g1["d_markov_w1"]), 1e-3)
    assert_norm("dW_c vs unsplit", to_np(rep["d_conf_w"]), to_np(g1["d_conf_w"]), 1e-3)
    del dz, dW2, g1, f1
    # sampled blocks against the oracle's per-shard protocol
    nb = wl.B * wl.N
    blocks = np.sort(np.random.default_rng(300 + G).choice(nb, size=12, replace=False))
    rows = (blocks[:, None] * wl.K + np.arange(wl.K)[None, :]).reshape(-1)
    inp = oracle_inputs(subset_blocks(d, blocks))
    tol = TOL["bf16"]
    stats = [oshard.shard_stats(inp, v0, v1) for v0, v1 in spans]
    lse_ref = oshard.merge_stats(stats)
    parts = torch.stack([s.fwd_stats() for s in shards])
    lse = merge_lse(parts)
    torch.cuda.synchronize()
    valid = np.isfinite(stats[0][:, 0])
    assert valid.any()
    for g, st in enumerate(stats):
        got = to_np(parts[g])[rows]
        assert np.all(np.isneginf(got[~valid])), "unsupervised rows must give -inf"
        ref = st[valid][:, [0, 2]] + np.log(st[valid][:, [1, 3]])
        assert_norm(f"shard {g} lse parts", got[valid], ref, 1e-5)
    assert_norm("merged lse", to_np(lse)[rows][valid], lse_ref[valid], 1e-5)
    terms_ref = [oshard.shard_terms(inp, v0, v1, lse_ref) for v0, v1 in spans]
    S_ref = np.sum([t[:, 1] for t in terms_ref], axis=0)
    y = inp.target_ids.astype(np.int64)
    for g, (v0, v1) in enumerate(spans):
        got = to_np(shards[g].fwd_terms(lse))[rows]
        owned = valid & (y >= v0) & (y < v1)
        assert np.array_equal(got[:, 3], owned.astype(np.float64)), "owner column"
        for j, k in enumerate(("L1_g", "S_g", "z'_y")):
            if np.any(terms_ref[g][:, j]):
                assert_norm(f"shard {g} {k}", got[:, j], terms_ref[g][:, j], tol)
            else:
                assert not np.any(got[:, j]), k
        dz_ref, dE_ref, _ = oshard.shard_grad(inp, ohp(hp), v0, v1, lse_ref, S_ref, GS)
        assert_grad(f"shard {g} dz", per[g]["d_draft_logits"][torch.as_tensor(rows, device=DEV)],
                    dz_ref, tol)
        assert_norm(f"shard {g} dE", to_np(per[g]["d_embed"])[rows], dE_ref, tol)
