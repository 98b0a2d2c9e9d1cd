"""Pins of the FP64 oracle against what the pages and the mathematics fix.

No GPU.  Each pin is independent of the oracle's own code: printed values,
closed forms, library routines (torch float64), brute force on tiny inputs and
finite differences.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import HParams
from tests.common import clone_inputs, oracle_inputs, tiny_inputs
from workloads import get_workload, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- printed values

def _disjoint_inputs(g, K=7):
    """One block of K slots, every slot a pair of disjoint saturated distributions."""
    V = g["vocab"]
    s = g["saturation_logit"]
    z = np.zeros((K, V)); z[:, g["draft_hot"]] = s
    t = np.zeros((K, V)); t[:, g["teacher_hot"]] = s
    return oracle.Inputs(B=1, N=1, K=K, z=z, target_ids=np.full(K, g["draft_hot"]),
                         eval_mask=np.ones(K), aligned=t)


def test_disjoint_saturated_raw_l1_is_two():
    g = _gold("disjoint_saturated.json")
    inp = _disjoint_inputs(g)
    fw = oracle.forward(inp, HParams())
    assert np.allclose(fw.l1, g["expected"]["raw_l1"], atol=1e-12)
    assert np.allclose(0.5 * fw.l1, g["expected"]["total_variation"], atol=1e-12)
    assert np.allclose(fw.accept, g["expected"]["accept"], atol=1e-12)
    tau_num, tau_den = fw.pairs["dspark tau"]
    assert tau_den == 1 and tau_num == pytest.approx(g["expected"]["tau_first_slot_rejected"])
    # the trained term is the raw L1 at weight 0.9 (not 1.8 x TV, not 0.9 x TV)
    hp = HParams(ce_alpha=0.0, l1_alpha=0.9, confidence_alpha=0.0, loss_decay_gamma=None)
    fw = oracle.forward(inp, hp)
    assert fw.loss == pytest.approx(0.9 * 2.0 * 7, rel=1e-12)


def test_recipe_constants_match_workloads():
    g = _gold("qwen3_8b_recipe.json")
    for idx in (2, 3):
        wl = get_workload(idx)
        assert wl.K == g["block_size"] and wl.gamma == g["loss_decay_gamma"]
        assert wl.r == g["markov_rank"] and wl.Vd == g["vocab_size"] == wl.Vt
    assert HParams().loss_decay_gamma == g["loss_decay_gamma"]


def test_loss_defaults_match_page():
    g = _gold("loss_defaults.json")
    hp = HParams()
    assert (hp.ce_alpha, hp.l1_alpha, hp.confidence_alpha, hp.loss_decay_gamma) == \
        (g["ce_alpha"], g["l1_alpha"], g["confidence_alpha"], g["loss_decay_gamma"])


def test_probability_tensor_size_pins_vocab_layout():
    g = _gold("probability_tensor_size.json")
    V = get_workload(3).Vd
    gib = g["batch"] * g["num_blocks"] * g["block_size"] * V * g["bytes_per_element"] / 2**30
    assert round(gib, 2) == g["gib_printed"]


# ----------------------------------------------------------------- closed forms

def test_identical_distributions_accept_one_tau_k_plus_one():
    inp = tiny_inputs(V=40)
    t = inp.H_t @ inp.LM.T
    e = inp.W1[inp.prev_ids.astype(int)]
    same = clone_inputs(inp, aligned=t.copy(), z=t - e @ inp.W2.T, H_t=None, LM=None)
    fw = oracle.forward(same, HParams())
    assert np.max(np.abs(fw.l1)) < 1e-12
    assert np.allclose(fw.accept, 1.0)
    tau_num, tau_den = fw.pairs["dspark tau"]
    assert tau_num / tau_den == pytest.approx(inp.K + 1, abs=1e-9)


@pytest.mark.parametrize("a,expected", [(0.8, 4.1611392), (0.5, 1.9921875), (0.0, 1.0), (1.0, 8.0)])
def test_tau_constant_accept_geometric_series(a, expected):
    K = 7
    closed = 1.0 + sum(a ** k for k in range(1, K + 1))       # geometric series
    assert closed == pytest.approx(expected, abs=1e-7)
    acc_num, acc_den, tau_num, tau_den = oracle.accept_report(np.full(K, a), np.ones(K), None, 1, 1, K)
    assert tau_den == 1 and tau_num == pytest.approx(closed, abs=1e-12)
    assert acc_den == K and acc_num == pytest.approx(K * a)


def test_decay_weights_properties():
    K, gamma = 7, 4.0
    w = oracle.decay_weights(K, gamma)
    assert w[0] == 1.0
    ratios = w[1:] / w[:-1]
    assert np.allclose(ratios, math.exp(-1.0 / gamma), rtol=1e-15)
    assert w[4] == pytest.approx(1.0 / math.e, rel=1e-15)      # k = gamma
    assert w.sum() == pytest.approx((1 - math.exp(-K / gamma)) / (1 - math.exp(-1 / gamma)), rel=1e-14)
    assert np.all(oracle.decay_weights(K, None) == 1.0)
    assert np.all(oracle.decay_weights(K, 0.0) == 1.0)
    # the weights the loss actually applies: w_k / w_0 = exp(-k / gamma) within each block
    fw = oracle.forward(tiny_inputs(V=16, N=2), HParams(loss_decay_gamma=gamma))
    wb = fw.w.reshape(-1, K)
    assert np.allclose(wb[:, 1:] / wb[:, :-1], math.exp(-1.0 / gamma), rtol=1e-15)


def test_l1_range_and_accept_relation():
    inp = tiny_inputs(V=50, N=4)
    fw = oracle.forward(inp, HParams())
    v = fw.m != 0
    assert np.all(fw.l1[v] >= 0) and np.all(fw.l1[v] <= 2.0)
    assert np.allclose(fw.accept[v], 1 - 0.5 * fw.l1[v])
    assert np.all(np.abs(fw.S[v]) <= 1.0 + 1e-12)


def test_softmax_gradient_rows_sum_to_zero():
    inp = tiny_inputs(V=30)
    gr = oracle.backward(inp, HParams(), grad_scale=0.37)
    assert np.max(np.abs(gr.dz.sum(axis=1))) < 1e-14


def test_loss_decomposition_into_pairs():
    inp = tiny_inputs(V=30, N=4)
    hp = HParams(ce_alpha=0.3, l1_alpha=0.6, confidence_alpha=0.7)
    fw = oracle.forward(inp, hp)
    ce, l1, cf = (fw.pairs[k][0] for k in ("dspark ce", "dspark l1", "dspark confidence"))
    assert fw.loss == pytest.approx(0.3 * ce + 0.6 * l1 + 0.7 * cf, rel=1e-14)
    for k in ("dspark ce", "dspark l1", "dspark confidence"):
        assert fw.pairs[k][1] == fw.num_tokens


# ----------------------------------------------------------------- masks and invariants

def test_cumprod_mask_example():
    # [1,1,0,1,1,1,1] -> [1,1,0,0,0,0,0]: the supervised part is a contiguous prefix
    m = oracle.effective_mask(np.array([1, 1, 0, 1, 1, 1, 1]), None, 1, 1, 7)
    assert m.tolist() == [1, 1, 0, 0, 0, 0, 0]
    m = oracle.effective_mask(np.array([1, 1, 1, 1, 1, 1, 1, 0.5, 0, 0, 0, 0, 0, 0]),
                              np.array([0, 1]), 1, 2, 7)
    assert m.tolist() == [0] * 7 + [1] + [0] * 6


def test_all_masked_gives_zero_loss_and_tokens():
    inp = tiny_inputs(V=20)
    inp = clone_inputs(inp, eval_mask=np.zeros_like(inp.eval_mask))
    fw = oracle.forward(inp, HParams())
    assert fw.loss == 0.0 and fw.num_tokens == 0
    gr = oracle.backward(inp, HParams())
    assert not np.any(gr.dz) and not np.any(gr.dW1) and not np.any(gr.dW2)


def test_garbage_in_masked_rows_changes_nothing():
    prefix = np.array([1, 1, 1, 0, 1, 0, 0] + [1] * 7 + [0] * 7)
    inp = tiny_inputs(V=24, prefix=prefix)
    fw = oracle.forward(inp, HParams())
    gr = oracle.backward(inp, HParams())
    m = fw.m
    bad = clone_inputs(inp)
    bad.z[m == 0] = np.nan
    bad.z[np.nonzero(m == 0)[0][::2]] = np.inf
    bad.prev_ids[m == 0] = -1
    bad.target_ids[m == 0] = -1
    bad.h_d[m == 0] = np.nan
    fw2 = oracle.forward(bad, HParams())
    gr2 = oracle.backward(bad, HParams())
    assert fw2.loss == fw.loss and fw2.pairs == fw.pairs
    assert np.array_equal(gr2.dz, gr.dz) and np.array_equal(gr2.dW1, gr.dW1)
    assert np.array_equal(gr2.dW2, gr.dW2) and np.array_equal(gr2.dW_c, gr.dW_c)
    assert fw2.conf_logit[m == 0].tolist() == [0.0] * int((m == 0).sum())


def test_data_parallel_split_is_additive():
    inp = tiny_inputs(V=24, B=2, N=2)
    hp = HParams()
    fw = oracle.forward(inp, hp)
    gr = oracle.backward(inp, hp, grad_scale=0.5)
    half = inp.R // 2
    parts = []
    for sl, bsl in ((slice(0, half), slice(0, 2)), (slice(half, None), slice(2, None))):
        p = clone_inputs(inp, B=1, z=inp.z[sl], target_ids=inp.target_ids[sl],
                         eval_mask=inp.eval_mask[sl], block_keep=inp.block_keep[bsl],
                         prev_ids=inp.prev_ids[sl], H_t=inp.H_t[sl], h_d=inp.h_d[sl])
        parts.append((oracle.forward(p, hp), oracle.backward(p, hp, grad_scale=0.5)))
    assert fw.loss == pytest.approx(sum(f.loss for f, _ in parts), rel=1e-13)
    assert fw.num_tokens == sum(f.num_tokens for f, _ in parts)
    for k in fw.pairs:
        assert fw.pairs[k][0] == pytest.approx(sum(f.pairs[k][0] for f, _ in parts), rel=1e-13)
        assert fw.pairs[k][1] == sum(f.pairs[k][1] for f, _ in parts)
    assert np.allclose(gr.dW2, sum(g.dW2 for _, g in parts), rtol=1e-12, atol=1e-15)
    assert np.allclose(gr.dW1, sum(g.dW1 for _, g in parts), rtol=1e-12, atol=1e-15)
    assert np.allclose(gr.dW_c, sum(g.dW_c for _, g in parts), rtol=1e-12, atol=1e-15)


def test_row_chunking_does_not_change_result():
    inp = tiny_inputs(V=24, N=4)
    a = oracle.forward(inp, HParams(), row_chunk=1)
    b = oracle.forward(inp, HParams(), row_chunk=1000)
    assert a.loss == pytest.approx(b.loss, rel=1e-14)


def test_teacher_free_mode():
    inp = tiny_inputs(V=24)
    nt = clone_inputs(inp, H_t=None, LM=None, h_d=None, W_c=None, b_c=None)
    with pytest.raises(ValueError):
        oracle.forward(nt, HParams())                       # l1_alpha defaults to 0.9
    fw = oracle.forward(nt, HParams(l1_alpha=0.0))
    assert not np.any(fw.l1)
    with pytest.raises(ValueError):                          # confidence head without teacher
        oracle.forward(clone_inputs(inp, H_t=None, LM=None), HParams(l1_alpha=0.0))


# ----------------------------------------------------------------- library routines

def _t(x):
    return torch.tensor(x, dtype=torch.float64)


def test_ce_bce_l1_bias_against_torch_library():
    inp = tiny_inputs(V=45, N=4)
    fw = oracle.forward(inp, HParams())
    v = np.nonzero(fw.m)[0]
    e = inp.W1[inp.prev_ids[v].astype(int)]
    # Markov bias == W2(W1[prev]) -- TorchSpec #132 "Testing"
    bias = F.linear(_t(e), _t(inp.W2))
    zp = _t(inp.z[v]) + bias
    ce = F.cross_entropy(zp, torch.tensor(inp.target_ids[v].astype(np.int64)), reduction="none")
    assert np.allclose(fw.ce[v], ce.numpy(), rtol=1e-13)
    t = F.linear(_t(inp.H_t[v]), _t(inp.LM))
    l1 = (F.softmax(zp, -1) - F.softmax(t, -1)).abs().sum(-1)
    assert np.allclose(fw.l1[v], l1.numpy(), rtol=1e-12)
    acc = (1 - 0.5 * l1).clamp(0, 1)
    c = F.linear(torch.cat([_t(inp.h_d[v]), _t(e)], 1), _t(inp.W_c), _t(inp.b_c)).squeeze(1)
    assert np.allclose(fw.conf_logit[v], c.numpy(), rtol=1e-12)
    bce = F.binary_cross_entropy_with_logits(c, acc, reduction="none")
    assert np.allclose(fw.bce[v], bce.numpy(), rtol=1e-12)


def test_reduces_to_plain_cross_entropy():
    inp = tiny_inputs(V=33, N=2)
    plain = clone_inputs(inp, W1=None, W2=None, prev_ids=None, h_d=None, W_c=None, b_c=None)
    fw = oracle.forward(plain, HParams(ce_alpha=1.0, l1_alpha=0.0, confidence_alpha=0.0,
                                       loss_decay_gamma=None))
    ref = F.cross_entropy(_t(inp.z), torch.tensor(inp.target_ids.astype(np.int64)), reduction="sum")
    assert fw.loss == pytest.approx(float(ref), rel=1e-13)


class _RoundGradBF16(torch.autograd.Function):
    """Identity forward; the incoming gradient rounded to bfloat16 on the way back."""

    @staticmethod
    def forward(ctx, x):
        return x.view_as(x)

    @staticmethod
    def backward(ctx, g):
        return g.to(torch.bfloat16).to(torch.float64)


def _torch_loss(inp, hp, grad_scale, round_bias_grad=False):
    """The objective assembled from torch float64 library ops, for autograd.
    ``round_bias_grad``: the gradient reaching the Markov bias W2 e is rounded
    to bf16 (what the weight products see when the logit gradient is bf16)."""
    B, N, K = inp.B, inp.N, inp.K
    m = torch.cumprod(torch.tensor(inp.eval_mask != 0, dtype=torch.float64).view(B, N, K), 2)
    if inp.block_keep is not None:
        m = m * torch.tensor(inp.block_keep != 0, dtype=torch.float64).view(B, N, 1)
    m = m.reshape(-1)
    z = _t(inp.z).requires_grad_(); W1 = _t(inp.W1).requires_grad_(); W2 = _t(inp.W2).requires_grad_()
    Wc = _t(inp.W_c).requires_grad_(); bc = _t(inp.b_c).requires_grad_(); hd = _t(inp.h_d).requires_grad_()
    e = W1[torch.tensor(inp.prev_ids.astype(np.int64))]
    bias = F.linear(e, W2)
    zp = z + (_RoundGradBF16.apply(bias) if round_bias_grad else bias)
    tl = F.linear(_t(inp.H_t), _t(inp.LM))
    ce = F.cross_entropy(zp, torch.tensor(inp.target_ids.astype(np.int64)), reduction="none")
    l1 = (F.softmax(zp, -1) - F.softmax(tl, -1)).abs().sum(-1)
    acc = (1 - 0.5 * l1).clamp(0, 1).detach()
    c = F.linear(torch.cat([hd, e], 1), Wc, bc).squeeze(1)
    bce = F.binary_cross_entropy_with_logits(c, acc, reduction="none")
    w = m * torch.exp(-(torch.arange(inp.R) % K).double() / hp.loss_decay_gamma)
    loss = (w * (hp.ce_alpha * ce + hp.l1_alpha * l1 + hp.confidence_alpha * bce)).sum()
    (loss * grad_scale).backward()
    return loss, dict(dz=z.grad, dW1=W1.grad, dW2=W2.grad, dW_c=Wc.grad, db_c=bc.grad, dh_d=hd.grad)


def test_gradients_against_torch_autograd():
    inp = tiny_inputs(V=37, N=4, prefix=np.array([1] * 7 + [1, 1, 1, 0, 0, 0, 0] + [1] * 7 + [1] * 7))
    hp = HParams(ce_alpha=0.2, l1_alpha=0.8, confidence_alpha=0.9)
    loss, ref = _torch_loss(inp, hp, 0.25)
    fw = oracle.forward(inp, hp)
    assert fw.loss == pytest.approx(float(loss.detach()), rel=1e-13)
    gr = oracle.backward(inp, hp, grad_scale=0.25)
    for k in ref:
        mine = getattr(gr, k)
        assert np.allclose(mine, ref[k].numpy().reshape(mine.shape), rtol=1e-10, atol=1e-14), k


def test_bf16_logit_gradient_in_the_weight_products():
    """Reading R19: with the logit gradient stored in bf16, the Markov weight
    products (dE = G W2, dW2 = G^T e) take that rounded G, as torch autograd
    does when the gradient reaching the bias is bf16; dz and the
    confidence-head gradients are the exact ones."""
    inp = tiny_inputs(V=37, N=4, prefix=np.array([1] * 7 + [1, 1, 1, 0, 0, 0, 0] + [1] * 7 + [1] * 7))
    hp = HParams(ce_alpha=0.4, l1_alpha=0.6, confidence_alpha=0.9)
    _, ref = _torch_loss(inp, hp, 0.25, round_bias_grad=True)
    gb = oracle.backward(inp, hp, grad_scale=0.25, g_bf16=True)
    for k in ref:
        mine = getattr(gb, k)
        assert np.allclose(mine, ref[k].numpy().reshape(mine.shape), rtol=1e-10, atol=1e-14), k
    gr = oracle.backward(inp, hp, grad_scale=0.25)
    assert np.array_equal(gb.dz, gr.dz) and np.array_equal(gb.dW_c, gr.dW_c)
    assert not np.allclose(gb.dW2, gr.dW2, rtol=1e-6, atol=0)  # the rounding reaches dW2


# ----------------------------------------------------------------- brute force

def _brute_row(z_row, t_row, y, e, W2, hd, Wc, bc):
    V = len(z_row)
    zp = [z_row[v] + sum(W2[v][j] * e[j] for j in range(len(e))) for v in range(V)]
    mz = max(zp); mt = max(t_row)
    sz = sum(math.exp(x - mz) for x in zp); st = sum(math.exp(x - mt) for x in t_row)
    p = [math.exp(x - mz) / sz for x in zp]; q = [math.exp(x - mt) / st for x in t_row]
    ce = -math.log(p[y])
    l1 = sum(abs(p[v] - q[v]) for v in range(V))
    acc = min(1.0, max(0.0, 1 - l1 / 2))
    feat = list(hd) + list(e)
    c = sum(Wc[i] * feat[i] for i in range(len(feat))) + bc
    sg = 1 / (1 + math.exp(-c))
    bce = -(acc * math.log(sg) + (1 - acc) * math.log(1 - sg))
    return ce, l1, acc, c, bce


def test_brute_force_tiny_vocab():
    inp = tiny_inputs(V=12, H=4, r=3, N=2)
    fw = oracle.forward(inp, HParams())
    T = inp.H_t @ inp.LM.T
    for row in range(inp.R):
        if not fw.m[row]:
            continue
        e = inp.W1[int(inp.prev_ids[row])]
        ce, l1, acc, c, bce = _brute_row(inp.z[row], T[row], int(inp.target_ids[row]), e,
                                         inp.W2, inp.h_d[row], inp.W_c[0], inp.b_c[0])
        assert fw.ce[row] == pytest.approx(ce, rel=1e-12)
        assert fw.l1[row] == pytest.approx(l1, rel=1e-12)
        assert fw.accept[row] == pytest.approx(acc, rel=1e-12)
        assert fw.conf_logit[row] == pytest.approx(c, rel=1e-12)
        assert fw.bce[row] == pytest.approx(bce, rel=1e-10)
    # tau by explicit loops over each block
    K = inp.K
    tau_sum = 0.0
    for blk in range(inp.B * inp.N):
        run, tau = 1.0, 1.0
        for k in range(K):
            r = blk * K + k
            run *= fw.accept[r] if fw.m[r] else 0.0
            tau += run
        tau_sum += tau
    assert fw.pairs["dspark tau"][0] == pytest.approx(tau_sum, rel=1e-13)


def test_finite_differences_every_element():
    """Central differences of the forward loss match the backward, element by element.

    The BCE label (accept) is detached (reading R6), so the differenced loss
    holds the label fixed at its unperturbed value.
    """
    inp = tiny_inputs(V=10, H=4, r=3, N=1, K=4, B=1)
    hp = HParams(ce_alpha=0.3, l1_alpha=0.7, confidence_alpha=0.5)
    hp_nc = HParams(ce_alpha=0.3, l1_alpha=0.7, confidence_alpha=0.0)
    gs = 0.8
    gr = oracle.backward(inp, hp, grad_scale=gs)
    accept0 = oracle.forward(inp, hp).accept.copy()

    def loss_of(x):
        f = oracle.forward(x, hp)
        frozen = np.sum(f.w * oracle.bce_with_logits(f.conf_logit, accept0))
        return gs * (oracle.forward(x, hp_nc).loss + hp.confidence_alpha * frozen)

    h = 1e-6
    for name in ("z", "W1", "W2", "W_c", "b_c", "h_d"):
        base = getattr(inp, name)
        fd = np.zeros_like(base, dtype=np.float64)
        for idx in np.ndindex(base.shape):
            xp = clone_inputs(inp); getattr(xp, name)[idx] += h
            xm = clone_inputs(inp); getattr(xm, name)[idx] -= h
            fd[idx] = (loss_of(xp) - loss_of(xm)) / (2 * h)
        ana = {"z": gr.dz, "W1": gr.dW1, "W2": gr.dW2, "W_c": gr.dW_c, "b_c": gr.db_c,
               "h_d": gr.dh_d}[name]
        assert np.allclose(ana, fd, rtol=1e-5, atol=1e-8), name


# ----------------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mutation", ["tv_half", "no_decay", "sign_flip", "no_cumprod", "label_grad",
                                      "rows_position_index", "head_invalid_passthrough"])
def test_pins_catch_planted_oracle_mistakes(monkeypatch, mutation):
    """Each plausible mistake planted in the oracle makes at least one pin fail."""
    import oracle.dspark_oracle as od
    if mutation == "tv_half":
        orig = od._row_terms
        def bad(inp, rows):
            t = orig(inp, rows); t["l1"] = 0.5 * t["l1"]; return t
        monkeypatch.setattr(od, "_row_terms", bad)
        pin = test_disjoint_saturated_raw_l1_is_two
    elif mutation == "no_decay":
        monkeypatch.setattr(od, "decay_weights", lambda K, g: np.ones(K))
        pin = test_decay_weights_properties
    elif mutation == "sign_flip":
        orig = od._row_terms
        def bad(inp, rows):
            t = orig(inp, rows); t["s"] = -t["s"]; t["S"] = -t["S"]; return t
        monkeypatch.setattr(od, "_row_terms", bad)
        pin = test_gradients_against_torch_autograd
    elif mutation == "no_cumprod":
        def bad_mask(ev, keep, B, N, K):
            m = (np.asarray(ev).reshape(B, N, K) != 0).astype(np.int64)
            if keep is not None:
                m = m * (np.asarray(keep).reshape(B, N, 1) != 0)
            return m.reshape(-1)
        monkeypatch.setattr(od, "effective_mask", bad_mask)
        monkeypatch.setattr(oracle, "effective_mask", bad_mask)
        pin = test_cumprod_mask_example
    elif mutation == "rows_position_index":
        # the subset's decay weights taken from list positions instead of row ids
        orig = od.forward_rows
        def bad(inp, hp, rows):
            out = orig(inp, hp, rows)
            dec = od.decay_weights(inp.K, hp.loss_decay_gamma)
            out["w"] = np.where(out["m"] != 0, dec[np.arange(len(rows)) % inp.K], 0.0)
            return out
        monkeypatch.setattr(od, "forward_rows", bad)
        monkeypatch.setattr(oracle, "forward_rows", bad)
        pin = test_forward_rows_equal_the_rows_of_forward
    elif mutation == "head_invalid_passthrough":
        # invalid slots passed through (z) instead of zeroed
        orig = od.markov_head_logits
        def bad(inp, valid):
            out = orig(inp, valid)
            v = np.asarray(valid) == 0
            out[v] = inp.z[v]
            return out
        monkeypatch.setattr(od, "markov_head_logits", bad)
        monkeypatch.setattr(oracle, "markov_head_logits", bad)
        pin = lambda: test_markov_head_alone(5)
    else:
        orig_sig = od.sigmoid
        monkeypatch.setattr(od, "sigmoid", lambda c: orig_sig(c) + 0.01)
        pin = test_finite_differences_every_element
    with pytest.raises(AssertionError):
        pin()


# ----------------------------------------------------------------- workloads

@pytest.mark.parametrize("idx", [0, 1])
def test_small_workloads_run_in_oracle(idx):
    wl = get_workload(idx)
    d = make_inputs(wl, "cpu")
    inp = oracle_inputs(d)
    fw = oracle.forward(inp, HParams())
    assert np.isfinite(fw.loss) and fw.num_tokens == int(fw.m.sum()) > 0
    v = fw.m != 0
    assert np.all(fw.l1[v] <= 2) and np.all(fw.accept[v] >= 0)


# --------------------------------------------------------------------------- batch construction

def test_build_blocks_hand_example():
    """A worked example, written out by hand from the definitions: tokens
    10..19, loss mask on positions 2..7 and 9, block size 4."""
    from oracle.batch import build_blocks, anchor_candidates
    ids = np.arange(10, 20, dtype=np.int32)[None, :]            # position p holds 10 + p
    lm = np.array([[0, 0, 1, 1, 1, 1, 1, 1, 0, 1]], dtype=np.uint8)
    # anchors: 2 (full block), 5 (prefix cut at position 8), 1 (anchor not in
    # the mask: dropped), 7 (first target 8 unsupervised: dropped), 9 (no target)
    anchors = np.array([[2, 5, 1, 7, 9]], dtype=np.int32)
    t, p, e, keep = build_blocks(ids, lm, anchors, 4)
    assert keep.tolist() == [1, 1, 0, 0, 0]
    # anchor 2: labels at 3..6, previous tokens at 2..5, all supervised
    assert t[0:4].tolist() == [13, 14, 15, 16]
    assert p[0:4].tolist() == [12, 13, 14, 15]
    assert e[0:4].tolist() == [1, 1, 1, 1]
    # anchor 5: labels at 6..9; position 8 is unsupervised, so slots 2 and 3
    # (positions 8 and 9) are cut although position 9 itself is supervised
    assert t[4:8].tolist() == [16, 17, 18, 19]
    assert p[4:8].tolist() == [15, 16, 17, 18]
    assert e[4:8].tolist() == [1, 1, 0, 0]
    # dropped blocks emit zeros
    assert t[8:].tolist() == [0] * 12 and p[8:].tolist() == [0] * 12 and e[8:].tolist() == [0] * 12
    assert anchor_candidates(lm)[0].tolist() == [0, 0, 1, 1, 1, 1, 1, 0, 0, 0]


def test_build_blocks_sequence_end():
    """A block running past the end of the sequence (by hand): tokens 10..19,
    every position supervised, anchor 8, block size 4."""
    from oracle.batch import build_blocks
    ids = np.arange(10, 20, dtype=np.int32)[None, :]
    lm = np.ones((1, 10), dtype=np.uint8)
    t, p, e, keep = build_blocks(ids, lm, np.array([[8]], dtype=np.int32), 4)
    assert keep.tolist() == [1]
    assert t.tolist() == [19, 0, 0, 0]
    assert p.tolist() == [18, 19, 0, 0]
    assert e.tolist() == [1, 0, 0, 0]


def test_build_blocks_properties():
    """Shift structure: slot k + 1's previous token is slot k's label; slot 0's
    previous token is the anchor token; the eval mask is a prefix per block."""
    from oracle.batch import build_blocks, anchor_candidates
    rng = np.random.default_rng(3)
    B, L, N, K = 3, 64, 6, 7
    ids = rng.integers(0, 5000, (B, L), dtype=np.int32)
    lm = (rng.random((B, L)) > 0.15).astype(np.uint8)
    cand = anchor_candidates(lm)
    anchors = np.stack([rng.choice(np.flatnonzero(cand[b]), N) for b in range(B)]).astype(np.int32)
    t, p, e, keep = build_blocks(ids, lm, anchors, K)
    assert keep.all()
    t, p, e = t.reshape(B, N, K), p.reshape(B, N, K), e.reshape(B, N, K)
    inside = (anchors[:, :, None] + np.arange(1, K)[None, None, :]) < L
    assert np.array_equal(np.where(inside, p[:, :, 1:], 0), np.where(inside, t[:, :, :-1], 0))
    for b in range(B):
        for n in range(N):
            a = anchors[b, n]
            assert p[b, n, 0] == ids[b, a]
            assert e[b, n, 0] == 1                    # the first target is valid by construction
            run = np.cumprod(e[b, n])
            assert np.array_equal(run, e[b, n])       # a contiguous prefix


# --------------------------------------------------------------------------- vocabulary shards

@pytest.mark.parametrize("cuts", [(0, 64, 128), (0, 40, 72, 128), (0, 8, 16, 24, 128)])
def test_vocab_shards_merge_to_the_unsplit_loss(cuts):
    """Splitting the draft vocabulary into column ranges and merging the
    exchanged partials reproduces the unsplit loss and gradient (fp64, to
    rounding): lse, L1, S, CE per row and every dz column."""
    from oracle import shard
    inp = tiny_inputs(V=128, H=16, r=8, N=3, seed=21)
    hp = oracle.HParams()
    fw = oracle.forward(inp, hp)
    gr = oracle.backward(inp, hp, grad_scale=0.5)
    bounds = list(zip(cuts[:-1], cuts[1:]))
    lse = shard.merge_stats([shard.shard_stats(inp, a, b) for a, b in bounds])
    m = fw.m != 0
    assert np.allclose(lse[m, 0], fw.lse_z[m], rtol=0, atol=1e-12)
    assert np.allclose(lse[m, 1], fw.lse_t[m], rtol=0, atol=1e-12)
    terms = sum(shard.shard_terms(inp, a, b, lse) for a, b in bounds)
    assert np.allclose(terms[m, 0], fw.l1[m], atol=1e-12)
    assert np.allclose(terms[m, 1], fw.S[m], atol=1e-12)
    assert np.allclose(lse[m, 0] - terms[m, 2], fw.ce[m], atol=1e-12)
    S = terms[:, 1]
    parts = [shard.shard_grad(inp, hp, a, b, lse, S, grad_scale=0.5) for a, b in bounds]
    dz = np.concatenate([p[0] for p in parts], axis=1)
    assert np.allclose(dz, gr.dz, rtol=0, atol=1e-14)
    dW2 = np.concatenate([p[2] for p in parts], axis=0)
    assert np.allclose(dW2, gr.dW2, rtol=0, atol=1e-13)
    # dE summed over shards plus the confidence term once gives dW1
    dE = sum(p[1] for p in parts)
    dW1 = np.zeros_like(gr.dW1)
    Hd = inp.h_d.shape[1]
    Wc = inp.W_c.reshape(-1)
    rows = np.nonzero(m)[0]
    dec = oracle.decay_weights(inp.K, hp.loss_decay_gamma)
    wr = dec[rows % inp.K]
    dc = 0.5 * wr * hp.confidence_alpha * (oracle.dspark_oracle.sigmoid(fw.conf_logit[rows]) -
                                           fw.accept[rows])
    dE[rows] += dc[:, None] * Wc[None, Hd:]
    np.add.at(dW1, inp.prev_ids[rows].astype(np.int64), dE[rows])
    assert np.allclose(dW1, gr.dW1, rtol=0, atol=1e-13)


def test_vocab_shard_owner_of_the_target_is_unique():
    from oracle import shard
    inp = tiny_inputs(V=64, H=16, r=8, N=2, seed=5)
    lse = shard.merge_stats([shard.shard_stats(inp, 0, 64)])
    parts = [shard.shard_terms(inp, a, b, lse) for a, b in ((0, 16), (16, 48), (48, 64))]
    owned = np.stack([p[:, 2] != 0 for p in parts])
    m = oracle.effective_mask(inp.eval_mask, inp.block_keep, inp.B, inp.N, inp.K) != 0
    assert np.all(owned[:, m].sum(axis=0) == 1)


# ----------------------------------------------------------------- row subsets and heads

def _ragged_problem():
    """Truncated prefixes, a non-prefix eval row, a dropped block (B=2, N=3, K=7)."""
    prefix = np.array([1, 1, 1, 0, 0, 0, 0] + [1] * 7 + [1, 0, 1, 1, 1, 1, 1]
                      + [1] * 7 + [1, 1, 1, 1, 1, 0, 0] + [1] * 7)
    inp = tiny_inputs(V=29, H=6, r=5, B=2, N=3, prefix=prefix)
    inp.block_keep = np.array([1, 1, 1, 1, 0, 1], dtype=np.uint8)
    return inp


def test_forward_rows_equal_the_rows_of_forward():
    """forward_rows / grad_rows on any subset of rows, in any order, equal the
    matching rows of forward / backward (rows are independent)."""
    inp = _ragged_problem()
    hp = HParams(ce_alpha=0.2, l1_alpha=0.8, confidence_alpha=0.6)
    fw = oracle.forward(inp, hp)
    gr = oracle.backward(inp, hp, grad_scale=0.3)
    rng = np.random.default_rng(3)
    for rows in (np.arange(inp.R), rng.permutation(inp.R), rng.permutation(inp.R)[:9],
                 np.array([inp.R - 1, 0, 15, 15])):
        fr = oracle.forward_rows(inp, hp, rows)
        for k in ("ce", "l1", "S", "bce", "conf_logit", "lse_z", "lse_t", "accept", "w", "m"):
            ref = getattr(fw, k)[rows]
            assert np.allclose(fr[k], ref, rtol=1e-13, atol=1e-15), k
        dz = oracle.grad_rows(inp, hp, rows, grad_scale=0.3)
        assert np.allclose(dz, gr.dz[rows], rtol=1e-13, atol=1e-16)
    # the decay weights of the rows follow the slot of each row, not its position in the list
    rows = np.array([5, 3, 1])
    assert np.allclose(oracle.forward_rows(inp, hp, rows)["w"],
                       oracle.decay_weights(7, hp.loss_decay_gamma)[[5, 3, 1]] * (fw.m[rows] != 0))


def _torch_conf_only(inp, rows):
    """F.linear of the confidence features: [h] alone, or [h ; W1[prev]]."""
    h = _t(inp.h_d[rows])
    if inp.with_markov_conf and inp.has_markov:
        h = torch.cat([h, F.embedding(torch.tensor(inp.prev_ids[rows].astype(np.int64)),
                                      _t(inp.W1))], 1)
    return F.linear(h, _t(inp.W_c), _t(inp.b_c)).squeeze(1).numpy()


def test_confidence_logit_without_markov_features():
    """with_markov=False: proj [1, hidden] over the hidden state alone ([HEADS]
    "Checkpoint Contract"); the embedding gets no confidence gradient."""
    inp = _ragged_problem()
    Hd = inp.h_d.shape[1]
    nm = clone_inputs(inp, with_markov_conf=False, W_c=inp.W_c[:, :Hd].copy())
    hp = HParams(ce_alpha=0.2, l1_alpha=0.8, confidence_alpha=0.6)
    fw = oracle.forward(nm, hp)
    v = np.nonzero(fw.m)[0]
    assert np.allclose(fw.conf_logit[v], _torch_conf_only(nm, v), rtol=1e-13)
    assert not np.any(fw.conf_logit[fw.m == 0])
    # autograd of the same objective with the hidden-only head
    B, N, K = nm.B, nm.N, nm.K
    m = torch.tensor(fw.m, dtype=torch.float64)
    z = _t(nm.z).requires_grad_(); W1 = _t(nm.W1).requires_grad_(); W2 = _t(nm.W2).requires_grad_()
    Wc = _t(nm.W_c).requires_grad_(); bc = _t(nm.b_c).requires_grad_(); hd = _t(nm.h_d).requires_grad_()
    e = W1[torch.tensor(nm.prev_ids.astype(np.int64))]
    zp = z + F.linear(e, W2)
    tl = F.linear(_t(nm.H_t), _t(nm.LM))
    ce = F.cross_entropy(zp, torch.tensor(nm.target_ids.astype(np.int64)), reduction="none")
    l1 = (F.softmax(zp, -1) - F.softmax(tl, -1)).abs().sum(-1)
    acc = (1 - 0.5 * l1).clamp(0, 1).detach()
    c = F.linear(hd, Wc, bc).squeeze(1)
    bce = F.binary_cross_entropy_with_logits(c, acc, reduction="none")
    w = m * torch.exp(-(torch.arange(nm.R) % K).double() / hp.loss_decay_gamma)
    term = hp.ce_alpha * ce + hp.l1_alpha * l1 + hp.confidence_alpha * bce
    loss = torch.where(m != 0, w * term, torch.zeros_like(term)).sum()
    (loss * 0.3).backward()
    assert fw.loss == pytest.approx(float(loss.detach()), rel=1e-13)
    gr = oracle.backward(nm, hp, grad_scale=0.3)
    for k, ref in (("dz", z.grad), ("dW1", W1.grad), ("dW2", W2.grad), ("dW_c", Wc.grad),
                   ("db_c", bc.grad), ("dh_d", hd.grad)):
        mine = getattr(gr, k)
        assert mine.shape == tuple(ref.shape) or mine.size == ref.numel(), k
        assert np.allclose(mine, ref.numpy().reshape(mine.shape), rtol=1e-10, atol=1e-14), k


@pytest.mark.parametrize("rank", [5, 0])
def test_markov_head_alone(rank):
    """The Markov head on its own: z + W2(W1[prev]) on valid slots ([TS132]
    "Testing": the bias equals W2 applied to W1[prev]); zero rows on invalid
    slots, never read there ([HEADS] "Inputs and Outputs")."""
    inp = _ragged_problem()
    if rank == 0:
        inp = clone_inputs(inp, W1=None, W2=None, prev_ids=None)
    valid = (np.arange(inp.R) % 3 != 1).astype(np.uint8)
    out = oracle.markov_head_logits(inp, valid)
    v = valid != 0
    ref = _t(inp.z[v])
    if rank:
        ref = ref + F.linear(F.embedding(torch.tensor(inp.prev_ids[v].astype(np.int64)),
                                         _t(inp.W1)), _t(inp.W2))
    assert np.allclose(out[v], ref.numpy(), rtol=1e-14, atol=1e-15)
    assert not np.any(out[~v])
    bad = clone_inputs(inp)
    bad.z[~v] = np.nan
    if rank:
        bad.prev_ids[~v] = -7
    assert np.array_equal(oracle.markov_head_logits(bad, valid), out)


@pytest.mark.parametrize("with_markov", [True, False])
def test_confidence_head_alone(with_markov):
    inp = _ragged_problem()
    Hd = inp.h_d.shape[1]
    if not with_markov:
        inp = clone_inputs(inp, with_markov_conf=False, W_c=inp.W_c[:, :Hd].copy())
    valid = (np.arange(inp.R) % 4 != 2).astype(np.uint8)
    v = valid != 0
    out = oracle.confidence_head_logits(inp, valid)
    assert np.allclose(out[v], _torch_conf_only(inp, np.nonzero(v)[0]), rtol=1e-13)
    assert not np.any(out[~v])
    bad = clone_inputs(inp)
    bad.h_d[~v] = np.inf
    bad.prev_ids[~v] = -3
    assert np.array_equal(oracle.confidence_head_logits(bad, valid), out)
    # with the loss's own mask the head is the loss's confidence logit
    fw = oracle.forward(inp, HParams())
    assert np.allclose(oracle.confidence_head_logits(inp, fw.m), fw.conf_logit, rtol=1e-14)
