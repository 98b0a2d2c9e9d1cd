"""Host-side checks of the C ABI: exports, validation codes, loud failures.

No GPU: every call here is rejected by host validation before any HIP call.
"""

from __future__ import annotations

import ctypes as C
import os
import re

import pytest
import torch

from speculative_decoding_draft_dspark_amd import _capi as capi
from speculative_decoding_draft_dspark_amd import DSparkBatch, DSparkError, dspark_loss_fwd

PKG = os.path.dirname(capi.__file__)


@pytest.fixture(scope="module")
def L():
    return capi.lib()


def test_library_exports_every_declared_symbol(L):
    names = capi.declared_functions()
    assert set(names) >= {"dspark_loss_fwd", "dspark_loss_bwd", "dspark_accept_report",
                          "dspark_workspace_size", "dspark_status_string"}
    for n in names:
        assert hasattr(L, n), n


def _shape(**kw):
    d = dict(batch=2, num_blocks=3, block_size=7, draft_vocab=512, target_vocab=600, hidden=64,
             conf_hidden=32, markov_rank=16, with_markov_conf=1, dtype=1, grad_dtype=1,
             options=0)
    d.update(kw)
    return capi.Shape(**d)


def test_workspace_size(L):
    s = _shape()
    n = L.dspark_workspace_size(C.byref(s))
    R, V = 42, 512
    assert n >= 2 * R * V * 4            # fp32 teacher + corrected draft logits
    assert n % 256 == 0
    for bad in (dict(batch=0), dict(draft_vocab=1001), dict(markov_rank=12), dict(dtype=7),
                dict(hidden=-8), dict(target_vocab=0), dict(options=4), dict(options=-1)):
        assert L.dspark_workspace_size(C.byref(_shape(**bad))) == 0, bad
    assert L.dspark_workspace_size(None) == 0


def test_deterministic_option_adds_the_fixed_point_accumulator(L):
    """DSPARK_OPT_DETERMINISTIC: 64-bit fixed-point sums [Vt, r] for dW1 (plus one
    float), only with a Markov head."""
    base = _shape()
    det = _shape(options=2)
    n0 = L.dspark_workspace_size(C.byref(base))
    n1 = L.dspark_workspace_size(C.byref(det))
    assert n1 - n0 >= 8 * base.target_vocab * base.markov_rank
    assert n1 - n0 <= 8 * base.target_vocab * base.markov_rank + 512
    nm = dict(markov_rank=0)
    assert L.dspark_workspace_size(C.byref(_shape(options=2, **nm))) == \
        L.dspark_workspace_size(C.byref(_shape(**nm)))
    assert L.dspark_workspace_size(C.byref(_shape(options=3))) > 0


def test_store_draft_logits_option_adds_the_corrected_logits_buffer(L):
    """DSPARK_OPT_STORE_DRAFT_LOGITS: an fp32 [R, Vd] z' in the workspace where the
    recompute sweeps are the default (bf16, supported rank, R and Vd multiples of 32);
    fp32 inputs always store it, so the bit changes nothing there."""
    R, V = 2 * 16 * 7, 512
    kw = dict(num_blocks=16, markov_rank=64)
    low = L.dspark_workspace_size(C.byref(_shape(**kw)))
    big = L.dspark_workspace_size(C.byref(_shape(options=capi.OPT_STORE_DRAFT_LOGITS, **kw)))
    assert big > 0 and low > 0
    # minus what only the recompute path holds: per-row partials and the sign
    # bits of p - q (2 bits per element, rows rounded up to whole 256-row tiles)
    signs = (R + 255) // 256 * 256 * V // 4
    assert big - low >= R * V * 4 - signs - (2 * 8) * R - 3 * 256
    f32 = dict(kw, dtype=0, grad_dtype=0)
    assert (L.dspark_workspace_size(C.byref(_shape(options=capi.OPT_STORE_DRAFT_LOGITS, **f32)))
            == L.dspark_workspace_size(C.byref(_shape(**f32))))


FAKE = 0x10000  # aligned host address; never dereferenced (validation fails first)


def _inputs(**over):
    d = {n: FAKE for n, _ in capi.InputsC._fields_}
    d["aligned_target_logits"] = None
    d.update(over)
    return capi.InputsC(**d)


def _fwd(L, shape=None, inp=None, ws=FAKE, wsbytes=1 << 40, out=None, hp=None):
    shape = shape or _shape()
    hp = hp or capi.HParamsC(0.1, 0.9, 1.0, 4.0)
    inp = inp or _inputs()
    out = out or capi.FwdOutC(FAKE, FAKE, FAKE, None, None, FAKE)
    return L.dspark_loss_fwd(C.byref(shape), C.byref(hp), C.byref(inp), ws, wsbytes,
                             C.byref(out), None)


def test_validation_codes(L):
    assert _fwd(L, inp=_inputs(draft_logits=None)) == -1
    assert _fwd(L, inp=_inputs(prev_ids=None)) == -1
    assert _fwd(L, inp=_inputs(conf_w=None)) == -1
    assert _fwd(L, shape=_shape(draft_vocab=100)) == -2
    assert _fwd(L, shape=_shape(grad_dtype=5)) == -3
    assert _fwd(L, inp=_inputs(target_hidden=None, lm_head=None)) == -4          # no teacher
    assert _fwd(L, inp=_inputs(target_hidden=None), hp=capi.HParamsC(1, 0, 0, 4)) == -4  # conf head
    assert _fwd(L, wsbytes=100) == -5
    assert _fwd(L, ws=None) == -5
    assert _fwd(L, inp=_inputs(lm_head=FAKE + 4)) == -6
    assert _fwd(L, out=capi.FwdOutC(FAKE, None, FAKE, None, None, FAKE)) == -1
    hp = capi.HParamsC(0.1, 0.9, 1.0, 4.0)
    o = capi.BwdOutC(None, FAKE, FAKE, FAKE, FAKE, None)
    s = _shape()
    assert L.dspark_loss_bwd(C.byref(s), C.byref(hp), C.byref(_inputs()), FAKE, 1 << 40, 1.0,
                             C.byref(o), None) == -1
    assert L.dspark_accept_report(1, 1, 7, None, FAKE, None, FAKE, None) == -1
    assert L.dspark_accept_report(1, 0, 7, FAKE, FAKE, None, FAKE, None) == -2
    assert L.dspark_accept_report(1, 1, 7, FAKE + 2, FAKE, None, FAKE, None) == -6


def test_status_strings(L):
    for code in capi.STATUS:
        assert len(L.dspark_status_string(code)) > 0
    assert L.dspark_status_string(123) == b"unknown status"


def test_binding_fails_loudly_on_cpu_tensors():
    z = torch.zeros(7, 64)
    b = DSparkBatch(B=1, N=1, K=7, draft_logits=z, target_ids=torch.zeros(7, dtype=torch.int32),
                    eval_mask=torch.ones(7, dtype=torch.uint8))
    with pytest.raises(DSparkError):
        dspark_loss_fwd(b)


def test_product_never_imports_the_oracle():
    for root, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert not re.search(r"\boracle\b", text), f


def test_missing_library_is_a_loud_error(monkeypatch, tmp_path):
    monkeypatch.setattr(capi, "_lib", None)
    monkeypatch.setattr(capi, "LIB_PATH", str(tmp_path / "libdspark.so"))
    with pytest.raises(DSparkError):
        capi.lib()


def test_head_ops_validation_codes(L):
    """The standalone head ops reject bad arguments on the host (no HIP call)."""
    E = {v: k for k, v in capi.STATUS.items()}
    ok = L.dspark_markov_logits_workspace_size(100, 512, 64, 1)
    assert ok > 0
    assert L.dspark_markov_logits_workspace_size(100, 500, 64, 1) == 0   # vocab % 8
    assert L.dspark_markov_logits_workspace_size(100, 512, 12, 1) == 0   # rank % 8
    assert L.dspark_markov_logits_workspace_size(100, 512, 64, 7) == 0   # dtype
    fake = C.c_void_p(4096)  # never dereferenced: every call below fails validation
    # markov: null output, bad dtype, bad shape, missing Markov weights, short workspace
    assert L.dspark_markov_logits(100, 512, 600, 64, 1, fake, fake, None, fake, fake, None,
                                  fake, ok, None) == E["ERR_NULL"]
    assert L.dspark_markov_logits(100, 512, 600, 64, 5, fake, fake, None, fake, fake, fake,
                                  fake, ok, None) == E["ERR_DTYPE"]
    assert L.dspark_markov_logits(100, 510, 600, 64, 1, fake, fake, None, fake, fake, fake,
                                  fake, ok, None) == E["ERR_SHAPE"]
    assert L.dspark_markov_logits(100, 512, 0, 64, 1, fake, fake, None, fake, fake, fake,
                                  fake, ok, None) == E["ERR_SHAPE"]
    assert L.dspark_markov_logits(100, 512, 600, 64, 1, fake, None, None, fake, fake, fake,
                                  fake, ok, None) == E["ERR_NULL"]
    assert L.dspark_markov_logits(100, 512, 600, 64, 1, fake, fake, None, fake, fake, fake,
                                  fake, ok - 1, None) == E["ERR_WORKSPACE"]
    assert L.dspark_markov_logits(100, 512, 600, 64, 1, C.c_void_p(4100), fake, None, fake,
                                  fake, fake, fake, ok, None) == E["ERR_ALIGN"]
    # confidence: no Markov features need no workspace; with them, the size rule holds
    assert L.dspark_confidence_logits_workspace_size(100, 64, 0, 1) == 0
    cw = L.dspark_confidence_logits_workspace_size(100, 64, 1, 1)
    assert cw >= 100 * 64 * 2 + 100
    assert L.dspark_confidence_logits(100, 0, 600, 64, 1, 1, fake, fake, None, fake, fake, fake,
                                      fake, fake, cw, None) == E["ERR_SHAPE"]
    assert L.dspark_confidence_logits(100, 32, 600, 64, 1, 1, None, fake, None, fake, fake,
                                      fake, fake, fake, cw, None) == E["ERR_NULL"]
    assert L.dspark_confidence_logits(100, 32, 600, 64, 1, 1, fake, fake, None, fake, fake,
                                      fake, fake, fake, cw - 1, None) == E["ERR_WORKSPACE"]
    # the no-allocation variant: same checks, and a problem beyond its scratch
    # (bf16 rank 256: 40000 rows need 20.5 MB of embeddings) is rejected up front
    na = L.dspark_confidence_logits_noalloc
    assert na(100, 0, 600, 64, 1, 1, fake, fake, None, fake, fake, fake, fake, None) == \
        E["ERR_SHAPE"]
    assert na(100, 32, 600, 64, 1, 1, None, fake, None, fake, fake, fake, fake, None) == \
        E["ERR_NULL"]
    assert na(100, 32, 600, 64, 1, 1, fake, None, None, fake, fake, fake, fake, None) == \
        E["ERR_NULL"]
    assert na(100, 32, 600, 64, 1, 1, fake, fake, None, fake, fake, fake, C.c_void_p(4100),
              None) == E["ERR_ALIGN"]
    assert L.dspark_confidence_logits_workspace_size(40000, 256, 1, 1) > 16 << 20
    assert na(40000, 32, 600, 256, 1, 1, fake, fake, None, fake, fake, fake, fake, None) == \
        E["ERR_SCRATCH"]


def test_build_blocks_validation_codes(L):
    E = {v: k for k, v in capi.STATUS.items()}
    fake = C.c_void_p(4096)  # never dereferenced: every call below fails validation
    args = [fake] * 7
    assert L.dspark_build_blocks(2, 64, 4, 7, None, *args[:6], None, None) == E["ERR_NULL"]
    assert L.dspark_build_blocks(2, 64, 4, 0, *args, None, None) == E["ERR_SHAPE"]
    assert L.dspark_build_blocks(0, 64, 4, 7, *args, None, None) == E["ERR_SHAPE"]
    assert L.dspark_build_blocks(2, 64, 1 << 40, 7, *args, None, None) == E["ERR_SHAPE"]


def test_vocab_shard_validation_codes(L):
    """The vocabulary-shard entry points take only shapes of the bias sweeps and
    reject bad arguments on the host (no HIP call)."""
    E = {v: k for k, v in capi.STATUS.items()}
    hp = capi.HParamsC(0.1, 0.9, 1.0, 4.0)
    inp = _inputs()
    good = _shape(num_blocks=16, markov_rank=64)          # R = 224, bf16, rank 64
    ws = L.dspark_workspace_size(C.byref(good))

    def stats(shape, lse=FAKE, flags=FAKE, wsbytes=ws):
        return L.dspark_shard_fwd_stats(C.byref(shape), C.byref(hp), C.byref(inp), FAKE,
                                        wsbytes, lse, flags, None)
    assert stats(good, lse=None) == E["ERR_NULL"]
    assert stats(good, flags=None) == E["ERR_NULL"]
    assert stats(good, wsbytes=ws - 1) == E["ERR_WORKSPACE"]
    assert stats(_shape(num_blocks=16, markov_rank=16)) == E["ERR_SHAPE"]       # rank 16
    assert stats(_shape(num_blocks=16, markov_rank=64, dtype=0, grad_dtype=0)) == E["ERR_SHAPE"]
    assert stats(_shape(num_blocks=16, markov_rank=64,
                        options=capi.OPT_STORE_DRAFT_LOGITS)) == E["ERR_SHAPE"]
    assert stats(_shape(num_blocks=3, markov_rank=64)) == E["ERR_SHAPE"]       # R = 42
    assert L.dspark_shard_fwd_terms(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, None,
                                    FAKE, None) == E["ERR_NULL"]
    assert L.dspark_shard_fwd_finish(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, FAKE,
                                     None, None) == E["ERR_NULL"]
    assert L.dspark_shard_bwd(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, 1.0, FAKE,
                              None, FAKE, None) == E["ERR_NULL"]
    assert L.dspark_shard_bwd(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, 1.0, FAKE + 2,
                              FAKE, FAKE, None) == E["ERR_ALIGN"]
    o = capi.BwdOutC(None, None, None, FAKE, FAKE, None)
    assert L.dspark_shard_bwd_finish(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, 1.0,
                                     FAKE, C.byref(o), None) == E["ERR_NULL"]   # d_markov_w1
    assert L.dspark_shard_merge_lse(0, 10, FAKE, FAKE, None) == E["ERR_SHAPE"]
    assert L.dspark_shard_merge_lse(2, -1, FAKE, FAKE, None) == E["ERR_SHAPE"]
    assert L.dspark_shard_merge_lse(2, 10, None, FAKE, None) == E["ERR_NULL"]
    assert L.dspark_shard_merge_lse(2, 0, None, None, None) == E["OK"]
    assert L.dspark_shard_merge_lse(2, 10, FAKE + 8, FAKE, None) == E["ERR_ALIGN"]
    assert stats(good, lse=FAKE + 8) == E["ERR_ALIGN"]
    assert L.dspark_shard_fwd_terms(C.byref(good), C.byref(hp), C.byref(inp), FAKE, ws, FAKE,
                                    FAKE + 8, None) == E["ERR_ALIGN"]


def test_bench_traffic_only_for_the_measured_workload():
    """The committed HBM byte counts are reported only for the workloads and
    GEMM code they were measured on."""
    import importlib.util
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    with open(os.path.join(root, "profiles", "logits_gemm_traffic.json")) as fh:
        rec = json.load(fh)
    for name, n in rec["bytes_per_launch"].items():
        got = bench._traffic("logits_gemm", name)
        assert got in (None, n)   # None once gemm.hip's code has changed
    assert bench._traffic("logits_gemm", "tiny-fp32-r28-v1024") is None


def test_bench_code_hash_ignores_comments_only(tmp_path):
    """The GEMM code hash behind the byte count: comment and whitespace edits
    keep it, a code edit changes it."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod2", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */\nint f(int x) {\n\n  // a note\n  return  x + 1;\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;  // one\n}\n")
    assert bench._code_sha256(str(a)) == bench._code_sha256(str(b))
    assert bench._code_sha256(str(a)) != bench._code_sha256(str(c))
