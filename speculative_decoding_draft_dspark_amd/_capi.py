"""ctypes mirror of include/dspark.h and the loader of libdspark.so.

Argument marshalling only.  Loading fails loudly when the library is absent.
"""

from __future__ import annotations

import ctypes as C
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "dspark.h")

DSPARK_F32, DSPARK_BF16 = 0, 1
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_DTYPE", -4: "ERR_NO_TARGET",
          -5: "ERR_WORKSPACE", -6: "ERR_ALIGN", -7: "ERR_HIP", -8: "ERR_SCRATCH"}
FLAG_TARGET_ID_RANGE, FLAG_PREV_ID_RANGE, FLAG_NONFINITE, FLAG_NO_TEACHER = 1, 2, 4, 8
OPT_STORE_DRAFT_LOGITS = 1
OPT_DETERMINISTIC = 2


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int64), ("num_blocks", C.c_int64), ("block_size", C.c_int64),
                ("draft_vocab", C.c_int64), ("target_vocab", C.c_int64), ("hidden", C.c_int64),
                ("conf_hidden", C.c_int64), ("markov_rank", C.c_int64),
                ("with_markov_conf", C.c_int32), ("dtype", C.c_int32), ("grad_dtype", C.c_int32),
                ("options", C.c_int32)]


class HParamsC(C.Structure):
    _fields_ = [("ce_alpha", C.c_float), ("l1_alpha", C.c_float),
                ("confidence_alpha", C.c_float), ("loss_decay_gamma", C.c_float)]


class InputsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "draft_logits", "target_ids", "eval_mask", "block_keep_mask", "prev_ids", "markov_w1",
        "markov_w2", "target_hidden", "lm_head", "aligned_target_logits", "conf_hidden", "conf_w",
        "conf_b")]


class FwdOutC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "loss", "num_tokens", "pairs", "accept_rate", "row_terms", "flags")]


class BwdOutC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "d_draft_logits", "d_markov_w1", "d_markov_w2", "d_conf_w", "d_conf_b", "d_conf_hidden")]


class DSparkError(RuntimeError):
    pass


_lib = None


def lib():
    """The loaded libdspark.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DSparkError(f"{LIB_PATH} is missing: build it with "
                          "`python -m speculative_decoding_draft_dspark_amd.build_lib`")
    L = C.CDLL(LIB_PATH)
    L.dspark_workspace_size.argtypes = [C.POINTER(Shape)]
    L.dspark_workspace_size.restype = C.c_size_t
    L.dspark_loss_fwd.argtypes = [C.POINTER(Shape), C.POINTER(HParamsC), C.POINTER(InputsC),
                                  C.c_void_p, C.c_size_t, C.POINTER(FwdOutC), C.c_void_p]
    L.dspark_loss_fwd.restype = C.c_int
    L.dspark_loss_bwd.argtypes = [C.POINTER(Shape), C.POINTER(HParamsC), C.POINTER(InputsC),
                                  C.c_void_p, C.c_size_t, C.c_float, C.POINTER(BwdOutC),
                                  C.c_void_p]
    L.dspark_loss_bwd.restype = C.c_int
    L.dspark_accept_report.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_void_p]
    L.dspark_accept_report.restype = C.c_int
    L.dspark_markov_logits_workspace_size.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int32]
    L.dspark_markov_logits_workspace_size.restype = C.c_size_t
    L.dspark_markov_logits.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                       C.c_void_p]
    L.dspark_markov_logits.restype = C.c_int
    L.dspark_confidence_logits_workspace_size.argtypes = [C.c_int64, C.c_int64, C.c_int32,
                                                          C.c_int32]
    L.dspark_confidence_logits_workspace_size.restype = C.c_size_t
    L.dspark_confidence_logits.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                           C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    L.dspark_confidence_logits.restype = C.c_int
    L.dspark_confidence_logits_noalloc.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                                   C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                   C.c_void_p, C.c_void_p]
    L.dspark_confidence_logits_noalloc.restype = C.c_int
    L.dspark_build_blocks.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int64] + \
        [C.c_void_p] * 9
    L.dspark_build_blocks.restype = C.c_int
    common = [C.POINTER(Shape), C.POINTER(HParamsC), C.POINTER(InputsC), C.c_void_p,
              C.c_size_t]
    L.dspark_shard_fwd_stats.argtypes = common + [C.c_void_p, C.c_void_p, C.c_void_p]
    L.dspark_shard_merge_lse.argtypes = [C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                         C.c_void_p]
    L.dspark_shard_fwd_terms.argtypes = common + [C.c_void_p, C.c_void_p, C.c_void_p]
    L.dspark_shard_fwd_finish.argtypes = common + [C.c_void_p, C.POINTER(FwdOutC), C.c_void_p]
    L.dspark_shard_bwd.argtypes = common + [C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_void_p]
    L.dspark_shard_bwd_finish.argtypes = common + [C.c_float, C.c_void_p, C.POINTER(BwdOutC),
                                                   C.c_void_p]
    for f in ("dspark_shard_fwd_stats", "dspark_shard_merge_lse", "dspark_shard_fwd_terms",
              "dspark_shard_fwd_finish", "dspark_shard_bwd", "dspark_shard_bwd_finish"):
        getattr(L, f).restype = C.c_int
    L.dspark_status_string.argtypes = [C.c_int]
    L.dspark_status_string.restype = C.c_char_p
    L.dspark_last_hip_error.argtypes = []
    L.dspark_last_hip_error.restype = C.c_char_p
    L.dspark_profile_enable.argtypes = [C.c_int]
    L.dspark_profile_enable.restype = C.c_int
    L.dspark_profile_read.argtypes = [C.c_void_p, C.c_void_p, C.c_int]
    L.dspark_profile_read.restype = C.c_int
    L.dspark_stage_name.argtypes = [C.c_int]
    L.dspark_stage_name.restype = C.c_char_p
    _lib = L
    return L


def check(status: int, what: str):
    if status != 0:
        msg = lib().dspark_status_string(status).decode()
        if status == -7:
            msg += ": " + lib().dspark_last_hip_error().decode()
        raise DSparkError(f"{what} failed with {STATUS.get(status, status)} ({msg})")


def declared_functions() -> list:
    """Names of the functions include/dspark.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def profile_enable(on: bool = True) -> None:
    """Turn the library's per-stage HIP-event timers on or off (clears totals)."""
    lib().dspark_profile_enable(1 if on else 0)


def profile_read() -> dict:
    """{stage name: (total ms, launches)} accumulated since profile_enable()."""
    L = lib()
    n = L.dspark_profile_read(None, None, 0)
    ms = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    L.dspark_profile_read(C.cast(ms, C.c_void_p), C.cast(cnt, C.c_void_p), n)
    return {L.dspark_stage_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}
