"""DSpark draft-training loss for AMD MI355X (gfx950): a C-ABI HIP library
(libdspark.so) and its thin Python binding."""

from .loss import (DSparkBatch, FwdResult, HParams, REPORT_KEYS, build_blocks, confidence_logits,
                   confidence_logits_noalloc,
                   dspark_accept_report, dspark_loss, dspark_loss_bwd, dspark_loss_fwd,
                   dspark_workspace_size, markov_logits)
from ._capi import DSparkError
from .shard import VocabShard, merge_lse, shard_loss
