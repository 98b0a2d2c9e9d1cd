"""The loss's forward + backward captured in a HIP graph (torch.cuda.CUDAGraph
over the C-ABI calls) and replayed: the library allocates nothing, never
synchronizes and clears its counters with fill kernels, so a replayed step
must equal the eager step.  Every replay is checked against the eager result,
with eager work and synchronizations between the replays.  All outputs are
compared bit for bit; dW1 too with DSPARK_OPT_DETERMINISTIC (fixed-point
sums), and within 1e-6 normwise with the default fp32-atomic scatter (any
order).
"""

from __future__ import annotations

import pytest
import torch

from speculative_decoding_draft_dspark_amd import (DSparkBatch, HParams, dspark_loss_bwd,
                                                   dspark_loss_fwd)
from tests.gpu_common import normwise, say, to_np
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GS = 0.0125


def _step(b, hp, ws, det=False):
    f = dspark_loss_fwd(b, hp, workspace=ws, deterministic=det)
    g = dspark_loss_bwd(b, hp, f, GS, conf_hidden_grad=True)
    return f, g


def _snapshot(f, g):
    out = {"loss": f.loss, "num_tokens": f.num_tokens, "pairs": f.pairs,
           "accept": f.accept_rate, "row_terms": f.row_terms, "flags": f.flags}
    out.update(g)
    return {k: v.detach().clone() for k, v in out.items()}


@pytest.mark.parametrize("idx,det", [(1, False), (4, False), (1, True)])
def test_graph_replay_matches_eager(idx, det):
    wl = get_workload(idx)
    say(f"[graph] {wl.name}: capture fwd + bwd, replay 3 times, deterministic={det}")
    d = make_inputs(wl, DEV)
    b = DSparkBatch.from_workload(d)
    hp = HParams(ce_alpha=0.3, l1_alpha=0.7, confidence_alpha=0.5)
    f0, g0 = _step(b, hp, None, det)
    ws = f0.workspace
    ref = _snapshot(f0, g0)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        _step(b, hp, ws, det)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fc, gc = _step(b, hp, ws, det)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays that overwrites the shared workspace
        _step(b, hp, ws, det)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(fc, gc)
        for k, v in ref.items():
            if k == "d_markov_w1" and not det:
                err = normwise(to_np(got[k]), to_np(v))
                assert err <= 1e-6, f"replay {rep}: {k} normwise {err:.2e}"
            else:
                assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager step"
    say(f"[graph] {wl.name}: 3 replays equal the eager step")
