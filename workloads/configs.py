"""The five workloads: shapes and value recipes.

Shapes follow the Qwen3-8B DSpark recipe (block_size 7, gamma 4.0,
markov_rank 256, vocabulary 151936) stated in TorchSpec pull request #132
(PR description) and the NeMo-RL "DSpark Auxiliary Heads" checkpoint contract.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    K: int
    Vd: int              # draft vocabulary (logits, L1)
    Vt: int              # target vocabulary (previous-token ids, W1 rows)
    H: int               # target hidden size (lm_head inner dimension)
    Hd: int              # confidence-head hidden size
    r: int               # markov rank
    dtype: str           # "f32" or "bf16": dtype of every float input
    gamma: float = 4.0
    seed: int = 1000
    recipe: str = ""

    @property
    def R(self) -> int:
        return self.B * self.N * self.K


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32-r28-v1024", B=1, N=4, K=7, Vd=1024, Vt=1024, H=64, Hd=64, r=16,
                 dtype="f32", seed=1001, recipe="tiny"),
        Workload("small-bf16-r224-v32000", B=2, N=16, K=7, Vd=32000, Vt=32000, H=1024, Hd=1024,
                 r=64, dtype="bf16", seed=1002, recipe="small"),
        Workload("qwen3-8b-r1792-v151936", B=4, N=64, K=7, Vd=151936, Vt=151936, H=4096,
                 Hd=4096, r=256, dtype="bf16", seed=1003, recipe="qwen"),
        Workload("large-batch-r14336-v151936", B=8, N=256, K=7, Vd=151936, Vt=151936, H=4096,
                 Hd=4096, r=256, dtype="bf16", seed=1004, recipe="large"),
        Workload("edge-r896-vd32000-vt151936", B=4, N=32, K=7, Vd=32000, Vt=151936, H=4096,
                 Hd=4096, r=256, dtype="bf16", seed=1005, recipe="edge"),
    ]
}

ORDER = list(WORKLOADS)


def get_workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index]]
    return WORKLOADS[name_or_index]
