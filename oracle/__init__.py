"""FP64 CPU oracle of the DSpark loss -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product path never does.
"""
from .dspark_oracle import (Inputs, HParams, Forward, Grads, effective_mask, decay_weights,
                            forward, backward, accept_report, forward_rows, grad_rows,
                            bce_with_logits, log_softmax_rows, markov_embedding,
                            draft_logits_corrected, confidence_logit,
                            markov_head_logits, confidence_head_logits)
