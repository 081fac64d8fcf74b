"""CPU fp64 oracle for the fused MHA forward, its split-over-keys form, its
backward, the attention KL divergence and the output projection.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path must not.
"""
from .attention import (  # noqa: F401
    attention_fwd,
    attention_fwd_bruteforce,
    attention_probs,
    causal_visible,
    scores,
    softmax_rows,
    weighted_values,
    log_sum_exp,
)
from .backward import attention_bwd, softmax_grad  # noqa: F401
from .split import attention_fwd_split, merge_splits, split_partials  # noqa: F401
from .kl import attention_kl, kl_online_terms  # noqa: F401
from .proj import out_proj, out_proj_bruteforce, out_proj_by_heads  # noqa: F401
