"""Plain, slow fp64 CPU oracle for blockwise online-softmax (ring) attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``blockwise_online_softmax_amd``) never imports it, and this package imports
nothing from the product path: the two share no kernels, helpers, tables or
constants.  Inputs come from the seeded generators in ``workloads.py``, which
hold none of the method's arithmetic.

Pages cited (by title and section):
  [M23]  "Module 23: Distributed Training" (learnllm), sections
         "Sequence Parallelism: Ring Attention", "The Math: One Block at a
         Time", "Exact by Construction", "The Causal Imbalance -- and the
         Striped Fix".
  [RAQA] "Explain ring attention and how it enables very long contexts across
         multiple devices?" (Transformer Architecture Q&A), sections "The
         ring", "The causal-mask problem", "A real-life example".
  [DT2]  "3.6 Distributed Training II: Tensor, Pipeline, Sequence & Expert
         Parallelism", sections "Ring Attention" and "Vocab-parallel
         cross-entropy".

Modules:
  attention  O1: ordinary softmax attention by its definition (+ log-sum-exp).
  ring       O2: the pages' blockwise recurrence run as a simulated ring.
  layouts    token->device maps (contiguous, striped, zigzag), positions and
             the causal pair count per device.
  merge      O3: merge of two partial results over disjoint key sets, as
             running states (m, l, o) or as finalized (out, lse).
  vocab_ce   O4: vocab-parallel cross-entropy (the page's three shard steps),
             the plain per-row definition and the gradient.
  parallel   O1 run by a pool of CPU processes over row ranges (no arithmetic
             of its own), for whole-output checks at full size and for the
             CPU baseline.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, printed page values, library routines, brute force).  What no
pin fixes is the exact value of N(0,1) outputs at the large shapes beyond O1's
own definition; that is stated where those tests live.
"""

from .attention import full_attention, attention_rows  # noqa: F401
from .ring import (  # noqa: F401
    init_state,
    absorb_block,
    finalize,
    ring_visit_order,
    ring_attention,
)
from .merge import merge_states, merge_outputs  # noqa: F401
from . import vocab_ce  # noqa: F401
from .layouts import (  # noqa: F401
    LAYOUTS,
    device_positions,
    permuted_positions,
    to_device_order,
    from_device_order,
    causal_block_work,
)
