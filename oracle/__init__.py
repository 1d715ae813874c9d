"""Plain, slow fp64 CPU oracle for one rank's lap of ring attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP product
path never calls, links or imports anything here, and nothing here imports the
product package: the two share no code, no constants and no helpers.

Sources (the three web pages the method is taken from):

* [P1] "GPU ring attention" explainer (aicassindra.com).
* [P2] "Ring attention" hard MCQ page (zenaique.com).
* [P3] "Ring Attention：把超长序列沿设备环流动" (charlestar.github.io).

Every function is pinned in ``tests/test_oracle_pins.py`` against something
other than itself (torch's scaled-dot-product attention in float64, closed
forms, brute force on tiny inputs, the ring table printed on [P3]).  None of
its results is "parity unpinned".
"""

from .attention import (  # noqa: F401
    EMPTY,
    FULL,
    PARTIAL,
    allowed_mask,
    backward_block,
    backward_row_terms,
    blockwise_attention,
    brute_force_pair_count,
    dense_attention,
    live_pair_count,
    merge_states,
    online_block_update,
    online_finalize,
    online_state_init,
    ring_visit_order,
    shard_capacity,
    tile_classes,
    token_owner,
    tokens_of_rank,
)
