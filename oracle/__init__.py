"""fp64 CPU oracle for the Gated DeltaNet (GDN) hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``gated_deltanet_03_amd``) never imports it, and this package never
imports the product path: the two share no code.

Contents
--------
``gdn_oracle``    token-by-token recurrence (optionally recording the states at
                  chunk boundaries), the input prologue (q/k l2norm, sigmoid
                  beta, softplus gate), compact capture, replay, snapshot
``chunked_form``  the chunked (UT / WY) reorganisation of the same recurrence in
                  fp64, used only as an independent cross-check of the recurrence

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(hand-worked example, exact-rational product form, closed forms, invariants).
The inverse-GQA head map (value head h reads key head h // (Hv/Hq)) is a
convention the pages do not define: "parity unpinned" beyond that convention.
The same holds for the prologue's formulas (the pages name gate and scaling
conventions but give none): each is pinned to its closed forms, not to a page.
"""

from .gdn_oracle import (  # noqa: F401
    sequence_bounds,
    recurrent,
    prologue,
    capture,
    replay,
    snapshot,
    record_width,
)
from .chunked_form import chunked  # noqa: F401
