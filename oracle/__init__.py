"""CPU oracle for the FVAttn block-sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables); inputs come from the
``workloads`` generator, which holds none of the method's arithmetic.

It is plain numpy, written for checking by eye rather than speed:

* ``blocks``    - video-aware 3D-tile block organisation;
* ``hilbert``   - the Hilbert-curve block organisation (tokens in curve
                  order, cut into consecutive 128-token blocks);
* ``routing``   - mean-pooled block scores, Top-p cut with a Top-k floor,
                  slack-aware augmentation, CSR lists (all in float64);
* ``attention`` - exact softmax attention restricted to the kept blocks.

Sources: the FVAttn pages (arXiv 2607.16190, "FVAttn: Adaptive Sparse
Attention with Runtime Load Balancing for Video Generation"): the abstract
(routing front end, materialised mask), the paperlayer.ai summary's section 2
"Background and Related Work" (dynamic block-sparse attention, Top-k vs Top-p)
and section 3 "FVAttn Design" (Sparse-routing frontend, Slack-Aware Sparse
Augmentation).  Each function cites its passage.

Pins: every function is pinned by ``tests/test_oracle_*.py`` against brute
force, closed forms, library routines and hand-worked fixtures in
``tests/golden/``.  The synthetic input generator is the only unpinned part
("parity unpinned": it is this project's own definition, not the pages').
"""
from .blocks import BlockLayout
from .hilbert import HilbertLayout
from . import routing, attention

__all__ = ["BlockLayout", "HilbertLayout", "routing", "attention"]
