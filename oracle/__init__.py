"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to anything here, and nothing here imports the
product path.

Everything is written from these pages:

* "Fast Inference and Training at Scale" (saravankumar25), sections 6.1 KV
  Caching, 6.2 Grouped Query Attention, 6.3 PagedAttention and 6.21
  FlashAttention (definition of attention, the standard nine-step algorithm,
  tiling and online softmax).
* "Hardware Co-Design" (mbrenndoerfer, Efficiency Frontiers), the online
  softmax update for m_i, l_i and O_i.
* "Week 13. GPUs and FlashAttention" (snula), Step 2 (per-row state m, d, o
  rescaled by e^(m_old - m_new); logsumexp kept per row; causal block skip)
  and "Common mistakes" (the -inf guard on fully masked blocks).
* "FlashAttention scaling, multi-GPU training and weight quantization"
  (itimpress.au), section 1 (rescaling postponed to the end of the inner loop).

The FP8 forward's reference lives in ``oracle.fp8``: the E4M3 encoding, the
power-of-two block scales and the rotation of Q and K ("FlashAttention
scaling, multi-GPU training and weight quantization", section 1, FP8 support:
block quantization and incoherent processing), and the exact attention of the
dequantized tensors.  It is pinned by ``tests/test_oracle_fp8_pins.py``
(format landmarks, brute-force rounding, exhaustive scale search, lossless
round trips, rotation invariance, planted mistakes).

Parity status: every public function is pinned by ``tests/test_oracle_pins.py``
against closed forms, a hand-derived worked example, library routines and
brute force; ``sdpa_backward`` against central finite differences, fp64 torch
autograd of a separately written forward, and the key-shift, value-sum and
constant-value closed forms; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    kv_head_of,
    sdpa,
    sdpa_rows,
    online_softmax_normalised,
    online_softmax_deferred,
    gather_pages,
    paged_decode,
    paged_multi_query,
    mla_decode,
    split_partials,
    merge_partials,
    sdpa_backward,
)
from . import fp8  # noqa: F401,E402
