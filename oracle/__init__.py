"""Plain FP64 CPU oracle of the chunkwise state scan — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never imports, links or executes it, and
this package shares no code with that path: the only thing both sides read is
the seeded inputs drawn by ``workloads``.

Contents
--------
gdr_ref   token-serial gated delta rule (outputs, pre-chunk states, final
          states), per-segment summaries (local state and transition
          product) and their serial composition.
abc_ref   token-serial ABC normalised slot recurrence (cumulative
          normaliser z, pre-chunk key/value slot states, final states).
abc_bwd_ref  the reverse (dH) recurrence of the ABC slot states: gradients
          of the states at chunk boundaries from gradients of the slot
          scores and of the value read.
gdr_bwd_ref  the reverse (gradient) recurrence of the gated delta rule:
          gradients at chunk boundaries, of the initial state and of the
          chunk form's write vectors.
kda_ref   the delta rule with a per-key-channel decay, token by token, and
          its per-chunk (WY) form for the prepared factors.

Every function is the plain definition, token by token, in float64 (or in
exact rationals when handed ``fractions.Fraction`` object arrays); there is
no blocking, chunking or reordering beyond recording the state at chunk
starts.
"""

from .gdr_ref import (  # noqa: F401
    CHUNK,
    chunk_counts,
    gdr_recurrent_fp64,
    gdr_scan_sequence,
    segment_bounds,
    gdr_segment_summaries_fp64,
    gdr_segment_compose_fp64,
)
from .abc_ref import abc_forward_fp64, abc_readout_sequence, abc_recurrent_fp64, abc_scan_sequence, abc_weighted_scan  # noqa: F401
from .abc_bwd_ref import abc_backward_fp64, abc_backward_sequence  # noqa: F401
from .chunked_ref import gdr_chunked_fp64, chunked_scan_sequence, chunk_factors  # noqa: F401
from .gdr_bwd_ref import gdr_backward_fp64, gdr_backward_sequence  # noqa: F401
from .kda_ref import kda_chunked_fp64, kda_recurrent_fp64, kda_scan_sequence  # noqa: F401
