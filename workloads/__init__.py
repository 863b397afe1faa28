"""Seeded synthetic inputs for the chunkwise state-scan workloads.

This package holds only input recipes: random draws, the token-level
normalisation of q/k, the gate pre-activations mapped through sigmoid /
log-sigmoid, and the cast into the storage dtype.  It contains none of the
scan arithmetic, so both the FP64 oracle tests and the HIP path can consume
the very same arrays without sharing any code of the method.
"""

from .synth import (  # noqa: F401
    GdrInputs,
    AbcInputs,
    CONFIGS,
    make_gdr,
    make_abc,
    make_config,
    random_lengths,
)
