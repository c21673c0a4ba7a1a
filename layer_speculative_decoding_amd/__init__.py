"""MI355X (gfx950) hot path of layer-parallel ("fuzzy") speculative decoding.

The computation lives in libspec.so (HIP kernels behind the C ABI of
include/spec.h); this package only marshals arguments (`api`) and drives the
round loop (`runtime`).
"""
from ._lib import (EXPORTS, SPEC_BF16, SPEC_F32, SPEC_MLP_PARALLEL, SPEC_MLP_SEQUENTIAL, SpecError,
                   LIB_PATH, load)

__all__ = ["EXPORTS", "SPEC_BF16", "SPEC_F32", "SPEC_MLP_PARALLEL", "SPEC_MLP_SEQUENTIAL", "SpecError",
           "LIB_PATH", "load"]
