"""Predictor-guided, neuron-aware sparse FFN for one AMD MI355X (gfx950).

The compute path is the HIP library libsffn.so (C ABI in include/sffn.h); this package only binds it
(``_lib``), packs stored layouts (``pack``) and drives a resident layer stack (``stack``). There is no
CPU fallback: calls fail if the library is missing.
"""
from ._lib import (  # noqa: F401
    ACT_RELU, ACT_REGLU, EXPORTS, SffnError, forward, forward_q4, lib, mask_words, predict, status_string,
    workspace_size,
)

__all__ = ["ACT_RELU", "ACT_REGLU", "EXPORTS", "SffnError", "forward", "forward_q4", "lib", "mask_words", "predict",
           "status_string", "workspace_size"]
