"""CPU oracle of the predictor-guided sparse FFN -- test infrastructure only.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The GPU library and its Python binding never do.
"""
from .sparse_ffn import (  # noqa: F401
    BAND, NORM_EPS, activations, band_neurons, dequant_q4_cols, dequant_q4_rows, ffn_dense, ffn_masked, layer,
    logical_weights, predictor_logits, layer_norm, stack, threshold_logit, token_masks, union_mask, with_hot_prefix,
)
