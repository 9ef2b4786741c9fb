"""CPU oracle of the predictor-guided sparse FFN (test infrastructure only).

This module is a plain, slow, fp64 NumPy statement of what the hot path
computes. It is test infrastructure: only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it. The GPU library never calls
it and shares no code with it.

Sources (the PowerInfer pages):
  * "Online stage: neuron-aware inference engine" (Turkish article) -- the
    engine predicts which neurons are active and skips the inactive ones; the
    sparse operators work on individual rows and columns of the weights.
  * "Adaptive sparsity predictors" (Turkish article) -- a small predictor per
    layer decides which MLP neurons fire; it runs on every token.
  * "Neuron placement and management" (Turkish article) -- neuron tables tie
    every stored neuron to its position in the original matrix, so results
    come out in original neuron order.
  * "Neuron-aware operator" (Turkish article) -- inactive neurons and their
    weights are skipped by the matrix products; no dense conversion.
  * Summary bullets and "Limitations/FAQ" (Indonesian digest) -- only ReLU,
    ReGLU and squared-ReLU FFNs are handled; ReLU output 0 is what makes a
    neuron inactive (Hacker News thread on the same page).
  * "Quantization" (Indonesian digest) -- INT4 Q4_0 weights.

Readings where the pages are silent (each is also listed in the design notes):
  * predictor: z = P2 (P1 x) + c, low rank, no nonlinearity between factors;
    active iff sigmoid(z) > t, i.e. z > ln(t / (1 - t)); strict inequality.
  * union over a batch of tokens: one mask M = OR over tokens; every token is
    computed over M.
  * ReLU FFN: a_k = max(0, W_up[k] x + b_up[k]); squared ReLU: a_k =
    max(0, W_up[k] x + b_up[k])^2; ReGLU: a_k = max(0, W_gate[k] x + b_gate[k]) * (W_up[k] x);
    y = W_down a, no down bias.
  * always-active prefix: the neurons stored first are the hottest ones ("Neuron placement and
    management"); a layer may declare its first n_hot stored neurons always active, and they join the
    predicted set whatever their logits (the GPU then reads no predictor rows for them).
  * Q4_0: blocks of 32 consecutive weights along d_model in every neuron's
    row (W_gate, W_up) or column (W_down), w = (q - 8) * s.
  * layer chaining: parameter-free normalisation of each token, x' = (y - mean(y)) / sqrt(var(y) + 1e-6)
    (population variance); it keeps every layer's input centred at unit scale, which the Zipf and predictor
    calibration of the synthetic workloads assume (weights of the Q4_0 workload have mean -s/2, so an
    uncentred stack drifts towards a common-mode input).

Parity pins: see tests/test_oracle_pins.py (brute force with exact rationals,
closed forms, library special cases, invariants).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

NORM_EPS = 1e-6
BAND = 1e-4


# ----------------------------------------------------------------------------- weights
def dequant_q4_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Q4_0 rows: q [N, K] integers in 0..15, s [N, K/32] scales; w[n, k] = (q[n, k] - 8) * s[n, k // 32].
    ("Quantization", Indonesian digest: INT4 Q4_0.) Exact in fp64."""
    q = np.asarray(q).astype(np.float64)
    s = np.asarray(s).astype(np.float64)
    N, K = q.shape
    assert s.shape == (N, K // 32) and K % 32 == 0
    return (q - 8.0) * np.repeat(s, 32, axis=1)


def dequant_q4_cols(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Q4_0 for W_down [D, F] with scale blocks of 32 along d_model (axis 0): s [D/32, F]."""
    return dequant_q4_rows(np.asarray(q).T, np.asarray(s).T).T


def logical_weights(t: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """fp64 logical weights of one layer from the generator's tensors (fp16 upcast exactly, or Q4_0
    dequantised exactly). Keys: P1 [r,D], P2 [F,r], W_gate [F,D] (ReGLU), W_up [F,D], W_down [D,F],
    b_gate / b_up [F], c [F] (optional)."""
    w: Dict[str, np.ndarray] = {}
    w["P1"] = np.asarray(t["P1"], dtype=np.float64)
    w["P2"] = np.asarray(t["P2"], dtype=np.float64)
    if "W_up" in t:
        for k in ("W_gate", "W_up", "W_down"):
            if k in t:
                w[k] = np.asarray(t[k], dtype=np.float64)
    else:
        if "Q_gate" in t:
            w["W_gate"] = dequant_q4_rows(t["Q_gate"], t["S_gate"])
        w["W_up"] = dequant_q4_rows(t["Q_up"], t["S_up"])
        w["W_down"] = dequant_q4_cols(t["Q_down"], t["S_down"])
    for k in ("b_gate", "b_up", "c"):
        if k in t and t[k] is not None:
            w[k] = np.asarray(t[k], dtype=np.float64)
    return w


# ----------------------------------------------------------------------------- predictor
def threshold_logit(t: float) -> float:
    """sigmoid(z) > t  <=>  z > ln(t / (1 - t)) for 0 < t < 1 (sigmoid is strictly increasing)."""
    assert 0.0 < t < 1.0
    return math.log(t / (1.0 - t))


def predictor_logits(P1: np.ndarray, P2: np.ndarray, x: np.ndarray, c: Optional[np.ndarray] = None) -> np.ndarray:
    """Low-rank predictor logits z[b, k] = sum_j P2[k, j] * (sum_d P1[j, d] * x[b, d]) + c[k]
    ("Adaptive sparsity predictors": a small per-layer predictor evaluated on every token). fp64."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    h = x @ np.asarray(P1, dtype=np.float64).T          # [B, r]
    z = h @ np.asarray(P2, dtype=np.float64).T          # [B, F]
    if c is not None:
        z = z + np.asarray(c, dtype=np.float64)[None, :]
    return z


def token_masks(z: np.ndarray, t: float) -> np.ndarray:
    """Per-token predicted-active masks [B, F]: sigmoid(z) > t, decided in logit space."""
    return np.asarray(z) > threshold_logit(t)


def union_mask(masks: np.ndarray) -> np.ndarray:
    """One mask for a batch: neuron k is computed for every token if any token predicts it active."""
    return np.any(np.atleast_2d(masks), axis=0)


def band_neurons(z: np.ndarray, t: float, eps: float = BAND) -> np.ndarray:
    """Neurons whose union membership is not decided beyond rounding: some token's logit lies within eps of
    the threshold and no token's logit exceeds the threshold by eps or more. [F] bool."""
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    tau = threshold_logit(t)
    near = np.any(np.abs(z - tau) < eps, axis=0)
    clearly_on = np.any(z > tau + eps, axis=0)
    return near & ~clearly_on


# ----------------------------------------------------------------------------- FFN
def activations(act: str, x: np.ndarray, w: Dict[str, np.ndarray]) -> np.ndarray:
    """Dense neuron activations a [B, F] (fp64).
    relu  : a = max(0, W_up x + b_up)
    sqrelu: a = max(0, W_up x + b_up)^2   (squared ReLU, Indonesian digest, summary bullets)
    reglu : a = max(0, W_gate x + b_gate) * (W_up x)"""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    u = x @ w["W_up"].T
    if act in ("relu", "sqrelu"):
        if "b_up" in w:
            u = u + w["b_up"][None, :]
        a = np.maximum(u, 0.0)
        return a * a if act == "sqrelu" else a
    if act == "reglu":
        g = x @ w["W_gate"].T
        if "b_gate" in w:
            g = g + w["b_gate"][None, :]
        return np.maximum(g, 0.0) * u
    raise ValueError(act)


def ffn_masked(act: str, x: np.ndarray, w: Dict[str, np.ndarray], mask: np.ndarray) -> np.ndarray:
    """Dense FFN with the activations of neurons outside ``mask`` set to zero, y [B, D]
    ("Neuron-aware operator": inactive neurons contribute nothing)."""
    a = activations(act, x, w)
    a = a * np.asarray(mask, dtype=np.float64)[None, :]
    return a @ w["W_down"].T


def ffn_dense(act: str, x: np.ndarray, w: Dict[str, np.ndarray]) -> np.ndarray:
    """Plain dense FFN y = W_down act(x)."""
    return activations(act, x, w) @ w["W_down"].T


def layer_norm(y: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """Parameter-free normalisation per token: x' = (y - mean(y)) / sqrt(mean((y - mean(y))^2) + eps)."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    c = y - np.mean(y, axis=1, keepdims=True)
    return c / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)


def with_hot_prefix(mask: np.ndarray, n_hot: int) -> np.ndarray:
    """The computed set when the first n_hot stored neurons are always active: M | {k < n_hot}."""
    m = np.array(mask, dtype=bool, copy=True)
    m[:max(0, int(n_hot))] = True
    return m


def layer(act: str, x: np.ndarray, w: Dict[str, np.ndarray], t: float = 0.5,
          n_hot: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One sparse-FFN layer for a batch x [B, D]: returns (z [B,F], computed mask [F], y [B,D]). The computed
    mask is the union of the tokens' predicted masks, plus the first n_hot stored neurons when n_hot > 0."""
    z = predictor_logits(w["P1"], w["P2"], x, w.get("c"))
    m = with_hot_prefix(union_mask(token_masks(z, t)), n_hot)
    return z, m, ffn_masked(act, x, w, m)


def stack(act: str, x: np.ndarray, layers, t: float = 0.5, n_hot=0):
    """Decode step through a stack: layer l consumes x_l, and x_{l+1} = layer_norm(y_l). ``n_hot`` is one
    always-active prefix length for every layer or a sequence of one per layer. Layers may differ in predictor
    rank. Returns the list of (z, mask, y) per layer."""
    out = []
    xl = np.atleast_2d(np.asarray(x, dtype=np.float64))
    hots = list(n_hot) if np.ndim(n_hot) else [int(n_hot)] * len(layers)
    for w, nh in zip(layers, hots):
        z, m, y = layer(act, xl, w, t, nh)
        out.append((z, m, y))
        xl = layer_norm(y)
    return out
