"""Stored layouts of one layer (set-up, off the hot path).

PowerInfer pages, Turkish article, "Neuron placement and management": neurons are stored in a chosen order
and a neuron table ties every stored neuron to its position in the original matrix. Here the chosen order
puts neurons by descending activation probability (hot neurons first) and ``perm[j]`` is the original id of
stored neuron j. Every per-neuron tensor is permuted the same way; W_down is stored transposed (row k =
column k) so that a neuron's down-projection weights are one contiguous row ("Neuron-aware operator":
operators work on individual rows and columns).

Q4_0 rows are packed as the library expects: for every block of 32 weights along d_model, byte i holds
element i in its low nibble and element 16 + i in its high nibble; the scales form a separate [F, D/32]
fp16 plane.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch


def hot_first_perm(probs: np.ndarray) -> np.ndarray:
    """Stored order: descending activation probability, ties by original id. perm[j] = original id."""
    return np.lexsort((np.arange(len(probs)), -np.asarray(probs))).astype(np.int64)


def pack_q4_rows(q: torch.Tensor) -> torch.Tensor:
    """q [N, K] uint8 values 0..15 -> [N, K/2] uint8 nibble bytes (K % 32 == 0)."""
    N, K = q.shape
    v = q.reshape(N, K // 32, 2, 16)
    return (v[:, :, 0, :] | (v[:, :, 1, :] << 4)).reshape(N, K // 2).contiguous()


def unpack_q4_rows(p: torch.Tensor) -> torch.Tensor:
    """Inverse of pack_q4_rows."""
    N, H = p.shape
    v = p.reshape(N, H // 16, 1, 16)
    return torch.cat([v & 15, v >> 4], dim=2).reshape(N, 2 * H).contiguous()


def pack_layer(t: Dict[str, torch.Tensor], perm: np.ndarray, device=None) -> Dict[str, torch.Tensor]:
    """Logical tensors of one layer (generator layout, see synthgen) -> stored layout on the same device.

    Output keys: P1 [r,D], P2 [F,r], c [F] (if given), b_gate or b_up [F], and either W_gate/W_up/W_downT
    [F,D] fp16 or Q_gate/S_gate, Q_up/S_up, Q_downT/S_downT (nibbles [F,D/2], scales [F,D/32]), perm [F] int32.
    """
    dev = device or t["P1"].device
    p = torch.as_tensor(perm, dtype=torch.long, device=dev)
    out = {"P1": t["P1"].contiguous(), "P2": t["P2"][p].contiguous(), "perm": p.to(torch.int32)}
    for k in ("c", "b_gate", "b_up"):
        if k in t and t[k] is not None:
            out[k] = t[k][p].contiguous()
    if "W_up" in t:
        if "W_gate" in t:
            out["W_gate"] = t["W_gate"][p].contiguous()
        out["W_up"] = t["W_up"][p].contiguous()
        out["W_downT"] = t["W_down"].t()[p].contiguous()
    else:
        if "Q_gate" in t:
            out["Q_gate"] = pack_q4_rows(t["Q_gate"][p])
            out["S_gate"] = t["S_gate"][p].contiguous()
        out["Q_up"] = pack_q4_rows(t["Q_up"][p])
        out["S_up"] = t["S_up"][p].contiguous()
        out["Q_downT"] = pack_q4_rows(t["Q_down"].t()[p])
        out["S_downT"] = t["S_down"].t()[p].contiguous()
    return out
