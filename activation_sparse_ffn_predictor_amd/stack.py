"""A resident sparse-FFN stack on one GPU: every layer's predictor and weights in HBM, one decode step =
sffn_predict + sffn_forward (or sffn_forward_q4) per layer, layer l+1 reading layer l's output through the
library's normalise-on-load option (a parameter-free LayerNorm). A step can be captured once into a HIP graph and replayed.

The pages' decode touches the whole model for every token (Turkish article, motivation section); the stack
is the FFN part of that, with the neuron order of every layer chosen hot-first (pack.hot_first_perm).

Layers may differ in predictor rank (Turkish article, "Adaptive sparsity predictors": the predictor is sized per
layer), and with ``hot_prefix`` each layer's saturated neurons, stored first, are declared always active so the
predictor reads no rows for them (sffn_predict_hot).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

import synthgen as sg

from . import _lib
from .pack import hot_first_perm, pack_layer


class SparseFFNStack:
    def __init__(self, wl: sg.Workload, device="cuda:0", layers: Optional[List[int]] = None, with_c: bool = True,
                 max_batch: int = 1, seed: int = sg.MASTER_SEED, hot_prefix: bool = False, fold_predictor: bool = True):
        self.wl = wl
        self.device = torch.device(device)
        self.layer_ids = list(range(wl.L)) if layers is None else list(layers)
        self.q4 = wl.wdtype == "q4"
        self.with_c = with_c
        self.max_batch = max_batch
        self.fold_predictor = fold_predictor
        self.ranks = [wl.rank(l) for l in self.layer_ids]
        self.n_hot = [sg.saturated_count(wl, l, seed) if hot_prefix else 0 for l in self.layer_ids]
        self.layers: List[Dict[str, torch.Tensor]] = []
        for l in self.layer_ids:
            logical = sg.layer_device(wl, l, self.device, seed=seed, with_c=with_c)
            perm = hot_first_perm(sg.neuron_probs(wl, l, seed))
            self.layers.append(pack_layer(logical, perm))
            del logical
        torch.cuda.synchronize(self.device)
        L, F, D = len(self.layer_ids), wl.F, wl.D
        self.nw = _lib.mask_words(F)
        self.mask = torch.zeros((L, self.nw), dtype=torch.int64, device=self.device)
        self.active = torch.zeros((L, F), dtype=torch.int32, device=self.device)
        self.n_active = torch.zeros((L,), dtype=torch.int32, device=self.device)
        self.y = torch.zeros((L, max_batch, D), dtype=torch.float32, device=self.device)
        self.ws = torch.zeros(_lib.workspace_size(max_batch, D, F, max(self.ranks)), dtype=torch.uint8,
                              device=self.device)
        self.x_in = torch.zeros((max_batch, D), dtype=torch.float32, device=self.device)
        self.graphs = {}

    # ------------------------------------------------------------------ one layer
    def layer_call(self, i: int, x: torch.Tensor, x_norm: bool, y: torch.Tensor, logits=None):
        """Predict + forward of stored layer i on input x [B, D]; writes self.mask[i], active[i], n_active[i], y."""
        t, wl = self.layers[i], self.wl
        if self.fold_predictor and x.shape[0] == 1 and not self.q4:
            # one token, fp16: sffn_decode (predictor stage 2 folded into the row gather where it applies)
            _lib.decode(wl.act, t["P1"], t["P2"], t.get("c"), wl.t, t.get("W_gate"), t.get("b_gate"), t["W_up"],
                        t.get("b_up"), t["W_downT"], x, self.mask[i], self.active[i], self.n_active[i:i + 1], y,
                        self.ws, x_norm=x_norm, n_hot=self.n_hot[i], logits=logits)
            return
        _lib.predict(t["P1"], t["P2"], t.get("c"), x, wl.t, self.mask[i], self.ws, logits=logits, x_norm=x_norm,
                     n_hot=self.n_hot[i])
        if self.q4:
            g = (t["Q_gate"], t["S_gate"]) if wl.act == "reglu" else None
            _lib.forward_q4(wl.act, g, t.get("b_gate"), (t["Q_up"], t["S_up"]), t.get("b_up"),
                            (t["Q_downT"], t["S_downT"]), x, self.mask[i], self.active[i], self.n_active[i:i + 1], y,
                            self.ws, x_norm=x_norm)
        else:
            _lib.forward(wl.act, t.get("W_gate"), t.get("b_gate"), t["W_up"], t.get("b_up"), t["W_downT"], x,
                         self.mask[i], self.active[i], self.n_active[i:i + 1], y, self.ws, x_norm=x_norm)

    def decode_path(self, i: int, B: int) -> int:
        """The kernels of layer i's call for B tokens: _lib.DECODE_FOLDED when sffn_decode runs the predictor's
        second stage inside the row gather, else DECODE_SEPARATE (sffn_predict, then the forward call)."""
        if not (self.fold_predictor and B == 1 and not self.q4):
            return _lib.DECODE_SEPARATE
        return _lib.decode_path(self.wl.act, False, self.wl.D, self.wl.F, self.ranks[i])

    def folded(self, i: int, B: int) -> bool:
        """Whether layer i's call for B tokens runs the predictor's second stage in the row-gather kernel."""
        return self.decode_path(i, B) != _lib.DECODE_SEPARATE

    # ------------------------------------------------------------------ decode step
    def step(self, B: int = 1):
        """One pass through every layer for the B tokens in self.x_in[:B]; outputs land in self.y[:, :B]."""
        x = self.x_in[:B]
        for i in range(len(self.layers)):
            y = self.y[i, :B]
            self.layer_call(i, x, i > 0, y)
            x = y

    def capture(self, B: int = 1):
        """Capture step(B) into a HIP graph (after one eager warm-up)."""
        self.step(B)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(B)
        self.graphs[B] = g
        return g

    def replay(self, B: int = 1):
        self.graphs[B].replay()

    # ------------------------------------------------------------------ accounting
    def active_weight_bytes_per_row(self) -> int:
        wl = self.wl
        row = (wl.D // 2 + 2 * (wl.D // 32)) if self.q4 else 2 * wl.D
        return wl.n_mats * row

    def predictor_bytes(self) -> int:
        """Predictor bytes one step reads over the whole stack: P1, and the rows of P2 outside the always-active
        prefix."""
        wl = self.wl
        return sum(2 * (r * wl.D + (wl.F - h) * r) for r, h in zip(self.ranks, self.n_hot))
