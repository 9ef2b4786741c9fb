"""Shared helpers of the GPU parity tests: run one layer through the C ABI and compare with the oracle.

Comparison rules (the pages leave ties open; the design notes list them):
  * set of predicted-active neurons: equal to the oracle's union mask after mapping stored ids back through
    the neuron table, except for band neurons (some token's oracle logit within 1e-4 of the threshold and no
    token clearly above it), which may go either way;
  * compaction: active[0:n] is strictly ascending, in range, and equal to the set bits of the mask;
  * y: per token, max |y_gpu - y_ref| <= 2e-3 * max |y_ref|, where y_ref is the oracle's masked FFN under the
    oracle mask with band neurons set as the GPU decided (either decision is valid); y_ref == 0 => y_gpu == 0;
  * always-active prefix (n_hot > 0): the first n_hot stored neurons must be set (they are never band neurons)
    and their logits are +infinity.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import synthgen as sg
from activation_sparse_ffn_predictor_amd import _lib
from activation_sparse_ffn_predictor_amd.pack import hot_first_perm, pack_layer

Y_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class LayerCase:
    wl: sg.Workload
    layer: int
    host: dict          # logical numpy tensors
    w: dict             # oracle fp64 weights
    dev: dict           # packed device tensors
    perm: np.ndarray


def make_case(wl, layer=0, device="cuda:0", with_c=True, perm="hot", from_device_generator=False):
    host = sg.layer_host(wl, layer, with_c=with_c)
    w = oracle.logical_weights(host)
    if perm == "hot":
        p = hot_first_perm(sg.neuron_probs(wl, layer))
    elif perm == "identity":
        p = np.arange(wl.F)
    else:
        p = np.random.default_rng(1234 + layer).permutation(wl.F)
    if from_device_generator:
        logical = sg.layer_device(wl, layer, device, with_c=with_c)
    else:
        logical = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in host.items()}
    dev = pack_layer(logical, p)
    del logical
    return LayerCase(wl, layer, host, w, dev, np.asarray(p))


def host_case(wl, layer=0, perm=None):
    """Oracle-side case of a layer whose device tensors live elsewhere (a resident stack): logical host tensors,
    fp64 weights and the stored order (hot-first by default, as the stack packs it)."""
    host = sg.layer_host(wl, layer)
    p = hot_first_perm(sg.neuron_probs(wl, layer)) if perm is None else perm
    return LayerCase(wl, layer, host, oracle.logical_weights(host), {}, np.asarray(p))


def run_gpu(case: LayerCase, x: torch.Tensor, x_norm=False, t=None, want_logits=True, n_hot=0):
    wl, d = case.wl, case.dev
    B, D = x.shape
    dev = x.device
    mask = torch.full((_lib.mask_words(wl.F),), -1, dtype=torch.int64, device=dev)   # garbage-filled outputs
    active = torch.full((wl.F,), -7, dtype=torch.int32, device=dev)
    n_active = torch.full((1,), -7, dtype=torch.int32, device=dev)
    y = torch.full((B, D), float("nan"), dtype=torch.float32, device=dev)
    logits = torch.full((B, wl.F), float("nan"), dtype=torch.float32, device=dev) if want_logits else None
    ws = torch.zeros(_lib.workspace_size(B, D, wl.F, wl.r), dtype=torch.uint8, device=dev)
    tt = wl.t if t is None else t
    _lib.predict(d["P1"], d["P2"], d.get("c"), x, tt, mask, ws, logits=logits, x_norm=x_norm, n_hot=n_hot)
    if wl.wdtype == "q4":
        g = (d["Q_gate"], d["S_gate"]) if wl.act == "reglu" else None
        _lib.forward_q4(wl.act, g, d.get("b_gate"), (d["Q_up"], d["S_up"]), d.get("b_up"), (d["Q_downT"], d["S_downT"]),
                        x, mask, active, n_active, y, ws, x_norm=x_norm)
    else:
        _lib.forward(wl.act, d.get("W_gate"), d.get("b_gate"), d["W_up"], d.get("b_up"), d["W_downT"], x, mask, active,
                     n_active, y, ws, x_norm=x_norm)
    torch.cuda.synchronize(dev)
    return dict(mask=mask.cpu().numpy().view(np.uint64), active=active.cpu().numpy(), n=int(n_active.item()),
                y=y.cpu().numpy().astype(np.float64),
                logits=None if logits is None else logits.cpu().numpy().astype(np.float64))


def run_decode(case: LayerCase, x: torch.Tensor, x_norm=False, t=None, want_logits=True, n_hot=0):
    """One token through sffn_decode (predictor and forward in one call); outputs as run_gpu."""
    wl, d = case.wl, case.dev
    B, D = x.shape
    dev = x.device
    mask = torch.full((_lib.mask_words(wl.F),), -1, dtype=torch.int64, device=dev)   # garbage-filled outputs
    active = torch.full((wl.F,), -7, dtype=torch.int32, device=dev)
    n_active = torch.full((1,), -7, dtype=torch.int32, device=dev)
    y = torch.full((B, D), float("nan"), dtype=torch.float32, device=dev)
    logits = torch.full((B, wl.F), float("nan"), dtype=torch.float32, device=dev) if want_logits else None
    ws = torch.full((_lib.workspace_size(B, D, wl.F, wl.r),), 0xA5, dtype=torch.uint8, device=dev)
    _lib.decode(wl.act, d["P1"], d["P2"], d.get("c"), wl.t if t is None else t, d.get("W_gate"), d.get("b_gate"),
                d["W_up"], d.get("b_up"), d["W_downT"], x, mask, active, n_active, y, ws, x_norm=x_norm, n_hot=n_hot,
                logits=logits)
    torch.cuda.synchronize(dev)
    return dict(mask=mask.cpu().numpy().view(np.uint64), active=active.cpu().numpy(), n=int(n_active.item()),
                y=y.cpu().numpy().astype(np.float64),
                logits=None if logits is None else logits.cpu().numpy().astype(np.float64))


def mask_bits(words: np.ndarray, F: int) -> np.ndarray:
    bits = np.unpackbits(words.astype("<u8").view(np.uint8), bitorder="little")
    return bits[:F].astype(bool)


def check(case: LayerCase, x_host: np.ndarray, res: dict, x_norm=False, t=None, tol=Y_TOL, n_hot=0):
    """Compare one GPU layer result with the oracle; raise AssertionError with details on mismatch.
    Returns a dict of statistics."""
    wl, F = case.wl, case.wl.F
    tt = wl.t if t is None else t
    xo = oracle.layer_norm(x_host) if x_norm else np.atleast_2d(x_host).astype(np.float64)
    z = oracle.predictor_logits(case.w["P1"], case.w["P2"], xo, case.w.get("c"))
    m_ref = oracle.union_mask(oracle.token_masks(z, tt))
    band = oracle.band_neurons(z, tt)
    hot = np.zeros(F, dtype=bool)                       # original ids of the always-active stored prefix
    hot[case.perm[:n_hot]] = True
    if n_hot:
        stored = oracle.with_hot_prefix(m_ref[case.perm], n_hot)   # the oracle's rule, in stored order
        m_ref = np.zeros(F, dtype=bool)
        m_ref[case.perm[stored]] = True
        band &= ~hot
    # GPU set in original ids
    bits = mask_bits(res["mask"], F)
    # bits beyond F must be zero
    nwords = res["mask"].shape[0]
    allbits = np.unpackbits(res["mask"].astype("<u8").view(np.uint8), bitorder="little")
    assert not allbits[F:nwords * 64].any(), "mask bits beyond F are set"
    m_gpu = np.zeros(F, dtype=bool)
    m_gpu[case.perm[bits]] = True
    diff = (m_gpu != m_ref) & ~band
    assert not diff.any(), f"active sets differ outside the band at {np.nonzero(diff)[0][:10]} (of {diff.sum()})"
    # compaction
    n = res["n"]
    assert n == int(bits.sum()), f"n_active {n} != popcount {int(bits.sum())}"
    ids = res["active"][:n]
    assert np.all(np.diff(ids) > 0) if n > 1 else True, "active ids not strictly ascending"
    assert np.array_equal(ids, np.nonzero(bits)[0]), "active ids differ from mask bits"
    # y under the oracle mask with band neurons as the GPU decided
    m_use = np.where(band, m_gpu, m_ref)
    y_ref = oracle.ffn_masked(wl.act, xo, case.w, m_use)
    y = res["y"]
    assert np.all(np.isfinite(y)), "non-finite y"
    errs = []
    for b in range(y.shape[0]):
        ymax = np.max(np.abs(y_ref[b]))
        err = np.max(np.abs(y[b] - y_ref[b]))
        if ymax == 0.0:
            assert err == 0.0, f"token {b}: y_ref == 0 but max|y| = {err}"
            errs.append(0.0)
        else:
            assert err <= tol * ymax, f"token {b}: max err {err:.3e} > {tol} * {ymax:.3e}"
            errs.append(err / ymax)
    if res.get("logits") is not None:
        lg = res["logits"][:, case.perm.argsort()]    # back to original ids
        assert np.all(np.isposinf(lg[:, hot])), "logits of the always-active prefix are not +inf"
        lerr = np.max(np.abs(lg[:, ~hot] - z[:, ~hot])) if (~hot).any() else 0.0
    else:
        lerr = None
    return dict(n=n, band=int(band.sum()), flips=int((m_gpu != m_ref).sum()), rel_err=max(errs) if errs else 0.0,
                logit_err=lerr, density=n / F)
