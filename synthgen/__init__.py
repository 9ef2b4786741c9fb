"""Seeded synthetic inputs for the predictor-guided sparse FFN.

This package makes inputs only; it holds no part of the sparse-FFN arithmetic
(no predictor, no threshold, no FFN). Both the CPU checker and the GPU path
draw their inputs from here.

Workloads follow the five FFN shapes the PowerInfer pages speak about
(ReLU-family FFNs of Falcon-40B and Llama2 7B/13B/70B, "Supported models"
and "Performance evaluation" sections), with sizes, weight distributions,
sparsity targets and Zipf hot-neuron profiles fixed per workload below.

Every weight and input element is a pure function of (seed, tensor tag,
layer or step, logical element index) through a counter-based generator
(Philox4x32-10, see ``csrc/synth.hip``), so any slice can be regenerated on
the host or filled in place on the GPU with identical bits.

Logical (un-permuted, un-transposed, unpacked) tensor shapes of one layer:
  P1      [r, D]  fp16     predictor first factor
  P2      [F, r]  fp16     predictor second factor
  c       [F]     fp32     predictor bias (calibrated reading; may be omitted)
  W_gate  [F, D]  fp16     ReGLU only, with b_gate [F] fp32
  W_up    [F, D]  fp16     with b_up [F] fp32 for ReLU
  W_down  [D, F]  fp16
  Q4_0 workloads replace each W by (q [same shape] uint8 in 0..15,
  s [blocks of 32 along d_model] fp16): W_gate/W_up scales [F, D/32],
  W_down scales [D/32, F]; w = (q - 8) * s.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

MASTER_SEED = 20231221

# tensor tags (the third Philox counter word)
TAG_P1, TAG_P2 = 1, 2
TAG_W_GATE, TAG_W_UP, TAG_W_DOWN = 3, 4, 5
TAG_Q_GATE, TAG_S_GATE, TAG_Q_UP, TAG_S_UP, TAG_Q_DOWN, TAG_S_DOWN = 6, 7, 8, 9, 10, 11
TAG_X_DECODE, TAG_X_PROMPT, TAG_X_TEST = 12, 13, 14

# standard deviation of the centred Irwin-Hall sum of eight 16-bit uniforms
IH8_STD = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)
Q4_LO, Q4_HI = 0.001, 0.01
ZIPF_CAP = 0.99


@dataclass(frozen=True)
class Workload:
    """One synthetic FFN-stack workload."""
    name: str
    index: int          # workload id, folded into the generator key
    D: int              # d_model
    F: int              # d_ffn (neurons)
    r: int              # predictor rank
    L: int              # layers
    act: str            # "relu" / "sqrelu" (W_up + b_up, W_down) or "reglu" (W_gate + b_gate, W_up, W_down)
    wdtype: str         # "f16" or "q4"
    sigma_w: float      # weight std (fp16 workloads)
    sigma_p: float      # predictor factor std
    zipf_s: float       # Zipf exponent of the hot-neuron profile
    density: float      # mean activation probability
    batches: Tuple[int, ...] = (1,)
    steps: int = 128    # decode steps
    prompt: int = 0     # prompt tokens handled as one union-mask batch (0 = none)
    t: float = 0.5      # predictor sigmoid threshold
    ranks: Optional[Tuple[int, ...]] = None   # per-layer predictor ranks, cycled over layers (None: r everywhere)

    def rank(self, layer: int) -> int:
        """Predictor rank of one layer."""
        return self.ranks[layer % len(self.ranks)] if self.ranks else self.r

    @property
    def n_mats(self) -> int:
        return 3 if self.act == "reglu" else 2

    def pre_std(self) -> float:
        """Std of one pre-activation W[k]·x for x ~ N(0, I)."""
        if self.wdtype == "q4":
            var_q = (16 ** 2 - 1) / 12.0 + 0.25            # E[(q-8)^2], q uniform on 0..15
            e_s2 = (Q4_LO ** 2 + Q4_LO * Q4_HI + Q4_HI ** 2) / 3.0
            return math.sqrt(self.D * var_q * e_s2)
        return self.sigma_w * math.sqrt(self.D)

    def logit_std(self, layer: int = 0) -> float:
        """Std of one predictor logit (P2 P1 x)[k] for x ~ N(0, I) at the layer's rank."""
        return self.sigma_p ** 2 * math.sqrt(self.rank(layer) * self.D)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("toy_relu", 0, D=512, F=2048, r=64, L=1, act="relu", wdtype="f16", sigma_w=0.02,
                 sigma_p=0.05, zipf_s=1.1, density=0.10, steps=1),
        Workload("relullama_7b", 1, D=4096, F=11008, r=256, L=32, act="reglu", wdtype="f16", sigma_w=0.02,
                 sigma_p=0.05, zipf_s=1.1, density=0.12, steps=128),
        Workload("llama2_13b", 2, D=5120, F=13824, r=256, L=40, act="reglu", wdtype="f16", sigma_w=0.02,
                 sigma_p=0.05, zipf_s=1.2, density=0.10, batches=(1, 4, 8), steps=128),
        Workload("falcon_40b", 3, D=8192, F=32768, r=512, L=60, act="relu", wdtype="f16", sigma_w=0.015,
                 sigma_p=0.05, zipf_s=1.1, density=0.05, steps=128),
        Workload("llama2_70b_q4", 4, D=8192, F=28672, r=512, L=80, act="reglu", wdtype="q4", sigma_w=0.0,
                 sigma_p=0.05, zipf_s=1.1, density=0.15, steps=64, prompt=64),
    ]
}
ALIASES = {"c1": "toy_relu", "c2": "relullama_7b", "c3": "llama2_13b", "c4": "falcon_40b", "c5": "llama2_70b_q4",
           "toy": "toy_relu", "7b": "relullama_7b", "13b": "llama2_13b", "40b": "falcon_40b", "70b": "llama2_70b_q4"}


def workload(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


# Per-layer rank schedule: multiples of the base rank, cycled over the layers (mean 1, so the stack holds as many
# predictor bytes as with the base rank everywhere). A stand-in for ranks sized per layer; no training is done.
RANK_FACTORS = (0.5, 1.0, 1.5, 1.0)


def with_rank_schedule(base: Workload, factors: Sequence[float] = RANK_FACTORS) -> Workload:
    """Copy of a workload whose layers cycle through ranks factor * r (multiples of 8); r becomes the largest."""
    ranks = tuple(max(8, int(round(f * base.r / 8.0)) * 8) for f in factors)
    return custom(base, r=max(ranks), ranks=ranks, name=base.name + "_adaptive_rank")


def custom(base: Workload, **kw) -> Workload:
    """A reduced or altered copy of a workload (test shapes)."""
    d = dict(base.__dict__)
    d.update(kw)
    return Workload(**d)


# ----------------------------------------------------------------------------- native fills
_lib_handle = None


def lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        h = ctypes.CDLL(LIB_PATH)
        u64, u32, vp, i32, f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        h.synth_fill_normal_f16.argtypes = [vp, i32, u64, u32, u32, u64, u64, f32, vp]
        h.synth_fill_normal_f32.argtypes = [vp, i32, u64, u32, u32, u64, u64, f32, vp]
        h.synth_fill_q4.argtypes = [vp, i32, u64, u32, u32, u64, u64, vp]
        h.synth_fill_uniform_f16.argtypes = [vp, i32, u64, u32, u32, u64, u64, f32, f32, vp]
        h.synth_philox4x32_10.argtypes = [ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(u32)]
        h.synth_f32_to_f16.argtypes = [vp, vp, u64]
        h.synth_f32_to_f16.restype = None
        for f in ("synth_fill_normal_f16", "synth_fill_normal_f32", "synth_fill_q4", "synth_fill_uniform_f16"):
            getattr(h, f).restype = i32
        h.synth_philox4x32_10.restype = None
        _lib_handle = h
    return _lib_handle


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> Tuple[int, int, int, int]:
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib().synth_philox4x32_10(c, k, o)
    return tuple(int(v) for v in o)


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    """The generator's own fp32 -> fp16 (round to nearest even) conversion, for tests."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.float16)
    lib().synth_f32_to_f16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def key_seed(wl_index: int, seed: int = MASTER_SEED) -> int:
    """64-bit Philox key of one workload."""
    return (int(seed) & 0xFFFFFFFF) | ((int(wl_index) & 0xFFFFFFFF) << 32)


def normal_scale(sigma: float) -> float:
    return float(np.float32(sigma / IH8_STD))


def _ptr_and_dev(buf):
    """(address, on_device, stream) of a numpy array or torch tensor."""
    if isinstance(buf, np.ndarray):
        assert buf.flags.c_contiguous
        return buf.ctypes.data, 0, None
    import torch  # only device fills need torch
    assert buf.is_contiguous()
    if buf.is_cuda:
        return buf.data_ptr(), 1, torch.cuda.current_stream(buf.device).cuda_stream
    return buf.data_ptr(), 0, None


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"synth fill failed (rc={rc})")


def fill_normal(out, key: int, tag: int, layer: int, sigma: float, start: int = 0):
    """Fill fp16/fp32 ``out`` (numpy or torch, host or device) with N(0, sigma^2) draws of elements
    start .. start+out.size-1 of the logical tensor."""
    p, dev, st = _ptr_and_dev(out)
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    is16 = (out.dtype == np.float16) if isinstance(out, np.ndarray) else (str(out.dtype) == "torch.float16")
    fn = lib().synth_fill_normal_f16 if is16 else lib().synth_fill_normal_f32
    _check(fn(p, dev, key, tag, layer, start, n, normal_scale(sigma), st))
    return out


def fill_q4(out, key: int, tag: int, layer: int, start: int = 0):
    p, dev, st = _ptr_and_dev(out)
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    _check(lib().synth_fill_q4(p, dev, key, tag, layer, start, n, st))
    return out


def fill_scales(out, key: int, tag: int, layer: int, start: int = 0):
    p, dev, st = _ptr_and_dev(out)
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    _check(lib().synth_fill_uniform_f16(p, dev, key, tag, layer, start, n, Q4_LO, Q4_HI - Q4_LO, st))
    return out


# ----------------------------------------------------------------------------- hot-neuron profile
def zipf_probs(F: int, s: float, mean: float, cap: float = ZIPF_CAP) -> np.ndarray:
    """Activation probability by rank 1..F: p(rank) = min(cap, C * rank^-s), C chosen by bisection so that
    mean(p) equals ``mean`` (fp64)."""
    ranks = np.arange(1, F + 1, dtype=np.float64)
    base = ranks ** (-s)
    lo, hi = 0.0, cap / base[-1] + 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * base).mean() < mean:
            lo = mid
        else:
            hi = mid
    return np.minimum(cap, hi * base)


def neuron_ranks(wl: Workload, layer: int, seed: int = MASTER_SEED) -> np.ndarray:
    """Zipf rank (1..F) of every neuron of one layer; hot neurons are scattered by a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), wl.index, int(layer), 7])))
    return rng.permutation(wl.F).astype(np.int64) + 1


def neuron_probs(wl: Workload, layer: int, seed: int = MASTER_SEED) -> np.ndarray:
    """Target activation probability p_k of every neuron (logical order), fp64."""
    p_by_rank = zipf_probs(wl.F, wl.zipf_s, wl.density)
    return p_by_rank[neuron_ranks(wl, layer, seed) - 1]


def saturated_count(wl: Workload, layer: int, seed: int = MASTER_SEED) -> int:
    """Neurons of one layer whose activation probability sits at the cap (the hottest ones; stored first in a
    hot-first order)."""
    return int(np.count_nonzero(neuron_probs(wl, layer, seed) >= ZIPF_CAP))


def _ndtri(p: np.ndarray) -> np.ndarray:
    from scipy.special import ndtri
    return ndtri(p)


def act_bias(wl: Workload, layer: int, seed: int = MASTER_SEED) -> np.ndarray:
    """Bias of the activation input (b_up for ReLU, b_gate for ReGLU): pre_std * Phi^-1(p_k), so that a neuron
    fires with probability p_k for x ~ N(0, I). fp32."""
    return (wl.pre_std() * _ndtri(neuron_probs(wl, layer, seed))).astype(np.float32)


def predictor_bias(wl: Workload, layer: int, seed: int = MASTER_SEED) -> np.ndarray:
    """Calibrated predictor bias c_k = logit_std * Phi^-1(p_k): the predictor marks neuron k with
    probability p_k for x ~ N(0, I) at threshold 0.5. fp32."""
    return (wl.logit_std(layer) * _ndtri(neuron_probs(wl, layer, seed))).astype(np.float32)


# ----------------------------------------------------------------------------- logical layer tensors
def layer_shapes(wl: Workload, layer: int = 0) -> Dict[str, Tuple[Tuple[int, ...], str, int]]:
    """name -> (shape, dtype, tag) of the logical tensors of one layer."""
    D, F, r = wl.D, wl.F, wl.rank(layer)
    s = {"P1": ((r, D), "f16", TAG_P1), "P2": ((F, r), "f16", TAG_P2)}
    if wl.wdtype == "f16":
        if wl.act == "reglu":
            s["W_gate"] = ((F, D), "f16", TAG_W_GATE)
        s["W_up"] = ((F, D), "f16", TAG_W_UP)
        s["W_down"] = ((D, F), "f16", TAG_W_DOWN)
    else:
        if wl.act == "reglu":
            s["Q_gate"] = ((F, D), "u8", TAG_Q_GATE)
            s["S_gate"] = ((F, D // 32), "f16", TAG_S_GATE)
        s["Q_up"] = ((F, D), "u8", TAG_Q_UP)
        s["S_up"] = ((F, D // 32), "f16", TAG_S_UP)
        s["Q_down"] = ((D, F), "u8", TAG_Q_DOWN)
        s["S_down"] = ((D // 32, F), "f16", TAG_S_DOWN)
    return s


def _fill_named(name: str, out, wl: Workload, layer: int, key: int, tag: int):
    if name in ("P1", "P2"):
        fill_normal(out, key, tag, layer, wl.sigma_p)
    elif name.startswith("W_"):
        fill_normal(out, key, tag, layer, wl.sigma_w)
    elif name.startswith("Q_"):
        fill_q4(out, key, tag, layer)
    else:
        fill_scales(out, key, tag, layer)


def layer_host(wl: Workload, layer: int, seed: int = MASTER_SEED, names: Optional[Sequence[str]] = None,
               with_c: bool = True) -> Dict[str, np.ndarray]:
    """Logical tensors of one layer as host numpy arrays (fp16 / uint8 / fp32)."""
    key = key_seed(wl.index, seed)
    out: Dict[str, np.ndarray] = {}
    for name, (shape, dt, tag) in layer_shapes(wl, layer).items():
        if names is not None and name not in names:
            continue
        a = np.empty(shape, dtype={"f16": np.float16, "u8": np.uint8}[dt])
        _fill_named(name, a, wl, layer, key, tag)
        out[name] = a
    bias = act_bias(wl, layer, seed)
    if wl.act == "reglu":
        out["b_gate"] = bias
    else:
        out["b_up"] = bias
    if with_c:
        out["c"] = predictor_bias(wl, layer, seed)
    return out


def layer_device(wl: Workload, layer: int, device="cuda", seed: int = MASTER_SEED, with_c: bool = True):
    """Logical tensors of one layer as torch tensors on ``device`` (filled in place by the device generator)."""
    import torch
    key = key_seed(wl.index, seed)
    tdt = {"f16": torch.float16, "u8": torch.uint8}
    out = {}
    for name, (shape, dt, tag) in layer_shapes(wl, layer).items():
        t = torch.empty(shape, dtype=tdt[dt], device=device)
        _fill_named(name, t, wl, layer, key, tag)
        out[name] = t
    bias = torch.from_numpy(act_bias(wl, layer, seed)).to(device)
    out["b_gate" if wl.act == "reglu" else "b_up"] = bias
    if with_c:
        out["c"] = torch.from_numpy(predictor_bias(wl, layer, seed)).to(device)
    return out


def inputs(wl: Workload, step: int, B: int, tag: int = TAG_X_DECODE, seed: int = MASTER_SEED, out=None):
    """Token inputs x [B, D] ~ N(0, 1) fp32 of one step (numpy unless ``out`` is given)."""
    key = key_seed(wl.index, seed)
    if out is None:
        out = np.empty((B, wl.D), dtype=np.float32)
    fill_normal(out, key, tag, step, 1.0)
    return out
