"""ctypes binding of libsffn.so: argument marshalling only, every computation runs in the HIP library.

Names and argument order follow include/sffn.h. Tensors are torch tensors on the GPU (device pointers are
taken with ``data_ptr()``); the stream is torch's current stream unless one is given.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# SFFN_LIB_PATH selects another build of the same library (the host-sanitized one of the CPU checks)
LIB_PATH = os.environ.get("SFFN_LIB_PATH") or os.path.join(HERE, "libsffn.so")

ACT_RELU, ACT_REGLU, ACT_SQRELU = 0, 1, 2
ACTS = {"relu": ACT_RELU, "reglu": ACT_REGLU, "sqrelu": ACT_SQRELU}

EXPORTS = ("sffn_status_string", "sffn_last_error", "sffn_workspace_size", "sffn_mask_words", "sffn_predict",
           "sffn_predict_hot", "sffn_forward", "sffn_forward_q4", "sffn_profile_begin", "sffn_profile_end",
           "sffn_forward_path", "sffn_decode", "sffn_decode_path", "sffn_decode_noalloc",
           "sffn_noalloc_scratch_bytes")
K_PRED_H, K_PRED_Z, K_ROWS, K_COLS = 0, 1, 2, 3


class SffnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class _Q4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p)]


_handle = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built (there is no fallback path)."""
    global _handle
    if _handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the sparse FFN has no non-HIP implementation)")
        h = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        h.sffn_status_string.argtypes, h.sffn_status_string.restype = [i32], ctypes.c_char_p
        h.sffn_last_error.argtypes, h.sffn_last_error.restype = [], ctypes.c_char_p
        h.sffn_workspace_size.argtypes, h.sffn_workspace_size.restype = [i32, i32, i32, i32], sz
        h.sffn_mask_words.argtypes, h.sffn_mask_words.restype = [i32], i32
        h.sffn_predict.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]
        h.sffn_predict.restype = i32
        h.sffn_predict_hot.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
        h.sffn_predict_hot.restype = i32
        h.sffn_forward.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        h.sffn_forward.restype = i32
        h.sffn_forward_q4.argtypes = [i32, _Q4, vp, _Q4, vp, _Q4, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        h.sffn_forward_q4.restype = i32
        h.sffn_decode.argtypes = [i32, vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp,
                                  vp, vp, sz, vp]
        h.sffn_decode.restype = i32
        h.sffn_decode_noalloc.argtypes = [i32, vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp,
                                          vp, vp, vp, vp]
        h.sffn_decode_noalloc.restype = i32
        h.sffn_noalloc_scratch_bytes.argtypes, h.sffn_noalloc_scratch_bytes.restype = [], sz
        h.sffn_decode_path.argtypes, h.sffn_decode_path.restype = [i32, i32, i32, i32, i32], i32
        h.sffn_profile_begin.argtypes, h.sffn_profile_begin.restype = [i32, i32], i32
        h.sffn_forward_path.argtypes, h.sffn_forward_path.restype = [i32, i32, i32, i32, i32], i32
        h.sffn_profile_end.argtypes, h.sffn_profile_end.restype = [ctypes.POINTER(ctypes.c_float), i32], i32
        _handle = h
    return _handle


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream, ref):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream(ref.device).cuda_stream


def _check(rc: int, where: str):
    if rc != 0:
        h = lib()
        raise SffnError(rc, where, f"{h.sffn_status_string(rc).decode()}: {h.sffn_last_error().decode()}")


def status_string(s: int) -> str:
    return lib().sffn_status_string(s).decode()


def workspace_size(B: int, D: int, F: int, r: int) -> int:
    return int(lib().sffn_workspace_size(B, D, F, r))


def mask_words(F: int) -> int:
    return int(lib().sffn_mask_words(F))


def predict(P1, P2, c, x, t: float, mask, ws, logits=None, x_norm: bool = False, stream=None, n_hot: int = 0):
    """sffn_predict (n_hot = 0) or sffn_predict_hot (stored neurons 0 .. n_hot-1 always active). P1 [r, D] fp16,
    P2 [F, r] fp16, c [F] fp32 or None, x [B, D] fp32, mask [ceil(F/64)] int64 (bit pattern), ws uint8
    workspace, logits [B, F] fp32 or None."""
    B, D = x.shape
    F, r = P2.shape
    if n_hot:
        rc = lib().sffn_predict_hot(_p(P1), _p(P2), _p(c), _p(x), int(bool(x_norm)), B, D, F, r, float(t), int(n_hot),
                                    _p(mask), _p(logits), _p(ws), _nbytes(ws), _stream(stream, x))
        _check(rc, "sffn_predict_hot")
        return
    rc = lib().sffn_predict(_p(P1), _p(P2), _p(c), _p(x), int(bool(x_norm)), B, D, F, r, float(t), _p(mask), _p(logits),
                            _p(ws), _nbytes(ws), _stream(stream, x))
    _check(rc, "sffn_predict")


def forward(act, W_gate, b_gate, W_up, b_up, W_downT, x, mask, active, n_active, y, ws, x_norm: bool = False,
            stream=None):
    """sffn_forward. W_gate/W_up/W_downT [F, D] fp16 in stored order, biases [F] fp32 or None,
    active [F] int32 and n_active [1] int32 outputs, y [B, D] fp32 output."""
    B, D = x.shape
    F = W_up.shape[0]
    rc = lib().sffn_forward(ACTS.get(act, act), _p(W_gate), _p(b_gate), _p(W_up), _p(b_up), _p(W_downT), _p(x),
                            int(bool(x_norm)), B, D, F, _p(mask), _p(active), _p(n_active), _p(y), _p(ws), _nbytes(ws),
                            _stream(stream, x))
    _check(rc, "sffn_forward")


def forward_q4(act, W_gate, b_gate, W_up, b_up, W_downT, x, mask, active, n_active, y, ws, x_norm: bool = False,
               stream=None):
    """sffn_forward_q4. Each W is a pair (q [F, D/2] uint8, s [F, D/32] fp16) or None (W_gate for ReLU)."""
    B, D = x.shape
    F = W_up[0].shape[0]
    g = _Q4(*(map(_p, W_gate))) if W_gate is not None else _Q4(None, None)
    rc = lib().sffn_forward_q4(ACTS.get(act, act), g, _p(b_gate), _Q4(*map(_p, W_up)), _p(b_up),
                               _Q4(*map(_p, W_downT)), _p(x), int(bool(x_norm)), B, D, F, _p(mask), _p(active),
                               _p(n_active), _p(y), _p(ws), _nbytes(ws), _stream(stream, x))
    _check(rc, "sffn_forward_q4")


def decode(act, P1, P2, c, t: float, W_gate, b_gate, W_up, b_up, W_downT, x, mask, active, n_active, y, ws,
           x_norm: bool = False, n_hot: int = 0, logits=None, stream=None):
    """sffn_decode: predictor and sparse FFN of one layer for one token (x [1, D]); fp16 weights as in forward."""
    B, D = x.shape
    F, r = P2.shape
    rc = lib().sffn_decode(ACTS.get(act, act), _p(P1), _p(P2), _p(c), float(t), int(n_hot), _p(W_gate), _p(b_gate),
                           _p(W_up), _p(b_up), _p(W_downT), _p(x), int(bool(x_norm)), D, F, r, _p(mask), _p(active),
                           _p(n_active), _p(y), _p(logits), _p(ws), _nbytes(ws), _stream(stream, x))
    _check(rc, "sffn_decode")


def decode_noalloc(act, P1, P2, c, t: float, W_gate, b_gate, W_up, b_up, W_downT, x, mask, active, n_active, y,
                   x_norm: bool = False, n_hot: int = 0, logits=None, stream=None):
    """sffn_decode_noalloc: sffn_decode with the library's own per-GPU device scratch as its workspace (no
    allocation; calls that overlap in time on one GPU race on the scratch)."""
    B, D = x.shape
    F, r = P2.shape
    rc = lib().sffn_decode_noalloc(ACTS.get(act, act), _p(P1), _p(P2), _p(c), float(t), int(n_hot), _p(W_gate),
                                   _p(b_gate), _p(W_up), _p(b_up), _p(W_downT), _p(x), int(bool(x_norm)), D, F, r,
                                   _p(mask), _p(active), _p(n_active), _p(y), _p(logits), _stream(stream, x))
    _check(rc, "sffn_decode_noalloc")


def noalloc_scratch_bytes() -> int:
    return int(lib().sffn_noalloc_scratch_bytes())


DECODE_SEPARATE, DECODE_FOLDED = 0, 1


def decode_path(act, q4: bool, D: int, F: int, r: int) -> int:
    """Which kernels sffn_decode runs for these sizes: DECODE_FOLDED (h, then the predictor's second stage inside
    the fused gather, then the sum of partials) or DECODE_SEPARATE (the sffn_predict and sffn_forward calls)."""
    return int(lib().sffn_decode_path(ACTS.get(act, act), int(bool(q4)), D, F, r))


PATH_DECODE, PATH_FUSED, PATH_UNION = 0, 1, 2


def forward_path(act, q4: bool, B: int, D: int, F: int) -> int:
    """Which kernels a forward call of these sizes runs (PATH_DECODE, PATH_FUSED or PATH_UNION)."""
    return int(lib().sffn_forward_path(ACTS.get(act, act), int(bool(q4)), B, D, F))


def profile_begin(kernel: int, max_launches: int):
    """Time every launch of `kernel` (K_PRED_H, K_PRED_Z, K_ROWS, K_COLS) with the kernel's own device timestamps
    (eager launches only)."""
    _check(lib().sffn_profile_begin(int(kernel), int(max_launches)), "sffn_profile_begin")


def _profile_times(fn, name, max_launches):
    buf = (ctypes.c_float * max(1, max_launches))()
    n = fn(buf, max_launches)
    if n < 0:
        _check(-n, name)
    return [float(buf[i]) for i in range(min(n, max_launches))]


def profile_end(max_launches: int):
    """Per-launch elapsed milliseconds of the bracketed launches (list of floats); frees the events."""
    return _profile_times(lib().sffn_profile_end, "sffn_profile_end", max_launches)
