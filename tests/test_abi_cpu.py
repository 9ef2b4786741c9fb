"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and rejects bad
arguments on the host before anything is enqueued (fake, never-dereferenced pointers)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sffn.h")

from activation_sparse_ffn_predictor_amd import _lib  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sffn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sffn_predict", "sffn_forward", "sffn_forward_q4", "sffn_workspace_size", "sffn_status_string",
              "sffn_last_error", "sffn_mask_words"):
        assert n in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    h = _lib.lib()
    for n in declared_functions():
        assert hasattr(h, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported


def test_status_strings_and_sizes():
    assert _lib.status_string(0) == "ok"
    assert "workspace" in _lib.status_string(4)
    assert _lib.mask_words(1) == 1 and _lib.mask_words(64) == 1 and _lib.mask_words(65) == 2
    # [a: F*B fp32, for B > 1 at least ceil(F/64)*64 x ceil(B/16)*16 fp32][B > 1: xn B*D fp32]
    # [partial y: 16*B*D fp32 (B > 1) or 256*D fp32 (B = 1)][B > 1: k-share partials KS*2*F*B fp32]
    # [B > 1: token fragments, 2 planes of 4 ceil(D/128) x ceil(B/16) kB, + 16 powers of two per token tile]
    # [B > 1: largest |a| per row tile (16 rows up to 4 tokens, else 64) and token][h: B*r fp32]
    assert _lib.workspace_size(1, 4096, 11008, 256) == 44032 + 256 * 4096 * 4 + 1024
    # (k shares: none up to 4 tokens, 8 up to 8, 4 up to 16, 2 up to 32; token fragments in whole quads of 4 k blocks)
    assert _lib.workspace_size(8, 512, 100, 64) == 8192 + 16384 + 262144 + 51200 + (32768 + 256) + 256 + 2048
    assert _lib.workspace_size(3, 40, 7, 8) == 4096 + 512 + 7680 + 0 + (8192 + 256) + 256 + 256
    assert _lib.workspace_size(64, 512, 100, 64) == 32768 + 131072 + 2097152 + 0 + (4 * 32768 + 256) + 512 + 16384


A = 0x10000          # fake, 256-byte aligned, never dereferenced
MIS = 0x10002        # fake, misaligned


def _predict(**kw):
    a = dict(P1=A, P2=A, c=None, x=A, x_norm=0, B=1, D=512, F=2048, r=64, t=0.5, mask=A, logits=None, ws=A,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _lib.lib().sffn_predict(*a.values())


def _forward(**kw):
    a = dict(act=0, Wg=None, bg=None, Wu=A, bu=A, WdT=A, x=A, x_norm=0, B=1, D=512, F=2048, mask=A, active=A,
             n_active=A, y=A, ws=A, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _lib.lib().sffn_forward(*a.values())


def _forward_q4(**kw):
    Q = _lib._Q4(A, A)
    a = dict(act=1, Wg=Q, bg=A, Wu=Q, bu=None, WdT=Q, x=A, x_norm=0, B=1, D=512, F=2048, mask=A, active=A, n_active=A,
             y=A, ws=A, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _lib.lib().sffn_forward_q4(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(P1=None), 1), (dict(x=None), 1), (dict(mask=None), 1), (dict(ws=None), 1),
    (dict(B=0), 2), (dict(B=65), 2), (dict(D=4), 2), (dict(D=100), 2), (dict(D=16392), 2), (dict(F=0), 2),
    (dict(r=4), 2), (dict(r=100), 2), (dict(r=1032), 2), (dict(B=64, r=1024), 2),
    (dict(t=0.0), 6), (dict(t=1.0), 6), (dict(t=float("nan")), 6),
    (dict(P1=MIS), 3), (dict(x=MIS), 3), (dict(ws=A + 16), 3),
    (dict(ws_bytes=100), 4),
    # P2 [F, r] fp16 of 4 GiB: the kernels address it with 31-bit byte offsets, so the shape is refused
    (dict(D=256, F=1 << 21, r=1024), 2), (dict(D=256, F=1 << 20, r=1024), 2),
])
def test_predict_rejects(kw, status):
    assert _predict(**kw) == status
    assert _lib.lib().sffn_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(act=7), 5), (dict(act=1, Wg=None), 5),
    (dict(Wu=None), 1), (dict(WdT=None), 1), (dict(y=None), 1), (dict(active=None), 1), (dict(n_active=None), 1),
    (dict(B=3, F=32769), 2), (dict(B=8, D=4096, F=40000), 2), (dict(F=1 << 21, D=1024), 2),
    (dict(Wu=MIS), 3), (dict(y=A + 4), 3),
    (dict(ws_bytes=16), 4),
])
def test_forward_rejects(kw, status):
    assert _forward(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(act=1, Wg=_lib._Q4(None, None)), 5), (dict(Wu=_lib._Q4(A, None)), 1), (dict(D=520), 2),
    (dict(WdT=_lib._Q4(MIS, A)), 3), (dict(ws_bytes=0), 4), (dict(B=16, F=32832), 2),
])
def test_forward_q4_rejects(kw, status):
    assert _forward_q4(**kw) == status


def test_profile_calls_reject_bad_arguments():
    h = _lib.lib()
    assert h.sffn_profile_begin(9, 4) == 6
    assert h.sffn_profile_begin(0, 0) == 6
    assert h.sffn_profile_end(None, 0) < 0         # nothing started


def test_union_batches_are_routed_not_rejected():
    # B = 3 and B = 16 take the union kernels: shape accepted, the fake workspace size is what fails
    assert _forward(B=3, ws_bytes=16) == 4
    assert _forward_q4(B=16, ws_bytes=16) == 4
    assert _predict(B=5, ws_bytes=16) == 4


def test_forward_path_routing():
    assert _lib.forward_path("reglu", False, 1, 5120, 13824) == _lib.PATH_FUSED
    assert _lib.forward_path("relu", False, 1, 8192, 32768) == _lib.PATH_FUSED
    assert _lib.forward_path("reglu", False, 1, 8192, 1000) == _lib.PATH_DECODE   # ReGLU wider than 5120
    assert _lib.forward_path("relu", False, 1, 64, 33000) == _lib.PATH_DECODE     # more than 32768 neurons
    assert _lib.forward_path("reglu", True, 1, 8192, 28672) == _lib.PATH_FUSED
    assert _lib.forward_path("reglu", True, 1, 16384, 2048) == _lib.PATH_DECODE   # Q4_0 rows wider than 8192
    assert _lib.forward_path("reglu", False, 2, 4096, 11008) == _lib.PATH_DECODE
    assert _lib.forward_path("reglu", False, 2, 16384, 1024) == _lib.PATH_UNION    # 2 D above 16384
    assert _lib.forward_path("reglu", False, 4, 4096, 11008) == _lib.PATH_UNION
    assert _lib.forward_path("reglu", False, 4, 4096, 40000) == _lib.PATH_DECODE   # F too large for the union
    assert _lib.forward_path("relu", False, 8, 2048, 40000) == _lib.PATH_DECODE
    assert _lib.forward_path("reglu", False, 4, 5120, 13824) == _lib.PATH_UNION
    assert _lib.forward_path("relu", True, 64, 8192, 28672) == _lib.PATH_UNION
    assert _lib.lib().sffn_forward_path(5, 0, 1, 64, 64) == -1


def _predict_hot(**kw):
    a = dict(P1=A, P2=A, c=None, x=A, x_norm=0, B=1, D=512, F=2048, r=64, t=0.5, n_hot=10, mask=A, logits=None, ws=A,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _lib.lib().sffn_predict_hot(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(n_hot=-1), 6), (dict(n_hot=2049), 6), (dict(P2=None), 1), (dict(r=12), 2), (dict(t=1.5), 6),
    (dict(mask=MIS), 3), (dict(ws_bytes=8), 4),
    (dict(n_hot=0, ws_bytes=8), 4), (dict(n_hot=2048, ws_bytes=8), 4), (dict(B=9, n_hot=5, ws_bytes=8), 4),
])
def test_predict_hot_rejects(kw, status):
    # n_hot in 0..F passes validation (the fake workspace size is what fails in the last three)
    assert _predict_hot(**kw) == status


def test_squared_relu_is_accepted_on_every_path():
    assert _forward(act=2, ws_bytes=16) == 4
    assert _forward(act=2, B=3, ws_bytes=16) == 4
    assert _forward_q4(act=2, Wg=_lib._Q4(None, None), bg=None, bu=A, ws_bytes=16) == 4
    assert _lib.forward_path("sqrelu", False, 1, 8192, 32768) == _lib.PATH_FUSED   # as ReLU: up to D = 8192
    assert _lib.forward_path("sqrelu", False, 1, 8704, 1000) == _lib.PATH_DECODE
    assert _lib.forward_path("sqrelu", True, 1, 8192, 28672) == _lib.PATH_FUSED
    assert _lib.forward_path("sqrelu", False, 2, 4096, 11008) == _lib.PATH_DECODE
    assert _lib.forward_path("sqrelu", False, 4, 4096, 11008) == _lib.PATH_UNION
    assert _lib.forward_path(3, False, 1, 512, 2048) == -1


def _decode(**kw):
    a = dict(act=1, P1=A, P2=A, c=None, t=0.5, n_hot=0, Wg=A, bg=A, Wu=A, bu=None, WdT=A, x=A, x_norm=0, D=512, F=2048,
             r=64, mask=A, active=A, n_active=A, y=A, logits=None, ws=A, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return _lib.lib().sffn_decode(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(act=5), 5), (dict(Wg=None), 5), (dict(P1=None), 1), (dict(y=None), 1), (dict(active=None), 1),
    (dict(r=12), 2), (dict(r=2048), 2), (dict(t=0.0), 6), (dict(n_hot=-1), 6), (dict(n_hot=2049), 6),
    (dict(P2=MIS), 3), (dict(y=A + 4), 3), (dict(ws=A + 16), 3), (dict(ws_bytes=1000), 4),
    # sizes outside the folded kernel take the separate calls and fail there the same way
    (dict(D=8192, ws_bytes=1000), 4), (dict(F=40000, D=64, ws_bytes=1000), 4), (dict(D=8192, n_hot=-2), 6),
    # P2 of 4 GiB (folded and separate routes alike)
    (dict(D=256, F=1 << 21, r=1024), 2), (dict(act=0, Wg=None, bg=None, bu=A, D=64, F=1 << 21, r=1024), 2),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def test_decode_paths_and_workspace():
    assert _lib.decode_path("reglu", False, 4096, 11008, 256) == _lib.DECODE_FOLDED
    assert _lib.decode_path("reglu", False, 4096, 11008, 384) == _lib.DECODE_SEPARATE   # 8 rounds per row
    assert _lib.decode_path("reglu", False, 5120, 13824, 256) == _lib.DECODE_SEPARATE   # rows wider than 4096
    assert _lib.decode_path("relu", False, 4096, 32768, 512) == _lib.DECODE_SEPARATE   # 2 row steps x 8 rounds
    assert _lib.decode_path("relu", False, 4096, 32768, 64) == _lib.DECODE_FOLDED      # 2 row steps x 1 round
    assert _lib.decode_path("reglu", False, 8192, 1000, 64) == _lib.DECODE_SEPARATE    # ReGLU wider than 5120
    assert _lib.decode_path("relu", True, 512, 1000, 64) == _lib.DECODE_SEPARATE       # Q4_0
    assert _lib.decode_path(9, False, 512, 1000, 64) == -1
    # one token: the activation region holds at least the 256 workgroups' 16-byte decision bitmaps
    assert _lib.workspace_size(1, 64, 1, 8) == 4096 + 256 * 64 * 4 + 256


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # the product path has no non-HIP implementation: without libsffn.so every call raises
    monkeypatch.setattr(_lib, "_handle", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libsffn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.workspace_size(1, 64, 64, 8)


def test_bench_refuses_more_than_one_gpu():
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout


def test_p2_just_below_the_limit_passes_validation():
    # F * r * 2 = 2 GiB - 2 KiB: accepted; the fake workspace size is what fails
    assert _predict(D=256, F=(1 << 20) - 1, r=1024, ws_bytes=16) == 4
    assert _predict_hot(D=256, F=(1 << 20) - 1, r=1024, n_hot=0, ws_bytes=16) == 4


def test_decode_noalloc_validates_sizes_first():
    h = _lib.lib()
    assert h.sffn_noalloc_scratch_bytes() == 16 << 20
    args = dict(act=0, P1=A, P2=A, c=None, t=0.5, n_hot=0, Wg=None, bg=None, Wu=A, bu=A, WdT=A, x=A, x_norm=0,
                D=16384, F=1 << 20, r=8, mask=A, active=A, n_active=A, y=A, logits=None, stream=None)
    assert h.sffn_decode_noalloc(*args.values()) == 4                        # scratch too small for these sizes
    assert "scratch" in h.sffn_last_error().decode()
    args.update(D=0)
    assert h.sffn_decode_noalloc(*args.values()) == 2
