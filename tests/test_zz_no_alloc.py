"""sffn_decode_noalloc (the library's own per-GPU scratch as workspace) against sffn_decode with a caller workspace
on the same inputs: two calls in a row, the second at smaller sizes (the scratch keeps the first call's contents),
each compared with the caller-workspace call (same kernels: identical masks, ids and outputs) and with the oracle.
Runs last (it shares the process-wide scratch with nothing else)."""
import numpy as np
import pytest
import torch

import synthgen as sg
from activation_sparse_ffn_predictor_amd import _lib
from parity_util import check, make_case, run_decode, say

pytestmark = pytest.mark.gpu


def run_noalloc(case, x):
    wl, d = case.wl, case.dev
    B, D = x.shape
    dev = x.device
    mask = torch.full((_lib.mask_words(wl.F),), -1, dtype=torch.int64, device=dev)   # garbage-filled outputs
    active = torch.full((wl.F,), -7, dtype=torch.int32, device=dev)
    n_active = torch.full((1,), -7, dtype=torch.int32, device=dev)
    y = torch.full((B, D), float("nan"), dtype=torch.float32, device=dev)
    logits = torch.full((B, wl.F), float("nan"), dtype=torch.float32, device=dev)
    _lib.decode_noalloc(wl.act, d["P1"], d["P2"], d.get("c"), wl.t, d.get("W_gate"), d.get("b_gate"), d["W_up"],
                        d.get("b_up"), d["W_downT"], x, mask, active, n_active, y, logits=logits)
    torch.cuda.synchronize(dev)
    return dict(mask=mask.cpu().numpy().view(np.uint64), active=active.cpu().numpy(), n=int(n_active.item()),
                y=y.cpu().numpy().astype(np.float64), logits=logits.cpu().numpy().astype(np.float64))


def test_noalloc_two_calls_second_smaller(gpu_ready):
    assert _lib.noalloc_scratch_bytes() == 16 << 20
    shapes = [sg.workload("llama2_13b"),                                             # separate kernels, 5.3 MB
              sg.custom(sg.workload("relullama_7b"), D=512, F=2000, r=64, L=1)]      # folded kernel, smaller
    for wl in shapes:
        assert _lib.workspace_size(1, wl.D, wl.F, wl.r) <= _lib.noalloc_scratch_bytes()
        case = make_case(wl, 0, gpu_ready)
        x = sg.inputs(wl, 3, 1, tag=sg.TAG_X_TEST)
        xt = torch.from_numpy(x).to(gpu_ready)
        say(f"[noalloc {wl.name} D={wl.D} F={wl.F} r={wl.r}] path {_lib.decode_path(wl.act, False, wl.D, wl.F, wl.r)}")
        ref = run_decode(case, xt)
        got = run_noalloc(case, xt)
        assert np.array_equal(got["mask"], ref["mask"]) and got["n"] == ref["n"]
        assert np.array_equal(got["active"][:got["n"]], ref["active"][:ref["n"]])
        assert np.array_equal(got["y"], ref["y"])
        st = check(case, x, got)
        say("   ", st)


def test_noalloc_rejects_sizes_beyond_the_scratch(gpu_ready):
    wl = sg.custom(sg.workload("toy_relu"), D=16384, F=1 << 20, r=8)
    assert _lib.workspace_size(1, wl.D, wl.F, wl.r) > _lib.noalloc_scratch_bytes()
    x = torch.zeros((1, wl.D), dtype=torch.float32, device=gpu_ready)
    z = torch.zeros(16, dtype=torch.float16, device=gpu_ready)
    P2 = torch.zeros((wl.F, wl.r), dtype=torch.float16, device=gpu_ready)
    out = torch.zeros(16, dtype=torch.int32, device=gpu_ready)
    with pytest.raises(_lib.SffnError) as ei:
        _lib.decode_noalloc("relu", z, P2, None, 0.5, None, None, z, None, z, x, out, out, out, x)
    assert ei.value.status == 4
