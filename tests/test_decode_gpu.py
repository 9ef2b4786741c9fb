"""GPU parity of sffn_decode (one token: predictor and sparse FFN in one call) against the CPU oracle, and against
the separate sffn_predict / sffn_forward calls on the same inputs.

Where the folded path applies, the predictor's second stage runs inside the row gather: every workgroup decides
the neurons it owns and gathers the active ones, and the mask and ascending ids are assembled beside the sum of
the partials. The cases cover every chunk-round count of a P2 row (r = 8 .. 1024, ragged ranks), owned-row counts
of one and two row steps (F up to 32768), tiny F (fewer neurons than workgroups), the always-active prefix, the
threshold extremes, normalised input, all three activations, and the sizes where sffn_decode falls back to the
separate calls.
"""
import numpy as np
import pytest
import torch

import synthgen as sg
from activation_sparse_ffn_predictor_amd import _lib
from parity_util import check, make_case, run_decode, run_gpu, say

pytestmark = pytest.mark.gpu


def _x(wl, B, step=0, tag=sg.TAG_X_TEST):
    return sg.inputs(wl, step, B, tag=tag)


def small(base, **kw):
    return sg.custom(sg.workload(base), **kw)


CASES = [
    ("relu_f16", small("c1", D=256, F=1000, r=72, L=1)),
    ("reglu_f16", small("c2", D=512, F=1250, r=64, L=1, density=0.2)),
    ("sqrelu_f16", small("c1", D=1024, F=3000, r=256, L=1, act="sqrelu", density=0.15)),
    ("reglu_r8", small("c2", D=256, F=700, r=8, L=1, density=0.3)),
    ("relu_r136", small("c1", D=512, F=5000, r=136, L=1, density=0.1)),        # 17 chunks: 4 rounds, ragged
    ("reglu_r256_one_step", small("c2", D=2048, F=16384, r=256, L=1, density=0.08)),
    ("reglu_two_steps", small("c2", D=2048, F=20000, r=128, L=1, density=0.08)),
    ("relu_f32768_r64", small("c1", D=1024, F=32768, r=64, L=1, density=0.05)),
    ("reglu_d4096", small("c2", D=4096, F=3000, r=128, L=1, density=0.1)),
]


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(gpu_ready, name, wl):
    assert _lib.decode_path(wl.act, False, wl.D, wl.F, wl.r) == _lib.DECODE_FOLDED, name
    case = make_case(wl, 0, gpu_ready)
    for step in range(2):
        x = _x(wl, 1, step)
        say(f"[decode {name}] step {step}")
        st = check(case, x, run_decode(case, torch.from_numpy(x).to(gpu_ready)))
        say("   ", st)
        assert st["logit_err"] < 1e-4


@pytest.mark.parametrize("name,wl", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_decode_equals_separate_calls(gpu_ready, name, wl):
    case = make_case(wl, 0, gpu_ready)
    x = torch.from_numpy(_x(wl, 1, 3)).to(gpu_ready)
    a, b = run_decode(case, x), run_gpu(case, x)
    # same decisions (the logits are the same sums in another order, so only band neurons could differ)
    assert np.array_equal(a["mask"], b["mask"]) and a["n"] == b["n"]
    assert np.array_equal(a["active"][:a["n"]], b["active"][:b["n"]])
    assert np.max(np.abs(a["y"] - b["y"])) <= 1e-5 * np.max(np.abs(b["y"]))
    c = run_decode(case, x)
    assert np.array_equal(a["y"], c["y"]) and np.array_equal(a["mask"], c["mask"])   # deterministic


@pytest.mark.parametrize("n_hot", [1, 255, 256, 257, 700, -1])
def test_decode_hot_prefix(gpu_ready, n_hot):
    wl = CASES[1][1]
    n_hot = wl.F if n_hot < 0 else n_hot
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, 1, 4)
    st = check(case, x, run_decode(case, torch.from_numpy(x).to(gpu_ready), n_hot=n_hot), n_hot=n_hot)
    say(f"[decode hot {n_hot}]", st)
    assert st["n"] >= n_hot


@pytest.mark.parametrize("F", [1, 63, 64, 65, 255, 257])
def test_decode_tiny_neuron_counts(gpu_ready, F):
    wl = small("c1", D=64, F=F, r=8, L=1, density=0.5)
    case = make_case(wl, 0, gpu_ready)
    for t in (1e-30, 0.5, 1.0 - 1e-7):
        x = _x(wl, 1, 3)
        res = run_decode(case, torch.from_numpy(x).to(gpu_ready), t=t)
        check(case, x, res, t=t)
        if t < 0.1:
            assert res["n"] == F
        if t > 0.9:
            assert res["n"] == 0 and np.all(res["y"] == 0.0)


@pytest.mark.parametrize("name,wl", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_decode_normalised_input_no_bias(gpu_ready, name, wl):
    for with_c in (True, False):
        case = make_case(wl, 0, gpu_ready, with_c=with_c)
        x = 2.9 * _x(wl, 1, 5) - 0.6
        check(case, x, run_decode(case, torch.from_numpy(x).to(gpu_ready), x_norm=True), x_norm=True)


@pytest.mark.parametrize("name,wl", [
    ("reglu_wide_d", small("c2", D=5632, F=900, r=16, L=1, density=0.1)),       # beyond the fused gather
    ("relu_many_neurons", small("c1", D=64, F=33000, r=8, L=1, density=0.01)),  # beyond 32768 neurons
    ("relu_r1024", small("c1", D=256, F=4000, r=1024, L=1, density=0.2)),        # 16 chunk rounds per row
    ("relu_f32768_r512", small("c1", D=1024, F=32768, r=512, L=1, density=0.05)),   # 2 row steps x 8 rounds
    ("reglu_d5120", small("c2", D=5120, F=3000, r=128, L=1, density=0.1)),       # rows wider than 4096
    ("relu_d8192", small("c1", D=8192, F=2000, r=64, L=1, density=0.1)),
])
def test_decode_falls_back_to_separate_calls(gpu_ready, name, wl):
    assert _lib.decode_path(wl.act, False, wl.D, wl.F, wl.r) == _lib.DECODE_SEPARATE
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, 1, 1)
    check(case, x, run_decode(case, torch.from_numpy(x).to(gpu_ready)))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_decode_full_size(gpu_ready, name):
    wl = sg.workload(name)
    layer = 0 if wl.L == 1 else 1
    folded = _lib.decode_path(wl.act, False, wl.D, wl.F, wl.r) == _lib.DECODE_FOLDED
    assert folded == (name in ("c1", "c2"))           # 13B and 40B keep the separate calls (measured no faster)
    say(f"[decode full {name}] generating layer {layer}")
    case = make_case(wl, layer, gpu_ready)
    for step in range(2):
        x = _x(wl, 1, step, tag=sg.TAG_X_DECODE)
        st = check(case, x, run_decode(case, torch.from_numpy(x).to(gpu_ready)))
        say(f"[decode full {name}] step {step}: {st}")
        assert abs(st["density"] - wl.density) < 0.05
