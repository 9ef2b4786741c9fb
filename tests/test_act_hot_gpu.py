"""GPU parity of the squared-ReLU activation and of the always-active stored prefix, through the C ABI, against
the CPU oracle on identical seeded inputs.

Squared ReLU (Indonesian digest, summary bullets: ReLU, ReGLU and squared-ReLU FFNs) runs through every forward
path: the fused single-token kernels, the decode kernels (wide rows, batches of 2, 4 and 8 beyond the union
limit) and the matrix-core union kernels, in fp16 and Q4_0. The always-active prefix (Turkish article, neuron
placement: the hottest neurons are stored first) runs through every predictor stage-2 kernel (1 token, 2..4
tokens, 5 and more).
"""
import numpy as np
import pytest
import torch

import synthgen as sg
from activation_sparse_ffn_predictor_amd import _lib
from parity_util import check, make_case, run_gpu, say

pytestmark = pytest.mark.gpu


def _x(wl, B, step=0, tag=sg.TAG_X_TEST):
    return sg.inputs(wl, step, B, tag=tag)


def small(base, **kw):
    return sg.custom(sg.workload(base), **kw)


SQ_SMALL = [
    ("sqrelu_f16", small("c1", D=256, F=1000, r=72, L=1, act="sqrelu")),
    ("sqrelu_q4", small("c5", D=256, F=333, r=8, L=1, act="sqrelu", density=0.25)),
]


@pytest.mark.parametrize("name,wl", SQ_SMALL, ids=[s[0] for s in SQ_SMALL])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 17, 64])
def test_sqrelu_small_layers(gpu_ready, name, wl, B):
    case = make_case(wl, 0, gpu_ready)
    for step in range(2):
        x = _x(wl, B, step)
        say(f"[{name}] B={B} step={step}")
        st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
        say("   ", st)


@pytest.mark.parametrize("name,wl,B,path", [
    ("fused_widest", small("c1", D=8192, F=600, r=16, L=1, density=0.2, act="sqrelu"), 1, _lib.PATH_FUSED),
    ("decode_wide_d", small("c1", D=8704, F=700, r=16, L=1, density=0.1, act="sqrelu"), 1, _lib.PATH_DECODE),
    ("decode_b2", small("c1", D=1024, F=900, r=16, L=1, density=0.2, act="sqrelu"), 2, _lib.PATH_DECODE),
    ("decode_b4_many", small("c1", D=1024, F=33000, r=16, L=1, density=0.02, act="sqrelu"), 4, _lib.PATH_DECODE),
    ("decode_b8_many", small("c1", D=512, F=33000, r=16, L=1, density=0.02, act="sqrelu"), 8, _lib.PATH_DECODE),
    ("q4_decode_b2", small("c5", D=1024, F=500, r=16, L=1, density=0.2, act="sqrelu"), 2, _lib.PATH_DECODE),
    ("q4_decode_wide_d", small("c5", D=16384, F=300, r=16, L=1, density=0.1, act="sqrelu"), 1, _lib.PATH_DECODE),
    ("union_b16", small("c1", D=512, F=2000, r=32, L=1, density=0.1, act="sqrelu"), 16, _lib.PATH_UNION),
])
def test_sqrelu_every_path(gpu_ready, name, wl, B, path):
    assert _lib.forward_path("sqrelu", wl.wdtype == "q4", B, wl.D, wl.F) == path
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 1)
    say(f"[{name}] B={B}")
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
    say("   ", st)


def test_sqrelu_normalised_input(gpu_ready):
    wl = SQ_SMALL[0][1]
    case = make_case(wl, 0, gpu_ready)
    for B in (1, 5):
        x = 1.9 * _x(wl, B, 3) - 0.4
        check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready), x_norm=True), x_norm=True)


@pytest.mark.parametrize("B", [1, 4])
def test_sqrelu_full_size_falcon_shape(gpu_ready, B):
    # the Falcon-40B layer shape (D = 8192, F = 32768) with a squared-ReLU activation
    wl = sg.custom(sg.workload("c4"), act="sqrelu")
    say(f"[sqrelu 40B shape B={B}] generating layer 1")
    case = make_case(wl, 1, gpu_ready)
    x = _x(wl, B, 0, tag=sg.TAG_X_DECODE)
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
    say(f"[sqrelu 40B shape B={B}]: {st}")
    assert abs(st["density"] - wl.density) < 0.05 * B


HOT_SMALL = [
    ("relu_f16", small("c1", D=256, F=1000, r=72, L=1)),
    ("reglu_f16", small("c2", D=512, F=1250, r=64, L=1, density=0.2)),
    ("reglu_q4", small("c5", D=512, F=700, r=40, L=1, density=0.3)),
]


@pytest.mark.parametrize("name,wl", HOT_SMALL, ids=[s[0] for s in HOT_SMALL])
@pytest.mark.parametrize("B", [1, 3, 8, 17])
@pytest.mark.parametrize("n_hot", [1, 63, 64, 65, 200, -1])
def test_hot_prefix_small_layers(gpu_ready, name, wl, B, n_hot):
    n_hot = wl.F if n_hot < 0 else n_hot
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 2)
    say(f"[{name}] B={B} n_hot={n_hot}")
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready), n_hot=n_hot), n_hot=n_hot)
    say("   ", st)
    assert st["n"] >= n_hot


@pytest.mark.parametrize("B", [1, 2, 6, 20])
def test_hot_prefix_alone_when_nothing_predicted(gpu_ready, B):
    # a threshold no logit reaches: exactly the prefix is computed
    wl = HOT_SMALL[1][1]
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 4)
    t = 1.0 - 1e-7
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), t=t, n_hot=97)
    check(case, x, res, t=t, n_hot=97)
    assert res["n"] == 97 and np.array_equal(res["active"][:97], np.arange(97))


def test_hot_prefix_rejects_out_of_range(gpu_ready):
    wl = HOT_SMALL[0][1]
    case = make_case(wl, 0, gpu_ready)
    x = torch.from_numpy(_x(wl, 1, 0)).to(gpu_ready)
    for bad in (-1, wl.F + 1):
        with pytest.raises(_lib.SffnError) as e:
            run_gpu(case, x, n_hot=bad)
        assert e.value.status == 6


@pytest.mark.parametrize("name,B", [("c3", 1), ("c3", 8), ("c4", 1), ("c5", 1)])
def test_hot_prefix_full_size(gpu_ready, name, B):
    # full-size layers with the saturated (always-hot) neurons declared as the prefix
    wl = sg.workload(name)
    n_hot = sg.saturated_count(wl, 1)
    say(f"[hot prefix {name} B={B}] n_hot={n_hot}, generating layer 1")
    case = make_case(wl, 1, gpu_ready)
    x = _x(wl, B, 0, tag=sg.TAG_X_DECODE)
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready), n_hot=n_hot), n_hot=n_hot)
    say(f"[hot prefix {name} B={B}]: {st}")
