"""GPU parity: the HIP path through the C ABI against the CPU oracle on identical seeded inputs."""
import numpy as np
import pytest
import torch

import synthgen as sg
from parity_util import check, make_case, run_gpu, say

pytestmark = pytest.mark.gpu


def _x(wl, B, step=0, tag=sg.TAG_X_TEST):
    return sg.inputs(wl, step, B, tag=tag)


def small(base, **kw):
    return sg.custom(sg.workload(base), **kw)


# reduced shapes: several 64-neuron tiles plus a ragged tail, ragged predictor rank
SMALL = [
    ("relu_f16", small("c1", D=256, F=1000, r=72, L=1)),
    ("reglu_f16", small("c2", D=512, F=1250, r=64, L=1, density=0.2)),
    ("reglu_q4", small("c5", D=512, F=700, r=40, L=1, density=0.3)),
    ("relu_q4", sg.custom(small("c5", D=256, F=333, r=8, L=1), act="relu", density=0.25)),
]


@pytest.mark.parametrize("name,wl", SMALL, ids=[s[0] for s in SMALL])
# 6 and 7 tokens: the last batch of the 16-row union kernel and the first of the 64-row one with the packed token
# plane; 9 tokens: the first with one fp16 value per token element
@pytest.mark.parametrize("B", [1, 2, 3, 4, 6, 7, 8, 9, 16, 17, 64])
def test_small_layers(gpu_ready, name, wl, B):
    case = make_case(wl, 0, gpu_ready)
    for step in range(3):
        x = _x(wl, B, step)
        say(f"[{name}] B={B} step={step}")
        res = run_gpu(case, torch.from_numpy(x).to(gpu_ready))
        st = check(case, x, res)
        say("   ", st)
        assert st["logit_err"] < 1e-4


@pytest.mark.parametrize("name,wl", SMALL[:3], ids=[s[0] for s in SMALL[:3]])
def test_normalised_input_and_no_predictor_bias(gpu_ready, name, wl):
    case = make_case(wl, 0, gpu_ready, with_c=False)
    x = 3.7 * _x(wl, 1, 5)                    # un-normalised input; the library normalises on load
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), x_norm=True)
    st = check(case, x, res, x_norm=True)
    say(name, st)
    assert 0.3 < st["density"] < 0.7          # no bias: about half the neurons are marked


@pytest.mark.parametrize("name,wl", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("B", [2, 5, 17, 33, 64])
def test_union_normalised_input(gpu_ready, name, wl, B):
    # from 17 tokens the normalisation is folded into the predictor (partials of P1 (x - x[0]) and row sums of P1)
    case = make_case(wl, 0, gpu_ready)
    x = 2.5 * _x(wl, B, 6) + 0.75            # un-normalised tokens; normalised per token on load
    say(f"[{name}] union B={B} x_norm")
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), x_norm=True)
    st = check(case, x, res, x_norm=True)
    say("   ", st)
    assert st["logit_err"] < 1e-4


@pytest.mark.parametrize("name,wl", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("B", [3, 40])
@pytest.mark.parametrize("scale", [1e-4, 1e4])
def test_union_token_range(gpu_ready, name, wl, B, scale):
    # tokens far from unit size without normalisation: the activations reach about scale^2 (ReGLU, squared ReLU),
    # beyond fp16's range either way, so the union kernels' per-token powers of two must carry them
    case = make_case(wl, 0, gpu_ready)
    x = scale * _x(wl, B, 7)
    say(f"[{name}] union B={B} x*{scale:g}")
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready))
    st = check(case, x, res)
    say("   ", st)
    assert np.all(np.isfinite(res["y"]))


@pytest.mark.parametrize("B", [3, 16])
@pytest.mark.parametrize("t,expect", [(1e-30, "all"), (1.0 - 1e-7, "none")])
def test_union_all_and_none_active(gpu_ready, B, t, expect):
    wl = SMALL[2][1]
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 1)
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), t=t)
    check(case, x, res, t=t)
    if expect == "all":
        assert res["n"] == wl.F
    else:
        assert res["n"] == 0 and np.all(res["y"] == 0.0)


@pytest.mark.parametrize("perm", ["identity", "random"])
def test_permutation_invariance(gpu_ready, perm):
    wl = SMALL[1][1]
    x = _x(wl, 1, 2)
    ys = []
    for p in ("hot", perm):
        case = make_case(wl, 0, gpu_ready, perm=p)
        res = run_gpu(case, torch.from_numpy(x).to(gpu_ready))
        check(case, x, res)
        ys.append(res["y"])
    assert np.max(np.abs(ys[0] - ys[1])) <= 1e-5 * np.max(np.abs(ys[0]))


@pytest.mark.parametrize("name,wl", [SMALL[1], SMALL[2]], ids=[SMALL[1][0], SMALL[2][0]])
@pytest.mark.parametrize("B", [4, 16])
@pytest.mark.parametrize("perm", ["identity", "random"])
def test_permutation_invariance_batches(gpu_ready, name, wl, B, perm):
    # union batches (matrix-core kernels): another stored neuron order gives the same set of original neurons and
    # the same outputs up to summation order
    x = _x(wl, B, 4)
    ys, sets = [], []
    for p in ("hot", perm):
        case = make_case(wl, 0, gpu_ready, perm=p)
        say(f"[{name}] B={B} perm={p}")
        res = run_gpu(case, torch.from_numpy(x).to(gpu_ready))
        check(case, x, res)
        ys.append(res["y"])
        ids = res["active"][:res["n"]]
        sets.append(set(case.perm[ids].tolist()))
    # each run matched the oracle outside the band (check), so the sets can differ only in band neurons; with
    # equal sets the outputs agree up to summation order
    if sets[0] == sets[1]:
        assert np.max(np.abs(ys[0] - ys[1])) <= 2e-3 * np.max(np.abs(ys[0]))


@pytest.mark.parametrize("t,expect", [(1e-30, "all"), (1.0 - 1e-7, "none")])
def test_all_and_none_active(gpu_ready, t, expect):
    wl = SMALL[0][1]
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, 1, 1)
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), t=t)
    check(case, x, res, t=t)
    if expect == "all":
        assert res["n"] == wl.F
    else:
        assert res["n"] == 0 and np.all(res["y"] == 0.0)


# one token with every neuron active: the fused kernels' blocks then take several passes of 8 rows each (n > 2048
# gives all 256 blocks 9-24 rows), and with n just above 512 the working block count rises from 64
@pytest.mark.parametrize("name,wl", [
    ("relu_f16_6000", small("c1", D=256, F=6000, r=16, L=1, density=0.5)),
    ("reglu_q4_3000", small("c5", D=256, F=3000, r=8, L=1, density=0.5)),
    ("relu_f16_520", small("c1", D=256, F=520, r=16, L=1, density=0.5)),
])
def test_fused_passes_all_active(gpu_ready, name, wl):
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, 1, 2)
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), t=1e-30)
    st = check(case, x, res, t=1e-30)
    say(f"[{name}] all active", st)
    assert res["n"] == wl.F


@pytest.mark.parametrize("F", [1, 63, 64, 65, 129])
@pytest.mark.parametrize("B", [1, 3])
def test_tiny_neuron_counts(gpu_ready, F, B):
    wl = small("c1", D=64, F=F, r=8, L=1, density=0.5)
    case = make_case(wl, 0, gpu_ready)
    for t in (1e-30, 0.5):
        x = _x(wl, B, 3)
        res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), t=t)
        check(case, x, res, t=t)


@pytest.mark.parametrize("r", [8, 136, 1024])
@pytest.mark.parametrize("B", [1, 2, 5, 8, 20, 32])
def test_predictor_rank_extremes(gpu_ready, r, B):
    # every stage-2 shape class: one chunk round (r = 8), a ragged last round (r = 136), the largest rank; from 17
    # tokens stage 2 runs on pre-split h fragments where they fit the token-fragment region (r = 8, 136 at D = 256)
    wl = small("c1", D=256, F=300, r=r, L=1, density=0.3)
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 1)
    say(f"[rank {r} B {B}]")
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
    assert st["logit_err"] < 1e-4


@pytest.mark.parametrize("B", [1, 6])
def test_minimum_d_q4(gpu_ready, B):
    wl = small("c5", D=32, F=200, r=8, L=1, density=0.5)
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, B, 0)
    check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))


@pytest.mark.parametrize("name,wl", [
    ("reglu_wide_d", small("c2", D=5632, F=900, r=16, L=1, density=0.1)),        # ReGLU wider than the fused kernel
    ("relu_wide_d", small("c1", D=8704, F=700, r=16, L=1, density=0.1)),         # ReLU wider than the fused kernel
    ("relu_many_neurons", small("c1", D=64, F=33000, r=8, L=1, density=0.01)),   # more mask words than threads
    ("relu_fused_widest", small("c1", D=8192, F=600, r=16, L=1, density=0.2)),
])
def test_single_token_path_boundaries(gpu_ready, name, wl):
    case = make_case(wl, 0, gpu_ready)
    for step in range(2):
        x = _x(wl, 1, step)
        say(f"[{name}] step {step}")
        st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
        say("   ", st)


def test_largest_union_f(gpu_ready):
    # the union kernels take F up to 32768 (512 mask words), a ragged D and many k splits of few rows
    wl = small("c1", D=200, F=32768, r=16, L=1, density=0.02)
    case = make_case(wl, 0, gpu_ready)
    x = _x(wl, 20, 0)
    st = check(case, x, run_gpu(case, torch.from_numpy(x).to(gpu_ready)))
    say("largest union F", st)


@pytest.mark.parametrize("B", [1, 4, 24])
def test_deterministic_reruns(gpu_ready, B):
    wl = SMALL[1][1]
    case = make_case(wl, 0, gpu_ready)
    x = torch.from_numpy(_x(wl, B, 4)).to(gpu_ready)
    a, b = run_gpu(case, x), run_gpu(case, x)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["mask"], b["mask"])


def test_device_generator_matches_host(gpu_ready):
    for name in ("c1", "c5"):
        wl = sg.workload(name)
        wl = sg.custom(wl, F=min(wl.F, 4096))
        host = sg.layer_host(wl, 3)
        dev = sg.layer_device(wl, 3, gpu_ready)
        for k, v in host.items():
            d = dev[k].cpu().numpy()
            assert np.array_equal(v.view(np.uint8), d.view(np.uint8)), (name, k)
    xh = sg.inputs(sg.workload("c2"), 7, 4)
    xd = torch.empty((4, 4096), dtype=torch.float32, device=gpu_ready)
    sg.inputs(sg.workload("c2"), 7, 4, out=xd)
    assert np.array_equal(xh, xd.cpu().numpy())


# full-size single layers of every workload (decode batch 1), input from the generator
FULL = ["c1", "c2", "c3", "c4", "c5"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(gpu_ready, name):
    wl = sg.workload(name)
    layer = 0 if wl.L == 1 else 1
    say(f"[full {name}] generating layer {layer}")
    case = make_case(wl, layer, gpu_ready)
    for step in range(2):
        x = _x(wl, 1, step, tag=sg.TAG_X_DECODE)
        res = run_gpu(case, torch.from_numpy(x).to(gpu_ready))
        st = check(case, x, res)
        say(f"[full {name}] step {step}: {st}")
        assert abs(st["density"] - wl.density) < 0.05


# full-size union batches: the decode batches of the 13B shape that exceed the decode kernels, the Falcon shape at
# B = 4, and the 70B Q4 prompt of 64 tokens
UNION_FULL = [("c3", 4, sg.TAG_X_DECODE, False), ("c3", 8, sg.TAG_X_DECODE, False),
              ("c4", 4, sg.TAG_X_DECODE, False), ("c5", 64, sg.TAG_X_PROMPT, False),
              ("c5", 64, sg.TAG_X_PROMPT, True)]


@pytest.mark.parametrize("name,B,tag,xn", UNION_FULL, ids=[f"{n}-B{b}{'-xnorm' if xn else ''}"
                                                          for n, b, _, xn in UNION_FULL])
def test_full_size_union(gpu_ready, name, B, tag, xn):
    wl = sg.workload(name)
    layer = 0 if wl.L == 1 else 2
    say(f"[full union {name} B={B} x_norm={xn}] generating layer {layer}")
    case = make_case(wl, layer, gpu_ready)
    x = _x(wl, B, 0, tag=tag)
    if xn:                                    # tokens off unit scale and centre, normalised by the library
        x = 1.9 * x - 0.4
    res = run_gpu(case, torch.from_numpy(x).to(gpu_ready), x_norm=xn)
    st = check(case, x, res, x_norm=xn)
    say(f"[full union {name} B={B} x_norm={xn}]: {st}")
