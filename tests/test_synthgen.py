"""Synthetic-input generator: known answers, determinism, slice regeneration, workload statistics."""
import os

import numpy as np
import pytest

import synthgen as sg

HERE = os.path.dirname(os.path.abspath(__file__))


def test_philox_known_answers():
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for row in rows:
        v = [int(h, 16) for h in row]
        assert sg.philox4x32_10(v[0:4], v[4:6]) == tuple(v[6:10])


def test_deterministic_and_sliceable():
    wl = sg.workload("c1")
    a = sg.layer_host(wl, 0)
    b = sg.layer_host(wl, 0)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    # rows 100..109 of W_up regenerate alone, bit for bit
    key = sg.key_seed(wl.index)
    part = np.empty((10, wl.D), dtype=np.float16)
    sg.fill_normal(part, key, sg.TAG_W_UP, 0, wl.sigma_w, start=100 * wl.D)
    assert np.array_equal(part.view(np.uint16), a["W_up"][100:110].view(np.uint16))
    # different layers / tags differ
    c = sg.layer_host(wl, 1)
    assert not np.array_equal(a["W_up"], c["W_up"])
    assert not np.array_equal(a["W_up"], a["W_down"].T)


def test_thread_count_does_not_change_bits(monkeypatch):
    wl = sg.workload("c1")
    key = sg.key_seed(wl.index)
    a = np.empty(300_000, dtype=np.float16)
    sg.fill_normal(a, key, sg.TAG_W_UP, 0, 0.02)
    monkeypatch.setenv("SYNTH_THREADS", "1")
    b = np.empty_like(a)
    sg.fill_normal(b, key, sg.TAG_W_UP, 0, 0.02)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_normal_moments_and_range():
    key = sg.key_seed(0)
    a = np.empty(1 << 20, dtype=np.float32)
    sg.fill_normal(a, key, sg.TAG_X_TEST, 0, 1.0)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1.0) < 5e-3
    assert np.abs(a).max() <= 262140 / sg.IH8_STD + 1e-3   # Irwin-Hall support
    q = np.empty(1 << 16, dtype=np.uint8)
    sg.fill_q4(q, key, sg.TAG_Q_UP, 0)
    assert q.max() == 15 and q.min() == 0 and abs(q.mean() - 7.5) < 0.1
    s = np.empty(1 << 16, dtype=np.float16)
    sg.fill_scales(s, key, sg.TAG_S_UP, 0)
    sf = s.astype(np.float64)
    assert sf.min() >= 0.001 - 1e-6 and sf.max() <= 0.01 + 1e-5 and abs(sf.mean() - 0.0055) < 1e-4


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_zipf_profile(name):
    wl = sg.workload(name)
    p = sg.zipf_probs(wl.F, wl.zipf_s, wl.density)
    assert abs(p.mean() - wl.density) < 1e-9
    assert p.max() <= sg.ZIPF_CAP and np.all(np.diff(p) <= 0) and p.min() > 0
    ranks = sg.neuron_ranks(wl, 0)
    assert sorted(ranks.tolist()) == list(range(1, wl.F + 1))


def test_firing_rate_matches_profile():
    wl = sg.workload("c1")
    t = sg.layer_host(wl, 0)
    X = np.stack([sg.inputs(wl, s, 1, tag=sg.TAG_X_TEST)[0] for s in range(4096)]).astype(np.float64)
    pre = X @ t["W_up"].astype(np.float64).T + t["b_up"].astype(np.float64)[None, :]
    rate = (pre > 0).mean(axis=0)
    p = sg.neuron_probs(wl, 0)
    assert abs(rate.mean() - wl.density) < 0.01
    tol = 5 * np.sqrt(p * (1 - p) / 4096) + 0.01
    assert np.mean(np.abs(rate - p) <= tol) > 0.995
    # calibrated predictor marks about the target share; without c it marks about half
    z = (X @ t["P1"].astype(np.float64).T) @ t["P2"].astype(np.float64).T
    assert abs(((z + t["c"][None, :]) > 0).mean() - wl.density) < 0.01
    assert abs((z > 0).mean() - 0.5) < 0.02


def test_fp16_conversion_is_round_to_nearest_even():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # exact ties between fp16 neighbours, fp16 subnormal range, overflow edge
    m = rng.integers(0, 1 << 10, size=20000).astype(np.uint32)
    e = rng.integers(100, 143, size=20000).astype(np.uint32)
    ties = ((e << 23) | (m << 13) | 0x1000).view(np.float32)
    edge = np.array([65504, 65519.99, 65520, 65536, 2 ** -24, 2 ** -25, 1.5 * 2 ** -25, 2 ** -26, 0.0, -0.0,
                     6.1e-5, 5.96e-8], dtype=np.float32)
    for v in (vals, ties, -ties, edge, -edge):
        ours = sg.f32_to_f16(v).view(np.uint16)
        with np.errstate(over="ignore"):
            ref = v.astype(np.float16).view(np.uint16)
        assert np.array_equal(ours, ref)


def test_rank_schedule_shapes_and_calibration():
    base = sg.workload("c3")
    wl = sg.with_rank_schedule(base)
    assert wl.ranks == (128, 256, 384, 256) and wl.r == 384
    assert np.mean(wl.ranks) == base.r                       # same predictor bytes as the fixed rank on average
    for layer, r in enumerate((128, 256, 384, 256, 128)):
        assert wl.rank(layer) == r
        shapes = sg.layer_shapes(wl, layer)
        assert shapes["P1"][0] == (r, wl.D) and shapes["P2"][0] == (wl.F, r)
    # at rank 128 the first 128 rows of P1 equal the base workload's (the generator is counter-based)
    small = sg.custom(sg.with_rank_schedule(sg.workload("c1")), F=256)
    t0 = sg.layer_host(small, 0, names=["P1"])
    tb = sg.layer_host(sg.custom(sg.workload("c1"), F=256), 0, names=["P1"])
    assert np.array_equal(t0["P1"], tb["P1"][:small.rank(0)])


def test_rank_schedule_predictor_density():
    # the calibrated bias follows each layer's rank: the predictor still marks about the target share
    wl = sg.custom(sg.with_rank_schedule(sg.workload("c1")), F=1024)
    X = np.stack([sg.inputs(wl, s, 1, tag=sg.TAG_X_TEST)[0] for s in range(512)]).astype(np.float64)
    for layer in range(4):
        t = sg.layer_host(wl, layer, names=["P1", "P2"])
        assert t["P1"].shape == (wl.rank(layer), wl.D)
        z = (X @ t["P1"].astype(np.float64).T) @ t["P2"].astype(np.float64).T + t["c"][None, :]
        assert abs((z > 0).mean() - wl.density) < 0.015, layer


def test_saturated_count_is_the_hot_first_prefix():
    from activation_sparse_ffn_predictor_amd.pack import hot_first_perm
    wl = sg.workload("c2")
    p = sg.neuron_probs(wl, 3)
    n = sg.saturated_count(wl, 3)
    perm = hot_first_perm(p)
    assert n > 0 and np.all(p[perm[:n]] >= sg.ZIPF_CAP) and np.all(p[perm[n:]] < sg.ZIPF_CAP)
