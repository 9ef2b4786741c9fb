"""Pins of the CPU oracle against things other than itself.

* exact-rational brute force on tiny dyadic inputs (every fp64 intermediate is
  exact there, so the oracle must match bit for bit);
* hand-worked closed forms;
* special cases that reduce to a library routine (torch.nn.functional.linear);
* invariants the pages fix: skipped neurons contribute nothing ("Neuron-aware
  operator"), neuron tables map results back to original order ("Neuron
  placement and management"), sigmoid threshold == logit threshold;
* planted mistakes: every mutant of the oracle must fail at least one pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle.sparse_ffn as sf

F0 = Fraction(0)


# ----------------------------------------------------------------------------- exact brute force
def _dyadic(rng, shape, lim=32, den=16):
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float64) / den


def _exact_layer(act, x, P1, P2, c, Wg, bg, Wu, bu, Wd, tau=F0, n_hot=0):
    """Scalar loops over exact rationals: the layer written out from its definition (the first n_hot stored
    neurons are computed whatever the predictor says)."""
    Fr = lambda v: Fraction(float(v))  # noqa: E731  (inputs are dyadic, conversion is exact)
    B, D = x.shape
    r, F = P1.shape[0], P2.shape[0]
    h = [[sum((Fr(P1[j, d]) * Fr(x[b, d]) for d in range(D)), F0) for j in range(r)] for b in range(B)]
    z = [[sum((Fr(P2[k, j]) * h[b][j] for j in range(r)), F0) + (Fr(c[k]) if c is not None else F0)
          for k in range(F)] for b in range(B)]
    mask = [k < n_hot or any(z[b][k] > tau for b in range(B)) for k in range(F)]
    a = [[F0] * F for _ in range(B)]
    for b in range(B):
        for k in range(F):
            u = sum((Fr(Wu[k, d]) * Fr(x[b, d]) for d in range(D)), F0)
            if act in ("relu", "sqrelu"):
                pre = u + (Fr(bu[k]) if bu is not None else F0)
                a[b][k] = (pre if act == "relu" else pre * pre) if pre > 0 else F0
            else:
                g = sum((Fr(Wg[k, d]) * Fr(x[b, d]) for d in range(D)), F0) + (Fr(bg[k]) if bg is not None else F0)
                a[b][k] = (g if g > 0 else F0) * u
    y = [[sum((a[b][k] * Fr(Wd[d, k]) for k in range(F) if mask[k]), F0) for d in range(D)] for b in range(B)]
    return z, mask, y


def _tiny_case(seed, act, B, D=8, F=16, r=4, with_c=True, tie=True):
    rng = np.random.default_rng(seed)
    x = _dyadic(rng, (B, D))
    P1, P2 = _dyadic(rng, (r, D)), _dyadic(rng, (F, r))
    Wg = _dyadic(rng, (F, D)) if act == "reglu" else None
    Wu, Wd = _dyadic(rng, (F, D)), _dyadic(rng, (D, F))
    bias = _dyadic(rng, (F,))
    c = _dyadic(rng, (F,)) if with_c else None
    if tie and with_c and B == 1:
        # force an exact tie z = 0 on neuron 3: strict '>' must leave it inactive
        zc = (x @ P1.T) @ P2.T
        c[3] = -zc[0, 3]
    w = {"P1": P1, "P2": P2, "W_up": Wu, "W_down": Wd}
    if c is not None:
        w["c"] = c
    if act == "reglu":
        w["W_gate"], w["b_gate"] = Wg, bias
    else:
        w["b_up"] = bias
    return x, w


def check_brute_force(act, B, seed, with_c=True, n_hot=0):
    x, w = _tiny_case(seed, act, B, with_c=with_c)
    z, m, y = sf.layer(act, x, w, 0.5, n_hot)
    ez, em, ey = _exact_layer(act, x, w["P1"], w["P2"], w.get("c"), w.get("W_gate"), w.get("b_gate"), w["W_up"],
                              w.get("b_up"), w["W_down"], n_hot=n_hot)
    ok = all(Fraction(float(z[b, k])) == ez[b][k] for b in range(B) for k in range(z.shape[1]))
    ok &= [bool(v) for v in m] == em
    ok &= all(Fraction(float(y[b, d])) == ey[b][d] for b in range(B) for d in range(y.shape[1]))
    return ok


@pytest.mark.parametrize("act", ["relu", "sqrelu", "reglu"])
@pytest.mark.parametrize("B", [1, 2, 3])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_exact(act, B, seed):
    assert check_brute_force(act, B, seed)


@pytest.mark.parametrize("act", ["relu", "sqrelu", "reglu"])
@pytest.mark.parametrize("n_hot", [1, 5, 16])
def test_brute_force_hot_prefix(act, n_hot):
    assert check_brute_force(act, 2, 3, n_hot=n_hot)


def test_brute_force_no_predictor_bias():
    assert check_brute_force("reglu", 2, 5, with_c=False)


def test_tie_is_inactive():
    x, w = _tiny_case(11, "relu", 1)
    z, m, _ = sf.layer("relu", x, w, 0.5)
    assert z[0, 3] == 0.0 and not m[3]


# ----------------------------------------------------------------------------- Q4_0
def check_q4_exact(seed=0):
    rng = np.random.default_rng(seed)
    N, K = 3, 64
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    s = (rng.integers(1, 64, size=(N, K // 32)) / 1024.0).astype(np.float16)
    w = sf.dequant_q4_rows(q, s)
    ok = True
    for n in range(N):
        for k in range(K):
            ok &= Fraction(float(w[n, k])) == (int(q[n, k]) - 8) * Fraction(float(s[n, k // 32]))
    # columns variant: W_down [D, F] with blocks of 32 along d_model (axis 0)
    qd = rng.integers(0, 16, size=(64, 5)).astype(np.uint8)
    sd = (rng.integers(1, 64, size=(2, 5)) / 512.0).astype(np.float16)
    wd = sf.dequant_q4_cols(qd, sd)
    for d in range(64):
        for f in range(5):
            ok &= Fraction(float(wd[d, f])) == (int(qd[d, f]) - 8) * Fraction(float(sd[d // 32, f]))
    return ok


def test_q4_dequant_exact():
    assert check_q4_exact()


def test_q4_block_hand_values():
    # one block: q = 0..15, 0..15 with scale 0.5 -> w = -4, -3.5, ..., 3.5 twice
    q = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :]
    s = np.array([[0.5]], dtype=np.float16)
    w = sf.dequant_q4_rows(q, s)[0]
    assert w[0] == -4.0 and w[8] == 0.0 and w[15] == 3.5 and w[16] == -4.0 and w[31] == 3.5


def test_q4_integer_then_scale_order():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(1, 256)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, size=(1, 8)).astype(np.float16)
    x = rng.standard_normal(256)
    blockwise = sum(float(s[0, j]) * float(np.dot(q[0, 32 * j:32 * j + 32].astype(np.float64) - 8, x[32 * j:32 * j + 32]))
                    for j in range(8))
    direct = float(sf.dequant_q4_rows(q, s)[0] @ x)
    assert abs(blockwise - direct) <= 1e-12 * max(1.0, abs(direct))


# ----------------------------------------------------------------------------- closed forms
def test_closed_form_relu_two_neurons():
    # u = W_up x + b = (3-1, -1+0.5) = (2, -0.5) -> a = (2, 0); y = W_down a = (2*1, 2*0) ... see below
    x = np.array([[3.0, -1.0]])
    w = {"P1": np.array([[1.0, 1.0]]), "P2": np.array([[1.0], [1.0]]), "c": np.array([0.0, 0.0]),
         "W_up": np.eye(2), "b_up": np.array([-1.0, 0.5]), "W_down": np.array([[1.0, 0.0], [3.0, 2.0]])}
    z, m, y = sf.layer("relu", x, w, 0.5)
    assert z.tolist() == [[2.0, 2.0]] and m.tolist() == [True, True]
    assert y.tolist() == [[2.0, 6.0]]                      # (1*2 + 0*0, 3*2 + 2*0)
    w["c"] = np.array([-5.0, 0.0])                         # predictor now skips neuron 0
    _, m, y = sf.layer("relu", x, w, 0.5)
    assert m.tolist() == [False, True] and y.tolist() == [[0.0, 0.0]]


def test_closed_form_sqrelu_two_neurons():
    # u = W_up x + b = (2, -0.5) -> a = (4, 0); y = W_down a = (1*4, 3*4)
    x = np.array([[3.0, -1.0]])
    w = {"P1": np.array([[1.0, 1.0]]), "P2": np.array([[1.0], [1.0]]), "c": np.array([0.0, 0.0]),
         "W_up": np.eye(2), "b_up": np.array([-1.0, 0.5]), "W_down": np.array([[1.0, 0.0], [3.0, 2.0]])}
    _, m, y = sf.layer("sqrelu", x, w, 0.5)
    assert m.tolist() == [True, True] and y.tolist() == [[4.0, 12.0]]


def check_hot_prefix_closed_form():
    # the predictor skips neuron 0 (z = -3); declared always active, it is computed anyway
    x = np.array([[3.0, -1.0]])
    w = {"P1": np.array([[1.0, 1.0]]), "P2": np.array([[1.0], [1.0]]), "c": np.array([-5.0, 0.0]),
         "W_up": np.eye(2), "b_up": np.array([-1.0, 0.5]), "W_down": np.array([[1.0, 0.0], [3.0, 2.0]])}
    _, m0, y0 = sf.layer("relu", x, w, 0.5)
    ok = m0.tolist() == [False, True] and y0.tolist() == [[0.0, 0.0]]
    _, m1, y1 = sf.layer("relu", x, w, 0.5, n_hot=1)
    ok &= m1.tolist() == [True, True] and y1.tolist() == [[2.0, 6.0]]
    w["c"] = np.array([0.0, -5.0])                         # a hot prefix never removes a predicted neuron
    _, m2, _ = sf.layer("relu", x, w, 0.5, n_hot=1)
    return ok and m2.tolist() == [True, False]


def test_closed_form_hot_prefix():
    assert check_hot_prefix_closed_form()


def test_hot_prefix_everything_is_dense():
    x, w = _tiny_case(9, "reglu", 2)
    _, m, y = sf.layer("reglu", x, w, 1.0 - 1e-15, n_hot=16)   # the predictor marks nothing, the prefix all
    assert m.all() and np.array_equal(y, sf.ffn_dense("reglu", x, w))


def test_hot_prefix_nested():
    x, w = _tiny_case(10, "relu", 3, tie=False)
    prev = None
    for n_hot in range(0, 17):
        _, m, _ = sf.layer("relu", x, w, 0.5, n_hot)
        assert m[:n_hot].all()
        if prev is not None:
            assert np.all(m >= prev) and (m.sum() - prev.sum()) <= 1
        prev = m


def test_closed_form_reglu():
    x = np.array([[1.0, 2.0]])
    w = {"P1": np.array([[1.0, 0.0]]), "P2": np.array([[1.0], [-1.0], [2.0]]), "c": np.zeros(3),
         "W_gate": np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]]), "b_gate": np.array([0.0, 0.0, 0.0]),
         "W_up": np.array([[0.0, 1.0], [1.0, 1.0], [1.0, 0.0]]),
         "W_down": np.array([[1.0, 10.0, 100.0], [0.0, 0.0, 1.0]])}
    # h = 1; z = (1, -1, 2) -> M = {0, 2}; g = (1, 2, -1), u = (2, 3, 1); a = (2, 6, 0); masked a = (2, 0, 0)
    z, m, y = sf.layer("reglu", x, w, 0.5)
    assert z.tolist() == [[1.0, -1.0, 2.0]] and m.tolist() == [True, False, True]
    assert y.tolist() == [[2.0, 0.0]]


def test_closed_form_threshold_and_union():
    # rank-1 predictor, t = sigmoid(0.6): z = (0.5, -0.5) token 0, (0.7, 0.1) token 1
    x = np.array([[0.25, 0.25], [0.35, 0.35]])
    P1 = np.array([[1.0, 1.0]])
    P2 = np.array([[1.0], [-1.0]])
    c = np.array([0.0, 0.0])
    t = 1.0 / (1.0 + np.exp(-0.6))
    z = sf.predictor_logits(P1, P2, x, c)
    assert np.allclose(z, [[0.5, -0.5], [0.7, -0.7]])
    masks = sf.token_masks(z, t)
    assert masks.tolist() == [[False, False], [True, False]]
    assert sf.union_mask(masks).tolist() == [True, False]


def test_layer_norm_closed_form():
    # y = (3, -1): mean 1, centred (2, -2), variance 4 -> (2, -2) / sqrt(4 + eps)
    y = np.array([[3.0, -1.0], [5.0, 5.0]])
    x = sf.layer_norm(y)
    s = np.sqrt(4.0 + sf.NORM_EPS)
    assert np.allclose(x[0], [2.0 / s, -2.0 / s], rtol=0, atol=1e-15)
    assert x[1].tolist() == [0.0, 0.0]                      # a constant token centres to zero
    z = sf.layer_norm(np.random.default_rng(0).standard_normal((3, 1000)) * 7 + 40)
    assert np.allclose(z.mean(axis=1), 0, atol=1e-12) and np.allclose((z * z).mean(axis=1), 1, atol=1e-6)


# ----------------------------------------------------------------------------- library special cases
def test_all_active_matches_torch_linear():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    D, F, r = 24, 40, 6
    x = rng.standard_normal((3, D))
    w = {"P1": rng.standard_normal((r, D)), "P2": rng.standard_normal((F, r)), "W_gate": rng.standard_normal((F, D)),
         "b_gate": rng.standard_normal(F), "W_up": rng.standard_normal((F, D)), "W_down": rng.standard_normal((D, F))}
    z, m, y = sf.layer("reglu", x, w, 1e-300)        # tau = ln(1e-300) ~ -690: every neuron active
    assert m.all()
    tx = torch.from_numpy(x)
    g = torch.nn.functional.linear(tx, torch.from_numpy(w["W_gate"]), torch.from_numpy(w["b_gate"]))
    u = torch.nn.functional.linear(tx, torch.from_numpy(w["W_up"]))
    ref = torch.nn.functional.linear(torch.relu(g) * u, torch.from_numpy(w["W_down"])).numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    w2 = {"P1": w["P1"], "P2": w["P2"], "W_up": w["W_up"], "b_up": w["b_gate"], "W_down": w["W_down"]}
    _, _, y2 = sf.layer("relu", x, w2, 1e-300)
    ref2 = torch.nn.functional.linear(
        torch.relu(torch.nn.functional.linear(tx, torch.from_numpy(w["W_up"]), torch.from_numpy(w["b_gate"]))),
        torch.from_numpy(w["W_down"])).numpy()
    assert np.max(np.abs(y2 - ref2)) <= 1e-12 * np.max(np.abs(ref2))
    _, _, y3 = sf.layer("sqrelu", x, w2, 1e-300)
    ref3 = torch.nn.functional.linear(
        torch.square(torch.relu(torch.nn.functional.linear(tx, torch.from_numpy(w["W_up"]),
                                                           torch.from_numpy(w["b_gate"])))),
        torch.from_numpy(w["W_down"])).numpy()
    assert np.max(np.abs(y3 - ref3)) <= 1e-12 * np.max(np.abs(ref3))


def test_none_active_gives_zero():
    rng = np.random.default_rng(5)
    D, F, r = 16, 32, 4
    x = rng.standard_normal((2, D))
    w = {"P1": 0.1 * rng.standard_normal((r, D)), "P2": 0.1 * rng.standard_normal((F, r)),
         "W_up": rng.standard_normal((F, D)), "b_up": rng.standard_normal(F), "W_down": rng.standard_normal((D, F))}
    z, m, y = sf.layer("relu", x, w, 1.0 - 1e-15)    # tau ~ 34.5, |z| << 1
    assert not m.any() and np.all(y == 0.0)


def test_sigmoid_threshold_equals_logit_threshold():
    from scipy.special import expit
    rng = np.random.default_rng(6)
    z = rng.standard_normal(20000) * 4
    for t in (0.05, 0.3, 0.5, 0.7, 0.95):
        tau = sf.threshold_logit(t)
        keep = np.abs(z - tau) > 1e-9
        assert np.array_equal((expit(z) > t)[keep], sf.token_masks(z[None, :], t)[0][keep])


# ----------------------------------------------------------------------------- invariants
def check_true_mask_equals_dense(act="reglu", seed=7):
    """Sparse FFN under the true firing mask equals the dense FFN, bit for bit when both are accumulated by the
    same sequential loop (the skipped terms are exact zeros)."""
    rng = np.random.default_rng(seed)
    D, F = 12, 48
    x = rng.standard_normal((1, D))
    w = {"W_gate": rng.standard_normal((F, D)), "b_gate": rng.standard_normal(F) - 0.5,
         "W_up": rng.standard_normal((F, D)), "b_up": rng.standard_normal(F) - 0.5, "W_down": rng.standard_normal((D, F))}
    a = sf.activations(act, x, w)[0]
    true_mask = a != 0.0
    assert 0 < true_mask.sum() < F
    y_masked = sf.ffn_masked(act, x, w, true_mask)[0]
    y_dense = sf.ffn_dense(act, x, w)[0]
    dense_loop = np.zeros(D)
    sparse_loop = np.zeros(D)
    for k in range(F):
        dense_loop = dense_loop + a[k] * w["W_down"][:, k]
        if true_mask[k]:
            sparse_loop = sparse_loop + a[k] * w["W_down"][:, k]
    return (np.array_equal(dense_loop, sparse_loop)
            and np.max(np.abs(y_masked - y_dense)) <= 1e-12 * np.max(np.abs(y_dense))
            and np.max(np.abs(y_masked - sparse_loop)) <= 1e-12 * np.max(np.abs(y_dense)))


@pytest.mark.parametrize("act", ["relu", "sqrelu", "reglu"])
def test_true_mask_equals_dense(act):
    assert check_true_mask_equals_dense(act)


def check_permutation_invariance(seed=8):
    """Storing neurons in another order (with the table mapping back) changes neither y nor the set of active
    original neurons."""
    rng = np.random.default_rng(seed)
    D, F, r = 10, 30, 5
    x = rng.standard_normal((2, D))
    w = {"P1": rng.standard_normal((r, D)), "P2": rng.standard_normal((F, r)), "c": rng.standard_normal(F),
         "W_gate": rng.standard_normal((F, D)), "b_gate": rng.standard_normal(F), "W_up": rng.standard_normal((F, D)),
         "W_down": rng.standard_normal((D, F))}
    perm = rng.permutation(F)                          # stored position j holds original neuron perm[j]
    wp = {"P1": w["P1"], "P2": w["P2"][perm], "c": w["c"][perm], "W_gate": w["W_gate"][perm],
          "b_gate": w["b_gate"][perm], "W_up": w["W_up"][perm], "W_down": w["W_down"][:, perm]}
    _, m, y = sf.layer("reglu", x, w)
    _, mp, yp = sf.layer("reglu", x, wp)
    back = np.zeros(F, dtype=bool)
    back[perm[mp]] = True
    return np.array_equal(back, m) and np.max(np.abs(y - yp)) <= 1e-12 * np.max(np.abs(y))


def test_permutation_invariance():
    assert check_permutation_invariance()


def test_masks_nested_in_threshold_and_union_contains_tokens():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((4, 500))
    prev = None
    for t in np.linspace(0.05, 0.95, 19):
        m = sf.token_masks(z, t)
        u = sf.union_mask(m)
        assert np.all(u[m.any(axis=0)]) and np.all(m <= u[None, :])
        if prev is not None:
            assert np.all(u <= prev)          # raising t can only remove neurons
        prev = u


def test_union_equals_per_token_calls():
    x, w = _tiny_case(12, "reglu", 3, tie=False)
    _, m, _ = sf.layer("reglu", x, w)
    single = np.zeros_like(m)
    for b in range(3):
        _, mb, _ = sf.layer("reglu", x[b:b + 1], w)
        single |= mb
    assert np.array_equal(single, m)


def test_band_rule():
    t = 0.5
    z = np.array([[5e-5, 2e-4, -1.0, 5e-5, -5e-5],
                  [-1.0, 5e-5, -1.0, -1.0, -2.0]])
    b = sf.band_neurons(z, t)
    # n0: near, not clearly on -> band; n1: one token clearly on -> decided; n2: off; n3: band; n4: near -> band
    assert b.tolist() == [True, False, False, True, True]


# ----------------------------------------------------------------------------- logical weights
def _q4_tiny(seed=31, D=64, F=64):
    """A tiny Q4_0 ReGLU layer with planted codes and scales: every plane draws its own values, so a plane routed
    to the wrong logical matrix, or a scale plane read in the wrong orientation, changes some element."""
    rng = np.random.default_rng(seed)
    t = {"P1": rng.integers(-8, 8, size=(4, D)).astype(np.float16) / np.float16(8),
         "P2": rng.integers(-8, 8, size=(F, 4)).astype(np.float16) / np.float16(8),
         "Q_gate": rng.integers(0, 16, size=(F, D)).astype(np.uint8),
         "S_gate": (rng.integers(1, 200, size=(F, D // 32)) / 1024.0).astype(np.float16),
         "Q_up": rng.integers(0, 16, size=(F, D)).astype(np.uint8),
         "S_up": (rng.integers(200, 400, size=(F, D // 32)) / 1024.0).astype(np.float16),
         "Q_down": rng.integers(0, 16, size=(D, F)).astype(np.uint8),
         "S_down": (rng.integers(400, 600, size=(D // 32, F)) / 1024.0).astype(np.float16),
         "b_gate": rng.standard_normal(F).astype(np.float32), "c": rng.standard_normal(F).astype(np.float32)}
    return t


def _fp16_tiny(seed=32, D=16, F=24):
    rng = np.random.default_rng(seed)
    return {"P1": rng.standard_normal((4, D)).astype(np.float16), "P2": rng.standard_normal((F, 4)).astype(np.float16),
            "W_gate": rng.standard_normal((F, D)).astype(np.float16),
            "W_up": rng.standard_normal((F, D)).astype(np.float16),
            "W_down": rng.standard_normal((D, F)).astype(np.float16),
            "b_gate": rng.standard_normal(F).astype(np.float32), "c": rng.standard_normal(F).astype(np.float32)}


def check_logical_weights():
    """Every logical matrix is the element-wise exact value of the plane it is named after: Q4_0 as
    (q - 8) * s with the scale of the element's 32-block along d_model (rows of W_gate / W_up, columns of
    W_down), fp16 upcast unchanged; biases and predictor factors pass through."""
    Fr = lambda v: Fraction(float(v))  # noqa: E731
    try:
        t = _q4_tiny()
        w = sf.logical_weights(t)
        F, D = t["Q_up"].shape
        ok = set(w) == {"P1", "P2", "W_gate", "W_up", "W_down", "b_gate", "c"}
        for name, q, s in (("W_gate", t["Q_gate"], t["S_gate"]), ("W_up", t["Q_up"], t["S_up"])):
            ok &= w[name].shape == (F, D)
            ok &= all(Fr(w[name][k, d]) == (int(q[k, d]) - 8) * Fr(s[k, d // 32]) for k in range(F) for d in range(D))
        ok &= w["W_down"].shape == (D, F)
        ok &= all(Fr(w["W_down"][d, k]) == (int(t["Q_down"][d, k]) - 8) * Fr(t["S_down"][d // 32, k])
                  for d in range(D) for k in range(F))
        for name in ("P1", "P2", "b_gate", "c"):
            ok &= np.array_equal(w[name], t[name].astype(np.float64))
        t = _fp16_tiny()
        w = sf.logical_weights(t)
        ok &= set(w) == {"P1", "P2", "W_gate", "W_up", "W_down", "b_gate", "c"}
        for name in t:
            ok &= w[name].dtype == np.float64 and w[name].shape == t[name].shape
            ok &= all(Fr(a) == Fr(b) for a, b in zip(w[name].ravel(), t[name].ravel()))
        return bool(ok)
    except (KeyError, AssertionError, ValueError, IndexError):
        return False


def test_logical_weights_planes():
    assert check_logical_weights()


# ----------------------------------------------------------------------------- stack (closed form)
def check_stack_closed_form():
    """Two ReLU layers worked by hand. Layer 1 (rank 1): x = (3, -1), h = 2, z = (2, 2), both neurons computed,
    u = (2, -0.5), a = (2, 0), y1 = (2, 6). The next input is y1 centred and scaled: mean 4, variance 4, so
    x2 = (-2, 2) / sqrt(4 + eps) = (-s, s). Layer 2 (rank 2, first neuron always active): h = x2,
    z = (-s, -s), so the predictor marks nothing and only neuron 0 is computed; u = (s, s), a = (s, 0),
    y2 = (s, 2 s)."""
    s = 2.0 / np.sqrt(4.0 + sf.NORM_EPS)
    l1 = {"P1": np.array([[1.0, 1.0]]), "P2": np.array([[1.0], [1.0]]), "c": np.array([0.0, 0.0]),
          "W_up": np.eye(2), "b_up": np.array([-1.0, 0.5]), "W_down": np.array([[1.0, 0.0], [3.0, 2.0]])}
    l2 = {"P1": np.eye(2), "P2": np.array([[1.0, 0.0], [0.0, -1.0]]), "c": np.array([0.0, 0.0]),
          "W_up": np.array([[-1.0, 0.0], [0.0, 1.0]]), "b_up": np.array([0.0, 0.0]),
          "W_down": np.array([[1.0, 0.0], [2.0, 5.0]])}
    try:
        out = sf.stack("relu", np.array([[3.0, -1.0]]), [l1, l2], 0.5, n_hot=[0, 1])
        (z1, m1, y1), (z2, m2, y2) = out
        ok = len(out) == 2 and z1.tolist() == [[2.0, 2.0]] and m1.tolist() == [True, True]
        ok &= y1.tolist() == [[2.0, 6.0]] and m2.tolist() == [True, False]
        ok &= np.allclose(z2, [[-s, -s]], rtol=1e-15, atol=0) and np.allclose(y2, [[s, 2 * s]], rtol=1e-15, atol=0)
        return bool(ok)
    except (KeyError, ValueError, IndexError):
        return False


def test_stack_two_layers_closed_form():
    assert check_stack_closed_form()


# ----------------------------------------------------------------------------- planted mistakes
def check_layer_norm():
    y = np.array([[3.0, -1.0]])
    s = np.sqrt(4.0 + sf.NORM_EPS)
    return np.allclose(sf.layer_norm(y)[0], [2.0 / s, -2.0 / s], rtol=0, atol=1e-15)


def _all_pins():
    return check_layer_norm() and (all(check_brute_force(act, B, s) for act in ("relu", "sqrelu", "reglu")
                                       for B in (1, 3) for s in (0, 1))
            and all(check_brute_force(act, 2, 3, n_hot=n) for act in ("relu", "reglu") for n in (1, 5))
            and check_q4_exact() and all(check_true_mask_equals_dense(a) for a in ("relu", "sqrelu", "reglu"))
            and check_permutation_invariance() and check_hot_prefix_closed_form()
            and check_logical_weights() and check_stack_closed_form())


def test_unmutated_oracle_passes_all_pins():
    assert _all_pins()


def _mut_predictor_transposed(P1, P2, x, c=None):
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    z = (x @ P1.T) @ P2.T
    return z[:, ::-1] + (c[None, :] if c is not None else 0)   # logits come out in the wrong neuron order


def _mut_predictor_no_bias(P1, P2, x, c=None):
    return (np.atleast_2d(x) @ P1.T) @ P2.T


def _mut_threshold_sign(z, t):
    return np.asarray(z) < sf.threshold_logit(t)


def _mut_threshold_ge(z, t):
    return np.asarray(z) >= sf.threshold_logit(t)


def _mut_reglu_swapped(act, x, w):
    x = np.atleast_2d(x)
    if act == "reglu":
        g = x @ w["W_gate"].T + w["b_gate"][None, :]
        u = x @ w["W_up"].T
        return np.maximum(u, 0.0) * g
    return np.maximum(x @ w["W_up"].T + w["b_up"][None, :], 0.0)


def _mut_relu_no_bias(act, x, w):
    x = np.atleast_2d(x)
    if act == "relu":
        return np.maximum(x @ w["W_up"].T, 0.0)
    return np.maximum(x @ w["W_gate"].T + w["b_gate"][None, :], 0.0) * (x @ w["W_up"].T)


def _mut_sqrelu_unsquared(act, x, w):
    x = np.atleast_2d(x)
    if act == "reglu":
        return np.maximum(x @ w["W_gate"].T + w["b_gate"][None, :], 0.0) * (x @ w["W_up"].T)
    return np.maximum(x @ w["W_up"].T + w["b_up"][None, :], 0.0)   # squared ReLU left unsquared


def _mut_sqrelu_square_before_relu(act, x, w):
    x = np.atleast_2d(x)
    if act == "reglu":
        return np.maximum(x @ w["W_gate"].T + w["b_gate"][None, :], 0.0) * (x @ w["W_up"].T)
    u = x @ w["W_up"].T + w["b_up"][None, :]
    return (u * u) if act == "sqrelu" else np.maximum(u, 0.0)


def _mut_hot_prefix_off_by_one(mask, n_hot):
    m = np.array(mask, dtype=bool, copy=True)
    m[:max(0, int(n_hot) - 1)] = True
    return m


def _mut_hot_prefix_ignored(mask, n_hot):
    return np.array(mask, dtype=bool, copy=True)


def _mut_q4_offset(q, s):
    q = np.asarray(q).astype(np.float64)
    return (q - 7.0) * np.repeat(np.asarray(s, dtype=np.float64), 32, axis=1)


def _mut_mask_ignored(act, x, w, mask):
    return sf.activations(act, x, w) @ w["W_down"].T


def _mut_norm_uncentred(y, eps=sf.NORM_EPS):
    y = np.atleast_2d(y)
    return y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)


def _mut_mask_first_token(masks):
    return np.atleast_2d(masks)[0]


def _mut_lw_gate_up_swapped(t):
    w = _LW(t)
    if "Q_gate" in t:
        w["W_gate"] = sf.dequant_q4_rows(t["Q_up"], t["S_up"])
        w["W_up"] = sf.dequant_q4_rows(t["Q_gate"], t["S_gate"])
    return w


def _mut_lw_scales_swapped(t):
    w = _LW(t)
    if "Q_gate" in t:
        w["W_gate"] = sf.dequant_q4_rows(t["Q_gate"], t["S_up"])
        w["W_up"] = sf.dequant_q4_rows(t["Q_up"], t["S_gate"])
    return w


def _mut_lw_down_scale_transposed(t):
    w = _LW(t)
    if "Q_down" in t:                                  # scale blocks taken along d_ffn instead of d_model
        w["W_down"] = sf.dequant_q4_rows(t["Q_down"], np.asarray(t["S_down"]).T)
    return w


def _mut_lw_fp16_gate_up_swapped(t):
    w = _LW(t)
    if "W_gate" in t:
        w["W_gate"], w["W_up"] = w["W_up"], w["W_gate"]
    return w


def _mut_stack_unnormalised(act, x, layers, t=0.5, n_hot=0):
    out, xl = [], np.atleast_2d(np.asarray(x, dtype=np.float64))
    hots = list(n_hot) if np.ndim(n_hot) else [int(n_hot)] * len(layers)
    for w, nh in zip(layers, hots):
        z, m, y = sf.layer(act, xl, w, t, nh)
        out.append((z, m, y))
        xl = y                                         # next layer fed the raw output
    return out


def _mut_stack_first_prefix_everywhere(act, x, layers, t=0.5, n_hot=0):
    hots = list(n_hot) if np.ndim(n_hot) else [int(n_hot)] * len(layers)
    return _STACK(act, x, layers, t, [hots[0]] * len(layers))


_LW = sf.logical_weights
_STACK = sf.stack


@pytest.mark.parametrize("name,mutant", [
    ("predictor_logits", _mut_predictor_transposed),
    ("predictor_logits", _mut_predictor_no_bias),
    ("token_masks", _mut_threshold_sign),
    ("token_masks", _mut_threshold_ge),
    ("activations", _mut_reglu_swapped),
    ("activations", _mut_relu_no_bias),
    ("activations", _mut_sqrelu_unsquared),
    ("activations", _mut_sqrelu_square_before_relu),
    ("with_hot_prefix", _mut_hot_prefix_off_by_one),
    ("with_hot_prefix", _mut_hot_prefix_ignored),
    ("dequant_q4_rows", _mut_q4_offset),
    ("ffn_masked", _mut_mask_ignored),
    ("union_mask", _mut_mask_first_token),
    ("layer_norm", _mut_norm_uncentred),
    ("logical_weights", _mut_lw_gate_up_swapped),
    ("logical_weights", _mut_lw_scales_swapped),
    ("logical_weights", _mut_lw_down_scale_transposed),
    ("logical_weights", _mut_lw_fp16_gate_up_swapped),
    ("stack", _mut_stack_unnormalised),
    ("stack", _mut_stack_first_prefix_everywhere),
])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(sf, name, mutant)
    assert not _all_pins()


