"""Pins of the oracle's fully connected layer, its backward with the SGD step, and the
logistic head with normalized entropy ("Meta DLRM", 02: bottom MLP, top MLP and a sigmoid
for the click probability; "DHEN" notes, 7.1 "Setup": NE, and Solution 16/17: NE = 1 for
the base-rate predictor, the softplus form of the cross-entropy).

Nothing here reuses the oracle's arithmetic: the forward is checked against Python loops,
the bf16 operand rounding against an integer-bit rounding written here, every gradient
against central finite differences of the loss it differentiates, and the head against
closed forms.  No GPU is used.
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc


def _brute_layer(X, W, b, relu):
    M, K = X.shape
    N = W.shape[0]
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0 if b is None else float(b[n])
            for k in range(K):
                acc += float(X[m, k]) * float(W[n, k])
            Y[m][n] = max(acc, 0.0) if relu else acc
    return np.array(Y)


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_dense_fwd_matches_loops(relu, with_bias):
    rng = np.random.default_rng(0)
    M, K, N = 7, 13, 5
    # small integers: every product and sum is exact, so the results must be equal
    X = rng.integers(-8, 9, (M, K)).astype(np.float64)
    W = rng.integers(-8, 9, (N, K)).astype(np.float64)
    b = rng.integers(-20, 21, N).astype(np.float64) if with_bias else None
    Y, Ym = orc.dense_fwd(X, W, b, relu, False)
    np.testing.assert_array_equal(Y, _brute_layer(X, W, b, relu))
    want_m = np.abs(X) @ np.abs(W).T + (0 if b is None else np.abs(b))
    np.testing.assert_array_equal(Ym, want_m)
    if relu:
        assert np.all(Y >= 0) and np.any(Y == 0)


def _bf16_rne_bits(x):
    """Nearest-even bf16 of binary32 values by integer arithmetic on their bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_dense_bf16_operands_are_rounded_nearest_even():
    # ties: 1 + 2^-8 is half an ulp above 1 (even) -> 1; 1 + 3 * 2^-8 -> 1 + 2^-6 (even)
    X = np.array([[1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9]])
    W = np.eye(3)
    Y, _ = orc.dense_fwd(X, W, None, False, True)
    np.testing.assert_array_equal(Y[0], [1.0, 1 + 2.0 ** -6, 1.0])
    rng = np.random.default_rng(1)
    X = rng.standard_normal((9, 40)).astype(np.float32)
    W = rng.standard_normal((6, 40)).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    Y, _ = orc.dense_fwd(X, W, b, True, True)
    Xr, Wr = _bf16_rne_bits(X), _bf16_rne_bits(W)
    want = np.maximum(Xr @ Wr.T + b.astype(np.float64), 0.0)
    np.testing.assert_allclose(Y, want, rtol=1e-12, atol=1e-12)


def _layer_loss(X, W, b, G, relu):
    Y, _ = orc.dense_fwd(X, W, b, relu, False)
    return float(np.sum(G * Y))


def _away_from_kinks(X, W, b, h):
    pre = X @ W.T + b
    return np.min(np.abs(pre)) > 100 * h


@pytest.mark.parametrize("relu", [False, True])
def test_dense_bwd_is_the_gradient(relu):
    """dX, the weight step and the bias step against central differences of
    L = sum(G * layer(X, W, b)); with lr = 1 the step is W - dL/dW."""
    rng = np.random.default_rng(2 + relu)
    M, K, N = 6, 5, 4
    h = 1e-6
    for _ in range(20):
        X = rng.standard_normal((M, K))
        W = rng.standard_normal((N, K)).astype(np.float32).astype(np.float64)
        b = rng.standard_normal(N).astype(np.float32).astype(np.float64)
        if _away_from_kinks(X, W, b, h):
            break
    G = rng.standard_normal((M, N))
    Y, _ = orc.dense_fwd(X, W, b, relu, False)
    out = orc.dense_bwd_sgd(X, W, b, relu, Y, G, False, 1.0)

    def fd(arr, idx):
        a0 = arr[idx]
        arr[idx] = a0 + h
        lp = _layer_loss(X, W, b, G, relu)
        arr[idx] = a0 - h
        lm = _layer_loss(X, W, b, G, relu)
        arr[idx] = a0
        return (lp - lm) / (2 * h)

    for idx in np.ndindex(M, K):
        assert abs(out["dX"][idx] - fd(X, idx)) < 1e-6
    step_w = W - out["W"]                       # = dL/dW, up to the binary32 rounding of W'
    for idx in np.ndindex(N, K):
        assert abs(step_w[idx] - fd(W, idx)) < 1e-5 * (1 + abs(W[idx]))
    step_b = b - out["b"]
    for n in range(N):
        assert abs(step_b[n] - fd(b, (n,))) < 1e-5 * (1 + abs(b[n]))
    if relu:                                    # rows where the unit is off get no gradient
        off = Y <= 0
        assert off.any()
        np.testing.assert_allclose(out["dX"], (G * ~off) @ W, rtol=0, atol=1e-13)


def test_dense_step_scales_with_lr_and_rounds_to_binary32():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((8, 3))
    W = rng.standard_normal((2, 3)).astype(np.float32).astype(np.float64)
    G = rng.standard_normal((8, 2))
    o1 = orc.dense_bwd_sgd(X, W, None, False, None, G, False, 0.01, want_dx=False)
    dW = G.T @ X
    np.testing.assert_array_equal(o1["W"], (W - 0.01 * dW).astype(np.float32).astype(np.float64))
    assert "dX" not in o1 and "b" not in o1


def test_dense_zero_rows_leave_parameters():
    W = np.ones((3, 4))
    b = np.full(3, 0.5)
    out = orc.dense_bwd_sgd(np.zeros((0, 4)), W, b, True, np.zeros((0, 3)), np.zeros((0, 3)),
                            False, 0.1)
    np.testing.assert_array_equal(out["W"], W)
    np.testing.assert_array_equal(out["b"], b)


def _mean_ce(s, y):
    return float(np.mean([math.log1p(math.exp(-abs(a))) + max(a, 0.0) - t * a
                          for a, t in zip(s, y)]))


def test_head_closed_forms():
    # s = 0: p = 1/2, ce = ln 2 for either label
    y = np.array([0, 1, 1, 0, 1.0])
    prob, dl, _, st, _ = orc.logistic_ne(np.zeros(5), y)
    np.testing.assert_allclose(prob, 0.5)
    assert abs(st[0] - 5 * math.log(2)) < 1e-14 and st[1] == 3
    np.testing.assert_allclose(dl, (0.5 - y) / 5)
    q = 0.6
    assert abs(st[2] - math.log(2) / -(q * math.log(q) + (1 - q) * math.log(1 - q))) < 1e-14
    # predicting the base rate everywhere gives NE = 1 exactly (up to rounding)
    for q_n in (1, 3, 7):
        y = np.zeros(10)
        y[:q_n] = 1
        q = q_n / 10
        s = np.full(10, math.log(q / (1 - q)))
        assert abs(orc.logistic_ne(s, y)[3][2] - 1.0) < 1e-12
    # far tails: the stable form keeps the tiny loss of a confident correct prediction
    _, _, _, st, _ = orc.logistic_ne(np.array([50.0, -50.0, 50.0]), np.array([1.0, 0.0, 0.0]))
    assert abs(st[0] - (2 * math.exp(-50) + 50 + math.log1p(math.exp(-50)))) < 1e-12
    one = orc.logistic_ne(np.array([50.0]), np.array([1.0]))[3][0]
    assert one > 0 and abs(one - math.exp(-50)) < 1e-12 * math.exp(-50)
    # a batch with one label value has no entropy: NE is undefined
    assert math.isnan(orc.logistic_ne(np.array([0.3, -1.0]), np.ones(2))[3][2])


def test_head_gradient_is_the_derivative_of_the_mean():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(12) * 3
    y = (rng.random(12) < 0.4).astype(np.float64)
    _, dl, _, st, _ = orc.logistic_ne(s, y)
    assert abs(st[0] / 12 - _mean_ce(s, y)) < 1e-14
    h = 1e-6
    for i in range(12):
        sp, sm = s.copy(), s.copy()
        sp[i] += h
        sm[i] -= h
        assert abs(dl[i] - (_mean_ce(sp, y) - _mean_ce(sm, y)) / (2 * h)) < 1e-8


def test_two_layers_and_head_chain():
    """The composition used by the training step: layer 1 (ReLU) -> layer 2 (linear, one
    logit) -> head.  The input gradient obtained by feeding each backward's dX to the layer
    below matches central differences of the mean cross-entropy."""
    rng = np.random.default_rng(6)
    M, K, H = 5, 4, 6
    X = rng.standard_normal((M, K))
    W1 = rng.standard_normal((H, K)).astype(np.float32).astype(np.float64)
    b1 = rng.standard_normal(H).astype(np.float32).astype(np.float64)
    W2 = rng.standard_normal((1, H)).astype(np.float32).astype(np.float64)
    y = np.array([1, 0, 1, 1, 0.0])

    def loss(Xv):
        a, _ = orc.dense_fwd(Xv, W1, b1, True, False)
        s, _ = orc.dense_fwd(a, W2, None, False, False)
        return orc.logistic_ne(s[:, 0], y)[3][0] / M

    A1, _ = orc.dense_fwd(X, W1, b1, True, False)
    S, _ = orc.dense_fwd(A1, W2, None, False, False)
    _, dl, _, _, _ = orc.logistic_ne(S[:, 0], y)
    g2 = orc.dense_bwd_sgd(A1, W2, None, False, None, dl[:, None], False, 0.0)
    g1 = orc.dense_bwd_sgd(X, W1, b1, True, A1, g2["dX"], False, 0.0)
    h = 1e-6
    for idx in np.ndindex(M, K):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        assert abs(g1["dX"][idx] - (loss(Xp) - loss(Xm)) / (2 * h)) < 1e-7
    # lr = 0 leaves every parameter as it was
    np.testing.assert_array_equal(g1["W"], W1)
    np.testing.assert_array_equal(g1["b"], b1)


def test_dense_bf16_bias_step_is_the_ones_column():
    """With bf16 operands the bias moves like the weight of an extra input fixed at 1: the
    same step as a bias-free layer whose input has a column of ones appended."""
    rng = np.random.default_rng(8)
    M, K, N = 40, 6, 3
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    G = rng.standard_normal((M, N)).astype(np.float32)
    o = orc.dense_bwd_sgd(X, W, b, False, None, G, True, 0.5)
    Xa = np.concatenate([X, np.ones((M, 1), np.float32)], axis=1)
    Wa = np.concatenate([W, b[:, None]], axis=1)
    oa = orc.dense_bwd_sgd(Xa, Wa, None, False, None, G, True, 0.5)
    np.testing.assert_array_equal(o["W"], oa["W"][:, :K])
    np.testing.assert_array_equal(o["b"], oa["W"][:, K])
    # and the rounding is there: the fp32-operand step differs
    o32 = orc.dense_bwd_sgd(X, W, b, False, None, G, False, 0.5)
    assert not np.array_equal(o["b"], o32["b"])
