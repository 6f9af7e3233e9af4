"""Pins of the oracle's interaction variants ("DHEN" notes, 3.1: inner products for i <= j;
Solution 2: the FM sum by the squared-norm identity; 3.3, eq. (7): the whole Gram matrix)
against facts that do not come from the oracle's own loops.

* The forward values are checked against a library routine (numpy matmul of Z with its
  transpose, the Gram matrix), read at the documented pair positions.
* Closed forms: F copies of one vector give C(F, 2) ||v||^2 for the FM sum and ||v||^2 on
  every self-dot.
* The gradients are checked with central finite differences of L = <dR, R(Z)>.  L is a
  quadratic in Z, so central differences are exact up to rounding.  A dropped factor 2 on
  the self-dots, or a wrong pair index, fails here.
No GPU is used.
"""
import numpy as np
import pytest

from oracle import oracle as orc


def _gram(Z):
    return Z @ np.transpose(Z, (0, 2, 1))


@pytest.mark.parametrize("B,F,d", [(3, 1, 4), (4, 5, 8), (2, 17, 3), (1, 33, 2)])
def test_self_fwd_is_the_gram_lower_triangle(B, F, d):
    rng = np.random.default_rng(F * 100 + d)
    Z = rng.standard_normal((B, F, d))
    R, Rm = orc.interaction_self_fwd(Z)
    G = _gram(Z)
    assert R.shape == (B, d + F * (F + 1) // 2)
    np.testing.assert_array_equal(R[:, :d], Z[:, 0])
    q = 0
    for i in range(F):
        for j in range(i + 1):
            np.testing.assert_allclose(R[:, d + q], G[:, i, j], rtol=1e-13, atol=1e-13)
            q += 1
    # the self-dots are the squared norms, and the magnitude bounds every entry
    diag = [i * (i + 1) // 2 + i for i in range(F)]
    np.testing.assert_allclose(R[:, d + np.array(diag)], (Z ** 2).sum(-1), rtol=1e-13)
    assert np.all(Rm >= np.abs(R) - 1e-12)


def test_self_and_strict_sets_agree_off_the_diagonal():
    rng = np.random.default_rng(3)
    B, F, d = 3, 7, 5
    Z = rng.standard_normal((B, F, d))
    Rs, _ = orc.interaction_self_fwd(Z)
    R, _ = orc.interaction_fwd(Z)
    for i in range(1, F):
        for j in range(i):
            np.testing.assert_array_equal(Rs[:, d + i * (i + 1) // 2 + j],
                                          R[:, d + i * (i - 1) // 2 + j])


def _fd_grad(f, Z, h=0.5):
    """Central differences of a quadratic scalar function (exact up to rounding)."""
    g = np.zeros_like(Z)
    for idx in np.ndindex(Z.shape):
        zp = Z.copy()
        zm = Z.copy()
        zp[idx] += h
        zm[idx] -= h
        g[idx] = (f(zp) - f(zm)) / (2 * h)
    return g


@pytest.mark.parametrize("F,d", [(1, 3), (4, 2), (6, 3)])
def test_self_bwd_is_the_derivative(F, d):
    rng = np.random.default_rng(F + 10 * d)
    B = 2
    Z = rng.standard_normal((B, F, d))
    dR = rng.standard_normal((B, d + F * (F + 1) // 2))
    dZ, dm = orc.interaction_self_bwd(Z, dR)
    want = _fd_grad(lambda z: float((orc.interaction_self_fwd(z)[0] * dR).sum()), Z)
    np.testing.assert_allclose(dZ, want, rtol=1e-10, atol=1e-10)
    assert np.all(dm >= np.abs(dZ) - 1e-12)


@pytest.mark.parametrize("B,F,d", [(5, 1, 4), (4, 2, 3), (3, 9, 16), (2, 27, 8)])
def test_fm_fwd_is_the_sum_of_pair_dots(B, F, d):
    rng = np.random.default_rng(B * F * d)
    Z = rng.standard_normal((B, F, d))
    out, om = orc.fm_fwd(Z)
    G = _gram(Z)
    want = np.array([np.tril(G[b], -1).sum() for b in range(B)])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    # the magnitude covers the self terms of the squared-norm form
    assert np.all(om >= 0.5 * (Z ** 2).sum((1, 2)) - 1e-12)


def test_fm_closed_form_for_equal_vectors():
    v = np.array([1.5, -2.0, 0.25, 3.0])
    for F in (1, 2, 5, 30):
        Z = np.tile(v, (1, F, 1))
        out, _ = orc.fm_fwd(Z)
        assert out[0] == F * (F - 1) // 2 * float(v @ v)


@pytest.mark.parametrize("F,d", [(1, 2), (3, 3), (7, 2)])
def test_fm_bwd_is_the_derivative(F, d):
    rng = np.random.default_rng(F * 7 + d)
    B = 3
    Z = rng.standard_normal((B, F, d))
    dout = rng.standard_normal(B)
    dZ, dm = orc.fm_bwd(Z, dout)
    want = _fd_grad(lambda z: float((orc.fm_fwd(z)[0] * dout).sum()), Z)
    np.testing.assert_allclose(dZ, want, rtol=1e-10, atol=1e-10)
    assert np.all(dm >= np.abs(dZ) - 1e-12)


# ----------------------------------------------------------------------------- Gram matrix
# "DHEN" notes, 3.3, eq. (7): a DCN-style layer takes the whole Gram matrix X X^T.

@pytest.mark.parametrize("B,F,d", [(3, 1, 4), (4, 5, 8), (2, 17, 3), (1, 33, 2)])
def test_gram_fwd_is_the_gram_matrix(B, F, d):
    rng = np.random.default_rng(F * 7 + d)
    Z = rng.standard_normal((B, F, d))
    R, Rm = orc.interaction_gram_fwd(Z)
    assert R.shape == (B, d + F * F)
    np.testing.assert_array_equal(R[:, :d], Z[:, 0])
    G = R[:, d:].reshape(B, F, F)
    np.testing.assert_allclose(G, _gram(Z), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(G, np.transpose(G, (0, 2, 1)))          # symmetric exactly
    np.testing.assert_allclose(np.diagonal(G, axis1=1, axis2=2), (Z ** 2).sum(-1), rtol=1e-13)
    np.testing.assert_allclose(Rm[:, d:].reshape(B, F, F), _gram(np.abs(Z)), rtol=1e-13)
    # its lower triangle with the diagonal is the self-dot pair set, value for value
    Rs, _ = orc.interaction_self_fwd(Z)
    si, sj = np.tril_indices(F, 0)
    np.testing.assert_array_equal(G[:, si, sj], Rs[:, d:])


@pytest.mark.parametrize("F,d", [(1, 3), (4, 2), (6, 3)])
def test_gram_bwd_is_the_derivative(F, d):
    rng = np.random.default_rng(F + 100 * d)
    B = 2
    Z = rng.standard_normal((B, F, d))
    dR = rng.standard_normal((B, d + F * F))
    dZ, dm = orc.interaction_gram_bwd(Z, dR)
    want = _fd_grad(lambda z: float((orc.interaction_gram_fwd(z)[0] * dR).sum()), Z)
    np.testing.assert_allclose(dZ, want, rtol=1e-10, atol=1e-10)
    assert np.all(dm >= np.abs(dZ) - 1e-12)


def test_gram_bwd_of_a_lower_triangle_is_the_self_bwd():
    """dG zero above the diagonal: S_ij = dG_(max,min), S_ii = 2 dG_ii, the self-dot set's
    chain rule exactly."""
    rng = np.random.default_rng(8)
    B, F, d = 3, 7, 5
    Z = rng.standard_normal((B, F, d))
    dRs = rng.standard_normal((B, d + F * (F + 1) // 2))
    dG = np.zeros((B, F, F))
    si, sj = np.tril_indices(F, 0)
    dG[:, si, sj] = dRs[:, d:]
    dR = np.concatenate([dRs[:, :d], dG.reshape(B, F * F)], axis=1)
    for bf16 in (False, True):
        got, _ = orc.interaction_gram_bwd(Z, dR, bf16=bf16)
        want, _ = orc.interaction_self_bwd(Z, dRs, bf16=bf16)
        np.testing.assert_array_equal(got, want)


def test_gram_bf16_operands_against_torch_cast():
    """bf16 mode: factors rounded with torch's own cast; the backward's S_ij is the binary32
    sum of the two mirrored gradients (numpy float32 addition), then rounded."""
    import torch

    def bf(x):
        return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()

    rng = np.random.default_rng(31)
    B, F, d = 3, 9, 16
    Z = rng.standard_normal((B, F, d))
    dR = rng.standard_normal((B, d + F * F)).astype(np.float32).astype(np.float64)
    Zb = bf(Z)
    R, _ = orc.interaction_gram_fwd(Z, bf16=True)
    np.testing.assert_allclose(R[:, d:].reshape(B, F, F), _gram(Zb), rtol=1e-13, atol=1e-13)
    g = dR[:, d:].reshape(B, F, F).astype(np.float32)
    S = bf((g + np.transpose(g, (0, 2, 1))).astype(np.float64))      # float32 sums
    want = np.matmul(S, Zb)
    want[:, 0, :] += dR[:, :d]
    dZ, dm = orc.interaction_gram_bwd(Z, dR, bf16=True)
    np.testing.assert_allclose(dZ, want, rtol=1e-12, atol=1e-12)
    wm = np.matmul(np.abs(S), np.abs(Zb))
    wm[:, 0, :] += np.abs(dR[:, :d])
    np.testing.assert_allclose(dm, wm, rtol=1e-12)
