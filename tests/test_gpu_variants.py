"""Interaction variants on the GPU through the C ABI, against the oracle ("DHEN" notes, 3.1:
the pair set with self-dots; Solution 2: the FM sum by the squared-norm identity; 3.3,
eq. (7): the whole Gram matrix).

The self-dot cases span the three arithmetic paths: the fp32 lane kernels (including a
shape whose LDS partials no longer fit, which falls back), the LDS-staged fp32 kernels, and
bf16 on matrix cores (single and several 32-row blocks), plus F = 1.  The FM cases span F
from 1 to 65 and dims below, at and above one wavefront of columns.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr
from tests.parity import RTOL_F32, assert_close, gamma
from tests.test_gpu_parity import DEV, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SELF_CASES = [
    ("f32", 128, 5, 16), ("f32", 2048, 9, 64), ("f32", 77, 1, 4), ("f32", 33, 27, 128),
    ("f32", 50, 16, 4),            # lanes shape, partials above 64 KiB: LDS-staged fallback
    ("f32", 19, 17, 48), ("f32", 64, 33, 16), ("f32", 45, 32, 256),
    ("bf16", 100, 27, 128), ("bf16", 67, 65, 128), ("bf16", 40, 5, 16), ("bf16", 9, 1, 32),
    ("bf16", 13, 100, 64), ("bf16", 6, 128, 128), ("bf16", 10, 17, 16),
]


def _inputs(B, F, d, width, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, F, d)).astype(np.float32)
    dR = rng.standard_normal((B, width)).astype(np.float32)
    return Z, dR


@pytest.mark.parametrize("compute,B,F,d", SELF_CASES)
def test_self_fwd_matches_oracle(compute, B, F, d):
    say("interaction_self_fwd", compute, B, F, d)
    P = F * (F + 1) // 2
    Z, _ = _inputs(B, F, d, d + P, 11)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    R = host(ctr.ctr_dot_interaction_self_fwd(dev(Z), code))
    want, mag = orc.interaction_self_fwd(Z.astype(np.float64), bf16=compute == "bf16")
    assert_close(R, want, mag, gamma(d), "self fwd")
    np.testing.assert_array_equal(R[:, :d], Z[:, 0, :])


@pytest.mark.parametrize("compute,B,F,d", SELF_CASES)
def test_self_bwd_matches_oracle(compute, B, F, d):
    say("interaction_self_bwd", compute, B, F, d)
    P = F * (F + 1) // 2
    Z, dR = _inputs(B, F, d, d + P, 12)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    dZ = host(ctr.ctr_dot_interaction_self_bwd(dev(Z), dev(dR), code))
    want, mag = orc.interaction_self_bwd(Z.astype(np.float64), dR.astype(np.float64),
                                         bf16=compute == "bf16")
    # F pair terms (the self term included) and the dense gradient
    assert_close(dZ, want, mag, gamma(F + 1), "self bwd")


def test_self_strided_output_and_strict_unchanged():
    B, F, d = 50, 9, 64
    P = F * (F + 1) // 2
    Z, _ = _inputs(B, F, d, 1, 13)
    big = torch.full((B, d + P + 12), -7.0, device=DEV)
    ctr.ctr_dot_interaction_self_fwd(dev(Z), ctr.CTR_F32, big)
    got = host(big)
    want, mag = orc.interaction_self_fwd(Z.astype(np.float64))
    assert_close(got[:, :d + P], want, mag, gamma(d), "strided self R")
    assert np.all(got[:, d + P:] == -7.0)
    # the strict entry point still writes F(F-1)/2 pairs
    Rs = host(ctr.ctr_dot_interaction_fwd(dev(Z), ctr.CTR_F32))
    assert Rs.shape == (B, d + F * (F - 1) // 2)


# ----------------------------------------------------------------------------- Gram matrix
# "DHEN" notes, 3.3, eq. (7): the whole F x F Gram matrix.  Shapes cover the fp32 lane
# kernels (F <= 16, dim = 4L), the LDS-staged fp32 kernels (F above 16, other dims), and
# bf16 on matrix cores over one to four 32-row blocks.
GRAM_CASES = [
    ("f32", 128, 5, 16), ("f32", 300, 16, 4), ("f32", 77, 1, 8), ("f32", 33, 27, 128),
    ("f32", 19, 17, 48), ("f32", 64, 9, 256),
    ("bf16", 100, 27, 128), ("bf16", 67, 65, 128), ("bf16", 40, 5, 16), ("bf16", 9, 1, 32),
    ("bf16", 13, 100, 64), ("bf16", 6, 128, 128), ("bf16", 10, 17, 16),
]


@pytest.mark.parametrize("compute,B,F,d", GRAM_CASES)
def test_gram_fwd_matches_oracle(compute, B, F, d):
    say("interaction_gram_fwd", compute, B, F, d)
    Z, _ = _inputs(B, F, d, 1, 21)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    R = host(ctr.ctr_dot_interaction_gram_fwd(dev(Z), code))
    want, mag = orc.interaction_gram_fwd(Z.astype(np.float64), bf16=compute == "bf16")
    assert_close(R, want, mag, gamma(d), "gram fwd")
    np.testing.assert_array_equal(R[:, :d], Z[:, 0, :])
    G = R[:, d:].reshape(B, F, F)
    np.testing.assert_array_equal(G, np.transpose(G, (0, 2, 1)))     # one dot, two places


@pytest.mark.parametrize("compute,B,F,d", GRAM_CASES)
def test_gram_bwd_matches_oracle(compute, B, F, d):
    say("interaction_gram_bwd", compute, B, F, d)
    Z, dR = _inputs(B, F, d, d + F * F, 22)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    dZ = host(ctr.ctr_dot_interaction_gram_bwd(dev(Z), dev(dR), code))
    want, mag = orc.interaction_gram_bwd(Z.astype(np.float64), dR.astype(np.float64),
                                         bf16=compute == "bf16")
    # fp32: the binary32 sum S_ij, F fused multiply-adds and the dense gradient; bf16: the
    # same S on both sides, F products exact in fp32 and the dense gradient
    assert_close(dZ, want, mag, gamma(F + 2 if compute == "f32" else F + 1), "gram bwd")
    if compute == "bf16":
        dZb = torch.empty((B, F, d), dtype=torch.bfloat16, device=DEV)
        ctr.ctr_dot_interaction_gram_bwd(dev(Z), dev(dR), code, dZb)
        np.testing.assert_array_equal(host(dZb), host(torch.from_numpy(dZ).to(torch.bfloat16)))


def test_gram_strided_output_and_bad_stride():
    B, F, d = 40, 6, 32
    Z, _ = _inputs(B, F, d, 1, 23)
    big = torch.full((B, d + F * F + 5), -3.0, device=DEV)
    ctr.ctr_dot_interaction_gram_fwd(dev(Z), ctr.CTR_F32, big)
    got = host(big)
    want, mag = orc.interaction_gram_fwd(Z.astype(np.float64))
    assert_close(got[:, :d + F * F], want, mag, gamma(d), "strided gram R")
    assert np.all(got[:, d + F * F:] == -3.0)
    small = torch.empty((B, d + F * F - 1), device=DEV)
    with pytest.raises(ctr.CtrError):
        ctr.ctr_dot_interaction_gram_fwd(dev(Z), ctr.CTR_F32, small)


FM_CASES = [(128, 5, 16), (2048, 9, 64), (77, 27, 128), (33, 1, 8), (50, 65, 128),
            (9, 2, 200), (1000, 101, 32)]


def _fm_inputs(B, F, d, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, F, d)).astype(np.float32)
    dout = rng.standard_normal(B).astype(np.float32)
    return Z, dout


@pytest.mark.parametrize("B,F,d", FM_CASES)
def test_fm_fwd_matches_oracle(B, F, d):
    say("fm_fwd", B, F, d)
    Z, _ = _fm_inputs(B, F, d, 21)
    out = host(ctr.ctr_fm_interaction_fwd(dev(Z)))
    want, mag = orc.fm_fwd(Z.astype(np.float64))
    assert_close(out, want, mag, RTOL_F32, "fm fwd")


@pytest.mark.parametrize("B,F,d", FM_CASES)
def test_fm_bwd_matches_oracle(B, F, d):
    say("fm_bwd", B, F, d)
    Z, dout = _fm_inputs(B, F, d, 22)
    dZ = host(ctr.ctr_fm_interaction_bwd(dev(Z), dev(dout)))
    want, mag = orc.fm_bwd(Z.astype(np.float64), dout.astype(np.float64))
    assert_close(dZ, want, mag, RTOL_F32, "fm bwd")


def test_fm_equals_sum_of_strict_pairs_on_gpu():
    # two GPU paths, O(F^2 d) pairs summed on the host in fp64 vs the O(F d) identity
    B, F, d = 64, 27, 128
    Z, _ = _fm_inputs(B, F, d, 23)
    R = host(ctr.ctr_dot_interaction_fwd(dev(Z), ctr.CTR_F32)).astype(np.float64)
    fm = host(ctr.ctr_fm_interaction_fwd(dev(Z)))
    _, mag = orc.fm_fwd(Z.astype(np.float64))
    assert_close(fm, R[:, d:].sum(axis=1), mag, 4 * RTOL_F32, "fm vs pairs")
