"""Pins of the oracle's ratio-m compression (`compress`): the per-channel
softmax of m tokens' logits weighting their values, the ratio-2 rule of the
pages (ai.info "Methodology in Plain English": compression without overlapping
source entries) widened to m tokens.  Each pin is fixed by the definition, not
by re-running it."""
import math

import numpy as np

import synth


def test_ratio_two_is_the_pair_rule(orc):
    x = synth.normal(91, "x", (64, 512))
    z = synth.normal(91, "z", (64, 512)) * np.float32(3.0)
    assert np.array_equal(orc.compress(x, z, 2).view(np.uint32), orc.compress_pairs(x, z).view(np.uint32))


def test_ratio_one_is_the_token(orc):
    x = synth.normal(92, "x", (5, 512))
    z = synth.normal(92, "z", (5, 512))
    assert np.array_equal(orc.compress(x, z, 1).view(np.uint32), x.view(np.uint32))


def test_equal_logits_give_the_mean(orc):
    for m in (3, 4, 8, 16):
        x = synth.normal(93, f"x{m}", (2 * m, 512))
        z = np.full((2 * m, 512), np.float32(0.7), np.float32)
        got = orc.compress(x, z, m).astype(np.float64)
        want = x.astype(np.float64).reshape(2, m, 512).sum(axis=1) / m
        assert np.allclose(got, want, rtol=2e-7, atol=1e-30), m


def test_one_dominant_logit_selects_its_token(orc):
    m = 5
    x = synth.normal(94, "x", (3 * m, 512))
    z = np.full((3 * m, 512), np.float32(-300.0), np.float32)
    pick = np.array([0, 3, 4])  # the token of each entry whose logit dominates
    for e, j in enumerate(pick):
        z[e * m + j] = 0.0
    got = orc.compress(x, z, m)
    want = np.stack([x[e * m + j] for e, j in enumerate(pick)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))  # exp(-300) vanishes next to 1


def test_worked_weights(orc):
    """Logits ln 1, ln 2, ln 4 weight 1 : 2 : 4, so values 1, 2, 4 give
    (1 + 4 + 16) / 7 = 3 (up to the fp32 logits' rounding)."""
    x = np.zeros((3, 512), np.float32)
    z = np.zeros((3, 512), np.float32)
    x[:, 0] = [1.0, 2.0, 4.0]
    z[:, 0] = [0.0, math.log(2.0), math.log(4.0)]
    x[:, 1] = [-5.0, 7.0, 0.5]     # equal logits: the mean
    got = orc.compress(x, z, 3)[0]
    assert abs(float(got[0]) - 3.0) < 1e-6
    assert abs(float(got[1]) - (2.5 / 3.0)) < 1e-6


def test_order_of_tokens_does_not_matter(orc):
    """Permuting an entry's tokens (values with their logits) changes only the
    rounding of the sums."""
    m = 6
    x = synth.normal(95, "x", (4 * m, 512))
    z = synth.normal(95, "z", (4 * m, 512)) * np.float32(2.0)
    perm = np.array([5, 2, 0, 4, 1, 3])
    idx = np.concatenate([e * m + perm for e in range(4)])
    a = orc.compress(x, z, m)
    b = orc.compress(x[idx], z[idx], m)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-30)


def test_cache_append_with_ratio_four(orc):
    """quantize_append at ratio 4 stores the compressed entries: the same
    bytes as quantising compress() of the tokens directly."""
    B, T, m = 2, 12, 4
    kv = synth.normal(96, "kv", (B, T, 512))
    lg = synth.normal(96, "lg", (B, T, 512))
    ik = synth.normal(96, "ik", (B, T // m, 64))
    c = orc.Cache(B, 10, m)
    orc.quantize_append(c, kv, ik, logits=lg)
    assert c.length.tolist() == [3, 3]
    for b in range(B):
        codes, scales = orc.quantize_main(orc.compress(kv[b], lg[b], m))
        assert np.array_equal(c.kv_codes[b, :3], codes) and np.array_equal(c.kv_scales[b, :3], scales)
