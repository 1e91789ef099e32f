"""Pins of the oracle's indexer-K projection (ai.info "Methodology in Plain
English": indexer K comes from a projection of the main KV entries): each is
checked against something other than the oracle's own formula."""
from fractions import Fraction

import numpy as np

import oracle as orc
import synth


def f32_round(x: Fraction) -> np.float32:
    """The fp32 value nearest to the exact rational x, ties to even (by search
    over the neighbours of a close candidate)."""
    c = np.float32(float(x))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(v)) - x)
        key = (d, int(np.float32(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def test_projection_selects_channels():
    """A one-hot w_ik picks channels: every output is exactly the chosen input."""
    e = synth.normal(41, "pe", (5, 512))
    sel = synth.integers(41, "sel", (64,), 0, 512)
    w = np.zeros((512, 64), np.float32)
    w[sel, np.arange(64)] = 1.0
    k = orc.project_ik(e, w)
    assert np.array_equal(k.view(np.uint32), e[:, sel].view(np.uint32))


def test_projection_exact_rational():
    """Against exact rational sums rounded once to fp32."""
    e = synth.normal(42, "pe", (3, 512))
    w = (synth.normal(42, "pw", (512, 64)) / np.float32(22.0)).astype(np.float32)
    k = orc.project_ik(e, w)
    ef = [[Fraction(float(v)) for v in row] for row in e]
    for r in range(3):
        for d in range(0, 64, 7):
            exact = sum(ef[r][c] * Fraction(float(w[c, d])) for c in range(512))
            assert k[r, d] == f32_round(exact), (r, d)


def test_projection_scales_with_weights():
    """Doubling w_ik (exact in fp32) doubles every output exactly."""
    e = synth.normal(43, "pe", (4, 512))
    w = synth.normal(43, "pw", (512, 64))
    assert np.array_equal(orc.project_ik(e, 2.0 * w), 2.0 * orc.project_ik(e, w))


def test_append_proj_ratio2_projects_the_compressed_entry():
    """At ratio 2 with equal logits the entry is the pair's mean, and the stored
    indexer K is that mean projected and quantised."""
    B, T = 2, 6
    x = synth.normal(44, "px", (B, T, 512))
    z = np.zeros((B, T, 512), np.float32)
    w = (synth.normal(44, "pw", (512, 64)) / np.float32(22.0)).astype(np.float32)
    c = orc.Cache(B, 8, 2)
    orc.quantize_append_proj(c, x, w, logits=z)
    mean = ((x[:, 0::2].astype(np.float64) + x[:, 1::2]) / 2).astype(np.float32)
    codes, scales = orc.quantize_ik(orc.project_ik(mean, w))
    assert np.array_equal(c.ik_codes[:, :3], codes)
    assert np.array_equal(c.ik_scales[:, :3].view(np.uint32), scales.view(np.uint32))
    assert list(c.length) == [3, 3]
