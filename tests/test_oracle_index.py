"""Pins of the oracle's indexer score, Top-512, candidate pool and Reindex."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth


def _e4m3_exact(codes):
    # exact values from a library implementation of OCP E4M3 (independent of the oracle)
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return [Fraction(float(v)) for v in t]


def test_score_hand_example(orc):
    # head 0 q = [448, 0...] -> s_q = 1, q8[0] = 448; key = [448, -1, ...] -> s_k = 1
    # dot_0 = 448 * 448 = 200704; head 1 q = [0, -448] -> dot = 448; head 2 q = [0, 448]
    # -> dot = -448 -> relu 0; head 3 all zero -> s_q = 0.  Weights (1, 2, 5, 7):
    # score = 1 * (200704 + 2 * 448) = 201600.
    iq = np.zeros((4, 64), np.float32)
    iq[0, 0] = 448.0
    iq[1, 1] = -448.0
    iq[2, 1] = 448.0
    q8, sq = orc.quantize_query(iq)
    assert list(sq) == [1.0, 1.0, 1.0, 0.0]
    k = np.zeros((1, 64), np.float32)
    k[0, 0], k[0, 1] = 448.0, -1.0
    k8, sk = orc.quantize_ik(k)
    w = np.array([1, 2, 5, 7], np.float32)
    assert orc.entry_score(q8, sq, w, k8[0], sk[0]) == 201600.0
    # the key scale multiplies the whole score; halving the key halves s_k
    k8b, skb = orc.quantize_ik(k * np.float32(0.5))
    assert np.array_equal(k8b, k8) and skb[0] == 0.5
    assert orc.entry_score(q8, sq, w, k8b[0], skb[0]) == 100800.0
    # a query scale: doubling head 1's query doubles its scale, not its codes
    iq2 = iq.copy()
    iq2[1] *= 2
    q8c, sqc = orc.quantize_query(iq2)
    assert np.array_equal(q8c, q8) and sqc[1] == 2.0
    assert orc.entry_score(q8c, sqc, w, k8[0], sk[0]) == 200704.0 + 2 * 2 * 448


def test_single_head_dot_is_exact(orc):
    """With unit scales and one head, the score is the exact dot when positive
    (the 64-term dot of E4M3 values fits in 53 bits), else 0."""
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    sq = np.array([1, 0, 0, 0], np.float32)
    for trial in range(300):
        if trial % 3 == 0:
            k8 = rng.choice(finite, 64).astype(np.uint8)
            qrow = rng.choice(finite, 64).astype(np.uint8)
        else:  # wide exponent spread: large and subnormal terms together
            k8 = rng.choice(finite, 64).astype(np.uint8)
            qrow = rng.choice(np.array([0x01, 0x02, 0x07, 0x7E, 0xFE, 0x7D, 0x81, 0x38], np.uint8), 64)
        q8 = np.zeros((4, 64), np.uint8)
        q8[0] = qrow
        exact = sum(a * b for a, b in zip(_e4m3_exact(qrow), _e4m3_exact(k8)))
        want = float(exact) if exact > 0 else 0.0
        assert Fraction(want) == max(exact, Fraction(0)), "the exact dot is representable"
        got = orc.entry_score(q8, sq, None, k8, 1.0)
        assert got == want, (trial, float(exact), got)


def test_multi_head_score_against_exact_rationals(orc):
    """Four heads with non-unit query and key scales and head weights (some
    negative, some zero) against the definition evaluated in exact rational
    arithmetic: s_k * sum_h w_h * s_qh * max(q8_h . k8, 0).  The oracle rounds
    the head products, the head sum and the key-scale product at fp64 precision,
    so it lies within a few units of 2^-53 of the sum of the terms' magnitudes
    (the usual bound for a sum whose terms may cancel)."""
    rng = np.random.default_rng(17)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n_pos = 0
    for trial in range(200):
        iq = rng.standard_normal((4, 64)).astype(np.float32) * np.float32(rng.choice([1e-3, 0.7, 3.0, 250.0]))
        if trial % 5 == 0:
            iq[rng.integers(0, 4)] = 0.0  # a zero head: s_q = 0
        q8, sq = orc.quantize_query(iq)
        k8 = rng.choice(finite, 64).astype(np.uint8)
        sk = np.float32(rng.choice([2.0 ** -9, 0.013, 1.0, 6.5]) * rng.uniform(0.5, 2.0))
        w = (rng.standard_normal(4) * 2).astype(np.float32)
        if trial % 4 == 0:
            w[rng.integers(0, 4)] = 0.0
        kv = _e4m3_exact(k8)
        exact, mag = Fraction(0), Fraction(0)
        for h in range(4):
            dot = sum(a * b for a, b in zip(_e4m3_exact(q8[h]), kv))
            term = Fraction(float(w[h])) * Fraction(float(sq[h])) * max(dot, Fraction(0))
            exact += term
            mag += abs(term)
        exact *= Fraction(float(sk))
        mag *= Fraction(float(sk))
        got = orc.entry_score(q8, sq, w, k8, float(sk))
        n_pos += exact > 0
        assert abs(Fraction(got) - exact) <= mag * Fraction(8, 2 ** 53), (trial, float(exact), got)
        if mag == abs(exact):  # no cancellation (non-negative weights): relative error bound
            assert abs(Fraction(got) - exact) <= abs(exact) * Fraction(4, 2 ** 53)
    assert n_pos > 20  # the cases are not all clipped to zero


def _cache_with_ik(orc, B, E, cap, seed_tag, cid=90, scale_rows=None):
    c = orc.Cache(B, cap, 1)
    for b in range(B):
        k = synth.normal_rows(cid, seed_tag, b * cap, E, 64)
        if scale_rows is not None:
            k = k * scale_rows
        codes, scales = orc.quantize_ik(k)
        c.ik_codes[b, :E] = codes
        c.ik_scales[b, :E] = scales
        c.length[b] = E
    return c


def _lexsort_topk(scores_row, visible, k):
    idx = np.nonzero(visible)[0]
    s = scores_row[idx]
    order = np.lexsort((idx, -s.astype(np.float64)))
    chosen = np.sort(idx[order[:k]])
    out = np.full(k, -1, np.int32)
    out[:len(chosen)] = chosen
    return out


@pytest.mark.parametrize("E", [1, 7, 511, 512, 513, 3000])
def test_full_topk_matches_full_sort(orc, E):
    B, Q, cap = 2, 3, 3100
    c = _cache_with_ik(orc, B, E, cap, "ik_sort")
    iq = synth.normal(91, f"iq{E}", (B, Q, 4, 64))
    q_pos = np.full((B, Q), E - 1, np.int32)  # every query sees the whole cache
    topk, _, scores = orc.index_topk(c, orc.FULL, iq, q_pos=q_pos, want_scores=True)
    for b in range(B):
        for q in range(Q):
            vis = np.arange(cap) < E
            assert np.array_equal(topk[b, q], _lexsort_topk(scores[b, q], vis, 512))


def test_relu_zero_ties_go_to_lower_index(orc):
    # keys all positive, queries all negative: every dot is negative, every score
    # is exactly +0, so Top-512 must be the 512 lowest indices
    B, E, cap = 1, 2000, 2000
    c = orc.Cache(B, cap, 1)
    k = np.abs(synth.normal_rows(92, "ik_pos", 0, E, 64)) + 0.1
    c.ik_codes[0], c.ik_scales[0] = orc.quantize_ik(k)
    c.length[0] = E
    iq = -np.abs(synth.normal(92, "iq_neg", (1, 1, 4, 64))) - 0.1
    topk, _, scores = orc.index_topk(c, orc.FULL, iq, want_scores=True)
    assert np.all(scores[0, 0] == 0) and not np.signbit(scores[0, 0]).any()
    assert np.array_equal(topk[0, 0], np.arange(512))


def test_planted_needles_are_selected_exactly(orc):
    B, E, cap = 1, 20000, 20000
    iq = synth.normal(93, "iq_needle", (1, 1, 4, 64))
    k = synth.normal_rows(93, "ik_needle", 0, E, 64) * np.float32(0.05)
    needles = np.sort(synth.integers(93, "needle_pos", (512,), 0, E))
    needles = np.unique(needles)
    # a needle key points along the sum of the four (positive-part) query heads
    direction = np.maximum(iq[0, 0], 0).sum(axis=0) + 1e-3
    k[needles] = direction / np.abs(direction).max() * 3.0
    c = orc.Cache(B, cap, 1)
    c.ik_codes[0], c.ik_scales[0] = orc.quantize_ik(k)
    c.length[0] = E
    topk, _, _ = orc.index_topk(c, orc.FULL, iq)
    got = topk[0, 0][topk[0, 0] >= 0]
    assert set(needles.tolist()) <= set(got.tolist())


def test_causal_visibility_ratio1_and_ratio2(orc):
    B, E, cap = 1, 300, 300
    for ratio in (1, 2):
        c = orc.Cache(B, cap, ratio)
        k = synth.normal_rows(94, "ik_causal", 0, E, 64)
        c.ik_codes[0], c.ik_scales[0] = orc.quantize_ik(k)
        c.length[0] = E
        ps = np.array([[0, 1, 2, 3, 57, 58, 599]], np.int32) if ratio == 2 else np.array([[0, 1, 5, 299]], np.int32)
        Q = ps.shape[1]
        iq = synth.normal(94, "iq_causal", (1, Q, 4, 64))
        topk, _, _ = orc.index_topk(c, orc.FULL, iq, q_pos=ps)
        for q in range(Q):
            p = int(ps[0, q])
            n_vis = min(E, (p + 1) // ratio)  # entry e visible iff (e+1)*r - 1 <= p
            got = topk[0, q]
            assert np.array_equal(got[got >= 0], np.arange(n_vis)), (ratio, p)
    # default positions: the last Q tokens of the sequence
    c = orc.Cache(1, 100, 1)
    c.ik_codes[0], c.ik_scales[0] = orc.quantize_ik(synth.normal_rows(94, "ik_c2", 0, 100, 64))
    c.length[0] = 100
    iq = synth.normal(94, "iq_c2", (1, 3, 4, 64))
    topk, _, _ = orc.index_topk(c, orc.FULL, iq)
    for q, n in enumerate((98, 99, 100)):
        assert np.array_equal(topk[0, q][topk[0, q] >= 0], np.arange(n))


def _check_pool(orc, topk, pool, scores, n_vis):
    p = pool[pool >= 0]
    assert np.all(pool[len(p):] == -1)
    assert np.all(np.diff(p) > 0)
    blocks = np.unique(p // 8)
    nblk_vis = (n_vis + 7) // 8
    assert len(blocks) == min(2048, nblk_vis)
    # each chosen block contributes all of its visible entries
    for blk in blocks:
        want = np.arange(blk * 8, min(blk * 8 + 8, n_vis))
        assert np.array_equal(p[(p >= blk * 8) & (p < blk * 8 + 8)], want)
    # top-512 is inside the pool
    t = topk[topk >= 0]
    assert set(t.tolist()) <= set(p.tolist())
    # no excluded block beats an included one under (max desc, block asc)
    bmax = np.array([scores[b * 8:min(b * 8 + 8, n_vis)].max() for b in range(nblk_vis)])
    inc = np.zeros(nblk_vis, bool)
    inc[blocks] = True
    if inc.all():
        return
    worst_in = min((bmax[b], -b) for b in np.nonzero(inc)[0])
    best_out = max((bmax[b], -b) for b in np.nonzero(~inc)[0])
    assert worst_in > best_out


@pytest.mark.parametrize("E", [100, 16384, 16390, 40003])
def test_pool_invariants(orc, E):
    B, cap = 1, 40008
    c = _cache_with_ik(orc, B, E, cap, "ik_pool")
    iq = synth.normal(95, f"iq_pool{E}", (1, 1, 4, 64))
    topk, pool, scores = orc.index_topk(c, orc.FULL, iq, want_pool=True, want_scores=True)
    _check_pool(orc, topk[0, 0], pool[0, 0], scores[0, 0], E)
    if E <= 16384:
        assert np.array_equal(pool[0, 0][:E], np.arange(E))


def test_reindex_with_full_queries_reproduces_full(orc):
    B, E, cap = 2, 50000, 50000
    c = _cache_with_ik(orc, B, E, cap, "ik_ri")
    iq = synth.normal(96, "iq_ri", (B, 1, 4, 64))
    topk, pool, _ = orc.index_topk(c, orc.FULL, iq, want_pool=True)
    topk_ri, _, _ = orc.index_topk(c, orc.REINDEX, iq, pool_in=pool)
    assert np.array_equal(topk, topk_ri)
    # with other queries Reindex differs from Full but stays inside the pool
    iq2 = synth.normal(96, "iq_ri2", (B, 1, 4, 64))
    topk2, _, _ = orc.index_topk(c, orc.REINDEX, iq2, pool_in=pool)
    for b in range(B):
        assert set(topk2[b, 0].tolist()) <= set(pool[b, 0].tolist())
    full2, _, _ = orc.index_topk(c, orc.FULL, iq2)
    assert not np.array_equal(full2, topk2)


def test_reindex_equals_full_when_pool_covers_context(orc):
    B, E, cap = 1, 9000, 9000
    c = _cache_with_ik(orc, B, E, cap, "ik_ri_small")
    iq = synth.normal(97, "iq_a", (B, 1, 4, 64))
    iq2 = synth.normal(97, "iq_b", (B, 1, 4, 64))
    _, pool, _ = orc.index_topk(c, orc.FULL, iq, want_pool=True)
    ri, _, _ = orc.index_topk(c, orc.REINDEX, iq2, pool_in=pool)
    full2, _, _ = orc.index_topk(c, orc.FULL, iq2)
    assert np.array_equal(ri, full2)


def test_head_weights_enter_linearly(orc):
    B, E, cap = 1, 600, 600
    c = _cache_with_ik(orc, B, E, cap, "ik_w")
    iq = synth.normal(98, "iq_w", (1, 1, 4, 64))
    w1 = np.ones((1, 1, 4), np.float32)
    w2 = np.full((1, 1, 4), 4.0, np.float32)  # a power of two scales every score exactly
    _, _, s1 = orc.index_topk(c, orc.FULL, iq, iw=w1, want_scores=True)
    _, _, s2 = orc.index_topk(c, orc.FULL, iq, iw=w2, want_scores=True)
    _, _, s0 = orc.index_topk(c, orc.FULL, iq, iw=None, want_scores=True)
    assert np.array_equal(s1, s0)
    assert np.array_equal(s2, s1 * 4)
