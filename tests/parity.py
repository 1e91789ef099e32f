"""Comparison rules between the GPU path and the CPU oracle.

* Bytes (FP4/FP8 codes, scales) and integer outputs: bit-exact.
* Top-K index sets: the GPU list must be ascending, unique and -1 padded, and
  its set must equal the oracle's except for pairs swapped across the selection
  boundary whose oracle scores both lie within 1e-6 relative of the oracle's
  K-th score (the boundary score S_b; when S_b == 0 the bound is 1e-6 times the
  best score).  The oracle's scores are the definition evaluated in fp64 (exact
  E4M3 dot products); the GPU sums the same exact products on the bf16 matrix
  cores in fp32 (within about 1e-7 relative of the exact dot on the largest
  dots) and takes the head sum and the key-scale product in fp32, so the two
  scores differ by rounding only, an order of magnitude inside that bound.
* Attention outputs: |gpu - ref| <= 2e-3 + 1e-2 * |ref| elementwise.
"""
import numpy as np

TOPK_REL = 1e-6
ATOL = 2e-3
RTOL = 1e-2


def check_sorted_list(lst, name):
    v = lst[lst >= 0]
    n = len(v)
    assert np.all(lst[n:] == -1), f"{name}: -1 padding not at the end"
    assert np.all(np.diff(v) > 0), f"{name}: not strictly ascending"
    return v


def topk_swaps(gpu, ref, scores, rel=TOPK_REL, name="topk"):
    """Number of allowed boundary swaps; raises AssertionError on any other difference.

    gpu, ref: 1-D index lists; scores: oracle score per index (dict-like or array)."""
    g = check_sorted_list(np.asarray(gpu), name)
    r = check_sorted_list(np.asarray(ref), name + " (oracle)")
    assert len(g) == len(r), f"{name}: {len(g)} selected vs oracle {len(r)}"
    gs, rs = set(g.tolist()), set(r.tolist())
    if gs == rs:
        return 0
    extra, missing = sorted(gs - rs), sorted(rs - gs)
    rsc = np.array([scores[i] for i in r], np.float64)
    sb = rsc.min()
    best = rsc.max()
    bound = rel * (abs(sb) if sb != 0 else abs(best))
    for i in extra + missing:
        assert abs(float(scores[i]) - sb) <= bound, (
            f"{name}: index {i} (score {scores[i]!r}) differs beyond the boundary rule; boundary {sb!r}, "
            f"extra {extra[:8]}, missing {missing[:8]}")
    return len(extra)


def pool_block_swaps(gpu_pool, ref_pool, scores, n_vis, rel=TOPK_REL, name="pool"):
    """Compare pools at block level (block maxima from oracle scores) and check
    that each chosen block contributes exactly its visible entries."""
    g = check_sorted_list(np.asarray(gpu_pool), name)
    r = check_sorted_list(np.asarray(ref_pool), name + " (oracle)")
    gb = np.unique(g // 8)
    rb = np.unique(r // 8)
    for blk in gb:
        want = np.arange(blk * 8, min(blk * 8 + 8, n_vis))
        got = g[(g >= blk * 8) & (g < blk * 8 + 8)]
        assert np.array_equal(got, want), f"{name}: block {blk} holds {got}, expected {want}"
    bmax = {}
    for blk in set(gb.tolist()) | set(rb.tolist()):
        bmax[blk] = max(float(scores[e]) for e in range(blk * 8, min(blk * 8 + 8, n_vis)))
    return topk_swaps(gb, rb, bmax, rel, name + " blocks")


def attn_close_conditioned(gpu, ref, row_keys, name="attend", max_frac=1e-4):
    """attn_close for outputs that may be ill-conditioned: an element outside
    2e-3 + 1e-2|ref| must lie within that plus kappa * delta, where kappa =
    sum_i P_i |V_i - ref| is the output's first-order change per unit change of
    every logit of its row and delta = 32 * 2^-24 * sm_scale * max_i sum_c
    |q_c k_ic| bounds an fp32 logit built from exact products by 16 chained
    accumulations of 32-product partial sums (each rounding at most half an
    ulp of that magnitude, the partial sums likewise).  row_keys(b, q, h) ->
    (keys [n][512] fp64, logits [n] fp64, sum_c |q_c k_c| * sm_scale [n]), from
    the oracle's dequantised rows.  At most max_frac of the elements may need
    the conditioning term.  Returns (max abs error, elements that needed it)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    rule = ATOL + RTOL * np.abs(ref)
    bad = np.argwhere(err > rule)
    assert len(bad) <= max_frac * err.size, f"{name}: {len(bad)} elements outside 2e-3 + 1e-2|ref|"
    rows = {}
    for b, q, h, c in bad.tolist():
        rows.setdefault((b, q, h), []).append(c)
    for (b, q, h), cs in rows.items():
        keys, logits, absdot = row_keys(b, q, h)
        pr = np.exp(logits - logits.max())
        pr /= pr.sum()
        delta = 32 * 2.0 ** -24 * absdot.max()
        for c in cs:
            kappa = float(np.sum(pr * np.abs(keys[:, c] - ref[b, q, h, c])))
            assert err[b, q, h, c] <= rule[b, q, h, c] + kappa * delta, (
                f"{name}: b{b} q{q} h{h} c{c}: error {err[b, q, h, c]:.3e} beyond the rule "
                f"{rule[b, q, h, c]:.3e} and the conditioning term {kappa * delta:.3e}")
    return float(err.max()), len(bad)


def attn_close(gpu, ref, name="attend"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    ok = err <= ATOL + RTOL * np.abs(ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{name}: {int((~ok).sum())} elements outside 2e-3 + 1e-2|ref|; first {idx.tolist()}, "
                             f"max abs err {err.max():.3e}")
    return float(err.max()), float((err / np.maximum(np.abs(ref), 1e-30))[np.abs(ref) > 1e-3].max(initial=0.0))
