"""A seeded sweep of random shapes through the whole path against the oracle.

Each case draws (from its own fixed seed) a batch size, ragged lengths, a
capacity, the compression ratio, the number of queries per sequence, whether
they carry explicit causal positions and head weights, and whether a pool is
built.  It runs Full scoring, Reindex over the Full call's pool (when there is
one) and attention over the Full Top-K on the GPU, and compares each with the
oracle under the usual rules: Top-K and pool sets under the boundary rule,
attention within 2e-3 + 1e-2|ref|.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity import attn_close, pool_block_swaps, topk_swaps

pytestmark = pytest.mark.gpu
SM = float(np.float32(1.0 / math.sqrt(512.0)))
CID = 80


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def draw(case):
    g = synth.generator(CID, "case", case)
    B = int(g.integers(1, 5))
    ratio = int(g.choice([1, 1, 2]))
    Q = int(g.choice([1, 2, 3, 4, 5, 6, 8, 9]))
    E_max = int(g.choice([300, 5000, 17000, 40000, 70000]))
    lengths = g.integers(0, E_max + 1, size=B)
    lengths[int(g.integers(0, B))] = E_max  # the longest sequence fills the capacity's bulk
    cap = E_max + int(g.integers(0, 100))
    explicit = bool(g.integers(0, 2))
    weights = bool(g.integers(0, 2))
    pool = bool(g.integers(0, 2))
    # positions: the last Q tokens of each sequence, or Q consecutive tokens
    # ending at a random one (from before the first entry to the last token)
    tokens = lengths.astype(np.int64) * ratio
    if explicit:
        last = np.array([int(g.integers(-2, max(1, tokens[b]))) for b in range(B)], np.int64)
        q_pos = (last[:, None] - (Q - 1) + np.arange(Q)[None, :]).astype(np.int32)
    else:
        q_pos = None
    return B, ratio, Q, lengths, cap, q_pos, weights, pool


@pytest.mark.parametrize("case", range(16))
def test_random_case(csa, orc, case):
    B, ratio, Q, lengths, cap, q_pos, weights, want_pool = draw(case)
    print(f"case {case}: B={B} r={ratio} Q={Q} lengths={lengths.tolist()} cap={cap} "
          f"q_pos={'given' if q_pos is not None else 'last'} weights={weights} pool={want_pool}", flush=True)
    oc = orc.Cache(B, cap, ratio)
    for b in range(B):
        n = int(lengths[b])
        oc.kv_codes[b, :n], oc.kv_scales[b, :n] = orc.quantize_main(synth.normal_rows(CID, f"kv{case}", b * cap, n,
                                                                                      512))
        oc.ik_codes[b, :n], oc.ik_scales[b, :n] = orc.quantize_ik(synth.normal_rows(CID, f"ik{case}", b * cap, n, 64))
        oc.length[b] = n
    gc = csa.Cache(B, cap, ratio)
    for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
        getattr(gc, name).copy_(dev(getattr(oc, name)))
    gc.host_len_bound = int(oc.length.max())
    iq = synth.normal(CID, f"iq{case}", (B, Q, 4, 64))
    iw = np.abs(synth.normal(CID, f"iw{case}", (B, Q, 4))) if weights else None
    if q_pos is None:
        pos = oc.length.astype(np.int64)[:, None] * ratio - Q + np.arange(Q)[None, :]
    else:
        pos = q_pos.astype(np.int64)

    # Full, with or without a pool
    ref_topk, ref_pool, scores = orc.index_topk(oc, orc.FULL, iq, iw=iw, q_pos=q_pos, want_pool=want_pool,
                                                want_scores=True)
    topk = torch.empty((B, Q, 512), dtype=torch.int32, device="cuda")
    pool = torch.empty((B, Q, csa.POOL), dtype=torch.int32, device="cuda") if want_pool else None
    csa.index_score_topk(gc, csa.FULL, dev(iq), topk, iw=dev(iw) if weights else None,
                         q_pos=dev(q_pos) if q_pos is not None else None, pool_out=pool)
    topk = host(topk)
    g_pool = host(pool) if want_pool else None
    for b in range(B):
        for q in range(Q):
            n_vis = int(min(lengths[b], cap, max(0, (pos[b, q] + 1) // ratio))) if pos[b, q] >= 0 else 0
            topk_swaps(topk[b, q], ref_topk[b, q], scores[b, q], name=f"case {case} b{b} q{q}")
            if want_pool:
                pool_block_swaps(g_pool[b, q], ref_pool[b, q], scores[b, q], n_vis,
                                 name=f"case {case} pool b{b} q{q}")

    # Reindex over the GPU's pool, with other queries
    if want_pool:
        rq = synth.normal(CID, f"rq{case}", (B, Q, 4, 64))
        r_ref, _, r_scores = orc.index_topk(oc, orc.REINDEX, rq, q_pos=q_pos, pool_in=g_pool, want_scores=True)
        rt = torch.empty((B, Q, 512), dtype=torch.int32, device="cuda")
        csa.index_score_topk(gc, csa.REINDEX, dev(rq), rt, q_pos=dev(q_pos) if q_pos is not None else None,
                             pool_in=dev(g_pool))
        rt = host(rt)
        for b in range(B):
            for q in range(Q):
                topk_swaps(rt[b, q], r_ref[b, q], r_scores[b, q], name=f"case {case} reindex b{b} q{q}")

    # attention over the GPU's Top-K (the same ids on both sides); the window
    # ring holds the last S tokens before each sequence's last query
    S = 128 + Q
    swa = np.zeros((B, S, 512), np.uint8)
    for b in range(B):
        n_tok = int(max(pos[b].max() + 1, 0))
        t0 = max(0, n_tok - S)
        if n_tok > t0:
            x = synth.normal_rows(CID, f"swa{case}", b * 1000000 + t0, n_tok - t0, 512).reshape(1, -1, 512)
            sub = np.zeros((1, S, 512), np.uint8)
            orc.swa_append(sub, x, np.array([n_tok], np.int32))
            swa[b] = sub[0]
    qf = torch.from_numpy(synth.normal(CID, f"q{case}", (B, Q, 16, 512))).to(torch.bfloat16)
    att_pos = pos.astype(np.int32)
    ref, _ = orc.attend(oc, topk, swa, qf.float().numpy(), SM, q_pos=att_pos)
    out = torch.empty((B, Q, 16, 512), dtype=torch.bfloat16, device="cuda")
    csa.sparse_attend(gc, dev(topk), dev(swa), qf.cuda(), out, SM, q_pos=dev(att_pos))
    mabs, _ = attn_close(host(out.float()), ref, name=f"case {case} attend")
    print(f"case {case}: ok, attention max abs err {mabs:.2e}", flush=True)


@pytest.mark.parametrize("case", range(8))
def test_random_ratio_m_case(csa, orc, case):
    """Ratios above 2 end to end: the cache is built by the compressing append
    from token rows and logits (bytes compared with the oracle's), then Full
    scoring with a pool and attention run over it."""
    g = synth.generator(CID, "rcase", case)
    m = int(g.choice([3, 4, 8]))
    B = int(g.integers(1, 4))
    Q = int(g.choice([1, 2, 5, 8]))
    n = int(g.integers(200, 3000))
    T, cap = n * m, n + int(g.integers(0, 40))
    print(f"ratio case {case}: m={m} B={B} Q={Q} entries={n} cap={cap}", flush=True)
    kv = synth.normal_rows(CID, f"rkv{case}", 0, B * T, 512).reshape(B, T, 512)
    lg = synth.normal_rows(CID, f"rlg{case}", 0, B * T, 512).reshape(B, T, 512)
    ik = synth.normal_rows(CID, f"rik{case}", 0, B * n, 64).reshape(B, n, 64)
    oc = orc.Cache(B, cap, m)
    orc.quantize_append(oc, kv, ik, logits=lg)
    gc = csa.Cache(B, cap, m)
    csa.quantize_append(gc, dev(kv), dev(ik), logits=dev(lg))
    for name in ("kv_codes", "kv_scales", "ik_codes", "length"):
        assert np.array_equal(host(getattr(gc, name)), getattr(oc, name)), name
    assert np.array_equal(host(gc.ik_scales).view(np.uint32), oc.ik_scales.view(np.uint32))

    iq = synth.normal(CID, f"riq{case}", (B, Q, 4, 64))
    ref_topk, ref_pool, scores = orc.index_topk(oc, orc.FULL, iq, want_pool=True, want_scores=True)
    topk = torch.empty((B, Q, 512), dtype=torch.int32, device="cuda")
    pool = torch.empty((B, Q, csa.POOL), dtype=torch.int32, device="cuda")
    csa.index_score_topk(gc, csa.FULL, dev(iq), topk, pool_out=pool)
    topk, g_pool = host(topk), host(pool)
    pos = n * m - Q + np.arange(Q)  # the last Q tokens (the default positions)
    for b in range(B):
        for q in range(Q):
            n_vis = min(n, (int(pos[q]) + 1) // m)
            topk_swaps(topk[b, q], ref_topk[b, q], scores[b, q], name=f"ratio case {case} b{b} q{q}")
            pool_block_swaps(g_pool[b, q], ref_pool[b, q], scores[b, q], n_vis, name=f"ratio case {case} pool")

    S = 128 + Q
    swa = np.zeros((B, S, 512), np.uint8)
    x = synth.normal_rows(CID, f"rswa{case}", 0, B * S, 512).reshape(B, S, 512)
    orc.swa_append(swa, x, np.full(B, n * m, np.int32))
    qf = torch.from_numpy(synth.normal(CID, f"rq{case}", (B, Q, 16, 512))).to(torch.bfloat16)
    ref, _ = orc.attend(oc, topk, swa, qf.float().numpy(), SM)
    out = torch.empty((B, Q, 16, 512), dtype=torch.bfloat16, device="cuda")
    csa.sparse_attend(gc, dev(topk), dev(swa), qf.cuda(), out, SM)
    mabs, _ = attn_close(host(out.float()), ref, name=f"ratio case {case} attend")
    print(f"ratio case {case}: ok, attention max abs err {mabs:.2e}", flush=True)
