"""Parity at the largest capacity the library accepts: 2^23 entries per sequence.

At this size the ordering of the selected ids runs with exactly its maximum
number of buckets (2,048: entries >> 12, blocks >> 9), the select kernel takes
its most shares per query (2,048 stretches of a few candidates each), and byte
offsets into the main-KV planes of a second sequence pass 2^32.

The oracle needs minutes to quantise and scan 2^23 rows, so the checks use what
holds at any size, plus samples the oracle computes one by one:
  * indexer codes are random valid E4M3 bytes with small scales, and 512
    planted entries (one per block, spread over the whole range, the last
    entry included) score far above every other; the Top-512 must be exactly
    them;
  * the pool must hold every planted block and 2,048 distinct full blocks in
    ascending order, and the oracle's block maxima of all its other blocks
    and of 4,096 sampled blocks outside it must not be out of order beyond the
    boundary rule;
  * Reindex over the GPU's pool is compared with the oracle's in full (the
    oracle reads only the pool entries);
  * attention over Top-K ids at the top of the range of two sequences, with
    only those rows (and the window) filled, is compared with the oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity import attn_close, topk_swaps

pytestmark = pytest.mark.gpu
SM = float(np.float32(1.0 / math.sqrt(512.0)))
CAP = 1 << 23
CID = 60


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


def needle_positions():
    """512 entries in distinct 8-entry blocks over the whole range, the first
    and the last entry included."""
    blocks = np.unique(np.linspace(0, CAP // 8 - 1, 512).astype(np.int64))
    assert blocks.size == 512
    off = synth.integers(CID, "needle_off", (512,), 0, 8).astype(np.int64)
    pos = blocks * 8 + off
    pos[0], pos[-1] = 0, CAP - 1
    return np.sort(pos)


@pytest.fixture(scope="module")
def full_cache(csa, orc):
    """One full sequence of 2^23 entries: random indexer codes and the needles,
    on both sides (the main-KV planes stay zero)."""
    print("max capacity: generating indexer codes", flush=True)
    g = synth.generator(CID, "codes", 0)
    codes = g.integers(0, 256, size=(1, CAP, 64), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    scales = g.uniform(1e-4, 1e-3, size=(1, CAP)).astype(np.float32)
    pos = needle_positions()
    codes[0, pos] = 0x7E  # +448 in every dimension
    scales[0, pos] = 1.0
    oc = orc.Cache(1, CAP, 1)
    oc.ik_codes[:] = codes
    oc.ik_scales[:] = scales
    oc.length[0] = CAP
    gc = csa.Cache(1, CAP, 1)
    gc.ik_codes.copy_(dev(codes))
    gc.ik_scales.copy_(dev(scales))
    gc.length.fill_(CAP)
    gc.host_len_bound = CAP
    del codes
    return oc, gc, pos


def sub_scores(orc, oc, iq, entries):
    """Oracle scores of the given entries, each scored on its own (a cache of
    just those rows, every one visible)."""
    n = entries.size
    sc = orc.Cache(1, n, 1)
    sc.ik_codes[0] = oc.ik_codes[0, entries]
    sc.ik_scales[0] = oc.ik_scales[0, entries]
    sc.length[0] = n
    _, _, s = orc.index_topk(sc, orc.FULL, iq, want_scores=True)
    return s[0, 0, :n]


@pytest.fixture(scope="module")
def full_result(csa, full_cache):
    """The GPU's Full call with a pool over the whole sequence."""
    oc, gc, pos = full_cache
    iq = np.abs(synth.normal(CID, "iq", (1, 1, 4, 64))) + np.float32(0.5)  # every product with a needle positive
    topk = torch.empty((1, 1, 512), dtype=torch.int32, device="cuda")
    pool = torch.empty((1, 1, csa.POOL), dtype=torch.int32, device="cuda")
    print("max capacity: Full call", flush=True)
    csa.index_score_topk(gc, csa.FULL, dev(iq), topk, pool_out=pool)
    return iq, host(topk)[0, 0], host(pool)[0, 0]


def test_full_topk_and_pool_at_max_capacity(orc, full_cache, full_result):
    oc, gc, pos = full_cache
    iq, topk, pool = full_result
    assert np.array_equal(topk, pos)  # ascending, exactly the needles
    # the pool: 2,048 distinct full blocks, ascending, every needle block among them
    assert (pool >= 0).all() and np.all(np.diff(pool) > 0)
    blocks = pool.reshape(2048, 8)
    assert np.array_equal(blocks, blocks[:, :1] + np.arange(8)) and np.all(blocks[:, 0] % 8 == 0)
    chosen = blocks[:, 0] // 8
    assert set((pos // 8).tolist()) <= set(chosen.tolist())
    # its boundary against the oracle's block maxima: the other chosen blocks
    # and a sample of the blocks left out
    print("max capacity: oracle block maxima of the sample", flush=True)
    others = np.setdiff1d(chosen, pos // 8)
    left = np.setdiff1d(np.arange(CAP // 8), chosen)
    sample = synth.generator(CID, "sample", 0).choice(left, 4096, replace=False)
    ents = np.concatenate([others, sample])[:, None] * 8 + np.arange(8)
    s = sub_scores(orc, oc, iq, ents.reshape(-1)).reshape(-1, 8).max(axis=1)
    s_in, s_out = s[:others.size], s[others.size:]
    lo, hi = s_in.min(), s_out.max()
    # a block left out may beat a chosen one only by the boundary tolerance
    assert hi <= lo + 1e-6 * max(abs(lo), 1e-30), (lo, hi)
    # and the order among equals: a left-out block with the lowest chosen
    # score must not have a lower block index than a chosen one of that score
    tie_out = sample[s_out == lo]
    tie_in = others[s_in == lo]
    if tie_out.size and tie_in.size:
        assert tie_out.min() > tie_in.max()


def test_reindex_at_max_capacity(csa, orc, full_cache, full_result):
    oc, gc, pos = full_cache
    pool = full_result[2].reshape(1, 1, -1)
    rq = synth.normal(CID, "rq", (1, 1, 4, 64))
    ref, _, scores = orc.index_topk(oc, orc.REINDEX, rq, pool_in=pool, want_scores=True)
    got = torch.empty((1, 1, 512), dtype=torch.int32, device="cuda")
    csa.index_score_topk(gc, csa.REINDEX, dev(rq), got, pool_in=dev(pool))
    topk_swaps(host(got)[0, 0], ref[0, 0], scores[0, 0], name="reindex at 2^23")


def test_attend_at_max_capacity(csa, orc):
    """Two sequences of 2^23 entries: ids at the top of the range, so the second
    sequence's main-KV rows sit past 2^32 bytes."""
    B, S = 2, 128
    ids = np.stack([np.linspace(0, CAP - 1, 512).astype(np.int32), np.arange(CAP - 512, CAP, dtype=np.int32)])
    assert np.unique(ids[0]).size == 512
    topk = ids.reshape(B, 1, 512)
    oc = orc.Cache(B, CAP, 1)
    gc = csa.Cache(B, CAP, 1)
    for b in range(B):
        rows = synth.normal_rows(CID, f"kv{b}", 0, 512, 512)
        codes, scales = orc.quantize_main(rows)
        oc.kv_codes[b, ids[b]] = codes
        oc.kv_scales[b, ids[b]] = scales
        idx = torch.from_numpy(ids[b].astype(np.int64)).cuda()
        gc.kv_codes[b].index_copy_(0, idx, dev(codes))
        gc.kv_scales[b].index_copy_(0, idx, dev(scales))
    oc.length[:] = CAP
    gc.length.fill_(CAP)
    gc.host_len_bound = CAP
    swa = np.zeros((B, S, 512), np.uint8)
    x = synth.normal_rows(CID, "swa", 0, B * S, 512).reshape(B, S, 512)
    orc.swa_append(swa, x, np.full(B, CAP, np.int32))
    qf = torch.from_numpy(synth.normal(CID, "q", (B, 1, 16, 512))).to(torch.bfloat16)
    ref, ref_lse = orc.attend(oc, topk, swa, qf.float().numpy(), SM)
    out = torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, 16), dtype=torch.float32, device="cuda")
    csa.sparse_attend(gc, dev(topk), dev(swa), qf.cuda(), out, SM, lse=lse)
    mabs, _ = attn_close(host(out.float()), ref, name="attend at 2^23")
    np.testing.assert_allclose(host(lse), ref_lse, rtol=1e-4, atol=1e-4)
    print(f"attend at 2^23: max abs err {mabs:.2e}", flush=True)
