"""The debug library (libcsa2_debug.so): device-side precondition checks.

On valid input it gives the release library's results byte for byte and
records nothing.  Each kind of violation (a Top-K id or pool entry past the
entries visible to its query, a cache length past the capacity, an append
that would pass it, a window length below the tokens appended) is recorded by
the kernel that meets it, which treats the item as absent; the next call with
work to do returns CSA2_EDEVICE and enqueues nothing, and the one after
returns OK.  Every bad value used here still addresses memory inside its
buffers, so even an unchecked kernel would stay in bounds.
"""
import math

import numpy as np
import pytest
import torch

import synth
from parity import attn_close

pytestmark = pytest.mark.gpu
SM = float(np.float32(1.0 / math.sqrt(512.0)))


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    csa.debug_lib()
    return csa


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def probe(csa):
    """Status of a small valid call (a one-token window append), through the
    library currently in use."""
    ring = torch.zeros((1, 128, 512), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, 1, 512), dtype=torch.float32, device="cuda")
    n = torch.ones(1, dtype=torch.int32, device="cuda")
    try:
        csa.swa_append(ring, x, n)
    except csa.CSA2Error as e:
        return e.status
    torch.cuda.synchronize()
    return csa.OK


def make_cache(csa, orc, B, cap, lengths, cid):
    oc = orc.Cache(B, cap, 1)
    for b in range(B):
        n = int(lengths[b])
        oc.kv_codes[b, :n], oc.kv_scales[b, :n] = orc.quantize_main(synth.normal_rows(cid, "kv", b * cap, n, 512))
        oc.ik_codes[b, :n], oc.ik_scales[b, :n] = orc.quantize_ik(synth.normal_rows(cid, "ik", b * cap, n, 64))
        oc.length[b] = n
    gc = csa.Cache(B, cap, 1)
    for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
        getattr(gc, name).copy_(dev(getattr(oc, name)))
    gc.host_len_bound = int(oc.length.max())
    return oc, gc


def decode_step(csa, gc, B, seed):
    """Append one entry, Full scoring with a pool, Reindex on that pool and
    attention with a fused one-token window append; every output."""
    kv = dev(synth.normal(seed, "kv", (B, 1, 512)))
    ik = dev(synth.normal(seed, "ik", (B, 1, 64)))
    csa.quantize_append(gc, kv, ik)
    iq = dev(synth.normal(seed, "iq", (B, 1, 4, 64)))
    topk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    pool = torch.empty((B, 1, csa.POOL), dtype=torch.int32, device="cuda")
    csa.index_score_topk(gc, csa.FULL, iq, topk, pool_out=pool)
    rq = dev(synth.normal(seed, "rq", (B, 1, 4, 64)))
    rtopk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    csa.index_score_topk(gc, csa.REINDEX, rq, rtopk, pool_in=pool)
    ring = torch.zeros((B, 128, 512), dtype=torch.uint8, device="cuda")
    q = torch.from_numpy(synth.normal(seed, "q", (B, 1, 16, 512))).to(torch.bfloat16).cuda()
    out = torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    xs = dev(synth.normal(seed, "swa", (B, 1, 512)))
    csa.sparse_attend(gc, rtopk, ring, q, out, SM, swa_x=xs, swa_len=gc.length)
    torch.cuda.synchronize()
    return {"kv_codes": gc.kv_codes, "ik_codes": gc.ik_codes, "length": gc.length, "topk": topk, "pool": pool,
            "rtopk": rtopk, "ring": ring, "out": out.view(torch.int16)}


def test_debug_matches_release_and_flags_nothing(csa, orc):
    B, cap = 2, 20003
    lengths = [20000, 9000]
    _, g_rel = make_cache(csa, orc, B, cap, lengths, 40)
    _, g_dbg = make_cache(csa, orc, B, cap, lengths, 40)
    rel = decode_step(csa, g_rel, B, 41)
    with csa.using(csa.debug_lib()):
        assert csa.version().endswith("debug")
        dbg = decode_step(csa, g_dbg, B, 41)
        assert probe(csa) == csa.OK
    for k in rel:
        assert torch.equal(rel[k], dbg[k]), k


def test_debug_flags_topk_ids_past_visible(csa, orc):
    B, E, cap = 1, 3000, 3016
    oc, gc = make_cache(csa, orc, B, cap, [E], 42)
    iq = synth.normal(42, "iq", (B, 1, 4, 64))
    topk, _, _ = orc.index_topk(oc, orc.FULL, iq)
    bad = topk.copy()
    bad[0, 0, 5] = E + 7   # inside the buffer, past the entries
    bad[0, 0, 9] = -3
    fixed = bad.copy()
    fixed[0, 0, 5] = -1
    fixed[0, 0, 9] = -1
    S = 128
    swa = np.zeros((B, S, 512), np.uint8)
    x = synth.normal_rows(42, "swa", E - S, S, 512).reshape(1, S, 512)
    orc.swa_append(swa, x, np.array([E], np.int32))
    qf = torch.from_numpy(synth.normal(42, "q", (B, 1, 16, 512))).to(torch.bfloat16)
    ref, _ = orc.attend(oc, fixed, swa, qf.float().numpy(), SM)
    out = torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
    with csa.using(csa.debug_lib()):
        csa.sparse_attend(gc, dev(bad), dev(swa), qf.cuda(), out, SM)
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK
    attn_close(host(out.float()), ref)  # the bad ids were skipped


def test_debug_flags_pool_entries_past_visible(csa, orc):
    B, E, cap = 1, 3000, 3016
    oc, gc = make_cache(csa, orc, B, cap, [E], 43)
    _, pool, _ = orc.index_topk(oc, orc.FULL, synth.normal(43, "f", (B, 1, 4, 64)), want_pool=True)
    n_valid = int((pool[0, 0] >= 0).sum())
    bad = pool.copy()
    bad[0, 0, n_valid] = E + 9  # still ascending, inside the cache, past the entries
    rq = dev(synth.normal(43, "r", (B, 1, 4, 64)))
    want = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
    csa.index_score_topk(gc, csa.REINDEX, rq, want, pool_in=dev(pool))
    got = torch.empty_like(want)
    with csa.using(csa.debug_lib()):
        csa.index_score_topk(gc, csa.REINDEX, rq, got, pool_in=dev(bad))
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK
    assert torch.equal(got, want)  # the bad entry was scored as absent


def test_debug_flags_capacity_and_length(csa):
    cap = 10
    gc = csa.Cache(2, cap, 1)
    gc.length.fill_(9)
    gc.host_len_bound = 0  # the host bound understates the device lengths
    kv = dev(synth.normal(44, "kv", (2, 3, 512)))
    ik = dev(synth.normal(44, "ik", (2, 3, 64)))
    with csa.using(csa.debug_lib()):
        csa.quantize_append(gc, kv, ik)  # 9 + 3 > 10 on the device: not made
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK
        assert host(gc.length).tolist() == [9, 9]
        assert not host(gc.kv_codes).any() and not host(gc.ik_codes).any()
        # a length past the capacity, met by the indexer (which reads at most
        # `capacity` entries)
        gc.length.fill_(cap + 5)
        topk = torch.empty((2, 1, 512), dtype=torch.int32, device="cuda")
        csa.index_score_topk(gc, csa.FULL, dev(synth.normal(44, "iq", (2, 1, 4, 64))), topk)
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK


def test_debug_flags_short_window_length(csa):
    S = 128
    x = dev(synth.normal(45, "x", (1, 3, 512)))
    with csa.using(csa.debug_lib()):
        ring = torch.zeros((1, S, 512), dtype=torch.uint8, device="cuda")
        csa.swa_append(ring, x, torch.ones(1, dtype=torch.int32, device="cuda"))  # 1 token, 3 appended
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK
        r = host(ring)
        assert r[0, 0].any() and not r[0, 1:].any()  # only position 0 (the last token) was written
        # the same through the attention call's fused append
        gc = csa.Cache(1, 16, 1)
        ring2 = torch.zeros((1, S, 512), dtype=torch.uint8, device="cuda")
        q = torch.zeros((1, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
        out = torch.empty_like(q)
        topk = torch.full((1, 1, 512), -1, dtype=torch.int32, device="cuda")
        csa.sparse_attend(gc, topk, ring2, q, out, SM, q_pos=torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                          swa_x=x, swa_len=torch.ones(1, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert probe(csa) == csa.EDEVICE
        assert probe(csa) == csa.OK
        r2 = host(ring2)
        assert np.array_equal(r2, r)  # the same single token in slot 0


@pytest.mark.parametrize("cid", [2, 4, 5])  # 16 x 128K, 4 x 1M, 16 x 128K with six queries
def test_debug_full_size_step_matches_release(csa, cid):
    """A whole group step at full size through the debug library records no
    violation and gives the release library's outputs and cache bytes."""
    import bench
    wl = bench.Workload(cid, replicas=2, extra_steps=4)  # two identical cache replicas
    wl.inputs[1] = wl.inputs[0]
    wl.step(0)
    torch.cuda.synchronize()
    rel = [t.clone() for t in wl.topk] + [wl.pool.clone()] + [o.clone() for o in wl.out]
    with csa.using(csa.debug_lib()):
        wl.step(1)
        torch.cuda.synchronize()
        assert probe(csa) == csa.OK
    dbg = list(wl.topk) + [wl.pool] + list(wl.out)
    for i, (a, b) in enumerate(zip(rel, dbg)):
        assert torch.equal(a, b), i
    for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
        assert torch.equal(getattr(wl.caches[0], name), getattr(wl.caches[1], name)), name
    for l in range(wl.L):
        assert torch.equal(wl.swas[0][l], wl.swas[1][l]), l


def test_debug_schedule_step_matches_release(csa):
    """The whole 38-layer schedule (ratio-2 encoder caches, two tokens per step,
    explicit positions, projected appends) through the debug library: nothing
    recorded, the release library's outputs and caches byte for byte."""
    import bench
    wl = bench.Schedule38(6, 4, 16384, 2)
    wl.inputs[1] = wl.inputs[0]

    def outputs():
        return [o for per_t in wl.out for o in per_t] + [wl.topk[k] for k in sorted(wl.topk)] + [wl.pool]

    wl.step(0)
    torch.cuda.synchronize()
    rel = [t.clone() for t in outputs()]
    with csa.using(csa.debug_lib()):
        wl.step(1)
        torch.cuda.synchronize()
        assert probe(csa) == csa.OK
    for i, (a, b) in enumerate(zip(rel, outputs())):
        assert torch.equal(a, b), i
    for n in wl.caches[0]:
        for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
            assert torch.equal(getattr(wl.caches[0][n], name), getattr(wl.caches[1][n], name)), (n, name)
