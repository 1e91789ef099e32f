"""Parity at the benchmark's full workload sizes, in the launch configuration
bench.py times (same Workload class, same kernels, same workspaces).

The GPU runs one whole group step over the full batch.  The oracle rebuilds the
first sequence(s) of the batch from the same seeded rows, runs the same step,
and the sampled sequences (and, for the 2048-query prefill, sampled query
slots) are compared stage by stage: cache codes bit-exact, every Top-K and the
pool under the boundary rule, attention within 2e-3 + 1e-2|ref| wherever the
two sides attended the same index set.
"""
import numpy as np
import pytest
import torch

import bench
from parity import attn_close, pool_block_swaps, topk_swaps

pytestmark = pytest.mark.gpu

# config id -> (sequences sampled by the oracle, query slots sampled or None)
CASES = {
    0: (1, None),
    1: (2, None),
    2: (2, None),
    3: (1, [0, 1, 2, 511, 1024, 1500, 2046, 2047]),
    4: (1, None),
    5: (2, None),
}


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4, 5])
def test_full_size_step(gpu, cid):
    hs, qsel = CASES[cid]
    print(f"config {cid}: building workload", flush=True)
    wl = bench.Workload(cid, replicas=1, extra_steps=8, keep_host_seqs=hs)
    wl.step(0)
    torch.cuda.synchronize()
    print(f"config {cid}: GPU step done, running the oracle on {hs} sequence(s)", flush=True)
    ost = bench.OracleStep(wl, qsel=qsel)
    res = ost.step(want_scores=True)
    gc = wl.caches[0]
    # cache after the step's append: every byte of the sampled sequences
    assert np.array_equal(gc.length[:hs].cpu().numpy(), ost.oc.length)
    n = int(ost.oc.length.max())
    for name in ("kv_codes", "kv_scales", "ik_codes"):
        g = getattr(gc, name)[:hs, :n].cpu().numpy()
        assert np.array_equal(g, getattr(ost.oc, name)[:, :n]), name
    assert np.array_equal(gc.ik_scales[:hs, :n].cpu().numpy().view(np.uint32),
                          ost.oc.ik_scales[:, :n].view(np.uint32))
    qs = list(range(wl.Q)) if qsel is None else qsel
    swaps = 0
    topk_layer = None
    for l, mode in enumerate(wl.group):
        r = res[l]
        if mode != "reuse":
            topk_layer = l
            g_topk = wl.topk[l][:hs].cpu().numpy()[:, qs]
            for b in range(hs):
                for j in range(len(qs)):
                    swaps += topk_swaps(g_topk[b, j], r["topk"][b, j], r["scores"][b, j], name=f"L{l} b{b} q{qs[j]}")
            if mode == "full_pool":
                g_pool = wl.pool[:hs].cpu().numpy()[:, qs]
                q_pos = ost.q_pos
                for b in range(hs):
                    for j in range(len(qs)):
                        # entries visible to this query (all of them at single-token decode)
                        n_vis = int(ost.oc.length[b]) if q_pos is None else min(int(ost.oc.length[b]),
                                                                                (int(q_pos[b, j]) + 1) // wl.r)
                        swaps += pool_block_swaps(g_pool[b, j], r["pool"][b, j], r["scores"][b, j], n_vis,
                                                  name=f"pool b{b} q{qs[j]}")
        g_out = wl.out[l][:hs].float().cpu().numpy()[:, qs]
        g_used = wl.topk[topk_layer][:hs].cpu().numpy()[:, qs]
        for b in range(hs):
            for j in range(len(qs)):
                if set(g_used[b, j].tolist()) != set(r["topk"][b, j].tolist()):
                    continue  # an allowed boundary swap: the two sides attended different sets
                attn_close(g_out[b, j], r["out"][b, j], name=f"L{l} b{b} q{qs[j]}")
    print(f"config {cid}: parity ok, {swaps} boundary swaps", flush=True)
