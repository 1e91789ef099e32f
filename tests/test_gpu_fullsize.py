"""Parity at the benchmark's full workload sizes, in the launch configuration
bench.py times (same Workload class, same kernels, same workspaces).

The GPU runs one whole group step over the full batch.  The oracle rebuilds
every sequence of the batch from the same seeded rows, runs the same step, and
every output is compared stage by stage: cache codes bit-exact, every Top-K and
the pool under the boundary rule, and every attention output within
2e-3 + 1e-2|ref|.  Where a boundary swap made the two sides select different
index sets, the oracle's attention is evaluated over the GPU's own list, so no
output goes unchecked.  The 2,048-query prefill compares 128 query slots spread
over the chunk (its oracle scores every query against 32K entries).
"""
import numpy as np
import pytest
import torch

import bench
from parity import attn_close, pool_block_swaps, topk_swaps

pytestmark = pytest.mark.gpu

# config id -> query slots compared, or None for all (every sequence is compared)
QSEL = {3: sorted(set(np.linspace(0, 2047, 128).round().astype(int).tolist()))}


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4, 5])
def test_full_size_step(gpu, cid):
    qsel = QSEL.get(cid)
    B = bench.synth.WORKLOADS[cid]["B"]
    print(f"config {cid}: building workload", flush=True)
    wl = bench.Workload(cid, replicas=1, extra_steps=8, keep_host_seqs=B)
    wl.step(0)
    torch.cuda.synchronize()
    hs = B
    qs = list(range(wl.Q)) if qsel is None else qsel
    # the Top-K list each GPU layer attended with (the latest indexing layer's)
    gpu_used, latest = [], None
    for l, mode in enumerate(wl.group):
        if mode != "reuse":
            latest = wl.topk[l].cpu().numpy()[:, qs]
        gpu_used.append(np.ascontiguousarray(latest))
    print(f"config {cid}: GPU step done, running the oracle on all {hs} sequences", flush=True)
    ost = bench.OracleStep(wl, qsel=qsel)
    res = ost.step(want_scores=True, gpu_used=gpu_used)
    gc = wl.caches[0]
    # cache after the step's append: every byte of every sequence
    assert np.array_equal(gc.length.cpu().numpy(), ost.oc.length)
    n = int(ost.oc.length.max())
    for name in ("kv_codes", "kv_scales", "ik_codes"):
        g = getattr(gc, name)[:, :n].cpu().numpy()
        assert np.array_equal(g, getattr(ost.oc, name)[:, :n]), name
    assert np.array_equal(gc.ik_scales[:, :n].cpu().numpy().view(np.uint32), ost.oc.ik_scales[:, :n].view(np.uint32))
    swaps, compared, swapped_sets, max_abs = 0, 0, 0, 0.0
    for l, mode in enumerate(wl.group):
        r = res[l]
        if mode != "reuse":
            g_topk = gpu_used[l]
            for b in range(hs):
                for j in range(len(qs)):
                    swaps += topk_swaps(g_topk[b, j], r["topk"][b, j], r["scores"][b, j], name=f"L{l} b{b} q{qs[j]}")
            if mode == "full_pool":
                g_pool = wl.pool.cpu().numpy()[:, qs]
                q_pos = ost.q_pos
                for b in range(hs):
                    for j in range(len(qs)):
                        # entries visible to this query (all of them at single-token decode)
                        n_vis = int(ost.oc.length[b]) if q_pos is None else min(int(ost.oc.length[b]),
                                                                                (int(q_pos[b, j]) + 1) // wl.r)
                        swaps += pool_block_swaps(g_pool[b, j], r["pool"][b, j], r["scores"][b, j], n_vis,
                                                  name=f"pool b{b} q{qs[j]}")
        g_out = wl.out[l].float().cpu().numpy()[:, qs]
        for b in range(hs):
            for j in range(len(qs)):
                swapped_sets += not np.array_equal(gpu_used[l][b, j], r["topk"][b, j])
                m, _ = attn_close(g_out[b, j], r["out_cmp"][b, j], name=f"L{l} b{b} q{qs[j]}")
                max_abs = max(max_abs, m)
                compared += 1
    assert compared == len(wl.group) * hs * len(qs)
    print(f"config {cid}: parity ok, {compared} attention outputs compared (max abs err {max_abs:.2e}), "
          f"{swaps} boundary swaps, {swapped_sets} outputs over a swapped set", flush=True)
