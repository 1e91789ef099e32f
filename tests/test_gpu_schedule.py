"""Parity of the whole 38-layer CSA2 schedule of a decode token (two tokens:
the first leaves the encoder's ratio-2 entry pending, the second completes
it), on a small batch and context, through the same Schedule38 class that
bench.py times.  Every layer of both tokens is compared with the oracle's
replay of the step: each indexing call's Top-K (and the pool) under the
boundary rule, every attention output within 2e-3 + 1e-2|ref| (over the GPU's
own Top-K list where a boundary swap made the lists differ), and every cache
byte after the step.
"""
import numpy as np
import pytest
import torch

import bench
from parity import attn_close, pool_block_swaps, topk_swaps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


# (sequences, context, sequences the oracle replays): every sequence, up to the
# benchmark's own 16 x 128K workload
@pytest.mark.parametrize("B,ctx,hs", [(2, 4096, 2), (1, 40000, 1), (16, 131072, 16)])
def test_schedule38_step(gpu, B, ctx, hs):
    print(f"schedule38 B={B} ctx={ctx}: building", flush=True)
    wl = bench.Schedule38(6, B, ctx, replicas=1, keep_host_seqs=hs)
    wl.step(0, record=True)
    torch.cuda.synchronize()
    print("GPU step done, running the oracle", flush=True)
    ost = bench.OracleSchedule38(wl)
    gpu_used = [[np.ascontiguousarray(wl.used[t][l][:hs].cpu().numpy()) for l in range(len(bench.SCHEDULE38))]
                for t in range(2)]
    res = ost.step(want_scores=True, gpu_used=gpu_used)
    for n, c in wl.caches[0].items():
        oc = ost.oc[n]
        assert np.array_equal(c.length[:hs].cpu().numpy(), oc.length), n
        m = int(oc.length.max())
        for f in ("kv_codes", "kv_scales", "ik_codes"):
            assert np.array_equal(getattr(c, f)[:hs, :m].cpu().numpy(), getattr(oc, f)[:, :m]), (n, f)
        assert np.array_equal(c.ik_scales[:hs, :m].cpu().numpy().view(np.uint32), oc.ik_scales[:, :m].view(np.uint32))
    swaps, compared = 0, 0
    for t in range(2):
        for l, (mode, cn) in enumerate(bench.SCHEDULE38):
            r = res[t][l]
            used = wl.used[t][l].cpu().numpy()
            if mode != "reuse":
                for b in range(hs):
                    swaps += topk_swaps(used[b, 0], r["topk"][b, 0], r["scores"][b, 0], name=f"t{t} L{l} b{b}")
            if mode == "full_pool":
                pool = wl.used_pool[t].cpu().numpy()
                for b in range(hs):
                    n_vis = wl.ctx + t + 1  # decoder entries visible to token t
                    swaps += pool_block_swaps(pool[b, 0], r["pool"][b, 0], r["scores"][b, 0], n_vis,
                                              name=f"t{t} pool b{b}")
            got = wl.out[t][l].float().cpu().numpy()
            for b in range(hs):
                # out_cmp: the oracle's attention over the list the GPU attended with
                attn_close(got[b, 0], r["out_cmp"][b, 0], name=f"t{t} L{l} b{b}")
                compared += 1
    print(f"schedule38 B={B} ctx={ctx}: {compared} attention outputs compared, {swaps} boundary swaps", flush=True)
    assert compared == 2 * 38 * hs
