"""HIP-graph replays of a whole group step give the eager results.

bench.py times steps captured in hipGraphs.  Here two cache replicas start
identical and get the same step inputs: replica 0 steps eagerly, replica 1 by
replaying one captured step.  They alternate, with synchronisations between
them, for several steps.  After every replay the Top-K lists, the pool, every
layer's attention output, every cache plane and every window ring must equal
the eager step's, byte for byte.  The step appends to the caches, so each
replay runs on the state the one before left.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


@pytest.mark.parametrize("cid", [0, 2, 5])  # 1 x 4K; 16 x 128K with pool and Reindex; six queries per sequence
def test_graph_replays_match_eager_steps(csa, cid):
    import bench
    wl = bench.Workload(cid, replicas=2, extra_steps=16)
    wl.inputs[1] = wl.inputs[0]
    wl.step(0)  # both replicas one step on, every kernel loaded before the capture
    wl.step(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.step(1)  # recorded, not run
    torch.cuda.synchronize()
    for rep in range(4):
        wl.step(0)
        torch.cuda.synchronize()
        eager = [t.clone() for t in wl.topk] + [wl.pool.clone()] + [o.clone() for o in wl.out]
        g.replay()
        torch.cuda.synchronize()
        replay = list(wl.topk) + [wl.pool] + list(wl.out)
        for i, (a, b) in enumerate(zip(eager, replay)):
            assert torch.equal(a, b), f"replay {rep}: output {i}"
        for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
            assert torch.equal(getattr(wl.caches[0], name), getattr(wl.caches[1], name)), f"replay {rep}: {name}"
        for l in range(wl.L):
            assert torch.equal(wl.swas[0][l], wl.swas[1][l]), f"replay {rep}: window of layer {l}"
        print(f"config {cid}: replay {rep} equals the eager step", flush=True)


@pytest.mark.parametrize("B,ctx", [(4, 16384), (16, 131072)])
def test_schedule38_graph_replays_match_eager_steps(csa, B, ctx):
    """The same check for the whole 38-layer schedule (two tokens per step,
    projected appends into three ratio-2 encoder caches and the decoder cache)."""
    import bench
    wl = bench.Schedule38(6, B, ctx, 2)
    wl.inputs[1] = wl.inputs[0]
    wl.step(0)
    wl.step(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.step(1)
    torch.cuda.synchronize()

    def outputs():
        outs = [o for per_t in wl.out for o in per_t]
        return outs + [wl.topk[k] for k in sorted(wl.topk)] + [wl.pool]

    for rep in range(3):
        wl.step(0)
        torch.cuda.synchronize()
        eager = [t.clone() for t in outputs()]
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outputs())):
            assert torch.equal(a, b), f"replay {rep}: output {i}"
        for n in wl.caches[0]:
            for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
                assert torch.equal(getattr(wl.caches[0][n], name), getattr(wl.caches[1][n], name)), \
                    f"replay {rep}: cache {n} {name}"
        for l in range(len(wl.swas[0])):
            assert torch.equal(wl.swas[0][l], wl.swas[1][l]), f"replay {rep}: window of layer {l}"
        print(f"schedule {B} x {ctx}: replay {rep} equals the eager step", flush=True)
