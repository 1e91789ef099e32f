"""Calls on different streams run concurrently when they share no output or
workspace: the library keeps no state between calls.

Two independent caches, each with its own inputs, outputs and workspaces, are
stepped (append, Full scoring with a pool, Reindex, attention with a fused
window append) on two streams at once, many times over, and every result must
equal the same steps run one after the other on the default stream.  Both
streams keep the default priority.
"""
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
SM = float(np.float32(1.0 / math.sqrt(512.0)))


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    return csa


class Lane:
    """One independent decode lane: a cache filled with its own rows, its own
    step inputs, outputs and workspaces."""

    def __init__(self, csa, seed, B=4, E=40000):
        self.csa, self.B = csa, B
        cap = E + 64
        self.c = csa.Cache(B, cap, 1)
        kv = torch.from_numpy(synth.normal_rows(seed, "kv", 0, B * E, 512).reshape(B, E, 512)).cuda()
        ik = torch.from_numpy(synth.normal_rows(seed, "ik", 0, B * E, 64).reshape(B, E, 64)).cuda()
        csa.quantize_append(self.c, kv, ik)
        self.ring = torch.zeros((B, 128, 512), dtype=torch.uint8, device="cuda")
        self.kv = [torch.from_numpy(synth.normal(seed, f"kv{i}", (B, 1, 512))).cuda() for i in range(8)]
        self.ik = [torch.from_numpy(synth.normal(seed, f"ik{i}", (B, 1, 64))).cuda() for i in range(8)]
        self.iq = [torch.from_numpy(synth.normal(seed, f"iq{i}", (B, 1, 4, 64))).cuda() for i in range(8)]
        self.rq = [torch.from_numpy(synth.normal(seed, f"rq{i}", (B, 1, 4, 64))).cuda() for i in range(8)]
        self.x = [torch.from_numpy(synth.normal(seed, f"x{i}", (B, 1, 512))).cuda() for i in range(8)]
        self.q = [torch.from_numpy(synth.normal(seed, f"q{i}", (B, 1, 16, 512))).to(torch.bfloat16).cuda()
                  for i in range(8)]
        self.topk = torch.empty((B, 1, 512), dtype=torch.int32, device="cuda")
        self.pool = torch.empty((B, 1, csa.POOL), dtype=torch.int32, device="cuda")
        self.rtopk = torch.empty_like(self.topk)
        self.out = torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device="cuda")
        self.ws_i = torch.zeros(csa.workspace_bytes(csa.OP_INDEX, B, 1, cap), dtype=torch.uint8, device="cuda")
        self.ws_a = torch.zeros(max(1, csa.workspace_bytes(csa.OP_ATTEND, B, 1, cap)), dtype=torch.uint8,
                                device="cuda")
        torch.cuda.synchronize()

    def snapshot(self):
        return [t.clone() for t in (self.c.kv_codes, self.c.ik_codes, self.c.length, self.ring)]

    def restore(self, snap):
        for t, s in zip((self.c.kv_codes, self.c.ik_codes, self.c.length, self.ring), snap):
            t.copy_(s)

    def step(self, i, stream):
        csa = self.csa
        csa.quantize_append(self.c, self.kv[i], self.ik[i], stream=stream)
        csa.index_score_topk(self.c, csa.FULL, self.iq[i], self.topk, pool_out=self.pool, ws=self.ws_i,
                             stream=stream)
        csa.index_score_topk(self.c, csa.REINDEX, self.rq[i], self.rtopk, pool_in=self.pool, ws=self.ws_i,
                             stream=stream)
        csa.sparse_attend(self.c, self.rtopk, self.ring, self.q[i], self.out, SM, ws=self.ws_a, stream=stream,
                          swa_x=self.x[i], swa_len=self.c.length)

    def results(self):
        return [t.clone() for t in (self.topk, self.pool, self.rtopk, self.out, self.c.kv_codes, self.c.length,
                                    self.ring)]


def test_two_streams_match_sequential(csa):
    a, b = Lane(csa, 70), Lane(csa, 71)
    snap_a, snap_b = a.snapshot(), b.snapshot()
    hb_a, hb_b = a.c.host_len_bound, b.c.host_len_bound
    # sequential reference on the default stream
    seq = []
    for i in range(8):
        a.step(i, None)
        b.step(i, None)
        torch.cuda.synchronize()
        seq.append((a.results(), b.results()))
    a.restore(snap_a)
    b.restore(snap_b)
    a.c.host_len_bound, b.c.host_len_bound = hb_a, hb_b
    torch.cuda.synchronize()
    # the same steps, the two lanes on two streams at once
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(8):
        a.step(i, sa)
        b.step(i, sb)
        torch.cuda.synchronize()
        ra, rb = a.results(), b.results()
        for k, (x, y) in enumerate(zip(ra, seq[i][0])):
            assert torch.equal(x, y), f"lane a step {i} result {k}"
        for k, (x, y) in enumerate(zip(rb, seq[i][1])):
            assert torch.equal(x, y), f"lane b step {i} result {k}"
