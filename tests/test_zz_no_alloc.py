"""csa2_sparse_attend_noalloc against csa2_sparse_attend: two calls in a row on
one GPU, the second smaller, each equal to the workspace entry point's result
(outputs, log-sum-exps and window rings) on the same inputs, and within the
attention tolerance of the oracle.  Both run the same kernels, so the outputs
are expected bit for bit."""
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
    return csa


def _case(csa, orc, B, Q, E, seed):
    cap = E + 4
    oc = orc.Cache(B, cap, 1)
    for b in range(B):
        kv = synth.normal_rows(seed, "kv", b * cap, E, 512)
        oc.kv_codes[b, :E], oc.kv_scales[b, :E] = orc.quantize_main(kv)
        k = synth.normal_rows(seed, "ik", b * cap, E, 64)
        oc.ik_codes[b, :E], oc.ik_scales[b, :E] = orc.quantize_ik(k)
        oc.length[b] = E
    q_pos = np.array([[E - Q + j for j in range(Q)] for _ in range(B)], np.int32)
    iq = synth.normal(seed, "iq", (B, Q, 4, 64))
    topk, _, _ = orc.index_topk(oc, orc.FULL, iq, q_pos=q_pos)
    S = 128 + Q
    swa = np.zeros((B, S, 512), np.uint8)
    x_old = synth.normal(seed, "swa", (B, S, 512))
    orc.swa_append(swa, x_old, np.full(B, E - Q, np.int32))  # ring before the step's Q new tokens
    x_new = synth.normal(seed, "xnew", (B, Q, 512))
    q = torch.from_numpy(synth.normal(seed, "q", (B, Q, 16, 512))).to(torch.bfloat16)
    return oc, q_pos, topk, swa, x_new, q


def _run(csa, oc, q_pos, topk, swa, x_new, q, noalloc):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B, Q = q.shape[0], q.shape[1]
    gc = csa.Cache(B, oc.cap, 1)
    gc.kv_codes.copy_(dev(oc.kv_codes))
    gc.kv_scales.copy_(dev(oc.kv_scales))
    gc.length.copy_(dev(oc.length))
    ring = dev(swa)
    out = torch.empty((B, Q, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Q, 16), dtype=torch.float32, device="cuda")
    seq = dev(oc.length.astype(np.int32))  # ratio 1: tokens after the append = entries
    args = dict(lse=lse, q_pos=dev(q_pos), swa_x=dev(x_new), swa_len=seq)
    if noalloc:
        csa.sparse_attend_noalloc(gc, dev(topk), ring, q.cuda(), out, SM, **args)
    else:
        csa.sparse_attend(gc, dev(topk), ring, q.cuda(), out, SM, **args)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), ring.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(csa, orc):
    # (B, Q, E): 48 queries in ten splits (the larger call), then 3 queries
    cases = [(16, 3, 6000, 51), (3, 1, 2500, 52)]
    for B, Q, E, seed in cases:
        print(f"no-alloc attention B={B} Q={Q} E={E}", flush=True)
        oc, q_pos, topk, swa, x_new, q = _case(csa, orc, B, Q, E, seed)
        ref_out, ref_lse, ref_ring = _run(csa, oc, q_pos, topk, swa, x_new, q, noalloc=False)
        out, lse, ring = _run(csa, oc, q_pos, topk, swa, x_new, q, noalloc=True)
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)
        assert np.array_equal(ring, ref_ring)
        # and both against the oracle (the ring after the append)
        ring_o = swa.copy()
        orc.swa_append(ring_o, x_new, oc.length.astype(np.int32))
        assert np.array_equal(ring, ring_o)
        want, _ = orc.attend(oc, topk, ring_o, q.float().numpy(), SM, q_pos=q_pos)
        mabs, _ = attn_close(out.float().numpy(), want, name=f"noalloc B={B} Q={Q}")
        print(f"  equal to the workspace call; max abs err vs oracle {mabs:.2e}", flush=True)
