#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

A step is one pass of the whole path over one batch: the Full layer's FP4
quantise-and-append of the new token, then for every layer of the group its
window append, its indexing call (Full with pool, Reindex, or none for Reuse)
and its attention.  The default workload is the decoder group Full(+pool) +
Reindex + 2 Reuse over 16 sequences of 128K context.  Three cache replicas
rotate so that the 256 MB Infinity Cache cannot keep the 143 MB of indexer K
resident between steps.  The steps run as hipGraphs: one graph steps every
replica once (a launch's fixed cost, about 8 us of idle GPU, is paid once per
cycle), and one graph per replica covers the steps left over.  Inputs are seeded synthetic N(0, 1) rows drawn on the device.

Prints one JSON line: metric, value (layer-steps/s; one layer-step advances
every sequence of the batch through one CSA2 layer), roofline of the dominant
kernel (the Full indexer call, timed with HIP events on its stream), and the
CPU oracle timed on the host as a correctness baseline.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "CSA2 decode layer-steps/sec and achieved HBM GB/s (% of peak) at 128K ctx"
UNIT = "layer-steps/s"
PEAK_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
SM_SCALE = float(np.float32(1.0 / math.sqrt(512.0)))
ROWS_PER_SEQ = 1 << 22          # row namespace of one sequence in the seeded generators
FILL_FLOATS = 32 * 1024 * 1024  # fp32 values per cache-fill chunk
MAIN_ROW, IDX_ROW, SWA_ROW = 288, 68, 512
# what the path computes in: E4M3 indexer keys and queries widened exactly to
# bf16 on the matrix cores; FP4 E2M1 x E4M3-scale main rows and E4M3 window
# rows widened exactly to fp16, with the bf16 query scaled exactly into fp16;
# fp32 accumulation and softmax throughout
DTYPE = "e4m3/e2m1 data; bf16 (indexer) and fp16 (attention) MFMA, fp32 accumulate"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Workload:
    """Device state of one workload: R cache replicas, per-layer windows, inputs,
    outputs and workspaces, and the step that runs the whole group."""

    def __init__(self, cid, replicas, extra_steps, keep_host_seqs=0):
        import fp4_kv_cache_index_amd as csa
        self.csa = csa
        w = synth.WORKLOADS[cid]
        self.cid, self.name = cid, w["name"]
        self.B, self.ctx, self.r, self.Q, self.group = w["B"], w["ctx"], w["ratio"], w["Q"], w["group"]
        self.decode = self.Q == 1
        self.L = len(self.group)
        B, r, Q = self.B, self.r, self.Q
        if self.decode:
            self.E_before = self.ctx // r          # entries present before the step
            self.T_step = 1                        # tokens appended per step
            self.S = 128
            cap = self.E_before + extra_steps + 16
        else:
            self.T_step = Q                        # the prefill chunk
            self.E_before = (self.ctx - Q) // r
            self.S = 128 + Q                       # ring holds every window of the chunk
            cap = self.ctx // r + 16
        self.cap = cap
        dev = "cuda"
        t0 = time.time()
        self.caches = [csa.Cache(B, cap, r) for _ in range(replicas)]
        c0 = self.caches[0]
        # ---- fill replica 0 with the context, keep host rows for the oracle sample
        self.host_rows = None
        hs = min(keep_host_seqs, B)
        if hs:
            self.host_rows = dict(kv=np.empty((hs, self.E_before * r, 512), np.float32),
                                  ik=np.empty((hs, self.E_before, 64), np.float32),
                                  lg=np.empty((hs, self.E_before * r, 512), np.float32) if r == 2 else None)
        T_fill = max(r, (FILL_FLOATS // (B * 512)) // r * r)
        tok = 0
        total_tok = self.E_before * r
        while tok < total_tok:
            T = min(T_fill, total_tok - tok)
            kv = torch.stack([synth.torch_normal_rows(cid, "kv", b * ROWS_PER_SEQ + tok, T, 512) for b in range(B)])
            ik = torch.stack([synth.torch_normal_rows(cid, "ik", b * ROWS_PER_SEQ + tok // r, T // r, 64)
                              for b in range(B)])
            lg = None
            if r == 2:
                lg = torch.stack([synth.torch_normal_rows(cid, "logit", b * ROWS_PER_SEQ + tok, T, 512)
                                  for b in range(B)])
            csa.quantize_append(c0, kv, ik, logits=lg)
            if hs:
                self.host_rows["kv"][:, tok:tok + T] = kv[:hs].cpu().numpy()
                self.host_rows["ik"][:, tok // r:(tok + T) // r] = ik[:hs].cpu().numpy()
                if r == 2:
                    self.host_rows["lg"][:, tok:tok + T] = lg[:hs].cpu().numpy()
            tok += T
        torch.cuda.synchronize()
        for c in self.caches[1:]:
            for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
                getattr(c, name).copy_(getattr(c0, name))
        for c in self.caches:
            c.host_len_bound = self.E_before
        log(f"filled {replicas} replica(s) of {B} x {self.E_before} entries in {time.time() - t0:.1f}s")

        # ---- per-layer windows: the S tokens before the step, then the step's own tokens
        tok_before = self.E_before * r
        self.swa_rows = [torch.stack([synth.torch_normal_rows(cid, f"swa{l}", b * ROWS_PER_SEQ + tok_before - 128,
                                                              128, 512) for b in range(B)]) for l in range(self.L)]
        self.swas = []
        seq_before = torch.full((B,), tok_before, dtype=torch.int32, device=dev)
        for _ in range(replicas):
            per = []
            for l in range(self.L):
                s = torch.zeros((B, self.S, 512), dtype=torch.uint8, device=dev)
                csa.swa_append(s, self.swa_rows[l], seq_before)
                per.append(s)
            self.swas.append(per)
        # ---- step inputs: one set per replica
        self.seq_after = torch.full((B,), tok_before + self.T_step, dtype=torch.int32, device=dev)
        self.q_pos = None
        if not self.decode:
            self.q_pos = (torch.arange(Q, dtype=torch.int32, device=dev) + tok_before).repeat(B, 1).contiguous()
        self.inputs = []
        for i in range(replicas):
            g = f"step{i}"
            inp = dict(
                kv=torch.stack([synth.torch_normal_rows(cid, g + "kv", b * ROWS_PER_SEQ, self.T_step, 512)
                                for b in range(B)]),
                ik=torch.stack([synth.torch_normal_rows(cid, g + "ik", b * ROWS_PER_SEQ, self.T_step // r, 64)
                                for b in range(B)]),
                lg=(torch.stack([synth.torch_normal_rows(cid, g + "lg", b * ROWS_PER_SEQ, self.T_step, 512)
                                 for b in range(B)]) if r == 2 else None),
                x=[torch.stack([synth.torch_normal_rows(cid, g + f"x{l}", b * ROWS_PER_SEQ, self.T_step, 512)
                                for b in range(B)]) for l in range(self.L)],
                iq=[synth.torch_normal_rows(cid, g + f"iq{l}", 0, B * Q * 4, 64).reshape(B, Q, 4, 64).contiguous()
                    for l in range(self.L)],
                q=[synth.torch_normal_rows(cid, g + f"q{l}", 0, B * Q * 16, 512).reshape(B, Q, 16, 512)
                   .to(torch.bfloat16).contiguous() for l in range(self.L)],
            )
            self.inputs.append(inp)
        # ---- outputs and workspaces
        self.topk = [torch.empty((B, Q, 512), dtype=torch.int32, device=dev) for _ in range(self.L)]
        self.pool = torch.empty((B, Q, csa.POOL), dtype=torch.int32, device=dev)
        self.out = [torch.empty((B, Q, 16, 512), dtype=torch.bfloat16, device=dev) for _ in range(self.L)]
        self.ws_idx = torch.zeros(max(1, csa.workspace_bytes(csa.OP_INDEX, B, Q, cap)), dtype=torch.uint8,
                                  device=dev)
        self.ws_att = torch.zeros(max(1, csa.workspace_bytes(csa.OP_ATTEND, B, Q, cap)), dtype=torch.uint8,
                                  device=dev)
        self.fused_full = self.decode and self.r == 1 and self.group[0] in ("full", "full_pool")
        torch.cuda.synchronize()

    # one pass of the whole group on replica i
    def step(self, i):
        csa = self.csa
        c, inp, swas = self.caches[i], self.inputs[i], self.swas[i]
        if not self.decode:
            c.length.fill_(self.E_before)
        c.host_len_bound = self.E_before if not self.decode else c.host_len_bound
        # a decode step at ratio 1 appends the Full layer's entry in its indexing call
        fused = self.fused_full
        if not fused:
            csa.quantize_append(c, inp["kv"], inp["ik"], logits=inp["lg"])
        seq = c.length if (self.decode and self.r == 1) else self.seq_after
        topk = None
        for l, mode in enumerate(self.group):
            if mode in ("full", "full_pool"):
                pool = self.pool if mode == "full_pool" else None
                if fused and l == 0:
                    csa.append_index_score_topk(c, inp["kv"], inp["ik"], inp["iq"][l], self.topk[l], q_pos=self.q_pos,
                                                pool_out=pool, ws=self.ws_idx)
                else:
                    csa.index_score_topk(c, csa.FULL, inp["iq"][l], self.topk[l], q_pos=self.q_pos, pool_out=pool,
                                         ws=self.ws_idx)
                topk = self.topk[l]
            elif mode == "reindex":
                csa.index_score_topk(c, csa.REINDEX, inp["iq"][l], self.topk[l], q_pos=self.q_pos,
                                     pool_in=self.pool, ws=self.ws_idx)
                topk = self.topk[l]
            # the layer's window append runs inside its attention launch
            csa.sparse_attend(c, topk, swas[l], inp["q"][l], self.out[l], SM_SCALE, q_pos=self.q_pos,
                              ws=self.ws_att, swa_x=inp["x"][l], swa_len=seq)

    def attend_layer(self, i):
        """Layer 0's attention on replica i (its window append included)."""
        inp = self.inputs[i]
        seq = self.caches[i].length if (self.decode and self.r == 1) else self.seq_after
        self.csa.sparse_attend(self.caches[i], self.topk[0], self.swas[i][0], inp["q"][0], self.out[0], SM_SCALE,
                               q_pos=self.q_pos, ws=self.ws_att, swa_x=inp["x"][0], swa_len=seq)

    def attend_bytes(self):
        """Algorithmic bytes of one layer's attention: the gathered rows and the window."""
        return self.B * self.Q * (512 * MAIN_ROW + 128 * SWA_ROW)

    def full_index(self, i):
        csa = self.csa
        mode = self.group[0]
        csa.index_score_topk(self.caches[i], csa.FULL, self.inputs[i]["iq"][0], self.topk[0], q_pos=self.q_pos,
                             pool_out=self.pool if mode == "full_pool" else None, ws=self.ws_idx)

    # algorithmic KV + indexer bytes of one step at E entries visible to the Full scan
    def step_bytes(self, E):
        B, Q, L = self.B, self.Q, self.L
        n_sel = min(512, E)
        by = 0
        for mode in self.group:
            if mode in ("full", "full_pool"):
                by += B * E * IDX_ROW if self.decode else B * self.E_before * IDX_ROW
            elif mode == "reindex":
                by += B * min(16384, E) * IDX_ROW
        by += L * B * Q * n_sel * MAIN_ROW
        by += L * B * Q * 128 * SWA_ROW
        return by


class OracleStep:
    """The oracle's copy of the first `hs` sequences of a workload: built from the
    same seeded rows (copied from where they were drawn), advanced by the same
    step inputs.  `qsel` restricts every layer to a subset of query slots."""

    def __init__(self, wl, qsel=None):
        import oracle as orc
        self.orc, self.wl = orc, wl
        h = wl.host_rows
        self.hs = hs = h["kv"].shape[0]
        r = wl.r
        self.oc = orc.Cache(hs, wl.cap, r)
        orc.quantize_append(self.oc, h["kv"], h["ik"], logits=h["lg"])
        self.swas = []
        tok_before = wl.E_before * r
        for l in range(wl.L):
            s = np.zeros((hs, wl.S, 512), np.uint8)
            orc.swa_append(s, wl.swa_rows[l][:hs].cpu().numpy(), np.full(hs, tok_before, np.int32))
            self.swas.append(s)
        self.qsel = qsel
        inp = wl.inputs[0]
        pick = (lambda a: a[:, qsel]) if qsel is not None else (lambda a: a)
        self.inp = dict(kv=inp["kv"][:hs].cpu().numpy(), ik=inp["ik"][:hs].cpu().numpy(),
                        lg=inp["lg"][:hs].cpu().numpy() if inp["lg"] is not None else None,
                        x=[t[:hs].cpu().numpy() for t in inp["x"]],
                        iq=[pick(t[:hs].cpu().numpy()) for t in inp["iq"]],
                        q=[pick(t[:hs].float().cpu().numpy()) for t in inp["q"]])
        self.q_pos = pick(wl.q_pos[:hs].cpu().numpy()) if wl.q_pos is not None else None

    def step(self, want_scores=False, gpu_used=None):
        """One group step; returns per-layer dict(topk, pool, scores, out, out_cmp).

        gpu_used[l], if given, is the Top-K list [hs][Q'][512] the GPU's layer l
        attended with; out_cmp is the oracle's attention over that list (its own
        `out` when the two lists agree), so that a boundary swap still leaves
        every attention output comparable."""
        orc, wl, oc, inp = self.orc, self.wl, self.oc, self.inp
        if not wl.decode:
            oc.length[:] = wl.E_before
        orc.quantize_append(oc, inp["kv"], inp["ik"], logits=inp["lg"])
        seq = (oc.length * wl.r).astype(np.int32) if wl.decode else \
            np.full(self.hs, wl.E_before * wl.r + wl.T_step, np.int32)
        res, topk, pool = [], None, None
        for l, mode in enumerate(wl.group):
            orc.swa_append(self.swas[l], inp["x"][l], seq)
            scores = None
            if mode in ("full", "full_pool"):
                topk, pool, scores = orc.index_topk(oc, orc.FULL, inp["iq"][l], q_pos=self.q_pos,
                                                    want_pool=mode == "full_pool", want_scores=want_scores)
            elif mode == "reindex":
                topk, _, scores = orc.index_topk(oc, orc.REINDEX, inp["iq"][l], q_pos=self.q_pos, pool_in=pool,
                                                 want_scores=want_scores)
            out, lse = orc.attend(oc, topk, self.swas[l], inp["q"][l], SM_SCALE, q_pos=self.q_pos)
            out_cmp = out
            if gpu_used is not None and not np.array_equal(gpu_used[l], topk):
                out_cmp, _ = orc.attend(oc, gpu_used[l], self.swas[l], inp["q"][l], SM_SCALE, q_pos=self.q_pos)
            res.append(dict(topk=topk, pool=pool if mode == "full_pool" else None, scores=scores, out=out, lse=lse,
                            out_cmp=out_cmp))
        return res


# The whole 38-layer CSA2 schedule of one decode token: three encoder groups of
# Full + 5 Reuse, each Full layer owning a ratio-2 cache, then the decoder's
# Full (+pool) + 3 Reuse and four groups of Reindex + 3 Reuse over the decoder's
# ratio-1 cache (technologiesdigest "CSA2"; ai.info "Methodology").
SCHEDULE38 = ([("full", "enc0")] + [("reuse", "enc0")] * 5 + [("full", "enc1")] + [("reuse", "enc1")] * 5 +
              [("full", "enc2")] + [("reuse", "enc2")] * 5 + [("full_pool", "dec")] + [("reuse", "dec")] * 3 +
              ([("reindex", "dec")] + [("reuse", "dec")] * 3) * 4)
ENC_CACHES = ("enc0", "enc1", "enc2")


class Schedule38:
    """Device state of the 38-layer schedule over B sequences of `ctx` tokens.

    A step is two decode tokens, at positions ctx and ctx + 1.  An encoder
    entry summarises two tokens, so the first token leaves it pending (the
    encoder layers see ctx / 2 entries) and the second completes it: each
    encoder Full layer appends the pair's entry before scoring.  The decoder
    appends one entry per token.  Every Full layer derives its indexer K by
    projecting its main-KV entries (csa2_quantize_append_proj, seeded
    N(0, 1/512) weights per cache).  Every step first resets the lengths, so
    each step sees the same context.  76 layer-steps per step."""

    def __init__(self, cid, B, ctx, replicas, keep_host_seqs=0):
        import fp4_kv_cache_index_amd as csa
        assert ctx % 2 == 0
        self.csa, self.cid, self.B, self.ctx = csa, cid, B, ctx
        w = synth.WORKLOADS.get(cid, {})
        self.name = w["name"] if (w.get("B"), w.get("ctx")) == (B, ctx) else f"sched38_b{B}_ctx{ctx}"
        self.r, self.Q, self.decode, self.tokens = 1, 1, False, 2
        self.group = [m for m, _ in SCHEDULE38]
        self.L = len(SCHEDULE38) * self.tokens
        self.S = 128
        self.E0 = {"dec": ctx}
        self.E0.update({n: ctx // 2 for n in ENC_CACHES})
        self.ratio = {"dec": 1}
        self.ratio.update({n: 2 for n in ENC_CACHES})
        dev = "cuda"
        t0 = time.time()
        self.w_ik_host = {n: (synth.normal(cid, f"w_ik_{n}", (512, 64)) / np.float32(math.sqrt(512.0)))
                          .astype(np.float32) for n in self.E0}
        self.w_ik = {n: torch.from_numpy(w).to(dev) for n, w in self.w_ik_host.items()}
        self.caches = [{n: csa.Cache(B, self.E0[n] + 8, self.ratio[n]) for n in self.E0} for _ in range(replicas)]
        hs = min(keep_host_seqs, B)
        self.host_rows = {} if hs else None
        T_fill = max(2, (FILL_FLOATS // (B * 512)) // 2 * 2)
        for n, c in self.caches[0].items():
            r = self.ratio[n]
            if hs:
                self.host_rows[n] = dict(kv=np.empty((hs, ctx, 512), np.float32),
                                         lg=np.empty((hs, ctx, 512), np.float32) if r == 2 else None)
            tok = 0
            while tok < ctx:
                T = min(T_fill, ctx - tok)
                kv = torch.stack([synth.torch_normal_rows(cid, f"kv_{n}", b * ROWS_PER_SEQ + tok, T, 512)
                                  for b in range(B)])
                lg = (torch.stack([synth.torch_normal_rows(cid, f"lg_{n}", b * ROWS_PER_SEQ + tok, T, 512)
                                   for b in range(B)]) if r == 2 else None)
                csa.quantize_append_proj(c, kv, self.w_ik[n], logits=lg)
                if hs:
                    h = self.host_rows[n]
                    h["kv"][:, tok:tok + T] = kv[:hs].cpu().numpy()
                    if r == 2:
                        h["lg"][:, tok:tok + T] = lg[:hs].cpu().numpy()
                tok += T
        torch.cuda.synchronize()
        for rep in self.caches[1:]:
            for n, c in rep.items():
                for f in ("kv_codes", "kv_scales", "ik_codes", "ik_scales", "length"):
                    getattr(c, f).copy_(getattr(self.caches[0][n], f))
        for rep in self.caches:
            for n, c in rep.items():
                c.host_len_bound = self.E0[n]
        log(f"filled {replicas} replica(s) of 3 encoder caches ({ctx // 2} entries) and a decoder cache "
            f"({ctx} entries) x {B} sequences in {time.time() - t0:.1f}s")
        # per-layer windows: the 128 tokens before the step
        nL = len(SCHEDULE38)
        self.swa_rows = [torch.stack([synth.torch_normal_rows(cid, f"swa{l}", b * ROWS_PER_SEQ + ctx - 128, 128, 512)
                                      for b in range(B)]) for l in range(nL)]
        seq_before = torch.full((B,), ctx, dtype=torch.int32, device=dev)
        self.swas = []
        for _ in range(replicas):
            per = []
            for l in range(nL):
                sw = torch.zeros((B, self.S, 512), dtype=torch.uint8, device=dev)
                csa.swa_append(sw, self.swa_rows[l], seq_before)
                per.append(sw)
            self.swas.append(per)
        # step inputs (one set per replica), token t at position ctx + t
        self.q_pos = [torch.full((B, 1), ctx + t, dtype=torch.int32, device=dev) for t in range(2)]
        self.seq = [torch.full((B,), ctx + t + 1, dtype=torch.int32, device=dev) for t in range(2)]
        rows = lambda tag, n, w: torch.stack([synth.torch_normal_rows(cid, tag, b * ROWS_PER_SEQ, n, w)
                                              for b in range(B)])
        self.inputs = []
        for i in range(replicas):
            g = f"s38step{i}"
            inp = dict(
                # encoder pair (2 tokens -> 1 entry) appended at the second token
                enc={n: dict(kv=rows(g + "kv" + n, 2, 512), lg=rows(g + "lg" + n, 2, 512)) for n in ENC_CACHES},
                dec=[dict(kv=rows(g + f"kvdec{t}", 1, 512)) for t in range(2)],
                x=[[rows(g + f"x{t}_{l}", 1, 512) for l in range(nL)] for t in range(2)],
                iq=[[(rows(g + f"iq{t}_{l}", 4, 64).reshape(B, 1, 4, 64).contiguous()
                      if SCHEDULE38[l][0] != "reuse" else None) for l in range(nL)] for t in range(2)],
                q=[[rows(g + f"q{t}_{l}", 16, 512).reshape(B, 1, 16, 512).to(torch.bfloat16).contiguous()
                    for l in range(nL)] for t in range(2)],
            )
            self.inputs.append(inp)
        self.topk = {n: torch.empty((B, 1, 512), dtype=torch.int32, device=dev) for n in ("enc", "dec_full", "dec_ri")}
        self.pool = torch.empty((B, 1, csa.POOL), dtype=torch.int32, device=dev)
        self.out = [[torch.empty((B, 1, 16, 512), dtype=torch.bfloat16, device=dev) for _ in range(nL)]
                    for _ in range(2)]
        capmax = max(c.capacity for c in self.caches[0].values())
        self.ws_idx = torch.zeros(max(1, csa.workspace_bytes(csa.OP_INDEX, B, 1, capmax)), dtype=torch.uint8,
                                  device=dev)
        self.ws_att = torch.zeros(max(1, csa.workspace_bytes(csa.OP_ATTEND, B, 1, capmax)), dtype=torch.uint8,
                                  device=dev)
        # the topk every layer attends with, per token (filled by step(); the test reads it)
        self.used = [[None] * nL for _ in range(2)]
        self.used_pool = [None, None]
        torch.cuda.synchronize()

    def step(self, i, record=False):
        """One step on replica i; with `record` (eager runs only) keep a copy of
        the Top-K (and pool) each layer attended with in self.used / self.used_pool."""
        csa = self.csa
        cs, inp, swas = self.caches[i], self.inputs[i], self.swas[i]
        for n, c in cs.items():
            c.length.fill_(self.E0[n])
            c.host_len_bound = self.E0[n]
        for t in range(2):
            if t == 1:
                for n in ENC_CACHES:
                    e = inp["enc"][n]
                    csa.quantize_append_proj(cs[n], e["kv"], self.w_ik[n], logits=e["lg"])
            csa.quantize_append_proj(cs["dec"], inp["dec"][t]["kv"], self.w_ik["dec"])
            topk = None
            for l, (mode, cn) in enumerate(SCHEDULE38):
                c = cs[cn]
                if mode == "full":
                    topk = self.topk["enc"]
                    csa.index_score_topk(c, csa.FULL, inp["iq"][t][l], topk, q_pos=self.q_pos[t], ws=self.ws_idx)
                elif mode == "full_pool":
                    topk = self.topk["dec_full"]
                    csa.index_score_topk(c, csa.FULL, inp["iq"][t][l], topk, q_pos=self.q_pos[t],
                                         pool_out=self.pool, ws=self.ws_idx)
                elif mode == "reindex":
                    topk = self.topk["dec_ri"]
                    csa.index_score_topk(c, csa.REINDEX, inp["iq"][t][l], topk, q_pos=self.q_pos[t],
                                         pool_in=self.pool, ws=self.ws_idx)
                if record:
                    if mode != "reuse":
                        snap = topk.clone()
                        if mode == "full_pool":
                            self.used_pool[t] = self.pool.clone()
                    self.used[t][l] = snap
                csa.sparse_attend(c, topk, swas[l], inp["q"][t][l], self.out[t][l], SM_SCALE, q_pos=self.q_pos[t],
                                  ws=self.ws_att, swa_x=inp["x"][t][l], swa_len=self.seq[t])

    def full_index(self, i):
        """The decoder's Full call (with the pool) on the step's second token."""
        self.csa.index_score_topk(self.caches[i]["dec"], self.csa.FULL, self.inputs[i]["iq"][1][18],
                                  self.topk["dec_full"], q_pos=self.q_pos[1], pool_out=self.pool, ws=self.ws_idx)

    def index_bytes(self):
        return self.B * (self.ctx + 2) * IDX_ROW

    def step_bytes(self, E=None):
        """Algorithmic KV + indexer bytes of one step (two tokens)."""
        B, by = self.B, 0
        for t in range(2):
            e_enc = self.ctx // 2 + t
            by += 3 * B * e_enc * IDX_ROW               # encoder Full scans
            by += B * (self.ctx + t + 1) * IDX_ROW       # decoder Full scan
            by += 4 * B * min(16384, self.ctx + t + 1) * IDX_ROW  # Reindex pools
            by += len(SCHEDULE38) * B * 512 * MAIN_ROW   # gathers
            by += len(SCHEDULE38) * B * 128 * SWA_ROW    # windows
        return by


class OracleSchedule38:
    """The oracle's replay of Schedule38's step on its first sequences, from the
    same seeded rows and step inputs (host copies)."""

    def __init__(self, wl):
        import oracle as orc
        self.orc, self.wl = orc, wl
        hs = next(iter(wl.host_rows.values()))["kv"].shape[0]
        self.hs = hs
        self.oc = {}
        for n, h in wl.host_rows.items():
            c = orc.Cache(hs, wl.caches[0][n].capacity, wl.ratio[n])
            orc.quantize_append_proj(c, h["kv"], wl.w_ik_host[n], logits=h["lg"])
            self.oc[n] = c
        self.swas = []
        for l in range(len(SCHEDULE38)):
            sw = np.zeros((hs, wl.S, 512), np.uint8)
            orc.swa_append(sw, wl.swa_rows[l][:hs].cpu().numpy(), np.full(hs, wl.ctx, np.int32))
            self.swas.append(sw)
        h = lambda x: None if x is None else x[:hs].float().cpu().numpy()
        inp = wl.inputs[0]
        self.inp = dict(enc={n: {k: h(v) for k, v in e.items()} for n, e in inp["enc"].items()},
                        dec=[{k: h(v) for k, v in d.items()} for d in inp["dec"]],
                        x=[[h(x) for x in xs] for xs in inp["x"]],
                        iq=[[h(x) for x in xs] for xs in inp["iq"]],
                        q=[[h(x) for x in xs] for xs in inp["q"]])
        self.q_pos = [np.full((hs, 1), wl.ctx + t, np.int32) for t in range(2)]

    def step(self, want_scores=False, gpu_used=None):
        """Returns res[t][l] = dict(topk, pool, scores, out, out_cmp) for token t and
        layer l; gpu_used[t][l] as in OracleStep.step (the ring and caches are as
        they were at that layer when out_cmp is computed)."""
        orc, wl, oc, inp = self.orc, self.wl, self.oc, self.inp
        for n, c in oc.items():
            c.length[:] = wl.E0[n]
        res = [[None] * len(SCHEDULE38) for _ in range(2)]
        for t in range(2):
            if t == 1:
                for n in ENC_CACHES:
                    e = inp["enc"][n]
                    orc.quantize_append_proj(oc[n], e["kv"], wl.w_ik_host[n], logits=e["lg"])
            orc.quantize_append_proj(oc["dec"], inp["dec"][t]["kv"], wl.w_ik_host["dec"])
            seq = np.full(self.hs, wl.ctx + t + 1, np.int32)
            topk, pool = None, None
            for l, (mode, cn) in enumerate(SCHEDULE38):
                c = oc[cn]
                orc.swa_append(self.swas[l], inp["x"][t][l], seq)
                scores, lpool = None, None
                if mode in ("full", "full_pool"):
                    topk, lpool, scores = orc.index_topk(c, orc.FULL, inp["iq"][t][l], q_pos=self.q_pos[t],
                                                         want_pool=mode == "full_pool", want_scores=want_scores)
                    if mode == "full_pool":
                        pool = lpool
                elif mode == "reindex":
                    topk, _, scores = orc.index_topk(c, orc.REINDEX, inp["iq"][t][l], q_pos=self.q_pos[t],
                                                     pool_in=pool, want_scores=want_scores)
                out, _ = orc.attend(c, topk, self.swas[l], inp["q"][t][l], SM_SCALE, q_pos=self.q_pos[t])
                out_cmp = out
                if gpu_used is not None and not np.array_equal(gpu_used[t][l], topk):
                    out_cmp, _ = orc.attend(c, gpu_used[t][l], self.swas[l], inp["q"][t][l], SM_SCALE,
                                            q_pos=self.q_pos[t])
                res[t][l] = dict(topk=topk, pool=lpool, scores=scores, out=out, out_cmp=out_cmp)
        return res


def cpu_baseline(wl, steps=3):
    """The oracle, as it stands, on the first sequences of the same workload."""
    t0 = time.time()
    ost = OracleSchedule38(wl) if isinstance(wl, Schedule38) else OracleStep(wl)
    log(f"oracle sample set up in {time.time() - t0:.1f}s ({ost.hs} sequences)")
    times = []
    for s_i in range(steps):
        t = time.time()
        ost.step()
        times.append(time.time() - t)
        log(f"oracle step {s_i}: {times[-1]:.2f}s")
    t_step = float(np.median(times))
    value = wl.L / t_step * ost.hs / wl.B
    cores = int(min(ost.orc.num_threads(), ost.hs * wl.Q))
    # one more step on a single thread, for the per-core rate, when it should
    # take well under a minute
    single = None
    n_thr = ost.orc.num_threads()
    if t_step * cores <= 40.0:
        ost.orc.set_threads(1)
        t = time.time()
        ost.step()
        t_one = time.time() - t
        ost.orc.set_threads(n_thr)
        single = wl.L / t_one * ost.hs / wl.B
        log(f"oracle step on one thread: {t_one:.2f}s")
    return dict(value=value, unit=UNIT, cores=cores, kind="oracle", single_thread_value=single,
                cpu_model=cpu_model(),
                sample=f"{steps} group steps of the first {ost.hs} of {wl.B} sequences (full context, all {wl.L} "
                       f"layers), median {t_step:.2f}s per step, scaled by {wl.B}/{ost.hs} to the whole batch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def pct(xs):
    """p10, median and p90 of a list of µs figures."""
    return [round(float(np.percentile(xs, q)), 2) for q in (10, 50, 90)]


COPY_BYTES = 256 << 20


def copy_calibration():
    """A plain device copy of known size, for scaling the rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters to bytes (run under the same counter pass)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def summarize_counters(fetch_csv, write_csv, workload_name, head=None):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of `bench.py --copy-calibration` into HBM bytes per Full indexer call.
    head: whether the call scores one query per workgroup (index_head; else the
    shared-load index_shared_head), then index_select; by default, whether the
    workload has fewer than four queries per sequence."""
    import csv
    import hashlib

    def per_kernel(path, counter):
        acc, copies = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, grid = r["Kernel_Name"], int(r["Grid_Size"])
            acc.setdefault((name, grid), []).append(float(r["Counter_Value"]))
            if "copyBuffer" in name:
                copies.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        # the calibration copies are the last three device copies of the run
        return acc, [v for _, v in sorted(copies)[-3:]]

    # the kernels of one Full call: a head kernel and the Full call's
    # index_select (<false, ...>; with a pool its grid is the larger, as it
    # also builds the pool)
    def full_call(acc, name, largest_grid=False):
        grids = [g for (n, g) in acc if name in n]
        return [v for (n, g), vals in acc.items()
                if name in n and (not largest_grid or g == max(grids)) for v in vals]

    if head is None:
        head = next(w for w in synth.WORKLOADS.values() if w["name"] == workload_name).get("Q", 1) < 4
    parts = (("head", "index_head_kernel<false>" if head else "index_shared_head_kernel<", False),
             ("select", "index_select_kernel<false,", True))
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        acc, copy = per_kernel(path, counter)
        kib_copy = float(np.median(copy)) if copy else float("nan")
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        for part, name, largest in parts:
            vals = full_call(acc, name, largest)
            out[f"{key}_kib_{part}"] = float(np.mean(vals)) if vals else None
        out[f"{key}_kib_copy_{COPY_BYTES >> 20}MiB"] = kib_copy
        out[f"{key}_factor"] = COPY_BYTES / (kib_copy * 1024.0)
    tot = 0.0
    for key in ("fetch", "write"):
        kib = sum(out[f"{key}_kib_{part}"] or 0.0 for part, _, _ in parts)
        tot += kib * 1024.0 * out[f"{key}_factor"]
    src = "index_head.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, "fp4_kv_cache_index_amd", "csrc", src), "rb").read()).hexdigest()
    out.update(source=src, source_sha256=sha, workload=workload_name, hbm_bytes_per_launch=round(tot))
    path = os.path.join(ROOT, "profiles", f"counters_index_full_{workload_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def traffic_from_profiles(wl, kernel_name):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter
    summaries, if they were taken on the kernel source as it is now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"counters_{kernel_name}_{wl.name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "fp4_kv_cache_index_amd", "csrc", rec["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def stream_ceiling(nbytes, reps=12, span=1 << 30, blocks=1024):
    """The streaming-read ceiling over `nbytes` (the Full scan's size): a plain
    non-temporal 16-byte-per-lane read kernel (libcsa2_roofline.so) over
    windows rotated through `span` bytes, so that the 256 MB Infinity Cache
    cannot serve a window twice in a row; a graph of `reps` reads, median of
    10 replays.  Returns GB/s."""
    import ctypes
    import fp4_kv_cache_index_amd as csa
    L = ctypes.CDLL(csa.ROOF_LIB_PATH)
    f = L.csa2roof_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    nbytes = nbytes // 16 * 16
    nwin = max(3, span // max(nbytes, 1))
    buf = torch.ones((nwin * nbytes) // 4 + 64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def reads():  # on the stream current at the call (graph capture runs on its own)
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(reps):
            rc = f(ctypes.c_void_p(buf.data_ptr() + (i % nwin) * nbytes), nbytes, ctypes.c_void_p(sink.data_ptr()),
                   blocks, sp)
            assert rc == 0, rc
    reads()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        reads()
    ts = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3 / reps)
    t = float(np.median(ts))
    del buf
    return nbytes / t / 1e9, t


def time_calls(call, n, R):
    """Mean and spread of `n` eager calls of call(i % R), each bracketed by HIP
    events on the current stream and queued behind a sleep so that host launch
    cost does not show."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(R):
        call(i)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)  # keep the GPU busy while the launches queue up
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        call(i % R)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in evs]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload preset (synth.WORKLOADS)")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--ctx", type=int, default=0, help="context tokens of the 38-layer schedule (0: the preset's)")
    ap.add_argument("--batch", type=int, default=0, help="sequences of the 38-layer schedule (0: the preset's)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the oracle sample (0: all)")
    ap.add_argument("--roofline-iters", type=int, default=30)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (scales the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters_index_full_<workload>.json from two rocprofv3 --pmc CSVs")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, synth.WORKLOADS[args.config]["name"])
        return
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported "
              "(it is not sharded across GPUs)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: run one process on one GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    import fp4_kv_cache_index_amd as csa
    csa.lib()
    R = max(1, args.replicas)
    # appends per replica: warm-up, timed steps and the spread pass (R >= 2 replicas
    # share them, so warm-up + steps covers all three)
    extra = args.warmup + args.steps * (2 if R == 1 else 1) + 4 * R + 8
    want_cpu = not args.no_cpu_baseline
    wl0 = synth.WORKLOADS[args.config]
    if wl0.get("schedule"):
        hs = (args.cpu_seqs or 1) if want_cpu else 0
        wl = Schedule38(args.config, args.batch or wl0["B"], args.ctx or wl0["ctx"], R, keep_host_seqs=hs)
    else:
        hs = (args.cpu_seqs or wl0["B"]) if want_cpu else 0
        wl = Workload(args.config, R, extra, keep_host_seqs=hs)

    # ---- capture one graph per replica, and one graph that steps every replica
    # once (a cycle), so that a launch's fixed cost is paid once per R steps;
    # each step does all of its work either way
    graphs = None
    if not args.no_graph:
        for i in range(R):  # eager warm-up outside capture
            wl.step(i)
        torch.cuda.synchronize()
        graphs = []
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                wl.step(i)
            graphs.append(g)
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle):
            for i in range(R):
                wl.step(i)
        torch.cuda.synchronize()

        def run_steps(i0, n, marks=None):  # steps i0 .. i0 + n - 1, replica i % R each
            i = i0
            while i < i0 + n:
                if marks is not None:
                    marks.append((i, torch.cuda.Event(enable_timing=True)))
                    marks[-1][1].record()
                if i % R == 0 and i + R <= i0 + n:
                    cycle.replay()
                    i += R
                else:
                    graphs[i % R].replay()
                    i += 1
    else:
        def run_steps(i0, n, marks=None):
            for i in range(i0, i0 + n):
                if marks is not None:
                    marks.append((i, torch.cuda.Event(enable_timing=True)))
                    marks[-1][1].record()
                wl.step(i % R)
    run_steps(0, args.warmup)
    torch.cuda.synchronize()
    E_start = int(wl.caches[0].length.max().item()) if wl.decode else 0
    log(f"warm-up done, timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    run_steps(args.warmup, args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    E_end = int(wl.caches[0].length.max().item()) if wl.decode else 0
    # the spread: the same steps again, untimed above, with an event before each
    # graph launch (the events stay out of the timed region)
    marks = []
    i_sp = args.warmup + args.steps
    run_steps(i_sp, args.steps, marks)
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_end.record()
    torch.cuda.synchronize()
    bounds = marks + [(i_sp + args.steps, ev_end)]
    step_us = [a[1].elapsed_time(b[1]) * 1e3 / (b[0] - a[0]) for a, b in zip(bounds, bounds[1:])]
    ms_per_step = wall * 1e3 / args.steps
    value = wl.L * args.steps / wall
    E_mid = (E_start + E_end) // 2 if wl.decode else wl.ctx // wl.r
    step_bytes = wl.step_bytes(E_mid)
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"{ms_per_step * 1e3:.1f} us/step (events {gpu_ms * 1e3 / args.steps:.1f} us), {value:.0f} layer-steps/s, "
        f"{step_gbps:.0f} GB/s on {step_bytes / 1e6:.1f} MB/step")

    # ---- dominant kernel: the Full indexer call, HIP events on its stream
    durs = time_calls(wl.full_index, args.roofline_iters, R)
    t_idx = float(np.mean(durs))
    E_idx = int(wl.caches[0].length.max().item()) if wl.decode else wl.ctx // wl.r
    # bytes: every indexer key of the batch once (the queries of a sequence share them);
    # FLOPs: 2 x 4 heads x 64 dims per (query, visible entry) pair
    idx_bytes = wl.B * E_idx * IDX_ROW
    if isinstance(wl, Schedule38):
        idx_bytes = wl.index_bytes()  # the decoder's Full call: one query per sequence
        pairs = idx_bytes // IDX_ROW
    elif wl.decode:
        pairs = wl.B * E_idx
    else:
        pos = wl.ctx - wl.Q + np.arange(wl.Q)
        pairs = int(np.minimum(E_idx, (pos + 1) // wl.r).sum()) * wl.B
    flops = 2 * 4 * 64 * pairs
    traffic = traffic_from_profiles(wl, "index_full")
    if getattr(wl, "Q", 1) < 4:
        kernel_name = "index_head + index_select (one csa2_index_score_topk Full call)"
    else:
        kernel_name = "index_shared_head + index_select (one csa2_index_score_topk Full call)"
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_GBPS * 1e9)  # FLOP per byte where the bf16 matrix cores take over
    if flops / idx_bytes < ridge:
        # decode (one or a few queries per sequence): bound by streaming the indexer keys
        achieved = idx_bytes / t_idx / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / PEAK_GBPS, 4), traffic=traffic, kernel=kernel_name,
                    bytes_per_launch=idx_bytes, avg_launch_us=round(t_idx * 1e6, 2),
                    launch_us_p10_p50_p90=pct([d * 1e6 for d in durs]))
        log(f"Full indexer call: {t_idx * 1e6:.1f} us, {achieved:.0f} GB/s on {idx_bytes / 1e6:.1f} MB")
    else:
        # a prefill chunk scores every query against every entry it sees: a dense
        # contraction on the bf16 matrix cores
        tflops = flops / t_idx / 1e12
        roof = dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(tflops / PEAK_BF16_TFLOPS, 4), traffic=traffic, kernel=kernel_name,
                    flops_per_launch=flops, avg_launch_us=round(t_idx * 1e6, 2),
                    launch_us_p10_p50_p90=pct([d * 1e6 for d in durs]))
        log(f"Full indexer call: {t_idx * 1e6:.1f} us, {tflops:.1f} TFLOP/s on {flops / 1e9:.2f} GFLOP")

    # ---- the streaming-read ceiling over the same bytes, for the fraction of what a plain read reaches
    if roof["bound"] == "hbm":
        ceil_gbps, ceil_t = stream_ceiling(idx_bytes)
        roof["ceiling_GBps"] = round(ceil_gbps, 1)
        roof["frac_of_ceiling"] = round(roof["achieved"] / ceil_gbps, 4)
        log(f"streaming-read ceiling over {idx_bytes / 1e6:.1f} MB: {ceil_gbps:.0f} GB/s ({ceil_t * 1e6:.1f} us)")
    # ---- attention of one layer (attention launch + split merge), HIP events on its stream
    roof_att = None
    if hasattr(wl, "attend_layer"):
        adurs = time_calls(wl.attend_layer, args.roofline_iters, R)
        t_att = float(np.mean(adurs))
        att_bytes = wl.attend_bytes()
        achieved = att_bytes / t_att / 1e9
        roof_att = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_GBPS, unit="GB/s",
                        frac=round(achieved / PEAK_GBPS, 4), traffic=None,
                        kernel="attend + merge (one csa2_sparse_attend call, layer 0)", bytes_per_launch=att_bytes,
                        avg_launch_us=round(t_att * 1e6, 2), launch_us_p10_p50_p90=pct([d * 1e6 for d in adurs]))
        log(f"attention layer: {t_att * 1e6:.1f} us, {achieved:.0f} GB/s on {att_bytes / 1e6:.2f} MB")
    if args.copy_calibration:
        copy_calibration()
    cpu = None
    if want_cpu:
        cpu = cpu_baseline(wl)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "step_us_p10_p50_p90": pct(step_us),
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context_tokens": wl.ctx, "ratio": wl.r,
                   "queries_per_seq": wl.Q, "group": list(wl.group), "replicas": R,
                   "hipgraph": graphs is not None, "steps_per_graph_launch": R if graphs is not None else 0},
        "step_algorithmic_bytes": step_bytes, "step_GBps": round(step_gbps, 1),
        **({"tokens_per_step": 2, "csa2_bytes_per_token_per_sequence": round(step_bytes / 2 / wl.B)}
           if isinstance(wl, Schedule38) else {}),
        "step_frac_of_peak": round(step_gbps / PEAK_GBPS, 4),
        "roofline": roof, "roofline_attention": roof_att, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
