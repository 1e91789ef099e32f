"""Pins of the oracle's attention, quantise-append, window append and the
footprint arithmetic."""
import math

import numpy as np
import pytest
import torch

import synth
from conftest import golden_lines

SM = float(np.float32(1.0 / math.sqrt(512.0)))  # the C-ABI passes the scale as fp32


def _e4m3_lib(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _filled_cache(orc, B, E, cap, cid, ratio=1):
    c = orc.Cache(B, cap, ratio)
    for b in range(B):
        kv = synth.normal_rows(cid, "kv", b * cap, E, 512)
        c.kv_codes[b, :E], c.kv_scales[b, :E] = orc.quantize_main(kv)
        k = synth.normal_rows(cid, "ik", b * cap, E, 64)
        c.ik_codes[b, :E], c.ik_scales[b, :E] = orc.quantize_ik(k)
        c.length[b] = E
    return c


def _textbook(q, keys, scale):
    """softmax(q K^T * scale) K in float64 numpy, q [H][D], keys [N][D]."""
    logits = (q.astype(np.float64) @ keys.T) * scale
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    return (p / l) @ keys, (m + np.log(l))[:, 0]


def test_footprint_890(orc):
    g = {l.split()[0]: int(l.split()[1]) for l in golden_lines("footprint.txt")}
    assert orc.main_entry_bytes() == 288
    assert orc.indexer_entry_bytes() == 68
    assert orc.footprint_bytes_per_token() == g["v41_flash"]
    assert round(g["v4_flash"] / orc.footprint_bytes_per_token()) == 4  # "roughly 1/4"
    assert round(g["v1"] / orc.footprint_bytes_per_token()) == g["ratio_v1_over_v41"]


@pytest.mark.parametrize("E,p", [(5, 4), (300, 299), (512, 511)])
def test_dense_special_case(orc, E, p):
    """With at most 512 visible entries Top-512 selects all of them, so the
    result is textbook dense softmax attention over every entry plus the window."""
    B, cap, S = 1, 600, 256
    c = _filled_cache(orc, B, E, cap, 80)
    iq = synth.normal(80, "iq", (1, 1, 4, 64))
    topk, _, _ = orc.index_topk(c, orc.FULL, iq)
    assert np.array_equal(topk[0, 0][:E], np.arange(E))
    swa = np.zeros((B, S, 512), np.uint8)
    xs = synth.normal(80, "swa", (B, p + 1, 512))
    orc.swa_append(swa, xs, np.array([p + 1], np.int32))
    q = _bf16(synth.normal(80, "q", (B, 1, 16, 512)))
    out, lse = orc.attend(c, topk, swa, q, SM)
    main = orc.dequant_main(c.kv_codes[0, :E], c.kv_scales[0, :E])
    lo = max(0, p - 127)
    win = _e4m3_lib(swa[0, [t % S for t in range(lo, p + 1)]])
    keys = np.concatenate([main, win])
    ref, ref_lse = _textbook(q[0, 0], keys, SM)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=1e-12, atol=1e-12)


def test_single_key_returns_that_key(orc):
    B, cap, S = 1, 8, 128
    c = orc.Cache(B, cap, 1)
    topk = np.full((1, 1, 512), -1, np.int32)
    swa = np.zeros((1, S, 512), np.uint8)
    x = synth.normal(81, "one", (1, 1, 512))
    orc.swa_append(swa, x, np.array([1], np.int32))  # token 0 only
    q = _bf16(synth.normal(81, "q1", (1, 1, 16, 512)))
    out, lse = orc.attend(c, topk, swa, q, SM, q_pos=np.array([[0]], np.int32))
    key = _e4m3_lib(swa[0, 0])
    for h in range(16):
        assert np.array_equal(out[0, 0, h], key)
        assert lse[0, 0, h] == pytest.approx(SM * float(q[0, 0, h].astype(np.float64) @ key), rel=1e-13)


def test_lse_merge_identity(orc):
    """Attention over (A u W) and (B u W) and W alone recombines into (A u B u W)."""
    B, E, cap, S = 1, 3000, 3000, 128
    c = _filled_cache(orc, B, E, cap, 82)
    iq = synth.normal(82, "iq", (1, 1, 4, 64))
    topk, _, _ = orc.index_topk(c, orc.FULL, iq)
    swa = np.zeros((1, S, 512), np.uint8)
    orc.swa_append(swa, synth.normal(82, "w", (1, S, 512)), np.array([E], np.int32))
    q = _bf16(synth.normal(82, "q", (1, 1, 16, 512)))
    none = np.full_like(topk, -1)
    ta, tb = none.copy(), none.copy()
    ta[0, 0, :200] = topk[0, 0, :200]
    tb[0, 0, :312] = topk[0, 0, 200:]
    o, l = orc.attend(c, topk, swa, q, SM)
    oa, la = orc.attend(c, ta, swa, q, SM)
    ob, lb = orc.attend(c, tb, swa, q, SM)
    ow, lw = orc.attend(c, none, swa, q, SM)
    m = np.maximum(np.maximum(la, lb), lw)
    tot = np.exp(la - m) + np.exp(lb - m) - np.exp(lw - m)
    np.testing.assert_allclose(np.log(tot) + m, l, rtol=1e-12)
    num = (oa * np.exp(la - m)[..., None] + ob * np.exp(lb - m)[..., None] - ow * np.exp(lw - m)[..., None])
    np.testing.assert_allclose(num / tot[..., None], o, rtol=1e-9, atol=1e-12)


def test_window_is_last_128_tokens_of_the_ring(orc):
    B, cap, S, p = 1, 8, 256, 300
    c = orc.Cache(B, cap, 1)
    topk = np.full((1, 1, 512), -1, np.int32)
    swa = np.zeros((1, S, 512), np.uint8)
    xs = synth.normal(83, "win", (1, p + 1, 512))
    orc.swa_append(swa, xs, np.array([p + 1], np.int32))
    # token 172 (outside the window) was overwritten in the ring by token 172+256?
    # no: 428 > p, so slot 172 still holds token 172 and must be ignored
    swa[0, 172 % S] = 0x7E  # 448 everywhere: would dominate if it were read
    q = _bf16(synth.normal(83, "q", (1, 1, 16, 512)))
    out, lse = orc.attend(c, topk, swa, q, SM, q_pos=np.array([[p]], np.int32))
    keys = _e4m3_lib(swa[0, [t % S for t in range(p - 127, p + 1)]])
    ref, ref_lse = _textbook(q[0, 0], keys, SM)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=1e-12)


def test_swa_append_ring_slots(orc):
    S = 128
    swa = np.zeros((2, S, 512), np.uint8)
    x = synth.normal(84, "x", (2, 3, 512))
    orc.swa_append(swa, x, np.array([130, 3], np.int32))
    # sequence 0: tokens 127, 128, 129 -> slots 127, 0, 1; sequence 1: tokens 0, 1, 2
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(swa[0, [127, 0, 1]], ref[0])
    assert np.array_equal(swa[1, [0, 1, 2]], ref[1])
    assert not swa[0, 2:127].any()


def test_quantize_append_positions_and_capacity(orc):
    B, cap = 2, 10
    c = orc.Cache(B, cap, 1)
    c.length[:] = [3, 7]
    kv = synth.normal(85, "kv", (B, 3, 512))
    ik = synth.normal(85, "ik", (B, 3, 64))
    orc.quantize_append(c, kv, ik)
    assert list(c.length) == [6, 10]
    for b, l0 in ((0, 3), (1, 7)):
        codes, scales = orc.quantize_main(kv[b])
        assert np.array_equal(c.kv_codes[b, l0:l0 + 3], codes)
        assert np.array_equal(c.kv_scales[b, l0:l0 + 3], scales)
        ic, isc = orc.quantize_ik(ik[b])
        assert np.array_equal(c.ik_codes[b, l0:l0 + 3], ic)
        assert np.array_equal(c.ik_scales[b, l0:l0 + 3], isc)
    with pytest.raises(orc.OracleError):
        orc.quantize_append(c, kv[:, :1], ik[:, :1])


def test_ratio2_compression_special_cases(orc):
    x = synth.normal(86, "x", (4, 512))
    # equal logits: the mean of the two tokens
    z = np.zeros((4, 512), np.float32)
    out = orc.compress_pairs(x, z)
    np.testing.assert_array_equal(out, ((x[0::2].astype(np.float64) + x[1::2]) / 2).astype(np.float32))
    # a decisive logit gap selects one token (exp(-200) underflows relative to 1)
    z2 = np.zeros((4, 512), np.float32)
    z2[0::2] = 200.0
    z2[1::2, :256] = 400.0
    z2[1::2, 256:] = -400.0
    out2 = orc.compress_pairs(x, z2)
    np.testing.assert_array_equal(out2[:, :256], x[1::2, :256])
    np.testing.assert_array_equal(out2[:, 256:], x[0::2, 256:])
    # shift invariance of the softmax (logits on a 2^-10 grid so the shift is exact)
    z3 = np.round(synth.normal(86, "z", (4, 512)) * 1024) / 1024
    np.testing.assert_array_equal(orc.compress_pairs(x, z3), orc.compress_pairs(x, z3 + 3.0))


def test_ratio2_append_uses_pairs(orc):
    B, cap, T = 1, 16, 8
    c = orc.Cache(B, cap, 2)
    kv = synth.normal(87, "kv", (B, T, 512))
    lg = synth.normal(87, "lg", (B, T, 512))
    ik = synth.normal(87, "ik", (B, T // 2, 64))
    orc.quantize_append(c, kv, ik, logits=lg)
    assert c.length[0] == 4
    comp = orc.compress_pairs(kv[0], lg[0])
    codes, scales = orc.quantize_main(comp)
    assert np.array_equal(c.kv_codes[0, :4], codes) and np.array_equal(c.kv_scales[0, :4], scales)
    with pytest.raises(orc.OracleError):
        orc.quantize_append(c, kv[:, :3], ik[:, :1], logits=lg[:, :3])  # T % r != 0
