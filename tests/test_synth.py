"""The seeded input generators both sides draw from: any row range of a host
tensor regenerates identically, chunk boundaries included; device rows are
reproduced per call and per whole chunk; distinct tags and workloads give
distinct streams."""
import zlib

import numpy as np
import torch

import synth


def test_row_ranges_regenerate_identically():
    C = synth.CHUNK_ROWS
    whole = synth.normal_rows(5, "rows", 0, 2 * C + 100, 3)
    for r0, n in [(0, 10), (C - 7, 20), (C, 5), (2 * C - 1, 101), (123, C + 50)]:
        assert np.array_equal(synth.normal_rows(5, "rows", r0, n, 3), whole[r0:r0 + n]), (r0, n)


def test_device_rows_per_call_and_per_chunk():
    """The torch-side generator (used for the large fills) on the CPU device.
    torch's normal draws are not prefix-consistent across draw sizes, so a
    row range is reproduced by the same call, and a whole chunk by any call
    that covers it; a partial range drawn alone may differ.  That is why the
    oracle side receives host copies of device rows instead of redrawing."""
    C = synth.CHUNK_ROWS
    a = synth.torch_normal_rows(5, "dev", 100, C + 40, 2, device="cpu")
    assert torch.equal(a, synth.torch_normal_rows(5, "dev", 100, C + 40, 2, device="cpu"))
    whole_first = synth.torch_normal_rows(5, "dev", 0, C, 2, device="cpu")
    assert torch.equal(synth.torch_normal_rows(5, "dev", 0, 2 * C, 2, device="cpu")[:C], whole_first)
    assert not torch.equal(whole_first[:40], synth.torch_normal_rows(5, "dev", C, 40, 2, device="cpu"))


def test_streams_are_distinct_and_deterministic():
    a = synth.normal(1, "a", (4, 8))
    assert np.array_equal(a, synth.normal(1, "a", (4, 8)))
    assert not np.array_equal(a, synth.normal(1, "b", (4, 8)))
    assert not np.array_equal(a, synth.normal(2, "a", (4, 8)))
    assert synth.tag_id("kv") == zlib.crc32(b"kv") & 0x7FFFFFFF
    s = synth.normal_rows(3, "big", 0, 20000, 64)
    assert abs(float(s.mean())) < 0.01 and abs(float(s.std()) - 1.0) < 0.01  # N(0, 1)
