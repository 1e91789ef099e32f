"""Host-side logic of bench.py that needs no GPU: it refuses more than one GPU,
reports HBM traffic only while the counter record matches the kernel source,
and turns the rocprofv3 counter CSVs into bytes per launch."""
import json
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


def test_percentiles():
    import bench
    assert bench.pct([1.0, 2.0, 3.0, 4.0, 5.0]) == [1.4, 3.0, 4.6]


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    """The committed record's hash matches its kernel source as it is, so its
    bytes are reported; once the source differs the figure is withheld (None)."""
    import bench

    class W:
        name = "f_ri_2ru_b16_ctx128k"

    rec = json.load(open(os.path.join(ROOT, "profiles", "counters_index_full_f_ri_2ru_b16_ctx128k.json")))
    assert bench.traffic_from_profiles(W, "index_full") == rec["hbm_bytes_per_launch"]
    # a copy of the tree whose measured source differs by one byte
    (tmp_path / "profiles").mkdir()
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "profiles" / "counters_index_full_f_ri_2ru_b16_ctx128k.json").write_text(json.dumps(rec))
    src = open(os.path.join(ROOT, "fp4_kv_cache_index_amd", "csrc", rec["source"]), "rb").read()
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc" / rec["source"]).write_bytes(src + b"\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles(W, "index_full") is None

    class Other:
        name = "no_such_workload"

    assert bench.traffic_from_profiles(Other, "index_full") is None


def test_counter_summary(tmp_path, monkeypatch):
    """Two synthetic counter CSVs of a many-query Full call: the last three
    device copies fix the scale factors, the Full call's select is the one with
    the larger grid (it also builds the pool), a Reindex call's kernels are left
    out, and each kernel's mean per dispatch is scaled."""
    import bench
    fields = "Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"

    def rows(counter, values):
        return fields + "".join(f'{i},"{k}",{g},{counter},{v}\n' for i, (k, g, v) in enumerate(values))

    copy = "__amd_rocclr_copyBuffer"
    head = "void csa2::index_shared_head_kernel<1, true>(csa2::SharedHeadArgs)"
    sel = "void csa2::index_select_kernel<false, csa2::SelAll>(csa2::SelectArgs)"
    fetch = [(copy, 4096, 999.0),  # an earlier copy: not a calibration copy
             (head, 270336, 70000.0),
             (head, 270336, 70002.0),
             (sel, 49152, 600.0),     # the Full call's (queries x kinds)
             ("void csa2::index_head_kernel<true>(csa2::HeadArgs)", 131072, 777.0),  # Reindex: left out
             ("void csa2::index_select_kernel<true, csa2::SelAll>(csa2::SelectArgs)", 24576, 12345.0),
             (copy, 65536, 131072.0), (copy, 65536, 131072.0), (copy, 65536, 131072.0)]
    write = [(copy, 4096, 999.0),
             (head, 270336, 9500.0),
             (sel, 49152, 1600.0),
             ("void csa2::index_select_kernel<true, csa2::SelAll>(csa2::SelectArgs)", 24576, 54321.0),
             (copy, 65536, 262144.0), (copy, 65536, 262144.0), (copy, 65536, 262144.0)]
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    f.write_text(rows("FETCH_SIZE", fetch))
    w.write_text(rows("WRITE_SIZE", write))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc" / "index_head.hip").write_bytes(b"// source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.summarize_counters(str(f), str(w), "wl_test", head=False)
    out = json.load(open(tmp_path / "profiles" / "counters_index_full_wl_test.json"))
    assert abs(out["fetch_factor"] - 2.0) < 1e-12 and abs(out["write_factor"] - 1.0) < 1e-12
    assert out["fetch_kib_head"] == 70001.0 and out["fetch_kib_select"] == 600.0
    want = ((70001.0 + 600.0) * 2.0 + (9500.0 + 1600.0)) * 1024
    assert out["hbm_bytes_per_launch"] == round(want)
    assert out["source"] == "index_head.hip" and len(out["source_sha256"]) == 64


def test_counter_summary_decode_kernels(tmp_path, monkeypatch):
    """The decode Full call: index_head plus the Full call's index_select (the
    larger grid: Top-512 and pool); Reindex instantiations are left out."""
    import bench
    fields = "Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"

    def rows(counter, values):
        return fields + "".join(f'{i},"{k}",{g},{counter},{v}\n' for i, (k, g, v) in enumerate(values))

    copy = "__amd_rocclr_copyBuffer"
    fetch = [("void csa2::index_head_kernel<false>(csa2::HeadArgs)", 262144, 70000.0),
             ("void csa2::index_select_kernel<false, csa2::SelAll>(csa2::SelectArgs)", 16384, 900.0),
             ("void csa2::index_head_kernel<true>(csa2::HeadArgs)", 131072, 11000.0),
             ("void csa2::index_select_kernel<true, csa2::SelAll>(csa2::SelectArgs)", 8192, 600.0),
             (copy, 65536, 131072.0), (copy, 65536, 131072.0), (copy, 65536, 131072.0)]
    write = [("void csa2::index_head_kernel<false>(csa2::HeadArgs)", 262144, 800.0),
             ("void csa2::index_select_kernel<false, csa2::SelAll>(csa2::SelectArgs)", 16384, 1000.0),
             ("void csa2::index_head_kernel<true>(csa2::HeadArgs)", 131072, 150.0),
             (copy, 65536, 262144.0), (copy, 65536, 262144.0), (copy, 65536, 262144.0)]
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    f.write_text(rows("FETCH_SIZE", fetch))
    w.write_text(rows("WRITE_SIZE", write))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "fp4_kv_cache_index_amd" / "csrc" / "index_head.hip").write_bytes(b"// source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.summarize_counters(str(f), str(w), "wl_test", head=True)
    out = json.load(open(tmp_path / "profiles" / "counters_index_full_wl_test.json"))
    assert out["fetch_kib_head"] == 70000.0 and out["fetch_kib_select"] == 900.0
    want = ((70000.0 + 900.0) * 2.0 + (800.0 + 1000.0)) * 1024
    assert out["hbm_bytes_per_launch"] == round(want)
    assert out["source"] == "index_head.hip"
