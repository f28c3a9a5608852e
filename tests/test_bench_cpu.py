"""Host logic of bench.py: the rocprofv3 counter and trace summaries (CPU only)."""
import csv
import json
import os

import bench


def write_rows(path, rows, fields):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def kernel_rows(counter, per_kernel):
    rows = []
    for (name, grid), vals in per_kernel.items():
        for v in vals:
            rows.append({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": v})
    return rows


def test_counter_summary_calibrates_against_the_copy(tmp_path):
    assert bench.C % 64 == 0          # the names below are those of the 64-token attention tile
    enc_grid = bench.OP_KERNELS["encode"][0][1]
    gib_kib = (1 << 30) / 1024
    fetch = {("hbm_probe::k_probe_copy(unsigned int const*)", 2097152): [gib_kib / 2] * 3,
             (f"void lynx::k_encode<{bench.C}, false>(lynx::EncodeArgs)", enc_grid): [1000.0, 1002.0],
             (f"void lynx::k_encode<{bench.C}, false>(lynx::EncodeArgs)", enc_grid // 2): [7.0],   # setup encode, ignored
             ("void lynx::k_decode<false, false>(lynx::DecodeArgs)", bench.OP_KERNELS["decode_anchor"][0][1]): [10.0],
             ("void lynx::k_decode<true, false>(lynx::DecodeArgs)", bench.OP_KERNELS["decode_full"][0][1]): [20.0],
             ("void lynx::k_attn_anchor<64, 1, 8, 12>(lynx::AttnArgs)", 4096): [30.0],
             ("lynx::k_attn_combine(lynx::AttnArgs)", 131072): [1.0],
             ("void lynx::k_verify<1>(lynx::(anonymous namespace)::VerifyArgs)", 131072): [40.0],
             ("lynx::k_verify_combine(lynx::(anonymous namespace)::VerifyArgs)", 8388608): [2.0]}
    write = {k: [v[0] * 2 for _ in v] for k, v in fetch.items()}
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    write_rows(fp, kernel_rows("FETCH_SIZE", fetch), fields)
    write_rows(wp, kernel_rows("WRITE_SIZE", write), fields)
    text = bench.counter_summary(str(fp), str(wp), str(out))
    rec = json.loads(out.read_text())
    assert abs(rec["calibration"]["fetch_factor"] - 2.0) < 1e-9
    assert abs(rec["calibration"]["write_factor"] - 1.0) < 1e-9
    assert rec["encode"]["bytes_per_launch"] == round(1001.0 * 1024 * 2 + 2000.0 * 1024 * 1)
    assert rec["attn_anchor"]["bytes_per_launch"] == round(31.0 * 1024 * 2 + 62.0 * 1024)
    assert rec["attn_verify"]["bytes_per_launch"] == round(42.0 * 1024 * 2 + 84.0 * 1024)
    assert rec["copy"]["bytes_per_launch"] == 2 << 30
    assert rec["encode"]["source_hash"] == bench.kernel_hash()
    assert "encode" in text and "calibration" in text


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    xyz = {"Grid_Size_X": 4096, "Grid_Size_Y": 128, "Grid_Size_Z": 1,
           "Workgroup_Size_X": 256, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1}
    rows = [dict(Kernel_Name="void lynx::k_decode<true, false>(lynx::DecodeArgs)", Start_Timestamp=1000,
                 End_Timestamp=1000 + d, **xyz) for d in (600000, 700000)]
    rows.append(dict(Kernel_Name="at::native::foo(int)", Start_Timestamp=0, End_Timestamp=5, **xyz))
    p = tmp_path / "k.csv"
    write_rows(p, rows, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"] + list(xyz))
    text = bench.trace_summary(str(p))
    assert "at::native" not in text
    line = [ln for ln in text.splitlines() if "k_decode" in ln][0].split()
    assert line[-6:-4] == ["524288", "256"]
    assert line[-4:] == ["2", "650.0", "600.0", "700.0"]


def test_load_traffic_rejects_a_stale_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({"encode": {"source_hash": "stale", "bytes_per_launch": 5},
                                                   "decode_full": {"source_hash": bench.kernel_hash(),
                                                                   "bytes_per_launch": 7}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: json.loads((prof / "traffic.json").read_text())
                        ["decode_full"]["source_hash"])
    assert bench.load_traffic("encode") is None
    assert bench.load_traffic("decode_full") == 7
    assert bench.load_traffic("attn_anchor") is None


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why, before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_codec_workloads_are_valid_shapes():
    """Every shape the codec-workloads report times is one the library accepts: whole pages,
    chunks that divide the page, and a segment size the oracle agrees with."""
    from decode_attention_lynx_amd import lynx
    from oracle import lynx_oracle as o
    for name, layers, tokens, kvh, pt, seed, settings, per_tensor in bench.CODEC_WORKLOADS:
        assert tokens % pt == 0 and layers > 0 and kvh > 0, name
        for c_, al in settings:
            assert pt % c_ == 0 and c_ in (8, 16, 32, 64, 128, 256) and al > 0, (name, c_)
            assert lynx.stream_sizes(pt, kvh, 128, c_) == o.segment_bytes(pt, kvh, 128, c_)


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """The counters' source hash survives a comment-only edit and changes with the code."""
    import shutil
    for s in bench.KERNEL_SOURCES:
        (tmp_path / s).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, s), tmp_path / s)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_hash()
    src = tmp_path / bench.KERNEL_SOURCES[0]
    text = src.read_text()
    src.write_text("// a comment line\n\n" + text.replace("\n", "   // trailing note\n", 1))
    assert bench.kernel_hash() == h0
    src.write_text(text.replace("kTileTokens", "kTileTokens + 0", 1))
    assert bench.kernel_hash() != h0


def test_cpu_baseline_reports_its_workers():
    """The oracle baseline runs one single-threaded worker per host core (at most 16) and
    states the core count and the sample it timed."""
    rec = bench.cpu_baseline(cpu_seconds=0.1)
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    assert rec["cores"] == n and rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and f"{n} single-threaded worker processes" in rec["sample"]


def test_util_summary_averages_every_counter_per_kernel(tmp_path):
    rows = kernel_rows("MfmaUtil", {("void lynx::k_verify<1>(lynx::VerifyArgs)", 131072): [30.0, 40.0]})
    rows += kernel_rows("VALUBusy", {("void lynx::k_verify<1>(lynx::VerifyArgs)", 131072): [50.0, 54.0],
                                     ("void lynx::k_decode<false, false>(lynx::DecodeArgs)", 16777216): [49.0]})
    rows += kernel_rows("VALUBusy", {("at::native::foo(int)", 64): [1.0]})
    p = tmp_path / "u.csv"
    write_rows(p, rows, ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
    text = bench.util_summary(str(p)).splitlines()
    assert text[0].split()[2:] == ["MfmaUtil", "VALUBusy"]
    assert not any("at::native" in ln for ln in text)
    ver = [ln for ln in text if "k_verify" in ln][0].split()
    assert ver[-3:] == ["131072", "35", "52"]
    dec = [ln for ln in text if "k_decode" in ln][0].split()
    assert dec[-2:] == ["nan", "49"]


def test_every_default_op_has_its_byte_and_flop_counts():
    """Each op the bench runs by default (the step and beyond it) has algorithmic bytes and
    elements, and the compute-bound ones their flops, so no report line divides by nothing."""
    next_ops = [o for o in bench.NEXT_OPS if o not in ("codec_two_streams", "encode_to_host")]
    assert {"attn_anchor_c32", "attn_anchor_paged", "attn_verify", "attn_verify_paged"} <= set(next_ops)
    for op in list(bench.STEP_OPS) + next_ops:
        assert bench.alg_bytes_per_elem(op) > 0 and bench.op_elems(op) > 0, op
    for op in ("attn_verify", "attn_verify_paged"):
        assert bench.op_flops(op) == 4.0 * bench.AB * bench.AM * bench.AHQ * bench.AT * bench.D


def test_workload_counter_summary_rates_the_codec_dispatches(tmp_path):
    """Per (kernel, grid) HBM bytes of the codec-workload counter runs against G * 64 elements of
    algorithmic bytes, with the copy calibration of profiles/traffic.json."""
    cal = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic.json")))["calibration"]
    grid = 4194304                                   # a 2.15 GB request: 268 M elements
    alg_enc = (3.0 + 8.0 / 64 + 8.0 / 256) * grid * 64
    fetch = {("void lynx::k_encode<64, false>(lynx::EncodeArgs)", grid):
             [alg_enc * 2 / 3 / 1024 / cal["fetch_factor"]] * 2,
             ("void lynx::k_decode<true, false>(lynx::DecodeArgs)", grid): [1.0],
             ("void lynx::k_page_finish(lynx::EncodeArgs)", 2048): [3.0]}
    write = {("void lynx::k_encode<64, false>(lynx::EncodeArgs)", grid):
             [alg_enc / 3 / 1024 / cal["write_factor"]] * 2,
             ("void lynx::k_decode<true, false>(lynx::DecodeArgs)", grid): [2.0],
             ("void lynx::k_page_finish(lynx::EncodeArgs)", 2048): [1.0]}
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    write_rows(fp, kernel_rows("FETCH_SIZE", fetch), fields)
    write_rows(wp, kernel_rows("WRITE_SIZE", write), fields)
    lines = bench.workload_counter_summary(str(fp), str(wp), chunk=64).splitlines()
    enc = [ln for ln in lines if "k_encode<64" in ln][0].split()
    assert enc[-1] == "1.0000" and int(enc[-2]) == round(alg_enc)
    dec = [ln for ln in lines if "k_decode<true" in ln][0].split()
    assert int(dec[-2]) == round((3.0 + 8.0 / 64 + 8.0 / 256) * grid * 64)
    fin = [ln for ln in lines if "k_page_finish" in ln][0].split()
    assert fin[-1] == "-"
