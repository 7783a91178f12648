"""Host-side logic of bench.py, without a GPU: the algorithmic byte count the
roofline divides by, the one-GPU guard, and the scaling of the HBM counters
by a copy of known size."""
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_headline_launch():
    """64 requests x 16384 tokens, 64 query / 8 KV heads, D = 128, 64-token
    pages, e4m3: the sum written out term by term."""
    B, L, Hq, Hkv, D, P = 64, 16384, 64, 8, 128, 64
    kv = B * L * Hkv * D * 2 * 1          # K and V, one byte per element
    table = B * (L // P) * 4              # one int32 page id per page
    q = B * Hq * D * 2                    # bf16 queries
    out = B * Hq * (D + 1) * 4            # fp32 out and lse
    small = 2 * Hkv * 4 + B * 4 + B * 4   # scales, lengths, status
    assert bench.algorithmic_bytes([L] * B, Hq, Hkv, D, P, 1) == kv + table + q + out + small
    assert bench.algorithmic_bytes([L] * B, Hq, Hkv, D, P, 1) == 2150711872
    # bf16 doubles only the KV term; no status without a check
    assert (bench.algorithmic_bytes([L] * B, Hq, Hkv, D, P, 2, checked=False)
            == 2 * kv + table + q + out + 2 * Hkv * 4 + B * 4)
    # a ragged batch counts its own pages (a partial last page is one entry)
    assert bench.algorithmic_bytes([1, 65], 8, 1, 64, 64, 1, checked=False) == \
        (66 * 64 * 2) + 3 * 4 + 2 * 8 * 64 * 2 + 2 * 8 * 65 * 4 + 8 + 8


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def _counter_dir(path, rows):
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy(tmp_path):
    """FETCH_SIZE and WRITE_SIZE (KiB) of one preset's kernel, each scaled by
    known bytes / counted bytes of a 1 GiB copy; the median launch counts;
    other kernels' rows are ignored; the summary states the algorithmic bytes."""
    preset = "decode_attn_e4m3_gqa8_16k_b64"
    attn = "void pafp8::(anonymous namespace)::" + bench.COUNTER_PRESETS[preset]["kernel"] + "(pafp8::AttnParams)"
    pmc = tmp_path / "pmc"
    _counter_dir(pmc / f"{preset}_fetch", [(attn, "FETCH_SIZE", v) for v in (1000.0, 1100.0, 1050.0)]
                 + [("other_kernel", "FETCH_SIZE", 9e9)])
    _counter_dir(pmc / f"{preset}_write", [(attn, "WRITE_SIZE", v) for v in (10.0, 12.0, 11.0)])
    gib_kib = (1 << 30) / 1024.0
    _counter_dir(pmc / "copy_fetch", [("copyBuffer", "FETCH_SIZE", gib_kib / 2), ("copyBuffer", "FETCH_SIZE", 4.0)])
    _counter_dir(pmc / "copy_write", [("copyBuffer", "WRITE_SIZE", gib_kib)])
    out = tmp_path / "summary.md"
    bench.summarize_counters(preset, str(pmc), str(out))
    vals = dict(line.split(":", 1) for line in out.read_text().splitlines()
                if ":" in line and not line.startswith(" "))
    # fetch counts half the copy's bytes -> factor 2; write counts them all -> factor 1
    assert float(vals["fetch_bytes_per_launch"]) == 1050.0 * 1024 * 2
    assert float(vals["write_bytes_per_launch"]) == 11.0 * 1024
    assert float(vals["traffic_bytes_per_launch"]) == 1050.0 * 1024 * 2 + 11.0 * 1024
    assert int(vals["algorithmic_bytes_per_launch"]) == 2150711872
    assert bench.read_traffic(str(out)) == 1050.0 * 1024 * 2 + 11.0 * 1024
    # figures taken on other sources are not used
    out.write_text(out.read_text().replace(vals["source_hash"].strip(), "0" * 16))
    assert bench.read_traffic(str(out)) is None


def test_counter_presets_name_their_bytes():
    """Every preset has algorithmic bytes from its workload definition (host
    only): the INT4 and hand-off figures written out, the others positive."""
    assert bench._preset_bytes("int4_gemv_28672x8192_m64") == \
        28672 * 8192 // 2 + 64 * 28672 * 2 + 64 * 8192 * 2 + 64 * 28672 * 4
    assert bench._preset_bytes("kv_fill_e4m3_handoff_8k_b8") == \
        2 * 8 * 8192 * 8 * 128 * 3 + 8 * 128 * 4 + 2 * 8 * 4 + 2 * 8 * 4
    for name in bench.COUNTER_PRESETS:
        assert bench._preset_bytes(name) > 0, name
    # the long-context preset counts the clean batch of four 256k-token requests
    assert bench._preset_bytes("decode_attn_wave_e4m3_gqa8_256k_b4_s64") == \
        bench.algorithmic_bytes([262144] * 4, 64, 8, 128, 64, 1)


def test_kernel_stats_summary(tmp_path):
    """The kernel-trace summary keeps the library's kernels only, names them
    without namespace and arguments, and divides the headline's algorithmic
    bytes by its average duration."""
    d = tmp_path / "stats" / "host"
    d.mkdir(parents=True)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["void pafp8::(anonymous namespace)::decode_attn_mfma_kernel<false, 128, true, false, "
                    "true>(pafp8::AttnParams)", 25, 8000000, 320000, 90, 310000, 330000, 1])
        w.writerow(["void pafp8::(anonymous namespace)::tag_check_kernel(int, int)", 25, 100000, 4000, 1,
                    3000, 5000, 1])
        w.writerow(["at::native::reduce_kernel<512, 1>(...)", 3, 600000, 200000, 9, 1, 2, 0])
    out = tmp_path / "summary.md"
    bench.summarize_kernel_stats("decode_attn_e4m3_gqa8_16k_b64", str(tmp_path / "stats"), str(out))
    text = out.read_text()
    assert "| decode_attn_mfma_kernel<false, 128, true, false, true> | 25 | 320000 |" in text
    assert "| tag_check_kernel | 25 | 4000 |" in text
    assert "reduce_kernel" not in text
    alg = bench._preset_bytes("decode_attn_e4m3_gqa8_16k_b64")
    assert f"achieved_GBps: {alg / 320000:.1f}" in text
