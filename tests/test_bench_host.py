"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the
algorithmic byte counts it prices the roofline with, and the traffic summary
lookup keyed to the profiled kernel's own sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_match_the_block_shapes():
    # per layer: bf16 router + fp32 bias, six routed experts and the shared one
    # (int4 codes + one bf16 scale per 128 inputs), as the scope table counts them
    assert bench.EXPERT_BYTES == 3 * (512 * 2048 // 2 + 512 * 2048 // 128 * 2) == 1622016
    assert bench.SHARED_BYTES == 3 * (1024 * 2048 // 2 + 1024 * 2048 // 128 * 2) == 3244032
    assert bench.LAYER_BYTES == 14025728
    assert bench.TOKEN_BYTES == 47 * 14025728 == 659209216
    assert bench.HEAD_BYTES == 150144 * (1024 + 32)
    assert bench.ATT_BYTES_PER_POS == 2048
    # one batch-1 full attention layer: 100,000 positions of k and v, q and out in fp32, 32 sinks
    assert bench.ATT_CALL_BYTES == 100000 * 2048 + 2 * 32 * 128 * 4 + 32 * 4 == 204832896


def test_traffic_summary_only_counts_for_its_own_sources(tmp_path):
    p = tmp_path / "traffic.txt"
    p.write_text(f"kernel_source_hash: {bench.kernel_source_hash('decode')}\nhbm_bytes_per_launch: 1234\n")
    assert bench.traffic_from_profiles(str(p), "decode") == 1234
    assert bench.traffic_from_profiles(str(p), "head") is None          # another kernel's sources
    assert bench.traffic_from_profiles(str(p), "attn") is None
    p.write_text("kernel_source_hash: 0000000000000000\nhbm_bytes_per_launch: 1234\n")
    assert bench.traffic_from_profiles(str(p), "decode") is None
    assert bench.traffic_from_profiles(str(tmp_path / "missing.txt")) is None


def test_prefill_roofline_takes_the_binding_roof():
    flops = sum(bench.prefill_flops(2048).values())
    moved = bench.ROUTER_BYTES + 256 * bench.EXPERT_BYTES + bench.SHARED_BYTES + 2 * 2048 * 2048 * 4
    r = bench.prefill_roofline(flops, moved, 450e-6)
    # 453 MB at 8 TB/s (56.6 us) outlasts 105 GFLOP at 2.5 PFLOP/s (42.1 us)
    assert r["bound"] == "hbm" and r["other_roof"]["bound"] == "mfma"
    assert abs(r["achieved"] - moved / 450e-6 / 1e9) < 0.1
    assert r["us_at_peak"]["hbm"] > r["us_at_peak"]["mfma"]
    r2 = bench.prefill_roofline(flops * 4, moved, 450e-6)     # four times the flops: the matrix cores bind
    assert r2["bound"] == "mfma" and r2["other_roof"]["bound"] == "hbm"
