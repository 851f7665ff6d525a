"""The benchmark's host-side contract, without a GPU: workload table, algorithmic byte counts, the committed
HBM-traffic summaries it reads, and the refusal of more than one GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_workload_table():
    names = ["qwen3-moe-t%d" % t for t in (1, 8, 64, 512)] + ["kimi-moe-t%d" % t for t in (1, 64, 256)] + \
            ["deepseek-moe-t%d" % t for t in (1, 32, 512, 4096)] + ["kimi-prefill-t8192"]
    for name in names:
        spec = bench.workload_spec(name)
        assert spec["name"] == name and spec.get("fmt", "int4") == "int4"
        mx = bench.workload_spec(name + "-mxfp4")
        assert mx["fmt"] == "mxfp4" and (mx["E"], mx["H"], mx["I"], mx["T"]) == (spec["E"], spec["H"], spec["I"],
                                                                                spec["T"])
    # expert-parallel shares state the global expert count their plans are hinted with
    assert bench.workload_spec("kimi-moe-t256")["global_experts"] == 384
    assert "global_experts" not in bench.workload_spec("qwen3-moe-t64")
    with pytest.raises(SystemExit):
        bench.workload_spec("no-such-workload")


def test_packed_weight_bytes():
    # 16-row x 256-k superblocks: 2304 bytes (INT4 codes + BF16 scales), 2176 (E2M1 codes + E8M0 scales)
    assert bench.packed_weight_bytes(16, 256) == 2304
    assert bench.packed_weight_bytes(16, 256, "mxfp4") == 2176
    assert bench.packed_weight_bytes(4096, 7168) == 4096 * 7168 * 9 // 16
    assert bench.packed_weight_bytes(4096, 7168, "mxfp4") == 4096 * 7168 * 17 // 32
    assert bench.packed_weight_bytes(17, 288) == 2 * 2 * 2304  # ragged shapes pad to whole superblocks


def test_committed_traffic_summaries_are_well_formed():
    """Every committed HBM-traffic summary names its workload and the hash of the kernel sources it was taken
    with; bench.py reports the figure only while the hash matches the sources (null otherwise), and a current
    decode figure lies near the algorithmic bytes."""
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "gate_up_silu_*_hbm_traffic.md")))
    assert paths
    for path in paths:
        workload = os.path.basename(path)[len("gate_up_silu_"):-len("_hbm_traffic.md")]
        spec = bench.workload_spec(workload)
        text = open(path).read()
        assert "workload: %s\n" % workload in text and "kernel_sources_sha256:" in text, path
        assert "traffic_bytes_per_launch:" in text and "rocprofv3" in text, path
        family = "prefill" if workload in ("deepseek-moe-t4096", "deepseek-moe-t4096-mxfp4",
                                           "kimi-prefill-t8192", "kimi-prefill-t8192-mxfp4") else "decode"
        traffic = bench.committed_traffic(workload, family)
        if traffic is not None and family == "decode":
            alg = bench.gate_up_algorithmic_bytes(spec)
            assert 0.95 * alg <= traffic <= 1.2 * alg, (workload, traffic, alg)


def test_stale_traffic_summary_is_not_reported(tmp_path, monkeypatch):
    """A summary taken with other kernel sources gives no traffic figure."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "workload: qwen3-moe-t64\nkernel_sources_sha256: %s\ntraffic_bytes_per_launch: 123\n"
    (prof / "gate_up_silu_qwen3-moe-t64_hbm_traffic.md").write_text(body % bench.kernel_sources_sha256("decode"))
    src = tmp_path / "weight_only_int4_amd" / "csrc"
    src.mkdir(parents=True)
    for rel in bench.KERNEL_SOURCES["decode"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            (tmp_path / rel).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_traffic("qwen3-moe-t64", "decode") == 123
    (tmp_path / bench.KERNEL_SOURCES["decode"][0]).write_bytes(b"// changed\n")
    assert bench.committed_traffic("qwen3-moe-t64", "decode") is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_roofline_bound_follows_arithmetic_intensity():
    """The reported roofline is the longer minimum time, bytes at the HBM peak or flops at the matrix peak (the
    ridge sits near 88 routed rows per expert), whichever kernel the plan runs: decode at 4 rows per expert
    and the prefill kernel at 16 rows stream weights, 128 rows per expert and the Kimi-K2 prefill share are
    matrix-bound."""
    for name, want in (("qwen3-moe-t64", "hbm"), ("deepseek-moe-t512", "hbm"), ("deepseek-moe-t512-mxfp4", "hbm"),
                       ("deepseek-moe-t4096", "mfma"), ("kimi-prefill-t8192", "mfma")):
        bound, nbytes, flops = bench.roofline_bound(bench.workload_spec(name))
        assert bound == want, (name, nbytes, flops)
