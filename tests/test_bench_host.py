"""Host-side checks of bench.py's contract and work model (no GPU): the
multi-GPU refusal, the algorithmic byte and flop counts at the Kimi-K3
shapes against sums written out independently here, and the names under
which the measured kernels are reported."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_workload  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_decode_algorithmic_bytes():
    """T=1, 16 distinct experts: 16 experts' gate, up and down codes (half a
    byte a weight) and exponents (a byte per 32), the two bf16 shared experts,
    the bf16 router, the token in and out."""
    d = get_workload("decode").dims
    per_expert = 3 * 3584 * 2048 // 2 + 3 * 3584 * 2048 // 32
    shared = 2 * 3 * 3584 * 2048 * 2
    router = 3584 * 896 * 2
    io = 2 * 3584 * 2
    want = 16 * per_expert + shared + router + io
    total_bytes, total_flops, st_bytes, _ = bench.algorithmic(d, 16, False)
    assert want == 281_688_064
    assert total_bytes == pytest.approx(want, rel=0, abs=0.5)
    # the per-stage split counts the token once more in each of the router,
    # gate/up and shared gate/up stages, which all read it
    assert sum(st_bytes.values()) == pytest.approx(total_bytes + 2 * 2 * 3584, rel=1e-12)
    # two flops per multiply-add: gate+up+down of 16 routes, 2 shared, router
    assert total_flops == 2 * (16 * 3 * 3584 * 2048 + 2 * 3 * 3584 * 2048 + 3584 * 896)


def test_prefill_algorithmic_flops():
    d = get_workload("prefill").dims
    _, total_flops, _, st_flops = bench.algorithmic(d, 896, False)
    assert st_flops["gate_up"] == 4 * 4096 * 16 * 3584 * 2048 == 1_924_145_348_608
    assert total_flops == 2 * 4096 * (16 * 3 * 3584 * 2048 + 2 * 3 * 3584 * 2048 + 3584 * 896)


def test_reported_kernel_names_match_the_profiled_kernels():
    """The large MXFP4 kernel carries a third template argument when it
    stages the exponent rows in LDS (K/32 a multiple of 16, at most 112): both
    Kimi-K3 GEMMs. Shared experts of up to 64 tokens use 16-row bf16 tiles."""
    d = get_workload("prefill").dims
    assert bench.stage_kernel("gate_up", True, True, d) == "gemm_large_kernel<true, true, true>"
    assert bench.stage_kernel("down", True, True, d) == "gemm_large_kernel<false, true, true>"
    assert bench.stage_kernel("shared_gate_up", True, True, d) == \
        "gemm_large_kernel<true, false, false>"
    assert bench.stage_kernel("shared_down", True, False, d) == "gemm_small_kernel<false>"
    wide = get_workload("prefill").dims.__class__(**{**get_workload("prefill").dims.__dict__, "L": 4096})
    assert bench.stage_kernel("gate_up", True, True, wide) == "gemm_large_kernel<true, true, false>"
    assert bench.stage_kernel("router", True, True, d) == "router_kernel<128>"
    assert bench.stage_kernel("router", True, False, get_workload("batched_decode").dims) == \
        "router_kernel<64>"
    # the router splits K over workgroups only when its tiles are few
    assert bench.stage_kernel("topk", True, True, d) == "topk_kernel<false>"
    assert bench.stage_kernel("topk", True, False, get_workload("batched_decode").dims) == \
        "topk_kernel<true>"
    assert bench.stage_kernel("topk", True, True, get_workload("skewed").dims, True) == \
        "topk_kernel<false>"


def test_stale_traffic_is_not_reported(tmp_path, monkeypatch):
    """Counter traffic taken on other sources of a kernel, or in another
    workload, is not reported; traffic of a kernel whose sources are
    unchanged is, for the workload it was taken in."""
    f = tmp_path / "t.json"
    f.write_text('{"kernels": {"decode_kernel": {"decode": '
                 '{"sources_sha": "0000", "traffic_bytes": 1}}}}')
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("decode_kernel", "decode") is None
    f.write_text('{"kernels": {"decode_kernel": {"decode": '
                 '{"sources_sha": "%s", "traffic_bytes": 7}}}}'
                 % bench.sources_sha("decode_kernel"))
    assert bench.measured_traffic("decode_kernel", "decode") == 7
    assert bench.measured_traffic("decode_kernel", "prefill") is None
    assert bench.measured_traffic("other", "decode") is None


def test_kernel_sources_hash_only_their_files():
    """The decode kernel's hash covers decode.hip and the headers, not the
    grouped path's files; the grouped GEMMs' covers experts.hip."""
    assert bench.sources_sha("decode_kernel") != bench.sources_sha("gemm_large_kernel<true, true, true>")
    assert bench.sources_sha("gemm_large_kernel<true, true, true>") == \
        bench.sources_sha("gemm_small_kernel<true, true, true>")
    assert bench.sources_sha() not in (bench.sources_sha("decode_kernel"),
                                       bench.sources_sha("gemm_large_kernel<true, true, true>"))


def test_quantised_runs_look_up_their_own_counters():
    """Counter summaries of quantised-activation runs are filed under the
    workload name `--extra` gives them (prefill_a4, batched_decode_a8)."""
    w = get_workload("prefill")
    assert bench.traffic_workload({"w": w, "act": "e2m1"}) == "prefill_a4"
    assert bench.traffic_workload({"w": w, "act": "e4m3"}) == "prefill_a8"
    assert bench.traffic_workload({"w": w, "act": "bf16"}) == "prefill"
    assert bench.traffic_workload({"w": w}) == "prefill"
