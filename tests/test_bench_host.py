"""Host-side checks of the benchmark's measurement code (no GPU): the
one-GPU guard, the decode-step byte count, the parity statistics and the
reduction of rocprofv3 counter files into per-launch HBM traffic."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_decode_step_bytes_by_hand():
    """Depth-12 shape, 32 sequences at mean length 600: the block and LM-head
    weights once, 32 rows of the embedding, K and V of 601 positions per
    sequence and layer read, one position written, the fp32 logits twice."""
    m = wl.depth_model(12)
    d, F, V = 768, 3072, 65536
    per_layer = d * d + 128 * d + 128 * d + d * d + F * d + d * F
    weights = 2 * (12 * per_layer + V * d) + 2 * 32 * d
    kv_read = 12 * 32 * 601 * 2 * 128 * 2
    kv_write = 12 * 32 * 2 * 128 * 2
    logits = 2 * 32 * V * 4
    assert bench.step_bytes(m, 32, 600.0, V) == weights + kv_read + kv_write + logits


def test_parity_stats_on_a_worked_case():
    ref = np.array([[0.0, 1.0, 0.5], [2.0, 0.0, 1.9], [0.0, 0.0, 3.0]])
    gpu = ref + np.array([[0.01, -0.02, 0.0], [0.0, 0.0, 0.15], [0.0, 0.04, 0.0]])
    st = bench.parity_stats(gpu, ref)
    assert st["rows"] == 3
    assert st["max_abs"] == pytest.approx(0.15)
    # row 1: the GPU's argmax (column 2, 2.05) differs from the oracle's (column 0)
    assert st["top1"] == pytest.approx(2 / 3, abs=1e-5)
    assert st["literal_max_met"] is False and st["literal_top1_met"] is False
    d = (gpu - ref).ravel()
    assert st["std"] == pytest.approx(float(np.std(d)), abs=1e-6)
    # the same rows split into blocks, with the chosen tokens given explicitly
    st2 = bench.parity_stats([gpu[:2], gpu[2:]], [ref[:2], ref[2:]], chosen=[[1, 0], [2]])
    assert st2["rows"] == 3 and st2["top1"] == pytest.approx(1.0)
    assert st2["max_abs"] == st["max_abs"]


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_known_copies(tmp_path):
    """Two prefills of 49 GEMM launches (the second counted), then the two
    copies of 1 GiB.  FETCH_SIZE is made to read half of the elementwise
    copy's 512 MiB source, WRITE_SIZE all of its 1 GiB output, so the factors
    are 2 and 1; every counted launch reads 1000 KiB and writes 300 KiB."""
    gemm = "void (anonymous namespace)::gemm_pp_kernel<256, 256, 2>(GemmArgs)"
    elem = "void at::native::vectorized_elementwise_kernel<4, at::native::float16tofloat32_copy_kernel>"
    blit = "__amd_rocclr_copyBuffer"
    fetch = [(gemm, 5.0)] * 49 + [(gemm, 1000.0)] * 49 + [(elem, 262144.0), (blit, 524288.0)]
    write = [(gemm, 7.0)] * 49 + [(gemm, 300.0)] * 49 + [(elem, 1048576.0), (blit, 1048576.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_counter_csv(fp, "FETCH_SIZE", fetch)
    _write_counter_csv(wp, "WRITE_SIZE", write)
    bench.summarize_traffic(str(fp), str(wp), str(out))
    t = json.loads(out.read_text())
    assert t["fetch"]["factor"] == pytest.approx(2.0)
    assert t["write"]["factor"] == pytest.approx(1.0)
    assert t["fetch"]["launches"] == 49 and t["write"]["launches"] == 49
    assert t["bytes_per_launch"] == pytest.approx((1000.0 * 2.0 + 300.0) * 1024.0)
    assert t["gemm_sources_sha256"] == bench.gemm_source_hash()


class _FakeProfile:
    """Stands in for the binding's profile reads with given launch records."""
    PROF_CLASSES = {"gemm": 0, "lmhead": 1}

    def __init__(self, recs):
        self.recs = recs

    def gpt_profile_read(self, cls):
        return {"launches": len(self.recs[cls])}

    def gpt_profile_read_launch(self, cls, i):
        return self.recs[cls][i]


def test_gemm_by_shape_tells_the_prefill_products_apart():
    """Depth-12 launches in layer order, twice, then the LM head: each is named
    by its flops and bytes (W1 and W2 differ only in bytes), and a shape's
    TFLOP/s is its flops over its summed time."""
    m, M = wl.depth_model(12), 16384

    def rec(N, K, out_b, ms):
        return {"ms": ms, "flops": 2.0 * M * N * K, "bytes": 2.0 * (M * K + N * K) + out_b * M * N}
    layer = [rec(1024, 768, 2, 0.040), rec(768, 768, 8, 0.030), rec(3072, 768, 2, 0.080), rec(768, 3072, 8, 0.090)]
    shapes = bench.gemm_by_shape(_FakeProfile({0: layer * 2, 1: [rec(65536, 768, 4, 2.0)]}), m, M)
    assert set(shapes) == {"qkv", "o", "w1", "w2", "lm_head"}
    assert (shapes["w1"]["N"], shapes["w1"]["K"]) == (3072, 768)
    assert (shapes["w2"]["N"], shapes["w2"]["K"]) == (768, 3072)
    assert shapes["w2"]["launches"] == 2 and shapes["w2"]["us_per_launch"] == pytest.approx(90.0)
    assert shapes["lm_head"]["achieved_tflops"] == pytest.approx(2.0 * M * 65536 * 768 / 2e-3 / 1e12, rel=1e-3)
    assert shapes["o"]["frac"] == pytest.approx(2.0 * M * 768 * 768 / 30e-6 / 1e12 / 2500.0, rel=1e-3)


def test_code_identity_ignores_comments_and_layout_only():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* result */\n}\n"
    b = "// a new header comment\nint f(int x)\n{\n    return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)
