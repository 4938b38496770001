"""Host logic of bench.py, on the CPU: the algorithmic bytes and FLOPs the
roofline divides by, the counter-file parsing and copy calibration behind
the HBM traffic figure, the committed counter summary matching the kernel
source, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from routed_expert_ffn_top_amd.inputs import CONFIGS  # noqa: E402


def test_algorithmic_olmoe_t4096_by_hand():
    # OLMoE shape: T=4096, d=2048, E=64, k=8, f=1024, bf16
    cfg = CONFIGS["olmoe_t4096"]
    alg = bench.layer_algorithmic(cfg)
    T, d, E, k, f = 4096, 2048, 64, 8, 1024
    R = T * k
    w_gu = E * 2 * f * d * 2            # every expert's gate and up slices, bf16
    assert alg["gate/up"][0] == w_gu + R * d * 2 + R * f * 2
    assert alg["gate/up"][1] == 4.0 * R * d * f
    assert alg["down"][0] == E * d * f * 2 + R * f * 2 + R * d * 4
    assert alg["down"][1] == 2.0 * R * d * f
    # the figures the roofline line quotes: 738 MB and 275 GFLOP for gate/up
    assert round(alg["gate/up"][0] / 1e6) == 738
    assert round(alg["gate/up"][1] / 1e9, 1) == 274.9
    # routed and expert FLOPs together are the layer's 6 R d f
    assert alg["gate/up"][1] + alg["down"][1] == 6.0 * R * d * f


def test_algorithmic_counts_shared_experts():
    # DeepSeek-V2-Lite shape: 64 routed experts top-6 plus 2 shared ones,
    # which every token uses and whose weights are read as well
    cfg = CONFIGS["dsv2lite_t4096"]
    alg = bench.layer_algorithmic(cfg)
    T, d, f = 4096, 2048, 1408
    R = T * (6 + 2)
    assert alg["gate/up"][0] == 66 * 2 * f * d * 2 + R * d * 2 + R * f * 2
    assert alg["down"][0] == 66 * d * f * 2 + R * f * 2 + R * d * 4
    assert alg["combine"][0] == R * d * 4 + 2 * T * d * 4


def _counter_csv(path, rows):
    with open(path, "w") as fh:
        fh.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for k, c, v in rows:
            fh.write(f'"{k}","{c}",{v}\n')


def test_pmc_average_per_kernel(tmp_path):
    p = tmp_path / "c.csv"
    _counter_csv(p, [("kA", "FETCH_SIZE", 10.0), ("kA", "FETCH_SIZE", 30.0), ("kB", "FETCH_SIZE", 5.0),
                     ("kA", "WRITE_SIZE", 99.0)])
    got = bench._pmc_per_kernel(str(p), "FETCH_SIZE")
    assert got == {"kA": (20.0, 2), "kB": (5.0, 1)}


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    # the copy kernel moves 1 GiB each way; its counters read half of that
    # (fetch) and all of it (write), so the factors must come out 2 and 1
    gu = "void moe::k_gemm_mfma_lds<256, 256, 4, 4, 2, true, false, false>(moe::GemmArgs)"
    cp = "at::native::vectorized_elementwise_kernel<4, MulFunctor>"
    gib_kib = float(1 << 20)
    f, w, cf, cw = (tmp_path / n for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _counter_csv(f, [(gu, "FETCH_SIZE", 1000.0), (gu, "FETCH_SIZE", 1000.0)])
    _counter_csv(w, [(gu, "WRITE_SIZE", 300.0)])
    _counter_csv(cf, [(cp, "FETCH_SIZE", gib_kib / 2)])
    _counter_csv(cw, [(cp, "WRITE_SIZE", gib_kib)])
    out = tmp_path / "s.txt"
    bench.summarize_pmc(str(f), str(w), str(cf), str(cw), str(out), "cmd")
    vals = dict(l.split(":", 1) for l in out.read_text().splitlines() if ":" in l and not l.startswith("#"))
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(1000.0 * 1024 * 2 + 300.0 * 1024)
    assert vals["kernel_source_hash"].strip() == bench.gemm_source_hash()


def test_committed_traffic_matches_kernel_source():
    # the committed gate/up counter summary was taken on the current kernel
    # source, so the bench line carries a traffic figure
    t = bench.read_traffic("olmoe_t4096", 0.0)
    assert t is not None and 0.7e9 < t < 2.0e9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
