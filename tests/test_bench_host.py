"""Host-side checks of bench.py (no GPU): the single-GPU guard, the HBM-traffic record the roofline
reads for the headline plan, and the shape of the context object."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_traffic_record_matches_the_headline_plan():
    """The headline plan (MXFP8 2048x14336x4096) runs the ping-pong kernel on 256x256 tiles with
    64-element steps; its HBM traffic comes from the committed FETCH_SIZE / WRITE_SIZE summary."""
    from block_scaled_quantized_amd import api
    b = load_bench()
    p = api.mxgemm_create(2048, 14336, 4096, api.MX_E4M3, api.MX_E4M3)
    tile = list(api.mxgemm_plan_info(p))
    api.mxgemm_destroy(p)
    assert tile == [256, 256, 64, 4]
    traffic, src = b.hbm_traffic("gemm_pp_ring_kernel", tile, (2048, 14336, 4096))
    assert src == "profiles/hbm_traffic_gemm_pp_mxfp8_prefill.md"
    algorithmic = 127_926_272   # A + SA + B + SB + C at the prefill shape
    assert algorithmic <= traffic < 4 * algorithmic
    assert b.hbm_traffic("gemm_pp_ring_kernel", tile, (2048, 14336, 8192)) == (None, None)


def test_context_names_its_source():
    b = load_bench()
    ctx = b.PAGES_CONTEXT
    assert ctx["source"].startswith("TileLang Metal Backend Internals")
    assert ctx["compare_with_detail"] == "fp16_gemm_4096x4096x4096"
    assert set(ctx["fp16_gemm_4096x4096x4096_tflops"]) == {"pytorch_mps", "mlx", "tilelang"}
