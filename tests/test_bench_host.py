"""Host-side checks of bench.py's accounting: the algorithmic bytes and flops that the
roofline fractions divide by, and the kernel patterns that select the dominant kernel in
rocprofv3 output.  The expected figures are worked by hand from the layer shapes."""
import re

import bench
import synth


def test_decode_gateup_bytes_and_flops():
    cfg = synth.get("qwen38max_decode")              # T=1, K=H=7168, I=2368, k=10, gated shared
    a = bench.algorithmic(cfg, 10, fused=True)
    row = 7168 * 17 // 32                             # one MXFP4 weight row: codes + scales = 3808 B
    assert row == 3808
    routed = 10 * 2 * 2368 * row                      # ten experts' gate and up
    shared = 2 * 2368 * row                           # the shared expert's gate and up (same launch)
    x_in, h_out, hs_out = 7168 * 2, 10 * 2368 * 4, 2368 * 4
    assert a["gu_bytes"] == routed + shared + x_in + h_out + hs_out == 198_500_096
    assert a["gu_flops"] == 2 * 10 * 2 * 7168 * 2368 + 2 * 1 * 2 * 7168 * 2368


def test_float_prefill_gateup_bytes_and_flops():
    cfg = synth.get("qwen38max_prefill_hot_float")   # T=512, ten hot experts, bf16 x, float32 h
    a = bench.algorithmic(cfg, 10, fused=False)
    routed = 10 * 2 * 2368 * 3808
    x_in, h_out = 512 * 7168 * 2, 512 * 10 * 2368 * 4
    assert a["gu_bytes"] == routed + x_in + h_out == 236_183_552
    assert a["gu_flops"] == 2 * 5120 * 2 * 7168 * 2368 == 347_623_915_520


def test_mx_prefill_gateup_bytes():
    cfg = synth.get("qwen38max_prefill_hot")         # MX activations: x and h as MXFP4 (17/32 B per value)
    a = bench.algorithmic(cfg, 10, fused=False)
    assert a["gu_bytes"] == 10 * 2 * 2368 * 3808 + 512 * 7168 * 17 // 32 + 5120 * 2368 * 17 // 32


def test_decode_down_combine_bytes_and_flops():
    cfg = synth.get("qwen38max_decode")
    a = bench.down_algorithmic(cfg, 10, fused=True)
    row = 2368 * 17 // 32                             # one MXFP4 down row over d_ff = 2368: 1258 B
    assert row == 1258
    routed, shared = 10 * 7168 * row, 7168 * row      # ten experts' down matrices and the shared one
    h_in, hs_in, out = 10 * 2368 * 4, 2368 * 4, 7168 * 4
    assert a["bytes"] == routed + shared + h_in + hs_in + out == 99_323_648
    assert a["flops"] == 2 * 11 * 7168 * 2368


def test_mx_prefill_down_bytes_and_flops():
    cfg = synth.get("qwen38max_prefill_hot")
    a = bench.down_algorithmic(cfg, 10, fused=False)
    assert a["bytes"] == 10 * 7168 * 1258 + 5120 * 2368 * 17 // 32 + 5120 * 7168 * 4
    assert a["flops"] == 2 * 5120 * 7168 * 2368


def test_roofline_picks_the_binding_roof():
    hbm = bench.roofline(198_500_096, 746_848_256, 40.0, bench.PEAK_TFLOPS["bf16"])
    assert hbm["bound"] == "hbm" and abs(hbm["achieved"] - 198_500_096 / 40e-6 / 1e9) < 0.1
    mfma = bench.roofline(237_000_000, 347_623_915_520, 100.0, bench.PEAK_TFLOPS["fp4"])
    assert mfma["bound"] == "mfma" and abs(mfma["frac"] - 347_623_915_520 / 100e-6 / 1e12 / 10100.0) < 1e-4


def test_dominant_kernel_patterns_select_one_instantiation():
    names = {
        "qwen38max_decode": ("void moe::gemv_flat_kernel<0, 0, 1, true, true>(moe::GemvParams)",
                             "void moe::gemv_kernel<0, 0, 1, true, false>(moe::GemvParams)"),
        "qwen38max_prefill_hot": ("void moe::mxgemm_kernel<true, true, true>(moe::GemmParams)",
                                  "void moe::mxgemm_kernel<true, false, true>(moe::GemmParams)"),
        "qwen38max_prefill_hot_float": ("void moe::fgemm_pair_kernel<false, true>(moe::FGemmParams)",
                                        "void moe::fgemm_pair_kernel<false, false>(moe::FGemmParams)"),
    }
    for wl, (routed, shared) in names.items():
        pat = re.compile(bench.dominant_kernel(synth.get(wl)))
        assert pat.search(routed), wl
        assert not pat.search(shared), wl


def test_more_than_one_gpu_is_refused_before_any_device_work():
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(here, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=here)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_latent_down_combine_bytes():
    cfg = synth.get("kimik3_latent_decode")          # T=4, k=8, latent 2048 (d_model of the experts), I=2048
    a = bench.down_algorithmic(cfg, 31, fused=False, combined=True)
    row = 2048 * 17 // 32                             # one MXFP4 down row over I = 2048: 1088 B
    assert a["bytes"] == 31 * 2048 * row + 32 * 2048 * 4 + 4 * 2048 * 4   # no shared rows: it is added after P_u
    assert bench.down_kernel(cfg, False, True) == r"down_combine_mfma_kernel"


def test_single_launch_step_entry_uses_the_layer_bytes():
    """The single-launch decode step's roofline divides the whole layer's algorithmic bytes
    (router, ten experts, the shared expert, x in and out once) by the launch time."""
    cfg = synth.get("qwen38max_decode")
    r = dict(single=True, D_ev=[10, 10], st_us=76.2, launches=2, phases=[["timed", 2]])
    (e,) = bench.kernel_entries(cfg, True, r)
    layer = 11 * 27_052_032 + 512 * 7168 * 2 + 7168 * 2 + 7168 * 2 + 7168 * 4
    assert layer == 304_969_728
    assert e["bytes_per_launch"] == layer and e["bound"] == "hbm"
    assert abs(e["achieved"] - layer / 76.2e-6 / 1e9) < 0.1
    assert re.search(e["kernel"], "void moe::decode_step_kernel<1>(moe::StepParams)")
