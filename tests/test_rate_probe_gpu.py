"""The instruction-rate probe (csrc/rate_probe.hip) reports physically sensible rates.

The probe measures per-CU per-shader-cycle throughput of v_exp_f32, the
unpacked fp32 FMA and the 32x32x16 bf16 MFMA.  Its figures are what the
benchmark reports as the exponential roof; here they are checked against
what the hardware can do at most: one 32x32x16 MFMA (32768 FLOP) per SIMD
every 32 cycles, four SIMDs per CU (4096 FLOP per clock per CU), and 16 fp32
lanes per SIMD per clock (64 FMAs per clock per CU, unpacked).
"""
import json
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "io_aware_exact_06_amd", "rate_probe")


@pytest.mark.gpu
def test_rate_probe_rates_are_physical():
    print("rate_probe", flush=True)
    assert os.path.exists(PROBE), "the package build makes the rate_probe executable"
    r = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    rates = json.loads(r.stdout.strip().splitlines()[-1])
    assert rates["cus"] > 0
    assert 0.8 * 4096 <= rates["mfma_bf16_flop_per_clk_per_cu"] <= 1.02 * 4096, rates
    assert 8 <= rates["fma_f32_per_clk_per_cu"] <= 1.02 * 64, rates
    assert 2 <= rates["exp_per_clk_per_cu"] <= 1.02 * 64, rates
    for k in ("exp_mhz", "fma_mhz", "mfma_mhz"):
        assert 300 <= rates[k] <= 2600, rates
