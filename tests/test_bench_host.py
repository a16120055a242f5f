"""Host logic of bench.py that needs no GPU: the clock read from rocminfo's
output, and which measured ceiling each line's dominant kernel is set
against."""
import bench

ROCMINFO = """
*******
Agent 1
*******
  Name:                    AMD EPYC 9575F 64-Core Processor
  Max Clock Freq. (MHz):   3300
*******
Agent 2
*******
  Name:                    gfx950
  Compute Unit:            256
  Max Clock Freq. (MHz):   2400
"""

CEILING = {"gate_up_shape_nontemporal": {"GB_per_s": 6800.0},
           "4GiB_4KiB_blocks_random_nontemporal": {"GB_per_s": 6500.0}}


def test_gpu_clock_is_the_gfx_agents():
    assert bench.gpu_max_clock_mhz(ROCMINFO) == 2400
    assert bench.gpu_max_clock_mhz("Name: cpu\n  Max Clock Freq. (MHz): 3000\n") is None
    assert bench.gpu_max_clock_mhz("") is None


def test_hbm_lines_use_the_read_kernels():
    lines = [{"roofline": {"bound": "hbm", "kernel": "gate_up_silu", "achieved": 6120.0}},
             {"roofline": {"bound": "hbm", "kernel": "attention", "achieved": 5200.0}}]
    bench.attach_measured_ceilings(lines, CEILING)
    a, b = lines[0]["roofline"]["measured_ceiling"], lines[1]["roofline"]["measured_ceiling"]
    assert a["value"] == 6800.0 and abs(a["frac"] - 0.9) < 1e-12 and "gate_up_shape" in a["source"]
    assert b["value"] == 6500.0 and abs(b["frac"] - 0.8) < 1e-12 and "random" in b["source"]


def test_gemm_lines_use_the_vendor_gemm_once_per_product(monkeypatch):
    calls = []

    def fake(M, N, K, reps=5):
        calls.append((M, N, K))
        return 1500.0

    monkeypatch.setattr(bench, "vendor_gemm_tflops", fake)
    mnk = [8192, 57344, 8192]
    lines = [{"roofline": {"bound": "mfma", "kernel": "gate_up_silu", "achieved": 1200.0, "product_mnk": mnk}},
             {"roofline": {"bound": "mfma", "kernel": "gate_up_silu", "achieved": 1350.0, "product_mnk": mnk}},
             {"roofline": {"bound": "mfma", "kernel": "moe_gate_up_silu", "achieved": 900.0}}]
    bench.attach_measured_ceilings(lines, CEILING)
    assert calls == [tuple(mnk)]
    assert abs(lines[0]["roofline"]["measured_ceiling"]["frac"] - 0.8) < 1e-12
    assert abs(lines[1]["roofline"]["measured_ceiling"]["frac"] - 0.9) < 1e-12
    assert "measured_ceiling" not in lines[2]["roofline"]  # grouped expert GEMMs: no vendor counterpart
