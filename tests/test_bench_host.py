"""Host-side contract of bench.py (no GPU): the multi-GPU flag is refused with a
message, the committed profile summaries parse and match the sources they were
taken from, every secondary row gets its CPU-oracle timing, and the JSON line
carries every field the benchmark contract names."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_traffic_summary_is_current_and_close_to_algorithmic():
    """The committed rocprofv3 summary of the one-pass kernel is for the current
    sources, and its calibrated bytes per launch are within 2% of the algorithmic
    bytes (32.125 B x the one-pass elements of the BERT-Large-shaped vector)."""
    traffic = bench.profile_traffic()
    if traffic is None:
        pytest.skip("profiles/compress_onepass_bert_large.md was taken from other sources (bench reports null traffic)")
    algorithmic = bench.B_COMPRESS_F32 * 303_889_410
    assert abs(traffic / algorithmic - 1.0) < 0.02


def test_quantizer_valu_summary_parses():
    valu = bench.valu_per_element()
    if not valu:
        pytest.skip("profiles/quantizers_valu.md was taken from other quantizer sources")
    assert set(valu) >= {"qsdp4_quantize", "qsdp8_quantize", "qsgd4_quantize", "qsgd8_quantize"}
    assert all(10.0 < v < 200.0 for v in valu.values())


def test_every_row_gets_a_cpu_oracle_timing():
    keys = ["warmup_adam_bert_large", "qsdp4_quantize", "qsdp4_dequantize", "qsdp8_quantize", "qsdp8_dequantize",
            "qsgd4_quantize", "qsgd8_quantize", "loco4_quantize", "qsdp4_seed_statistic", "allreduce_16x64M", "full_step_16x64M_f16_mask",
            "full_step_16x64M_f16_mask_packed_m", "gpu_share_of_16_64M_f16_mask",
            "gpu_share_of_16_64M_f16_mask_packed_m", "compress_bert_large_packed_m", "compress_gpt2_xl_bf16"]
    from error_compensated_bit_amd import workloads as W
    qg = W.QsgdWorkload()
    keys += [f"qsgd{b}_reduce_{qg.W}x{qg.shard}" for b in (4, 8)]
    rows = {k: {} for k in keys}
    bench.cpu_row_baselines(rows, budget_s=0.0)
    for k in keys:
        c = rows[k].get("cpu_oracle")
        assert c is not None, k
        assert c["value"] > 0 and c["cores"] == 1 and c["kind"] == "oracle" and c["unit"]


def test_headline_line_carries_every_field_of_the_contract():
    """The JSON line built from made-up measurements of the BERT-Large workload has the
    fields the benchmark contract names, with the roofline and CPU baseline objects."""
    import json
    from error_compensated_bit_amd import workloads as W
    wl = W.bert_like()
    bpe = bench.B_COMPRESS_F32
    head = {"params_per_s": 1.7e11, "seconds_per_call": 1.97e-3, "gbps": 5460.0, "onepass_ms": 1.76,
            "onepass_gbps": 5550.0, "onepass_elements": 303_889_410, "plan": {"tiles": 1}, "kernels": {}}
    base = {"value": 1.57e8, "unit": "params/s", "cores": 1, "kind": "oracle", "sample": "two chunks",
            "cpu_model": "x", "host_cpus": 16, "cpus_allowed": [0], "pinned_core": 0}
    ceiling = {"gbps_5r3w": 5800.0, "grid_5r3w": 1024, "block_5r3w": 1024, "elements": 1, "kernel": "probe"}
    line = json.loads(json.dumps(bench.headline_line(wl, bpe, head, base, ceiling, {}, 30, 3)))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 30 and line["warmup"] == 3
    assert line["unit"] == "params/s" and line["higher_is_better"] is True and line["vs_baseline"] is None
    assert "workload" in line["config"] and "model" not in line["config"]
    r = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - 5550.0 / 8000.0) < 1e-12
    assert abs(r["bytes_per_launch"] - bpe * 303_889_410) < 1.0
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in line["cpu_baseline"], k
    assert line["cpu_baseline"]["kind"] == "oracle"
