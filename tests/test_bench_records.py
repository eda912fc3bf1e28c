"""Host logic of bench.py's per-(config, op) records (no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_op_records_cover_every_call():
    line = {"copy_GBps": 6400.0, "steps": 400, "parity_sampled_rows": True,
            "roofline": {"avg_launch_us": 30.0, "algorithmic_bytes_per_launch": 176226304},
            "cpu_baseline": {"seconds": 9.5, "host_cpus": 16},
            "per_call": {"act_predict_R": {"us": 20.0, "bytes": 33554512, "launches": 320},
                         "attn_prune_compress_V_seq": {"us": 12.0, "bytes": 52428800, "launches": 320},
                         "gemm_dense_fp8": {"us": 290.0, "bytes": 310378496, "launches": 320,
                                            "TFLOPs": 1690.0, "mfma_frac": 0.338}}}
    recs = bench.op_records(line, "gpu", "rocm")
    assert [r["op"] for r in recs] == ["headline_prune_quantize_fp8", "act_predict_R",
                                       "attn_prune_compress_V_seq", "gemm_dense_fp8"]
    head, act, v, gemm = recs
    assert head["config"] == "C4" and head["shape"] == [16384, 4096]
    assert abs(head["GBps"] - 176226304 / 30e-6 / 1e9) < 0.1
    assert abs(head["pct_copy"] - 100 * head["GBps"] / 6400.0) < 0.01
    assert head["parity_sampled_rows"] is True and head["oracle_seconds"] == 9.5
    assert act["config"] == "C1" and act["tensors_per_s"] == 50000.0
    assert v["config"] == "C3" and v["shape"] == [8, 16384, 128]
    assert gemm["config"] == "C1 x C2" and gemm["mfma_frac"] == 0.338
