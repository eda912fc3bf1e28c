#!/usr/bin/env python3
"""Benchmark of the online 2:4 prune-and-compress hot path on one MI355X.

Workload: a linear-layer activation X [4096 tokens, 4096 hidden] in bf16, rows
N(0,1) with 4 outlier hidden channels (x50), the setting of the paper's 2x/4x
tier comparisons (Qin, "Is 2:4 Sparsity Still Worth It?", paper-daily.com
English summary, sections 2-4).

One step = the whole hot path over one batch (one X):
  1. fused online 2:4 prune + compress + FP8-e4m3 quantization of the kept
     values with a per-token scale (the call the metric names),
  2. the dense rivals: per-token FP8-e4m3 and INT8 quantization,
  3. predicted R for (2:4+FP8 vs FP8) and (2:4+FP8 vs INT8): energy loss,
     error energies and R in one read of X.
Inputs and outputs rotate over a pool larger than the 256 MB last-level
cache, so every step streams from HBM.  Steps are replayed from HIP graphs
(torch.cuda.graph) to keep host launch cost out of the measurement.

Prints ONE JSON line (see the repository's design notes for the fields).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--pool", type=int, default=16, help="X copies rotated (>= 512 MB total)")
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--hidden", type=int, default=4096)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of X the CPU oracle processes per baseline pass")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat baseline passes until this much CPU time is spent (max 8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of graphs")
    return ap.parse_args()


COUNTED_SOURCES = ["kernels_prune.hip", "kernels_quant.hip", "device_common.hpp", "dispatch.hpp",
                   "launch.hpp"]


def source_hash() -> str:
    """sha256 over the sources the measured row kernels are compiled from (the
    prune and quantizer kernels and the headers they include), to tell whether
    stored counters still describe the kernels that run."""
    import hashlib

    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for name in COUNTED_SOURCES:
        with open(os.path.join(root, "pruning_quantization_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, tokens: int, hidden: int):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for the
    library's copy kernel of known size).  None when no summary matches this
    workload or the kernel sources changed after the counters were taken."""
    if (tokens, hidden) != (4096, 4096):
        return None, "no counters for this shape"
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "pmc_traffic_bench_act4096x4096.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != source_hash():
        return None, "kernel sources changed since the counters were taken"
    k = d["kernels"].get(kernel)
    if k is None:
        return None, "kernel not in the counter summary"
    return k["traffic_bytes"], "profiles/pmc_traffic_bench_act4096x4096.json"


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the hot path has no "
                          "cross-GPU step (rows shard independently), so --gpus must be 1"}))
        sys.exit(2)

    import torch
    import pruning_quantization_amd as S
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, H = a.tokens, a.hidden

    # ---- inputs: same seeded bytes for GPU and oracle --------------------------------
    x_bits = W.activation_x(a.seed, T, H)
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    pool = [x0] + [x0.clone() for _ in range(a.pool - 1)]

    kept = ["fp8", "fp8"]
    dense = ["fp8", ("int", 8)]

    def outputs():
        return {
            "pq": (torch.empty(T, H // 2, dtype=torch.uint8, device=dev),
                   torch.empty(T, H // 8, dtype=torch.uint8, device=dev),
                   torch.empty(T, dtype=torch.float32, device=dev)),
            "fp8": (torch.empty(T, H, dtype=torch.uint8, device=dev),
                    torch.empty(T, dtype=torch.float32, device=dev),
                    torch.empty(1, dtype=torch.float32, device=dev)),
            "int8": (torch.empty(T, H, dtype=torch.int8, device=dev),
                     torch.empty(T, dtype=torch.float32, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev)),
            "R": torch.empty(1, 2, 5, dtype=torch.float64, device=dev),
            "pc": (torch.empty(T, H // 2, dtype=torch.bfloat16, device=dev),
                   torch.empty(T, H // 8, dtype=torch.uint8, device=dev)),
            "p48": (torch.empty(T, H // 2, dtype=torch.bfloat16, device=dev),
                    torch.empty(T, H // 16, dtype=torch.uint8, device=dev)),
            "R48": torch.empty(1, 2, 5, dtype=torch.float64, device=dev),
            "pqr": (torch.empty(T, H // 2, dtype=torch.uint8, device=dev),
                    torch.empty(T, H // 8, dtype=torch.uint8, device=dev),
                    torch.empty(T, dtype=torch.float32, device=dev)),
            "Rr": torch.empty(1, 2, 5, dtype=torch.float64, device=dev),
            "had": torch.empty(T, H, dtype=torch.bfloat16, device=dev),
            "sfp4": (torch.empty(T, H // 4, dtype=torch.uint8, device=dev),
                     torch.empty(T, H // 16, dtype=torch.uint8, device=dev),
                     torch.empty(T, H // 32, dtype=torch.uint8, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev)),
        }

    outs = [outputs() for _ in range(a.pool)]
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)

    def call_pq(i):
        S.prune_quantize(pool[i], "fp8", out=outs[i]["pq"])

    def call_fp8(i):
        S.quantize(pool[i], "fp8", out=outs[i]["fp8"])

    def call_int8(i):
        S.quantize(pool[i], ("int", 8), out=outs[i]["int8"])

    def call_R(i):
        S.predict_R(pool[i], kept, dense, out=outs[i]["R"], workspace=ws)

    calls = {"prune_quantize_fp8": call_pq, "quantize_fp8": call_fp8,
             "quantize_int8": call_int8, "predict_R": call_R}

    # timed one by one beside the step, not part of it: plain 2:4 compression and
    # the pairwise 4:8 pattern with its predicted R
    def call_pc(i):
        S.prune_compress(pool[i], out=outs[i]["pc"])

    def call_p48(i):
        S.prune_compress_pairs48(pool[i], out=outs[i]["p48"])

    def call_R48(i):
        S.predict_R_pairs48(pool[i], kept, dense, out=outs[i]["R48"], workspace=ws)

    def call_sfp4(i):  # sparse FP4: pairwise 4:8 with NVFP4 kept values
        S.prune_quantize_pairs48(pool[i], "nvfp4", out=outs[i]["sfp4"], workspace=ws)

    # Hadamard rotation in blocks of 128 along K, fused into the load
    def call_pqr(i):
        S.prune_quantize_rot(pool[i], 128, "fp8", out=outs[i]["pqr"])

    def call_Rr(i):
        S.predict_R_rot(pool[i], 128, kept, dense, out=outs[i]["Rr"], workspace=ws)

    def call_had(i):
        S.hadamard(pool[i], 128, out=outs[i]["had"])

    # whole-row rotation (one 4096-element block per row)
    def call_pqK(i):
        S.prune_quantize_rot(pool[i], H, "fp8", out=outs[i]["pqr"])

    def call_RK(i):
        S.predict_R_rot(pool[i], H, kept, dense, out=outs[i]["Rr"], workspace=ws)

    # operator-level output error of Y = X W^T against a synthetic MLP weight
    # W [14336, H] (bf16 N(0, 0.02^2)): reference + 2:4+FP8 and dense FP8 sides
    n_w = 14336
    w_op = torch.from_numpy(W.weight_w(a.seed + 1, n_w, H).view(np.int16)).view(torch.bfloat16).to(dev)
    op_sides = [("2:4", ("fp8", 0)), ("dense", ("fp8", 0))]
    op_out = torch.empty(T, 1 + len(op_sides), dtype=torch.float64, device=dev)
    op_ws = torch.empty(T * 2 * H * 2 + (1 + len(op_sides)) * T * ((n_w + 127) // 128) * 4 + (1 << 20),
                        dtype=torch.uint8, device=dev)

    def call_op(i):
        S.operator_error(pool[i], w_op, op_sides, out=op_out, workspace=op_ws)

    # GEMMs that consume the prepared X against W: 2:4-compressed X on the
    # sparse MFMA, dense bf16 X, and the e4m3 codes of the dense FP8 rival
    # (W quantized once, offline)
    c_gemm = torch.empty(T, n_w, dtype=torch.float32, device=dev)
    w_codes, w_scales = S.quantize(w_op, "fp8")

    def call_gsp(i):
        S.sparse_gemm(outs[i]["pc"][0], outs[i]["pc"][1], w_op, out=c_gemm)

    def call_gde(i):
        S.dense_gemm(pool[i], w_op, out=c_gemm)

    def call_g8(i):
        S.fp8_gemm(outs[i]["fp8"][0], outs[i]["fp8"][1], w_codes, w_scales, out=c_gemm)

    # predicted R of the other two scoring workloads (one tensor each, not
    # rotated: both calls are VALU-bound): the MLP weight W with Wanda 2:4
    # (norms of X's channels) over the equal-bits sweep 2:4+INT-2m vs dense
    # INT-(m+1), m = 2..8; and the heavy-tailed 4x-tier activation, 2:4+FP8 vs
    # MXFP4 and NVFP4 per block of 128 rows
    norms = S.col_l2norm(x0)
    sweep_kept = [("int", 2 * m) for m in range(2, 9)]
    sweep_dense = [("int", m + 1) for m in range(2, 9)]
    r_sweep = torch.empty(1, len(sweep_kept), 5, dtype=torch.float64, device=dev)
    n_h = 16384
    x_heavy = torch.from_numpy(W.student_t_x(a.seed + 2, n_h, H).view(np.int16)).view(torch.bfloat16).to(dev)
    r_heavy = torch.empty(n_h // 128, 2, 5, dtype=torch.float64, device=dev)
    ws_big = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def call_Rw(i):
        S.predict_R(w_op, sweep_kept, sweep_dense, score="wanda", col_norm=norms, out=r_sweep,
                    workspace=ws_big)

    def call_Rh(i):
        S.predict_R(x_heavy, ["fp8", "fp8"], ["mxfp4", "nvfp4"], rows_per_block=128, out=r_heavy,
                    workspace=ws_big)

    # the remaining workloads' own calls, each on its operand at full size
    # (operands below the 256 MB last-level cache rotate over copies):
    # Wanda 2:4 of W; the attention operands Q, K (pruned along head_dim), V
    # (pruned along the sequence: a strided operand) and P; the 4x tier's
    # fused 2:4+FP8 and its MXFP4 / NVFP4 rivals
    heavy2 = [x_heavy, x_heavy.clone()]
    pc_w = (torch.empty(n_w, H // 2, dtype=torch.bfloat16, device=dev),
            torch.empty(n_w, H // 8, dtype=torch.uint8, device=dev))

    def bf(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q_att = bf(W.attention_qkv(a.seed + 3, 32, 16384, 128)).view(-1, 128)
    q_pool = [q_att, q_att.clone()]
    k_att = bf(W.attention_qkv(a.seed + 4, 8, 16384, 128)).view(-1, 128)
    k_pool = [k_att] + [k_att.clone() for _ in range(7)]
    v_att = bf(W.attention_qkv(a.seed + 5, 8, 16384, 128))
    v_pool = [v_att] + [v_att.clone() for _ in range(7)]
    p_att = bf(W.attention_p(a.seed + 6, 32, 4096, 4096)).view(-1, 4096)
    pc_q = (torch.empty(32 * 16384, 64, dtype=torch.bfloat16, device=dev),
            torch.empty(32 * 16384, 16, dtype=torch.uint8, device=dev))
    pc_k = (torch.empty(8 * 16384, 64, dtype=torch.bfloat16, device=dev),
            torch.empty(8 * 16384, 16, dtype=torch.uint8, device=dev))
    pc_v = (torch.empty(8, 128, 8192, dtype=torch.bfloat16, device=dev),
            torch.empty(8, 128, 2048, dtype=torch.uint8, device=dev))
    pc_p = (torch.empty(32 * 4096, 2048, dtype=torch.bfloat16, device=dev),
            torch.empty(32 * 4096, 512, dtype=torch.uint8, device=dev))
    r_p = torch.empty(32, 2, 5, dtype=torch.float64, device=dev)
    pq_h = (torch.empty(n_h, H // 2, dtype=torch.uint8, device=dev),
            torch.empty(n_h, H // 8, dtype=torch.uint8, device=dev),
            torch.empty(n_h, dtype=torch.float32, device=dev))
    mx_h = (torch.empty(n_h, H // 2, dtype=torch.uint8, device=dev),
            torch.empty(n_h, H // 32, dtype=torch.uint8, device=dev),
            torch.empty(1, dtype=torch.float32, device=dev))
    nv_h = (torch.empty(n_h, H // 2, dtype=torch.uint8, device=dev),
            torch.empty(n_h, H // 16, dtype=torch.uint8, device=dev),
            torch.empty(1, dtype=torch.float32, device=dev))

    def call_pcw(i):
        S.prune_compress(w_op, score="wanda", col_norm=norms, out=pc_w)

    def call_pcq(i):
        S.prune_compress(q_pool[i % 2], out=pc_q)

    def call_pck(i):
        S.prune_compress(k_pool[i % 8], out=pc_k)

    def call_pcv(i):
        S.prune_compress(v_pool[i % 8], axis=1, out=pc_v)

    def call_pcp(i):
        S.prune_compress(p_att, out=pc_p)

    def call_Rp(i):
        S.predict_R(p_att, ["none", "none"], ["fp8", ("int", 8)], rows_per_block=4096, out=r_p,
                    workspace=ws_big)

    def call_pqh(i):
        S.prune_quantize(heavy2[i % 2], "fp8", out=pq_h)

    def call_mxh(i):
        S.quantize(heavy2[i % 2], "mxfp4", out=mx_h)

    def call_nvh(i):
        S.quantize(heavy2[i % 2], "nvfp4", out=nv_h, workspace=ws_big)

    side_calls = {"prune_compress_2of4": call_pc, "prune_compress_pairs48": call_p48,
                  "predict_R_pairs48": call_R48, "prune_quantize_pairs48_nvfp4": call_sfp4,
                  "hadamard128": call_had, "prune_quantize_fp8_rot128": call_pqr,
                  "predict_R_rot128": call_Rr, "prune_quantize_fp8_rot_row": call_pqK,
                  "predict_R_rot_row": call_RK, "operator_error_2sides": call_op,
                  "gemm_sparse24_bf16": call_gsp, "gemm_dense_bf16": call_gde,
                  "gemm_dense_fp8": call_g8, "predict_R_wanda_sweep_W": call_Rw,
                  "predict_R_heavy_blocks128": call_Rh, "prune_compress_wanda_W": call_pcw,
                  "prune_compress_attn_Q": call_pcq, "prune_compress_attn_K": call_pck,
                  "prune_compress_attn_V_seq": call_pcv, "prune_compress_attn_P": call_pcp,
                  "predict_R_attn_P_heads": call_Rp, "prune_quantize_fp8_heavy": call_pqh,
                  "quantize_mxfp4_heavy": call_mxh, "quantize_nvfp4_heavy": call_nvh}

    def step(i):
        for f in calls.values():
            f(i)

    # algorithmic bytes per call (input read once + every output written once)
    xb = T * H * 2
    alg = {
        "prune_quantize_fp8": xb + T * H // 2 + T * H // 8 + T * 4,
        "quantize_fp8": xb + T * H + T * 4,
        "quantize_int8": xb + T * H + T * 4,
        "predict_R": xb + 2 * 5 * 8,
    }
    step_bytes = sum(alg.values())
    alg.update({
        "prune_compress_2of4": xb + xb // 2 + T * H // 8,
        "prune_compress_pairs48": xb + xb // 2 + T * H // 16,
        "predict_R_pairs48": xb + 2 * 5 * 8,
        # one read of X (the kept-maximum pre-pass reads it a second time)
        "prune_quantize_pairs48_nvfp4": xb + T * H // 4 + T * H // 16 + T * H // 32 + 4,
        "hadamard128": 2 * xb,
        "prune_quantize_fp8_rot128": xb + T * H // 2 + T * H // 8 + T * 4,
        "predict_R_rot128": xb + 2 * 5 * 8,
        "prune_quantize_fp8_rot_row": xb + T * H // 2 + T * H // 8 + T * 4,
        "predict_R_rot_row": xb + 2 * 5 * 8,
        "operator_error_2sides": xb + n_w * H * 2,
        "gemm_sparse24_bf16": xb // 2 + T * H // 8 + n_w * H * 2 + T * n_w * 4,
        "gemm_dense_bf16": xb + n_w * H * 2 + T * n_w * 4,
        "gemm_dense_fp8": T * H + n_w * H + T * n_w * 4,
        "predict_R_wanda_sweep_W": n_w * H * 2 + H * 4 + len(sweep_kept) * 5 * 8,
        # one read of X (the NVFP4 tensor-maximum pass reads it a second time)
        "predict_R_heavy_blocks128": n_h * H * 2 + (n_h // 128) * 2 * 5 * 8,
        "prune_compress_wanda_W": n_w * H * 2 + n_w * H + n_w * H // 8 + H * 4,
        "prune_compress_attn_Q": 32 * 16384 * 128 * 2 + 32 * 16384 * 64 * 2 + 32 * 16384 * 16,
        "prune_compress_attn_K": 8 * 16384 * 128 * 2 + 8 * 16384 * 64 * 2 + 8 * 16384 * 16,
        "prune_compress_attn_V_seq": 8 * 16384 * 128 * 2 + 8 * 16384 * 64 * 2 + 8 * 16384 * 16,
        "prune_compress_attn_P": 32 * 4096 * 4096 * 2 + 32 * 4096 * 2048 * 2 + 32 * 4096 * 512,
        "predict_R_attn_P_heads": 32 * 4096 * 4096 * 2 + 32 * 2 * 5 * 8,
        "prune_quantize_fp8_heavy": n_h * H * 2 + n_h * H // 2 + n_h * H // 8 + n_h * 4,
        "quantize_mxfp4_heavy": n_h * H * 2 + n_h * H // 2 + n_h * H // 32,
        # one read of X (the tensor-maximum pass reads it a second time)
        "quantize_nvfp4_heavy": n_h * H * 2 + n_h * H // 2 + n_h * H // 16 + 4,
    })
    # MFMA work of the compute-bound call: the reference product plus, per side,
    # the product of the [hi | lo] residual (2K deep)
    flops = {"operator_error_2sides": 2.0 * T * n_w * H * (1 + 2 * len(op_sides)),
             "gemm_sparse24_bf16": 2.0 * T * n_w * H, "gemm_dense_bf16": 2.0 * T * n_w * H,
             "gemm_dense_fp8": 2.0 * T * n_w * H}
    mfma_peak = {"gemm_dense_fp8": 5000.0, "gemm_sparse24_bf16": 5000.0}  # sparse: 2x dense bf16

    # ---- spot parity against the oracle (not timed) ---------------------------------
    step(0)
    for f in side_calls.values():
        for i in range(a.pool):
            f(i)
    torch.cuda.synchronize()
    import oracle as O
    rows = np.r_[0:8, T - 8:T]
    wc, wm, wsc = O.prune_quantize(x_bits[rows], "bf16", O.QSpec("fp8"))
    c, m, s = (t.cpu().numpy() for t in outs[0]["pq"])
    parity = bool(np.array_equal(c[rows], wc) and np.array_equal(m[rows], wm)
                  and np.array_equal(s[rows].view(np.uint32), wsc.view(np.uint32)))
    wv, wm = O.prune_compress_pairs48(x_bits[rows], "bf16")
    v48, m48 = (t.cpu().view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
                for t in outs[0]["p48"])
    parity = parity and bool(np.array_equal(m48[rows], wm)
                             and np.array_equal(v48[rows].view(np.uint16), wv.view(np.uint16)))

    # ---- warmup ----------------------------------------------------------------------
    for w in range(a.warmup):
        step(w % a.pool)
    torch.cuda.synchronize()

    # ---- graphs: one per pool entry (1 step) and one per call over the ring ----------
    use_graphs = not a.eager
    step_graphs, call_graphs = [], {}
    if use_graphs:
        try:
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                for i in range(a.pool):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cap):
                        step(i)
                    step_graphs.append(g)
                for name, f in {**calls, **side_calls}.items():
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cap):
                        for i in range(a.pool):
                            f(i)
                    call_graphs[name] = g
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            for g in step_graphs:
                g.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported -> eager launches
            print(f"# graph capture failed ({e}); timing eager launches", file=sys.stderr)
            use_graphs = False

    # ---- timed region: exactly K steps ------------------------------------------------
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for k in range(a.steps):
        if use_graphs:
            step_graphs[k % a.pool].replay()
        else:
            step(k % a.pool)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / a.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- per-call kernel durations (HIP events around ring replays) ------------------
    per_call = {}
    reps = max(1, a.steps // a.pool)
    for name, f in {**calls, **side_calls}.items():
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            if use_graphs:
                call_graphs[name].replay()
            else:
                for i in range(a.pool):
                    f(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * a.pool)
        per_call[name] = {"us": round(us, 3), "GBps": round(alg[name] / (us * 1e-6) / 1e9, 1)}
        if name in flops:
            tf = flops[name] / (us * 1e-6) / 1e12
            pk = mfma_peak.get(name, 2500.0)
            per_call[name].update({"TFLOPs": round(tf, 1), "mfma_peak_TFLOPs": pk,
                                   "mfma_frac": round(tf / pk, 4)})

    # ---- copy baseline: library copy kernel over the same rotation -------------------
    src = [p.view(torch.uint8).view(-1) for p in pool]
    dst = [torch.empty_like(s_) for s_ in src]
    for i in range(a.pool):
        S.copy(src[i], dst[i])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        for i in range(a.pool):
            S.copy(src[i], dst[i])
    e1.record()
    torch.cuda.synchronize()
    copy_us = e0.elapsed_time(e1) * 1e3 / (reps * a.pool)
    copy_gbps = 2 * xb / (copy_us * 1e-6) / 1e9

    # torch's device-to-device copy as a second copy baseline; the better one counts
    e0.record()
    for r in range(reps):
        for i in range(a.pool):
            dst[i].copy_(src[i])
    e1.record()
    torch.cuda.synchronize()
    tcopy_us = e0.elapsed_time(e1) * 1e3 / (reps * a.pool)
    copy_gbps = max(copy_gbps, 2 * xb / (tcopy_us * 1e-6) / 1e9)

    dom = "prune_quantize_fp8"
    achieved = per_call[dom]["GBps"]
    kname = "k_prune_quantize<BF16T, 128, 4, false, 2, 0, 0>"
    traffic, traffic_note = measured_traffic(kname, T, H)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "traffic_note": traffic_note, "kernel": kname,
                "algorithmic_bytes_per_launch": alg[dom], "avg_launch_us": per_call[dom]["us"]}

    # ---- CPU baseline: the oracle on a bounded sample of the same step ---------------
    cpu = None
    if not a.no_cpu_baseline:
        n = min(a.cpu_rows, T)
        sub = x_bits[:n]
        passes = 0
        t1 = time.perf_counter()
        while True:
            O.prune_quantize(sub, "bf16", O.QSpec("fp8"))
            O.quantize_rows(sub, "bf16", O.QSpec("fp8"))
            O.quantize_rows(sub, "bf16", O.QSpec("int", 8))
            O.predict_R(sub, "bf16", [O.QSpec(k) for k in kept],
                        [O.QSpec("fp8"), O.QSpec("int", 8)])
            passes += 1
            dt = time.perf_counter() - t1
            if dt >= a.cpu_seconds or passes >= 8:
                break
        cpu = {"value": round(passes * step_bytes * n / T / dt / 1e9, 4), "unit": "GB/s",
               "cores": 1, "kind": "oracle", "host_cpus": os.cpu_count(),
               "seconds": round(dt, 2),
               "sample": f"{passes} pass(es) of rows 0..{n - 1} of the {T}-row X through all "
                         "four calls of one step (numpy, single-threaded)"}

    line = {
        "metric": "fused 2:4 prune+compress+quant GB/s (% of HBM peak); predicted-R tensors/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "linear-layer activation X 4096x4096 bf16, N(0,1) rows with 4 "
                               "outlier channels x50; step = 2:4 prune+compress+FP8 (per-token), "
                               "dense FP8 and INT8 (per-token), predicted R for 2 pairs",
                   "tokens": T, "hidden": H, "pool": a.pool, "graphs": use_graphs},
        "fused_prune_quant_GBps": achieved,
        "fused_prune_quant_pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "fused_prune_quant_pct_copy": round(100 * achieved / copy_gbps, 2),
        "predicted_R_tensors_per_s": round(1e6 / per_call["predict_R"]["us"], 1),
        # the weight W [14336, 4096] with all 7 equal-bits pairs; the heavy-tailed
        # X [16384, 4096] with all 128 row blocks x 2 pairs
        "predicted_R_wanda_sweep_W_tensors_per_s": round(
            1e6 / per_call["predict_R_wanda_sweep_W"]["us"], 1),
        "predicted_R_heavy_blocks128_tensors_per_s": round(
            1e6 / per_call["predict_R_heavy_blocks128"]["us"], 1),
        "step_tensors_per_s": round(1e3 / ms_step, 1),
        "copy_GBps": round(copy_gbps, 1),
        # [PD §3] speed question at equal nominal tier: dense FP8 (online
        # quantization of X + FP8 GEMM) time over 2:4 bf16 (online
        # prune+compress of X + sparse GEMM) time; above 1 = 2:4 faster
        "speed_2of4_bf16_vs_dense_fp8": round(
            (per_call["quantize_fp8"]["us"] + per_call["gemm_dense_fp8"]["us"])
            / (per_call["prune_compress_2of4"]["us"] + per_call["gemm_sparse24_bf16"]["us"]), 3),
        "per_call": per_call,
        "parity_sampled_rows": parity,
        "wall_s": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
