#!/usr/bin/env python3
"""Benchmark of the online 2:4 prune-and-compress hot path on one MI355X.

Headline (`value`): the fused online 2:4 prune + compress + FP8-e4m3
quantization of the kept values (one per-token scale) on the 4x-tier
activation X [16384 tokens, 4096 hidden] bf16 with Student-t(4) entries
(Qin, "Is 2:4 Sparsity Still Worth It?", paper-daily.com English summary,
section 3: the fused kernel reads the operand once and writes kept values and
indices once).  One step = one such call on one X; the X copies rotate over
1 GiB (4x the 256 MB last-level cache), so every step streams from HBM.
Steps are replayed from HIP graphs to keep host launch cost out.

Beside it, each on its own operand at full size:
  * the same X through the other calls of its workload (dense MXFP4 and
    NVFP4, predicted R per block of 128 rows);
  * the linear-layer activation X [4096, 4096] (4 outlier channels x50) through
    fused 2:4+FP8, dense FP8 and INT8 and predicted R (the four-call step);
  * the weight W [14336, 4096] (Wanda 2:4, the equal-bits INT sweep), the
    attention operands Q, K, V, P, pairwise 4:8, rotations, operator error and
    the GEMMs;
  * the copy baseline: the library's copy kernel and a device-to-device copy,
    each over 1 GiB, graph-replayed; the faster counts.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
VALU_PEAK_TOPS = 39.3216    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, non-packed lane-ops
ROOT = os.path.dirname(os.path.abspath(__file__))

# the headline kernel: fused 2:4 + FP8, bf16 rows of 4096 on two-wave teams
HEAD_KERNEL = "k_prune_quantize<BF16T, 128, 4, false, 2, 0, 0>"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--pool", type=int, default=8,
                    help="copies of the headline X rotated (128 MiB each; >= 4 for 512 MB)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--side-reps", type=int, default=20,
                    help="graph replays of each side call's rotation ring")
    ap.add_argument("--copy-mib", type=int, default=1024, help="copy-baseline buffer size")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="rows of the headline X per oracle pass of the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="repeat oracle passes until this much time is spent (max 8 passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline call and the copy baseline (for profiling)")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of graphs")
    ap.add_argument("--markers", action="store_true",
                    help="launch a one-workgroup copy before each measured phase, so that a "
                         "profile's dispatches can be split by phase")
    ap.add_argument("--ops-jsonl", default=None,
                    help="also write one JSON line per (config, op) to this file")
    return ap.parse_args()


# (config, operand shape) of each timed call, by name prefix; the configs are
# the five workloads: C0 tiny fp32 (a parity case only, not timed), C1 the
# linear-layer activation, C2 the MLP weight, C3 the attention operands, C4
# the heavy-tailed activation
OP_SHAPES = [
    ("headline", "C4", [16384, 4096]), ("act_", "C1", [4096, 4096]),
    ("weight_", "C2", [14336, 4096]), ("heavy_", "C4", [16384, 4096]),
    ("attn_prune_compress_Q", "C3", [32, 16384, 128]), ("attn_prune_compress_K", "C3", [8, 16384, 128]),
    ("attn_prune_compress_V_seq", "C3", [8, 16384, 128]), ("attn_prune_compress_P", "C3", [32, 4096, 4096]),
    ("attn_predict_R_P", "C3", [32, 4096, 4096]), ("operator_error", "C1 x C2", [4096, 4096]),
    ("gemm_", "C1 x C2", [4096, 4096]),
]


def op_records(line, gpu, rocm):
    """One record per (config, op) from a bench line: the metrics the line
    holds for that call, in one flat object."""
    copy = line["copy_GBps"]
    calls = [("headline_prune_quantize_fp8", {"us": line["roofline"]["avg_launch_us"],
                                              "bytes": line["roofline"]["algorithmic_bytes_per_launch"],
                                              "launches": line["steps"]})]
    calls += list(line["per_call"].items())
    out = []
    for name, c in calls:
        cfg, shape = next((cf, sh) for pre, cf, sh in OP_SHAPES if name.startswith(pre))
        elems = int(np.prod(shape))
        gbps = c["bytes"] / (c["us"] * 1e-6) / 1e9
        rec = {"config": cfg, "op": name, "dtype": "bf16", "shape": shape,
               "algorithmic_bytes": c["bytes"], "us": c["us"], "GBps": round(gbps, 1),
               "Gelem_per_s": round(elems / (c["us"] * 1e-6) / 1e9, 2),
               "pct_copy": round(100 * gbps / copy, 2), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
               "launches": c["launches"], "gpu": gpu, "rocm": rocm}
        if "predict_R" in name:
            rec["tensors_per_s"] = round(1e6 / c["us"], 1)
        if "TFLOPs" in c:
            rec.update({"TFLOPs": c["TFLOPs"], "mfma_frac": c["mfma_frac"]})
        if name.startswith("headline"):
            rec["parity_sampled_rows"] = line["parity_sampled_rows"]
            if line.get("cpu_baseline"):
                rec["oracle_seconds"] = line["cpu_baseline"]["seconds"]
                rec["host_cpus"] = line["cpu_baseline"]["host_cpus"]
        out.append(rec)
    return out


def source_hash(names) -> str:
    """sha256 over kernel sources, to tell whether stored counters still
    describe the kernels that run."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "pruning_quantization_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_counters(fname: str):
    """A committed rocprofv3 counter summary under profiles/, or None when it
    is absent or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None, f"no counter summary {fname}"
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != source_hash(d.get("sources", [])):
        return None, f"kernel sources changed since {fname} was taken"
    return d, f"profiles/{fname}"


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
    use_graphs = not a.eager
    cur = torch.cuda.current_stream

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def capture(fn):
        """HIP graph of fn() captured on a side stream (replayed on the current one)."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(cur())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn()
        cur().wait_stream(cap)
        torch.cuda.synchronize()
        return g

    def elapsed_us(run):
        """HIP events on the current stream (the one the library launches on)
        around run(); microseconds."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    # ================================================================================
    # Headline: fused 2:4 prune + compress + FP8 of the heavy-tailed X [16384, 4096].
    # Runs first, so its launches are the first of its kernel in a profile: the
    # pool fill (parity), the warmup, then the timed steps.
    # ================================================================================
    NH, H = 16384, 4096
    hx_bits = W.student_t_x(a.seed + 2, NH, H)
    hpool = [bf(hx_bits)]
    hpool += [hpool[0].clone() for _ in range(a.pool - 1)]
    houts = [(torch.empty(NH, H // 2, dtype=torch.uint8, device=dev),
              torch.empty(NH, H // 8, dtype=torch.uint8, device=dev),
              torch.empty(NH, dtype=torch.float32, device=dev)) for _ in range(a.pool)]
    head_bytes = NH * H * 2 + NH * H // 2 + NH * H // 8 + NH * 4

    def head(i):
        S.prune_quantize(hpool[i], "fp8", out=houts[i])

    mark_buf = torch.zeros(2, 16, dtype=torch.uint8, device=dev)
    phases = []

    def marker(name):
        """Progress line on stderr; with --markers also a one-workgroup copy of
        16 bytes that opens phase `name` in a profile."""
        print(f"# {name}", file=sys.stderr, flush=True)
        if a.markers:
            S.copy(mark_buf[0], mark_buf[1])
            phases.append(name)

    marker("headline_fill")
    for i in range(a.pool):
        head(i)
    torch.cuda.synchronize()
    import oracle as O
    rows = np.r_[0:16, NH - 16:NH]
    wc, wm, wsc = O.prune_quantize(hx_bits[rows], "bf16", O.QSpec("fp8"))
    parity = True
    for i in (0, a.pool - 1):
        c, m, s = (t.cpu().numpy() for t in houts[i])
        parity = parity and bool(np.array_equal(c[rows], wc) and np.array_equal(m[rows], wm)
                                 and np.array_equal(s[rows].view(np.uint32), wsc.view(np.uint32)))

    # ---- graphs for the timed steps, captured before the copy baseline so that no
    # idle gap precedes the timed region: a ring of RING launches over the pool
    # (a few hundred nodes or fewer run back to back; a 128-node ring measured
    # 0.06 us between kernels, an 8-node ring 1.1 us) and the K % RING rest --------
    RING = 128
    if use_graphs:
        ring = capture(lambda: [head(k % a.pool) for k in range(RING)]) if a.steps >= RING else None
        rest = a.steps % RING
        tail = capture(lambda: [head(k % a.pool) for k in range(rest)]) if rest else None

        def timed():
            for _ in range(a.steps // RING):
                ring.replay()
            if tail is not None:
                tail.replay()
    else:
        def timed():
            for k in range(a.steps):
                head(k % a.pool)

    # ================================================================================
    # Copy baseline: the library's copy kernel and a device-to-device copy over
    # copy_mib each, graph-replayed like the calls; the faster counts.  It runs
    # right before the headline's warmup, so the GPU is at sustained clocks
    # when the timed steps start.
    # ================================================================================
    nbytes = a.copy_mib << 20
    csrc = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    csrc.fill_(0x5A)
    cdst = torch.empty_like(csrc)
    creps = 30
    S.copy(csrc, cdst)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    marker("copy")
    if use_graphs:
        gk = capture(lambda: S.copy(csrc, cdst))
        gd = capture(lambda: cdst.copy_(csrc))
        kcopy_us = elapsed_us(lambda: [gk.replay() for _ in range(creps)]) / creps
        dcopy_us = elapsed_us(lambda: [gd.replay() for _ in range(creps)]) / creps
    else:
        kcopy_us = elapsed_us(lambda: [S.copy(csrc, cdst) for _ in range(creps)]) / creps
        dcopy_us = elapsed_us(lambda: [cdst.copy_(csrc) for _ in range(creps)]) / creps
    kcopy = 2 * nbytes / (kcopy_us * 1e-6) / 1e9
    dcopy = 2 * nbytes / (dcopy_us * 1e-6) / 1e9
    copy_gbps = max(kcopy, dcopy)
    del csrc, cdst

    # ---- headline warmup (W steps), then exactly K timed steps ----------------------
    marker("headline_warmup")
    for w in range(a.warmup):
        head(w % a.pool)
    marker("headline_timed")
    t0 = time.perf_counter()
    head_us_total = elapsed_us(timed)
    wall = time.perf_counter() - t0
    us_step = head_us_total / a.steps
    value = head_bytes / (us_step * 1e-6) / 1e9
    head_dispatches = {"parity_fill": a.pool, "warmup": a.warmup, "timed": a.steps}

    counters, counters_note = load_counters("pmc_traffic_heavy16384x4096.json")
    traffic = None
    if counters is not None and HEAD_KERNEL in counters.get("kernels", {}):
        traffic = counters["kernels"][HEAD_KERNEL]["traffic_bytes"]
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "traffic_note": counters_note, "kernel": HEAD_KERNEL,
                "algorithmic_bytes_per_launch": head_bytes, "avg_launch_us": round(us_step, 3)}

    per_call = {}
    extra = {}
    if not a.headline_only:
        per_call, extra = side_calls(a, S, W, O, torch, dev, bf, capture, elapsed_us, hx_bits,
                                     hpool, use_graphs, marker)

    # ================================================================================
    # CPU baseline: the oracle on a bounded sample of the headline workload.
    # ================================================================================
    cpu = None
    if not a.no_cpu_baseline:
        n = min(a.cpu_rows, NH)
        sub = np.ascontiguousarray(hx_bits[:n])
        passes = 0
        t1 = time.perf_counter()
        while True:
            O.prune_quantize(sub, "bf16", O.QSpec("fp8"))
            passes += 1
            dt = time.perf_counter() - t1
            if dt >= a.cpu_seconds or passes >= 8:
                break
        cpu = {"value": round(passes * head_bytes * n / NH / dt / 1e9, 5), "unit": "GB/s",
               "cores": 1, "kind": "oracle", "host_cpus": os.cpu_count(),
               "seconds": round(dt, 2),
               "sample": f"{passes} pass(es) of the fused 2:4 + FP8 call over rows 0..{n - 1} of "
                         f"the {NH}-row X (numpy, single-threaded)"}

    line = {
        "metric": "fused 2:4 prune+compress+quant GB/s (% of HBM peak); predicted-R tensors/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us_step * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "4x-tier activation X 16384x4096 bf16, Student-t(4) entries; step = "
                               "one fused 2:4 prune + compress + FP8-e4m3 call (per-token scale "
                               "of the kept values)",
                   "tokens": NH, "hidden": H, "pool": a.pool,
                   "pool_bytes": a.pool * NH * H * 2, "graphs": use_graphs},
        "fused_prune_quant_GBps": round(value, 1),
        "fused_prune_quant_pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "fused_prune_quant_pct_copy": round(100 * value / copy_gbps, 2),
        "copy_GBps": round(copy_gbps, 1),
        "copy": {"bytes": nbytes, "k_copy_GBps": round(kcopy, 1), "dtod_GBps": round(dcopy, 1),
                 "k_copy_us": round(kcopy_us, 2), "dtod_us": round(dcopy_us, 2)},
        "headline_dispatches": head_dispatches,
        **({"marker_phases": phases} if a.markers else {}),
        "parity_sampled_rows": parity,
        "wall_s": round(wall, 4),
        **extra,
        "per_call": per_call,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    if a.ops_jsonl:
        with open(a.ops_jsonl, "w") as fh:
            props = torch.cuda.get_device_properties(dev)
            gpu = f"{props.name} ({getattr(props, 'gcnArchName', '')})"
            for rec in op_records(line, gpu, torch.version.hip):
                fh.write(json.dumps(rec) + "\n")


def side_calls(a, S, W, O, torch, dev, bf, capture, elapsed_us, hx_bits, hpool, use_graphs, marker):
    """Every other call of the path, each on its own operand at full size, timed
    as graph replays of a rotation ring (>= 512 MB of operand per ring where
    the operand is smaller than that).  Returns (per_call, extra keys)."""
    T = H = 4096
    NW, NH = 14336, 16384
    seed = a.seed
    alloc = lambda *shape, dt=torch.uint8: torch.empty(*shape, dtype=dt, device=dev)  # noqa: E731

    # ---- linear-layer activation X [4096, 4096]: 16 copies (512 MiB) ----------------------
    x_bits = W.activation_x(seed, T, H)
    xpool = [bf(x_bits)]
    xpool += [xpool[0].clone() for _ in range(15)]
    xout = [{"pq": (alloc(T, H // 2), alloc(T, H // 8), alloc(T, dt=torch.float32)),
             "fp8": (alloc(T, H), alloc(T, dt=torch.float32), alloc(1, dt=torch.float32)),
             "int8": (alloc(T, H, dt=torch.int8), alloc(T, dt=torch.float32), alloc(1, dt=torch.float32)),
             "R": alloc(1, 2, 5, dt=torch.float64),
             "pc": (alloc(T, H // 2, dt=torch.bfloat16), alloc(T, H // 8)),
             "p48": (alloc(T, H // 2, dt=torch.bfloat16), alloc(T, H // 16)),
             "R48": alloc(1, 2, 5, dt=torch.float64),
             "pqr": (alloc(T, H // 2), alloc(T, H // 8), alloc(T, dt=torch.float32)),
             "Rr": alloc(1, 2, 5, dt=torch.float64),
             "had": alloc(T, H, dt=torch.bfloat16),
             "sfp4": (alloc(T, H // 4), alloc(T, H // 16), alloc(T, H // 32), alloc(1, dt=torch.float32))}
            for _ in range(16)]
    ws = alloc(1 << 20)
    ws_big = alloc(64 << 20)
    kept, dense = ["fp8", "fp8"], ["fp8", ("int", 8)]

    act_calls = {
        "act_prune_quantize_fp8": lambda i: S.prune_quantize(xpool[i], "fp8", out=xout[i]["pq"]),
        "act_quantize_fp8": lambda i: S.quantize(xpool[i], "fp8", out=xout[i]["fp8"]),
        "act_quantize_int8": lambda i: S.quantize(xpool[i], ("int", 8), out=xout[i]["int8"]),
        "act_predict_R": lambda i: S.predict_R(xpool[i], kept, dense, out=xout[i]["R"], workspace=ws),
    }
    xb = T * H * 2
    alg = {"act_prune_quantize_fp8": xb + T * H // 2 + T * H // 8 + T * 4,
           "act_quantize_fp8": xb + T * H + T * 4, "act_quantize_int8": xb + T * H + T * 4,
           "act_predict_R": xb + 2 * 5 * 8}
    step_bytes = sum(alg.values())

    rings = {}  # name -> (callable(i), ring length)
    for name, f in act_calls.items():
        rings[name] = (f, 16)
    rings.update({
        "act_prune_compress_2of4": (lambda i: S.prune_compress(xpool[i], out=xout[i]["pc"]), 16),
        "act_prune_compress_pairs48": (lambda i: S.prune_compress_pairs48(xpool[i], out=xout[i]["p48"]), 16),
        "act_predict_R_pairs48": (lambda i: S.predict_R_pairs48(xpool[i], kept, dense, out=xout[i]["R48"],
                                                                workspace=ws), 16),
        "act_prune_quantize_pairs48_nvfp4": (lambda i: S.prune_quantize_pairs48(
            xpool[i], "nvfp4", out=xout[i]["sfp4"], workspace=ws), 16),
        "act_hadamard128": (lambda i: S.hadamard(xpool[i], 128, out=xout[i]["had"]), 16),
        "act_prune_quantize_fp8_rot128": (lambda i: S.prune_quantize_rot(xpool[i], 128, "fp8",
                                                                         out=xout[i]["pqr"]), 16),
        "act_predict_R_rot128": (lambda i: S.predict_R_rot(xpool[i], 128, kept, dense, out=xout[i]["Rr"],
                                                           workspace=ws), 16),
        "act_prune_quantize_fp8_rot_row": (lambda i: S.prune_quantize_rot(xpool[i], H, "fp8",
                                                                          out=xout[i]["pqr"]), 16),
        "act_predict_R_rot_row": (lambda i: S.predict_R_rot(xpool[i], H, kept, dense, out=xout[i]["Rr"],
                                                            workspace=ws), 16),
    })
    alg.update({
        "act_prune_compress_2of4": xb + xb // 2 + T * H // 8,
        "act_prune_compress_pairs48": xb + xb // 2 + T * H // 16,
        "act_predict_R_pairs48": xb + 2 * 5 * 8,
        # one read of X (the kept-maximum pre-pass reads it a second time)
        "act_prune_quantize_pairs48_nvfp4": xb + T * H // 4 + T * H // 16 + T * H // 32 + 4,
        "act_hadamard128": 2 * xb,
        "act_prune_quantize_fp8_rot128": xb + T * H // 2 + T * H // 8 + T * 4,
        "act_predict_R_rot128": xb + 2 * 5 * 8,
        "act_prune_quantize_fp8_rot_row": xb + T * H // 2 + T * H // 8 + T * 4,
        "act_predict_R_rot_row": xb + 2 * 5 * 8,
    })

    # ---- weight W [14336, 4096]: 5 copies (560 MiB); norms of the activation's channels ----
    norms = S.col_l2norm(xpool[0])
    wpool = [bf(W.weight_w(seed + 1, NW, H))]
    wpool += [wpool[0].clone() for _ in range(4)]
    sweep_kept = [("int", 2 * m) for m in range(2, 9)]
    sweep_dense = [("int", m + 1) for m in range(2, 9)]
    r_sweep = alloc(1, len(sweep_kept), 5, dt=torch.float64)
    pc_w = (alloc(NW, H // 2, dt=torch.bfloat16), alloc(NW, H // 8))
    rings.update({
        "weight_prune_compress_wanda": (lambda i: S.prune_compress(wpool[i], score="wanda",
                                                                   col_norm=norms, out=pc_w), 5),
        "weight_predict_R_wanda_sweep": (lambda i: S.predict_R(
            wpool[i], sweep_kept, sweep_dense, score="wanda", col_norm=norms, out=r_sweep,
            workspace=ws_big), 5),
    })
    alg.update({
        "weight_prune_compress_wanda": NW * H * 2 + NW * H + NW * H // 8 + H * 4,
        "weight_predict_R_wanda_sweep": NW * H * 2 + H * 4 + len(sweep_kept) * 5 * 8,
    })

    # ---- heavy-tailed X [16384, 4096]: the headline pool (1 GiB) ----------------------------
    npool = len(hpool)
    mx_h = (alloc(NH, H // 2), alloc(NH, H // 32), alloc(1, dt=torch.float32))
    nv_h = (alloc(NH, H // 2), alloc(NH, H // 16), alloc(1, dt=torch.float32))
    r_heavy = alloc(NH // 128, 2, 5, dt=torch.float64)
    rings.update({
        "heavy_quantize_mxfp4": (lambda i: S.quantize(hpool[i], "mxfp4", out=mx_h), npool),
        "heavy_quantize_nvfp4": (lambda i: S.quantize(hpool[i], "nvfp4", out=nv_h, workspace=ws_big),
                                 npool),
        "heavy_predict_R_blocks128": (lambda i: S.predict_R(
            hpool[i], ["fp8", "fp8"], ["mxfp4", "nvfp4"], rows_per_block=128, out=r_heavy,
            workspace=ws_big), npool),
    })
    alg.update({
        "heavy_quantize_mxfp4": NH * H * 2 + NH * H // 2 + NH * H // 32,
        # one read of X (the tensor-maximum pass reads it a second time)
        "heavy_quantize_nvfp4": NH * H * 2 + NH * H // 2 + NH * H // 16 + 4,
        "heavy_predict_R_blocks128": NH * H * 2 + (NH // 128) * 2 * 5 * 8,
    })

    # ---- attention operands: Q 2 x 256 MiB, K / V 16 x 32 MiB, P 1 GiB ------------------
    q_att = bf(W.attention_qkv(seed + 3, 32, 16384, 128)).view(-1, 128)
    q_pool = [q_att, q_att.clone()]
    k_att = bf(W.attention_qkv(seed + 4, 8, 16384, 128)).view(-1, 128)
    k_pool = [k_att] + [k_att.clone() for _ in range(15)]
    v_att = bf(W.attention_qkv(seed + 5, 8, 16384, 128))
    v_pool = [v_att] + [v_att.clone() for _ in range(15)]
    p_att = bf(W.attention_p(seed + 6, 32, 4096, 4096)).view(-1, 4096)
    pc_q = (alloc(32 * 16384, 64, dt=torch.bfloat16), alloc(32 * 16384, 16))
    pc_k = (alloc(8 * 16384, 64, dt=torch.bfloat16), alloc(8 * 16384, 16))
    pc_v = (alloc(8, 128, 8192, dt=torch.bfloat16), alloc(8, 128, 2048))
    pc_p = (alloc(32 * 4096, 2048, dt=torch.bfloat16), alloc(32 * 4096, 512))
    r_p = alloc(32, 2, 5, dt=torch.float64)
    rings.update({
        "attn_prune_compress_Q": (lambda i: S.prune_compress(q_pool[i], out=pc_q), 2),
        "attn_prune_compress_K": (lambda i: S.prune_compress(k_pool[i], out=pc_k), 16),
        "attn_prune_compress_V_seq": (lambda i: S.prune_compress(v_pool[i], axis=1, out=pc_v), 16),
        "attn_prune_compress_P": (lambda i: S.prune_compress(p_att, out=pc_p), 1),
        "attn_predict_R_P_heads": (lambda i: S.predict_R(
            p_att, ["none", "none"], ["fp8", ("int", 8)], rows_per_block=4096, out=r_p,
            workspace=ws_big), 1),
    })
    qkv = 16384 * 128
    alg.update({
        "attn_prune_compress_Q": 32 * qkv * 2 + 32 * qkv + 32 * qkv // 8,
        "attn_prune_compress_K": 8 * qkv * 2 + 8 * qkv + 8 * qkv // 8,
        "attn_prune_compress_V_seq": 8 * qkv * 2 + 8 * qkv + 8 * qkv // 8,
        "attn_prune_compress_P": 32 * 4096 * 4096 * 2 + 32 * 4096 * 2048 * 2 + 32 * 4096 * 512,
        "attn_predict_R_P_heads": 32 * 4096 * 4096 * 2 + 32 * 2 * 5 * 8,
    })

    # ---- operator-level error and the GEMMs on X [4096, 4096] x W^T -------------------------
    w_op = wpool[0]
    op_sides = [("2:4", ("fp8", 0)), ("dense", ("fp8", 0))]
    op_out = alloc(T, 1 + len(op_sides), dt=torch.float64)
    op_ws = alloc(T * 2 * H * 2 + (1 + len(op_sides)) * T * ((NW + 127) // 128) * 4 + (1 << 20))
    c_gemm = alloc(T, NW, dt=torch.float32)
    w_codes, w_scales = S.quantize(w_op, "fp8")
    rings.update({
        "operator_error_2sides": (lambda i: S.operator_error(xpool[i], w_op, op_sides, out=op_out,
                                                             workspace=op_ws), 4),
        "gemm_sparse24_bf16": (lambda i: S.sparse_gemm(xout[i]["pc"][0], xout[i]["pc"][1], w_op,
                                                       out=c_gemm), 4),
        "gemm_dense_bf16": (lambda i: S.dense_gemm(xpool[i], w_op, out=c_gemm), 4),
        "gemm_dense_fp8": (lambda i: S.fp8_gemm(xout[i]["fp8"][0], xout[i]["fp8"][1], w_codes,
                                                w_scales, out=c_gemm), 4),
    })
    alg.update({
        "operator_error_2sides": xb + NW * H * 2,
        "gemm_sparse24_bf16": xb // 2 + T * H // 8 + NW * H * 2 + T * NW * 4,
        "gemm_dense_bf16": xb + NW * H * 2 + T * NW * 4,
        "gemm_dense_fp8": T * H + NW * H + T * NW * 4,
    })
    flops = {"operator_error_2sides": 2.0 * T * NW * H * (1 + 2 * len(op_sides)),
             "gemm_sparse24_bf16": 2.0 * T * NW * H, "gemm_dense_bf16": 2.0 * T * NW * H,
             "gemm_dense_fp8": 2.0 * T * NW * H}
    mfma_peak = {"gemm_dense_fp8": 5000.0, "gemm_sparse24_bf16": 5000.0}  # sparse: 2x dense bf16

    # first launches (fills every output the GEMMs consume), then graphs
    marker("side_fill")
    for name, (f, n) in rings.items():
        for i in range(n):
            f(i)
    torch.cuda.synchronize()
    # each call's graph walks its rotation ring until it holds at least 64
    # launches (short graphs add about a microsecond between kernels), and is
    # replayed until about side_reps * 16 launches are timed
    graphs, nodes = {}, {}
    for name, (f, n) in rings.items():
        nodes[name] = n * -(-64 // n)
        if use_graphs:
            graphs[name] = capture(lambda f=f, n=n, m=nodes[name]: [f(k % n) for k in range(m)])
    if use_graphs:
        step_graph = capture(lambda: [f(i) for i in range(16) for f in act_calls.values()])

    per_call = {}
    for name, (f, n) in rings.items():
        marker(name)
        m = nodes[name]
        reps = max(1, -(-a.side_reps * 16 // m))
        if use_graphs:
            us = elapsed_us(lambda: [graphs[name].replay() for _ in range(reps)]) / (reps * m)
        else:
            us = elapsed_us(lambda: [f(k % n) for _ in range(reps) for k in range(m)]) / (reps * m)
        per_call[name] = {"us": round(us, 3), "GBps": round(alg[name] / (us * 1e-6) / 1e9, 1),
                          "bytes": alg[name], "launches": reps * m}
        if name in flops:
            tf = flops[name] / (us * 1e-6) / 1e12
            pk = mfma_peak.get(name, 2500.0)
            per_call[name].update({"TFLOPs": round(tf, 1), "mfma_peak_TFLOPs": pk,
                                   "mfma_frac": round(tf / pk, 4)})

    # the activation's four-call step: one graph of 16 steps (one per pool entry)
    marker("act_step")
    nsteps = 16 * a.side_reps
    if use_graphs:
        step_us = elapsed_us(lambda: [step_graph.replay() for _ in range(a.side_reps)]) / nsteps
    else:
        step_us = elapsed_us(lambda: [f(k % 16) for k in range(nsteps)
                                      for f in act_calls.values()]) / nsteps

    # VALU roofline of the predict_R energy kernels (counter summary + live time)
    valu, valu_note = load_counters("pmc_valu_energy.json")
    r_roof = {}
    for name, key in (("weight_predict_R_wanda_sweep", "weight_sweep"),
                      ("heavy_predict_R_blocks128", "heavy_blocks128"),
                      ("act_predict_R", "act")):
        ent = {"bound": "alu", "peak": VALU_PEAK_TOPS, "unit": "T lane-ops/s",
               "call_us": per_call[name]["us"]}
        if valu is not None and key in valu.get("calls", {}):
            c = valu["calls"][key]
            alg_ops = c["algorithmic_lane_ops"]
            issued = c["valu_lane_ops"]
            t = per_call[name]["us"] * 1e-6
            ent.update({"achieved": round(alg_ops / t / 1e12, 3),
                        "frac": round(alg_ops / t / 1e12 / VALU_PEAK_TOPS, 4),
                        "issued": round(issued / t / 1e12, 3),
                        "issue_frac": round(issued / t / 1e12 / VALU_PEAK_TOPS, 4),
                        "algorithmic_lane_ops_per_elem": c["algorithmic_lane_ops_per_elem"],
                        "issued_lane_ops_per_elem": c["valu_lane_ops_per_elem"]})
        else:
            ent.update({"achieved": None, "frac": None, "note": valu_note})
        r_roof[key] = ent

    extra = {
        "predicted_R_tensors_per_s": round(1e6 / per_call["heavy_predict_R_blocks128"]["us"], 1),
        "predicted_R_note": "heavy-tailed X [16384, 4096]: 128 row blocks x (2:4+FP8 vs MXFP4, vs "
                            "NVFP4), NVFP4 tensor maximum included",
        "predicted_R_weight_sweep_tensors_per_s": round(
            1e6 / per_call["weight_predict_R_wanda_sweep"]["us"], 1),
        "predicted_R_act_tensors_per_s": round(1e6 / per_call["act_predict_R"]["us"], 1),
        "roofline_predict_R": r_roof,
        "act_step": {"workload": "linear-layer activation X 4096x4096 bf16, 4 outlier channels x50; "
                                 "2:4+FP8 (per-token), dense FP8 and INT8, predicted R for 2 pairs",
                     "us": round(step_us, 3), "GBps": round(step_bytes / (step_us * 1e-6) / 1e9, 1),
                     "bytes": step_bytes},
        # [PD §3] speed question at equal nominal tier: dense FP8 (online
        # quantization of X + FP8 GEMM) time over 2:4 bf16 (online
        # prune+compress of X + sparse GEMM) time; above 1 = 2:4 faster
        "speed_2of4_bf16_vs_dense_fp8": round(
            (per_call["act_quantize_fp8"]["us"] + per_call["gemm_dense_fp8"]["us"])
            / (per_call["act_prune_compress_2of4"]["us"] + per_call["gemm_sparse24_bf16"]["us"]), 3),
    }
    return per_call, extra


if __name__ == "__main__":
    main()
