"""Every call captured in one HIP graph (torch.cuda.graph) and replayed: each
replay must reproduce the eager outputs bit for bit.

Between replays the outputs are overwritten with a fill pattern and the same
shared workspace is used by eager calls on another operand, so a replay that
depended on state left by the capture run (a counter or partial sum that
should have been cleared, a stale workspace word) shows up as a mismatch.
The library issues no memset and allocates nothing, so its launches are the
only graph nodes."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import pruning_quantization_amd as S  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import DEV, t_bf16, t_f32  # noqa: E402

WS_BYTES = 64 << 20


def _calls(x, xf, w, norm, ws, ca, cb):
    """(name, fn(out) -> out) for every entry point: fn(None) allocates the
    outputs, fn(out) writes into them."""
    def q3(out):
        # quantize takes (codes, scales, tensor scale) and returns two of them
        # for INT / FP8 / MXFP4
        return None if out is None else (out[0], out[1], out[2] if len(out) > 2 else _ts)
    _ts = torch.empty(1, dtype=torch.float32, device=DEV)

    calls = [
        ("prune_compress", lambda o: S.prune_compress(x, out=o)),
        ("prune_compress_wanda", lambda o: S.prune_compress(x, score="wanda", col_norm=norm, out=o)),
        ("prune_compress_f32", lambda o: S.prune_compress(xf, out=o)),
        ("prune_quantize_fp8", lambda o: S.prune_quantize(x, "fp8", out=o, workspace=ws)),
        ("prune_quantize_int8", lambda o: S.prune_quantize(x, ("int", 8), out=o, workspace=ws)),
        ("prune_quantize_int4_wanda", lambda o: S.prune_quantize(x, ("int", 4), score="wanda",
                                                                 col_norm=norm, out=o, workspace=ws)),
        ("prune_quantize_mxfp4", lambda o: S.prune_quantize(x, "mxfp4", out=o, workspace=ws)),
        ("prune_quantize_nvfp4", lambda o: S.prune_quantize(x, "nvfp4", out=o, workspace=ws)),
        ("quantize_fp8", lambda o: S.quantize(x, "fp8", out=q3(o), workspace=ws)),
        ("quantize_int4", lambda o: S.quantize(x, ("int", 4), out=q3(o), workspace=ws)),
        ("quantize_mxfp4", lambda o: S.quantize(x, "mxfp4", out=q3(o), workspace=ws)),
        ("quantize_nvfp4", lambda o: S.quantize(x, "nvfp4", out=q3(o), workspace=ws)),
        ("quantize_f32_int8", lambda o: S.quantize(xf, ("int", 8), out=q3(o), workspace=ws)),
        ("prune_compress_pairs48", lambda o: S.prune_compress_pairs48(x, out=o)),
        ("prune_quantize_pairs48_nvfp4", lambda o: S.prune_quantize_pairs48(x, "nvfp4", out=o,
                                                                            workspace=ws)),
        ("hadamard128", lambda o: S.hadamard(x, 128, out=o, workspace=ws)),
        ("quantize_rot64_fp8", lambda o: S.quantize_rot(x, 64, "fp8", out=q3(o), workspace=ws)),
        ("prune_quantize_rot_row_fp8", lambda o: S.prune_quantize_rot(x, x.shape[-1], "fp8", out=o,
                                                                      workspace=ws)),
        ("col_l2norm", lambda o: S.col_l2norm(x, out=o, workspace=ws)),
        ("error_energy_blocks", lambda o: S.error_energy(x, "fp8", ("int", 8), rows_per_block=64,
                                                         out=o, workspace=ws)),
        ("predict_R", lambda o: S.predict_R(x, ["fp8", "fp8"], ["fp8", ("int", 8)], out=o,
                                            workspace=ws)),
        ("predict_R_blocks_fp4", lambda o: S.predict_R(x, ["fp8", "fp8"], ["mxfp4", "nvfp4"],
                                                       rows_per_block=128, out=o, workspace=ws)),
        ("predict_R_wanda", lambda o: S.predict_R(x, [("int", 4)], [("int", 4)], score="wanda",
                                                  col_norm=norm, out=o, workspace=ws)),
        ("predict_R_f32", lambda o: S.predict_R(xf, ["fp8"], [("int", 8)], out=o, workspace=ws)),
        ("predict_R_pairs48", lambda o: S.predict_R_pairs48(x, ["fp8"], ["fp8"], out=o, workspace=ws)),
        ("predict_R_rot128", lambda o: S.predict_R_rot(x, 128, ["fp8"], [("int", 8)], out=o,
                                                       workspace=ws)),
        ("predict_R_rot_row", lambda o: S.predict_R_rot(x, x.shape[-1], ["fp8"], [("int", 8)], out=o,
                                                        workspace=ws)),
        ("operator_error", lambda o: S.operator_error(x, w, [("2:4", "fp8"), ("dense", "fp8")],
                                                      out=o, workspace=ws)),
        ("dense_gemm", lambda o: S.dense_gemm(x, w, out=o)),
        ("fp8_gemm", lambda o: S.fp8_gemm(*ca, *cb, out=o)),
    ]
    return calls


def _flat(out):
    return list(out) if isinstance(out, (tuple, list)) else [out]


def _bytes(t):
    return t.contiguous().view(torch.uint8).reshape(-1)


def test_graph_replays_match_eager():
    rng = np.random.default_rng(20240611)
    # 300 rows (several workgroups and a ragged last one) of 4096 elements,
    # with outlier channels as in the activation workload
    x = t_bf16(W.activation_x(11, 300, 4096))
    xf = t_f32(rng.standard_normal((193, 1024)))
    w = t_bf16(W.weight_w(12, 320, 4096))
    norm = S.col_l2norm(x)
    other = t_bf16(W.activation_x(13, 300, 4096))  # eager work between replays
    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device=DEV)
    ca, cb = S.quantize(x, "fp8"), S.quantize(w, "fp8")  # fp8_gemm operands
    calls = _calls(x, xf, w, norm, ws, ca, cb)

    outs = {n: f(None) for n, f in calls}
    torch.cuda.synchronize()
    # a second eager pass into the same buffers is the reference
    for n, f in calls:
        f(outs[n])
    torch.cuda.synchronize()
    ref = {n: [_bytes(t).clone() for t in _flat(o)] for n, o in outs.items()}

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for n, f in calls:
                f(outs[n])
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs.values():
            for t in _flat(o):
                _bytes(t).fill_(0xA5 + rep)
        # eager library work on another operand through the same workspace
        S.predict_R(other, ["fp8", "fp8"], ["fp8", ("int", 8)], workspace=ws)
        S.predict_R(other, ["fp8"], ["nvfp4"], rows_per_block=64, workspace=ws)
        S.quantize(other, "nvfp4", workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, o in outs.items():
            got = [_bytes(t) for t in _flat(o)]
            assert len(got) == len(ref[n]), n
            for i, (a, b) in enumerate(zip(got, ref[n])):
                assert torch.equal(a, b), f"replay {rep}: {n} output {i} differs from the eager result"
