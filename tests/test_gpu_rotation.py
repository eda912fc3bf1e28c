"""GPU parity of the block Hadamard rotation ([PD §4]) and of the calls that
fuse it into their load, against the oracle's rotate() followed by the
unrotated oracle functions.

Bit-exact wherever the oracle's exactness predicate holds (every test input
is checked), energies within 1e-6 relative."""
import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import pruning_quantization_amd as S  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import raw_np, to_dev  # noqa: E402
from test_gpu_parity import assert_same, check_pq, qs_oracle, rel_close  # noqa: E402

DTYPES = ["bf16", "f16", "f32"]
BLOCKS = [8, 16, 32, 64, 128, 256, 512]


def rot_inputs(seed, rows, k, dtype, kind="normal"):
    """Gaussian (or small-integer, tie-rich) operands; fp32 ones carry bf16
    values so that every block's Hadamard sums are exact in fp64."""
    rng = np.random.default_rng(seed)
    if kind == "ints":
        a = rng.integers(-4, 5, size=(rows, k)).astype(np.float64) * 2.0 ** rng.integers(-3, 3, size=(rows, k))
        a[rng.random((rows, k)) < 0.1] = -0.0
        a[: max(1, rows // 8)] = 0.0                                   # all-zero rows
    else:
        a = rng.standard_normal((rows, k))
        a[:, rng.integers(0, k, size=2)] *= 40.0                      # outlier channels
    if dtype == "bf16":
        raw = W.to_bf16_bits(a)
        raw[(a == 0) & np.signbit(a)] = 0x8000
    elif dtype == "f16":
        raw = a.astype(np.float16)
    else:
        raw = W.bf16_bits_to_f32(W.to_bf16_bits(a)).astype(np.float32)
        raw[(a == 0) & np.signbit(a)] = -0.0
    return raw


def exact(raw, dtype, n):
    ok = O.rotation_exact(raw, dtype, n)
    assert ok.all(), f"test input breaks the exactness condition in {(~ok).sum()} blocks"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", BLOCKS)
def test_hadamard(dtype, n):
    for k, kind in ((n, "normal"), (4 * n, "ints"), (max(n, 1024), "normal"), (max(2 * n, 4096), "normal")):
        raw = rot_inputs(n + k, 23, k, dtype, kind)
        exact(raw, dtype, n)
        got = S.hadamard(to_dev(raw, dtype), n)
        assert_same(raw_np(got), O.rotate(raw, dtype, n), f"rotate n={n} k={k} {kind}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [1024, 2048, 4096])
def test_hadamard_long_blocks(dtype, n):
    # blocks over one wave's 512 elements: stages across a lane's units
    for k, kind in ((n, "normal"), (8192, "ints"), (8192, "normal")):
        raw = rot_inputs(n + k + 1, 13, k, dtype, kind)
        exact(raw, dtype, n)
        got = S.hadamard(to_dev(raw, dtype), n)
        assert_same(raw_np(got), O.rotate(raw, dtype, n), f"rotate n={n} k={k} {kind}")


def test_hadamard_transposed_and_strided():
    rng = np.random.default_rng(3)
    raw = W.to_bf16_bits(rng.standard_normal((2, 256, 40)))
    got = S.hadamard(to_dev(raw, "bf16"), 128, axis=1)
    rows = np.ascontiguousarray(np.swapaxes(raw, 1, 2)).reshape(-1, 256)
    assert_same(raw_np(got).reshape(-1, 256), O.rotate(rows, "bf16", 128), "transposed")
    full = W.to_bf16_bits(rng.standard_normal((30, 1024 + 64)))
    got = S.hadamard(to_dev(full, "bf16")[:, :1024], 256)
    assert_same(raw_np(got), O.rotate(np.ascontiguousarray(full[:, :1024]), "bf16", 256), "strided")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [16, 128, 512, 1024, 2048])
def test_quantize_rot(dtype, n):
    k = 2048
    raw = rot_inputs(7 * n, 37, k, dtype)
    exact(raw, dtype, n)
    x = to_dev(raw, dtype)
    rot = O.rotate(raw, dtype, n)
    for q in (("fp8", 0), ("int", 8), ("int", 4)):
        c, s = S.quantize_rot(x, n, q)
        wc, ws = O.quantize_rows(rot, dtype, O.QSpec(*q))
        assert_same(raw_np(c), wc, f"codes {q}")
        assert_same(raw_np(s), ws, f"scales {q}")
    c, s = S.quantize_rot(x, n, "mxfp4")
    wc, ws = O.quantize_mxfp4(rot, dtype)
    assert_same(raw_np(c), wc, "mx codes")
    assert_same(raw_np(s), ws, "mx scales")
    c, s, t = S.quantize_rot(x, n, "nvfp4")
    wc, ws, wt = O.quantize_nvfp4(rot, dtype)
    assert_same(raw_np(c), wc, "nv codes")
    assert_same(raw_np(s), ws, "nv scales")
    assert_same(raw_np(t), np.array([wt], dtype=np.float32), "nv tensor scale")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [8, 128, 256, 1024])
def test_prune_quantize_rot(dtype, n):
    k = 1024
    for kind in ("normal", "ints"):
        raw = rot_inputs(11 * n, 29, k, dtype, kind)
        exact(raw, dtype, n)
        x = to_dev(raw, dtype)
        rot = O.rotate(raw, dtype, n)
        for q in (("fp8", 0), ("int", 4), ("nvfp4", 0), ("mxfp4", 0)):
            check_pq(S.prune_quantize_rot(x, n, q), O.prune_quantize(rot, dtype, O.QSpec(*q)),
                     f"2:4 rot {q} {kind}")
            check_pq(S.prune_quantize_rot(x, n, q, pattern="pairs4:8"),
                     O.prune_quantize_pairs48(rot, dtype, O.QSpec(*q)), f"4:8 rot {q} {kind}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [32, 128, 4096])
def test_predict_R_rot(dtype, n):
    k = 4096
    raw = rot_inputs(13 * n, 41, k, dtype)
    exact(raw, dtype, n)
    x = to_dev(raw, dtype)
    rot = O.rotate(raw, dtype, n)
    kept = ["fp8", "none", ("int", 4), "nvfp4"]
    dense = [("int", 8), "fp8", "mxfp4", "nvfp4"]
    ok, od = [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense]
    for pat in ("2:4", "pairs4:8"):
        got = S.predict_R_rot(x, n, kept, dense, pattern=pat, rows_per_block=16)
        rel_close(raw_np(got), O.predict_R(rot, dtype, ok, od, rows_per_block=16, pattern=pat))


def test_whole_row_rotation_on_4096_rows():
    # the whole-row rotation of a 4096-wide operand through every fused call
    raw = rot_inputs(5, 300, 4096, "bf16")
    exact(raw, "bf16", 4096)
    x = to_dev(raw, "bf16")
    rot = O.rotate(raw, "bf16", 4096)
    for q in (("fp8", 0), ("int", 8)):
        c, s = S.quantize_rot(x, 4096, q)
        wc, ws = O.quantize_rows(rot, "bf16", O.QSpec(*q))
        assert_same(raw_np(c), wc, f"codes {q}")
        assert_same(raw_np(s), ws, f"scales {q}")
    for q in (("fp8", 0), ("nvfp4", 0)):
        check_pq(S.prune_quantize_rot(x, 4096, q), O.prune_quantize(rot, "bf16", O.QSpec(*q)),
                 f"2:4 rot4096 {q}")
        check_pq(S.prune_quantize_rot(x, 4096, q, pattern="pairs4:8"),
                 O.prune_quantize_pairs48(rot, "bf16", O.QSpec(*q)), f"4:8 rot4096 {q}")
    c, s = S.quantize_rot(x, 4096, "mxfp4")
    wc, ws = O.quantize_mxfp4(rot, "bf16")
    assert_same(raw_np(c), wc, "mx codes")
    assert_same(raw_np(s), ws, "mx scales")


def test_rotation_raises_R_on_outlier_activations():
    # the pages' direction [PD §4] on the GPU: rotating X with 4 outlier
    # channels x50 raises R against FP8 and INT8
    raw = W.activation_x(0, 512, 4096)
    x = to_dev(raw, "bf16")
    kept, dense = ["fp8", "fp8"], ["fp8", ("int", 8)]
    r0 = raw_np(S.predict_R(x, kept, dense))[0]
    r1 = raw_np(S.predict_R_rot(x, 128, kept, dense))[0]
    assert (r1[:, 4] > 1.3 * r0[:, 4]).all()


@pytest.mark.parametrize("k,n", [(3072, 1024), (6144, 2048), (8192, 4096), (1024, 1024)])
def test_long_blocks_rows_not_filling_team_registers(k, n):
    # long blocks on whole-workgroup teams: rows whose units do not fill the
    # last register of 256 lanes (K = 3072, 6144), two 4096-element blocks
    # per row, and a row of one 1024-element block (half the lanes idle)
    raw = rot_inputs(k + n, 37, k, "bf16")
    exact(raw, "bf16", n)
    x = to_dev(raw, "bf16")
    rot = O.rotate(raw, "bf16", n)
    assert_same(raw_np(S.hadamard(x, n)), rot, f"rotate k={k} n={n}")
    check_pq(S.prune_quantize_rot(x, n, ("fp8", 0)), O.prune_quantize(rot, "bf16", O.QSpec("fp8", 0)),
             f"2:4 rot k={k} n={n}")
    c, s = S.quantize_rot(x, n, ("int", 8))
    wc, ws = O.quantize_rows(rot, "bf16", O.QSpec("int", 8))
    assert_same(raw_np(c), wc, f"codes k={k} n={n}")
    assert_same(raw_np(s), ws, f"scales k={k} n={n}")
    kept, dense = ["fp8", ("int", 4)], [("int", 8), "fp8"]
    ok, od = [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense]
    for rpb in (0, 16):
        got = S.predict_R_rot(x, n, kept, dense, rows_per_block=rpb)
        rel_close(raw_np(got), O.predict_R(rot, "bf16", ok, od, rows_per_block=rpb))
