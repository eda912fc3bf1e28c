"""GPU parity: the HIP library (through its C ABI) against the CPU oracle,
element by element on the same seeded inputs.

Bar: bit-exact masks, metadata, kept values, codes and scales; energies and
R within 1e-6 relative; Wanda norms within 1 fp32 ulp.  Shapes span several
tiles/teams and ragged tails; inputs include ties, signed zeros, subnormals,
all-zero rows and saturating values.
"""
import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import pruning_quantization_amd as S  # noqa: E402
from gpu_util import raw_np, random_raw, tie_heavy_raw, to_dev  # noqa: E402

DTYPES = ["bf16", "f16", "f32"]
# K values: team shapes 16x1 .. 256x16 and ragged unit counts
KS = [8, 24, 128, 136, 256, 520, 1024, 4096, 4104, 8192, 16384]


def inputs(seed, rows, k, dtype, kind):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        return tie_heavy_raw(rng, (rows, k), dtype)
    raw = random_raw(rng, (rows, k), dtype)
    return raw


def assert_same(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert got.dtype == want.dtype, (what, got.dtype, want.dtype)
    if got.dtype.kind == "f":           # compare bit patterns (keeps -0 and +0 apart)
        ui = {2: np.uint16, 4: np.uint32, 8: np.uint64}[got.dtype.itemsize]
        got, want = got.view(ui), want.view(ui)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


# ---------------------------------------------------------------------------
# prune_compress
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [8, 24, 128, 520, 4096, 4104])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_prune_compress_magnitude(dtype, k, kind):
    rows = 37
    raw = inputs(k * 7 + len(dtype), rows, k, dtype, kind)
    x = to_dev(raw, dtype)
    v, m = S.prune_compress(x)
    torch.cuda.synchronize()
    wv, wm = O.prune_compress(raw, dtype)
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(v), wv, "values")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prune_compress_strided_rows(dtype):
    # rows taken from a wider buffer: row stride > K exercises the row-team path
    rng = np.random.default_rng(5)
    full = random_raw(rng, (50, 1024 + 64), dtype)
    x = to_dev(full, dtype)[:, :1024]
    v, m = S.prune_compress(x)
    wv, wm = O.prune_compress(np.ascontiguousarray(full[:, :1024]), dtype)
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(v), wv, "values")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [24, 128, 4096])
def test_prune_compress_wanda(dtype, k):
    rng = np.random.default_rng(k)
    raw = tie_heavy_raw(rng, (29, k), dtype)
    norm = (rng.integers(0, 5, size=k) * 0.75).astype(np.float32)  # ties and zeros
    norm[: k // 8] = rng.random(k // 8).astype(np.float32) * 3
    x = to_dev(raw, dtype)
    n = torch.from_numpy(norm).cuda()
    v, m = S.prune_compress(x, score="wanda", col_norm=n)
    wv, wm = O.prune_compress(raw, dtype, "wanda", norm)
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(v), wv, "values")


@pytest.mark.parametrize("view", ["batch_strided", "row_strided", "k16", "k4112", "k8192"])
def test_prune_compress_wanda_bf16_rows(view):
    # bf16 Wanda rows with K % 16 == 0 run on persistent whole-workgroup teams
    # (norms held per lane, several rows per workgroup when rows exceed the
    # grid, batches stepped with the rows); ragged pair counts and strided views
    rng = np.random.default_rng(len(view))
    if view == "batch_strided":
        full = tie_heavy_raw(rng, (2 * 1600, 528), "bf16").reshape(2, 1600, 528)
        raw = np.ascontiguousarray(full[:, :1500, :])
        x = to_dev(full, "bf16")[:, :1500, :]
    elif view == "row_strided":
        full = random_raw(rng, (3000, 544), "bf16")
        raw = np.ascontiguousarray(full[:, :528])
        x = to_dev(full, "bf16")[:, :528]
    else:
        k = int(view[1:])
        raw = random_raw(rng, (37 if k > 16 else 3000, k), "bf16")
        x = to_dev(raw, "bf16")
    k = raw.shape[-1]
    norm = (rng.integers(0, 5, size=k) * 0.75).astype(np.float32)
    norm[: k // 2] = rng.random(k // 2).astype(np.float32) * 3
    n = torch.from_numpy(norm).cuda()
    v, m = S.prune_compress(x, score="wanda", col_norm=n)
    flat = raw.reshape(-1, k)
    wv, wm = O.prune_compress(flat, "bf16", "wanda", norm)
    assert_same(raw_np(m).reshape(-1, k // 8), wm, "meta")
    assert_same(raw_np(v).reshape(-1, k // 2), wv, "values")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 136, 72), (1, 256, 128), (3, 40, 8), (2, 16392, 128)])
def test_prune_compress_transposed(dtype, shape):
    # V [heads, seq, dim] pruned along seq (axis 1)
    rng = np.random.default_rng(sum(shape))
    raw = random_raw(rng, shape, dtype)
    x = to_dev(raw, dtype)
    v, m = S.prune_compress(x, axis=1)
    assert v.shape == (shape[0], shape[2], shape[1] // 2)
    rows = np.ascontiguousarray(np.swapaxes(raw, 1, 2)).reshape(-1, shape[1])
    wv, wm = O.prune_compress(rows, dtype)
    assert_same(raw_np(m).reshape(-1, shape[1] // 8), wm, "meta")
    assert_same(raw_np(v).reshape(-1, shape[1] // 2), wv, "values")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 256, 128), (3, 512, 64), (2, 1024, 192), (8, 16384, 128)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_prune_compress_transposed_register_blocks(dtype, shape, kind):
    # 16-bit V with dims % 64 == 0 and seq % 256 == 0: the kernel that transposes
    # 8 x 8 blocks in registers (the V shape of 16K-token attention included)
    rng = np.random.default_rng(sum(shape) + len(kind))
    flat = (shape[0] * shape[1], shape[2])
    raw = (tie_heavy_raw(rng, flat, dtype) if kind == "ties" else random_raw(rng, flat, dtype)).reshape(shape)
    x = to_dev(raw, dtype)
    v, m = S.prune_compress(x, axis=1)
    rows = np.ascontiguousarray(np.swapaxes(raw, 1, 2)).reshape(-1, shape[1])
    pick = np.unique(np.r_[0:9, rows.shape[0] - 9:rows.shape[0],
                           rng.choice(rows.shape[0], size=min(40, rows.shape[0]), replace=False)])
    wv, wm = O.prune_compress(rows[pick], dtype)
    assert_same(raw_np(m).reshape(-1, shape[1] // 8)[pick], wm, "meta")
    assert_same(raw_np(v).reshape(-1, shape[1] // 2)[pick], wv, "values")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_transposed_rows_not_filling_chunks(dtype):
    # rows along the contiguous axis padded to 72 (16-byte aligned positions)
    # but only 68 / 3 used: tiles end inside a 16-byte chunk
    rng = np.random.default_rng(77)
    for used in (68, 3):
        raw = random_raw(rng, (2, 136, 72), dtype)
        x = to_dev(raw, dtype)[:, :, :used]
        rows = np.ascontiguousarray(np.swapaxes(raw[:, :, :used], 1, 2)).reshape(-1, 136)
        v, m = S.prune_compress(x, axis=1)
        wv, wm = O.prune_compress(rows, dtype)
        assert_same(raw_np(m).reshape(-1, 17), wm, f"meta {used}")
        assert_same(raw_np(v).reshape(-1, 68), wv, f"values {used}")
        c, sc = S.quantize(x, "fp8", axis=1)                       # staged through the transpose
        wc, ws = O.quantize_rows(rows, dtype, O.QSpec("fp8"))
        assert_same(raw_np(sc).reshape(-1), ws, f"fp8 scales {used}")
        assert_same(raw_np(c).reshape(-1, 136), wc, f"fp8 codes {used}")


# ---------------------------------------------------------------------------
# prune_quantize
# ---------------------------------------------------------------------------

QS = [("fp8", 0), ("int", 2), ("int", 3), ("int", 4), ("int", 8), ("int", 9), ("int", 16)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", KS)
def test_prune_quantize_fp8_int8(dtype, k):
    rows = 21 if k <= 4104 else 5
    for kind in ("normal", "ties"):
        raw = inputs(k + 3, rows, k, dtype, kind)
        x = to_dev(raw, dtype)
        for fmt, bits in (("fp8", 0), ("int", 8)):
            c, m, s = S.prune_quantize(x, (fmt, bits))
            wc, wm, ws = O.prune_quantize(raw, dtype, O.QSpec(fmt, bits))
            assert_same(raw_np(m), wm, f"meta {fmt}")
            assert_same(raw_np(s), ws, f"scales {fmt}")
            assert_same(raw_np(c), wc, f"codes {fmt}")


@pytest.mark.parametrize("dtype,rows,k,q,sample", [
    ("bf16", 16384, 4096, ("fp8", 0), False),    # the 16384-token activation, every row
    ("bf16", 16384, 4096, ("int", 8), False),
    ("f16", 20000, 512, ("fp8", 0), False),      # one-wave teams, four rows per workgroup
    ("bf16", 6000, 16384, ("int", 16), True),    # whole-workgroup teams
])
def test_prune_quantize_many_rows(dtype, rows, k, q, sample):
    # 16-bit magnitude 2:4 + INT/FP8 at full operand sizes (the grid's last
    # workgroups, ragged team counts, whole-workgroup teams): every row, or a
    # spread sample of rows, against the oracle, bit for bit
    rng = np.random.default_rng(rows + k)
    raw = random_raw(rng, (rows, k), dtype, scale=3.0)
    raw[rows // 3] = 0                                # an all-zero row
    x = to_dev(raw, dtype)
    c, m, s = S.prune_quantize(x, q)
    pick = (np.unique(np.r_[0:8, rows - 8:rows, rng.choice(rows, 300, replace=False)])
            if sample else np.arange(rows))
    wc, wm, ws = O.prune_quantize(raw[pick], dtype, O.QSpec(*q))
    assert_same(raw_np(m)[pick], wm, "meta")
    assert_same(raw_np(s)[pick], ws, "scales")
    assert_same(raw_np(c)[pick], wc, "codes")


@pytest.mark.parametrize("fmt,bits", QS)
@pytest.mark.parametrize("score", ["magnitude", "wanda"])
def test_prune_quantize_formats(fmt, bits, score):
    rng = np.random.default_rng(bits + 100)
    k = 1024
    raw = inputs(bits, 45, k, "bf16", "normal")
    norm = (rng.random(k) * 2).astype(np.float32)
    x = to_dev(raw, "bf16")
    n = torch.from_numpy(norm).cuda() if score == "wanda" else None
    c, m, s = S.prune_quantize(x, (fmt, bits), score=score, col_norm=n)
    wc, wm, ws = O.prune_quantize(raw, "bf16", O.QSpec(fmt, bits), score, norm if n is not None else None)
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(s), ws, "scales")
    assert_same(raw_np(c), wc, "codes")


def test_prune_quantize_k32768_and_tiny_rows():
    rng = np.random.default_rng(9)
    raw = random_raw(rng, (3, 32768), "bf16")
    raw[1] = 0x8000                         # all -0
    raw[2, ::3] = 0x0001                    # subnormals mixed in
    x = to_dev(raw, "bf16")
    c, m, s = S.prune_quantize(x, ("fp8", 0))
    wc, wm, ws = O.prune_quantize(raw, "bf16", O.QSpec("fp8"))
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(s), ws, "scales")
    assert_same(raw_np(c), wc, "codes")


# ---------------------------------------------------------------------------
# dense quantizers
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [8, 128, 136, 1024, 4096, 16384])
@pytest.mark.parametrize("fmt,bits", [("fp8", 0), ("int", 3), ("int", 8), ("int", 12)])
def test_quantize_rows(dtype, k, fmt, bits):
    rows = 19 if k <= 4096 else 4
    raw = inputs(k + bits, rows, k, dtype, "ties" if k % 3 else "normal")
    x = to_dev(raw, dtype)
    c, s = S.quantize(x, (fmt, bits))
    wc, ws = O.quantize_rows(raw, dtype, O.QSpec(fmt, bits))
    assert_same(raw_np(s), ws, "scales")
    assert_same(raw_np(c), wc, "codes")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [32, 96, 1024, 4096, 4128])
def test_quantize_mxfp4(dtype, k):
    for kind in ("normal", "ties"):
        raw = inputs(k, 23, k, dtype, kind)
        x = to_dev(raw, dtype)
        c, s = S.quantize(x, "mxfp4")
        wc, ws = O.quantize_mxfp4(raw, dtype)
        assert_same(raw_np(s), ws, "e8m0")
        assert_same(raw_np(c), wc, "codes")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [16, 48, 1024, 4096, 4112])
def test_quantize_nvfp4(dtype, k):
    for kind in ("normal", "ties"):
        raw = inputs(k + 1, 23, k, dtype, kind)
        x = to_dev(raw, dtype)
        c, s, ts = S.quantize(x, "nvfp4")
        wc, ws, wts = O.quantize_nvfp4(raw, dtype)
        assert raw_np(ts)[0] == wts
        assert_same(raw_np(s), ws, "e4m3 block scales")
        assert_same(raw_np(c), wc, "codes")
    # caller-supplied tensor maximum
    t = np.float32(37.5)
    c, s, ts = S.quantize(x, "nvfp4", tensor_amax=torch.tensor([t], device="cuda"))
    wc, ws, wts = O.quantize_nvfp4(raw, dtype, tensor_amax=float(t))
    assert raw_np(ts)[0] == wts
    assert_same(raw_np(s), ws, "block scales (given T)")
    assert_same(raw_np(c), wc, "codes (given T)")


# ---------------------------------------------------------------------------
# energies and predicted R
# ---------------------------------------------------------------------------

PAIRS_C2 = [(("int", 2 * m), ("int", m + 1)) for m in range(2, 9)]


def rel_close(got, want, rtol=1e-6):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    same_nonfinite = (np.isnan(got) & np.isnan(want)) | (np.isinf(got) & (got == want))
    ok = same_nonfinite | (np.abs(got - want) <= rtol * np.abs(want)) | ((want == 0) & (got == 0))
    assert ok.all(), f"{(~ok).sum()} of {ok.size} differ; first got {got[~ok][:3]} want {want[~ok][:3]}"


def qs_oracle(q):
    return O.QSpec(q) if isinstance(q, str) else O.QSpec(*q)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [32, 128, 1024, 4096, 16384])
def test_error_energy(dtype, k):
    rows = 40 if k <= 4096 else 6
    raw = inputs(k + 11, rows, k, dtype, "normal")
    x = to_dev(raw, dtype)
    for kept, dense in [("fp8", ("int", 8)), (("int", 4), "fp8"), ("none", "mxfp4"), ("fp8", "nvfp4")]:
        got = S.error_energy(x, kept, dense, rows_per_block=16)
        want = O.error_energy(raw, dtype, qs_oracle(kept), qs_oracle(dense), rows_per_block=16)
        rel_close(raw_np(got), want)


def test_predict_R_sweep_and_wanda():
    rng = np.random.default_rng(21)
    k = 4096
    raw = inputs(21, 33, k, "bf16", "normal")
    norm = (rng.random(k) * 3).astype(np.float32)
    x = to_dev(raw, "bf16")
    kept = [p[0] for p in PAIRS_C2]
    dense = [p[1] for p in PAIRS_C2]
    for score in ("magnitude", "wanda"):
        n = torch.from_numpy(norm).cuda() if score == "wanda" else None
        got = S.predict_R(x, kept, dense, score=score, col_norm=n)
        want = O.predict_R(raw, "bf16", [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                           score, norm if n is not None else None)
        rel_close(raw_np(got), want)


def wanda_colliding_inputs(seed, rows, k):
    """bf16 weights and fp32 norms whose Wanda products |w| * n often round to
    the same fp32 value (or agree in all but their last 8 bits) while the exact
    products differ or tie: |w| from {0, 0.5, 1, 1.5, 2, 3} (random signs),
    norms from values such as fp32(1/3), fp32(2/3), 1 + 2^-23 and 1 + 2^-20,
    so that e.g. 3 * fp32(1/3) and 1 * 1 fall on one fp32 but rank apart
    exactly.  The selection must still be the exact one (ties to the lower
    position)."""
    rng = np.random.default_rng(seed)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0])
    w = mags[rng.integers(0, len(mags), size=(rows, k))] * rng.choice([-1.0, 1.0], size=(rows, k))
    import workloads as W
    raw = W.to_bf16_bits(w)
    cands = np.array([1.0, np.float32(1 / 3), np.float32(2 / 3), 1 + 2.0 ** -23, 1 + 2.0 ** -20,
                      0.5, 2.0, 0.0, np.float32(1 / 3) * (1 + 2.0 ** -22)], dtype=np.float32)
    norm = cands[rng.integers(0, len(cands), size=k)].astype(np.float32)
    return raw, norm


@pytest.mark.parametrize("k", [1088, 4096])
def test_wanda_energies_with_colliding_fp32_products(k):
    # the energy kernels rank Wanda scores by fp32 products and fall back to
    # the exact fp64 ranking where those leave the kept set open
    raw, norm = wanda_colliding_inputs(k, 70, k)
    x = to_dev(raw, "bf16")
    n = torch.from_numpy(norm).cuda()
    for kept, dense, rpb in [([("int", 4), "fp8"], [("int", 3), ("int", 8)], 0),
                             ([("int", 6), "mxfp4"], ["nvfp4", ("int", 4)], 16)]:
        got = S.predict_R(x, kept, dense, score="wanda", col_norm=n, rows_per_block=rpb)
        want = O.predict_R(raw, "bf16", [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                           "wanda", norm, rows_per_block=rpb)
        rel_close(raw_np(got), want)
    # the prune kernels rank the same way
    v, m = S.prune_compress(x, score="wanda", col_norm=n)
    wv, wm = O.prune_compress(raw, "bf16", "wanda", norm)
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(v), wv, "values")
    for fmt, bits in (("fp8", 0), ("int", 4)):
        c, m, s = S.prune_quantize(x, (fmt, bits), score="wanda", col_norm=n)
        wc, wm, ws = O.prune_quantize(raw, "bf16", O.QSpec(fmt, bits), "wanda", norm)
        assert_same(raw_np(m), wm, f"meta {fmt}")
        assert_same(raw_np(s), ws, f"scales {fmt}")
        assert_same(raw_np(c), wc, f"codes {fmt}")


def test_predict_R_blocks_degenerate_and_deterministic():
    raw = inputs(5, 300, 256, "bf16", "ties")
    raw[:128] = 0                                   # first block all zero -> NaN
    x = to_dev(raw, "bf16")
    kept = ["fp8", "fp8", "none"]
    dense = ["mxfp4", "nvfp4", ("int", 8)]
    a = S.predict_R(x, kept, dense, rows_per_block=128)
    b = S.predict_R(x, kept, dense, rows_per_block=128)
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))     # bitwise repeatable
    want = O.predict_R(raw, "bf16", [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                       rows_per_block=128)
    assert np.isnan(raw_np(a)[0]).all()
    rel_close(raw_np(a), want)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,rows", [(4096, 300), (16384, 40)])
def test_predict_R_whole_operand_multi_wave_teams(dtype, k, rows):
    """Whole-operand predict_R (one block, per-workgroup partial slots): rows
    of 4096 and 16384 elements run on teams of two and four waves, and a
    workgroup can hold two teams.  Regression for teams of several waves that
    added into one shared slot: the sums must match the oracle and repeat bit
    for bit."""
    raw = inputs(k + rows, rows, k, dtype, "normal")
    x = to_dev(raw, dtype)
    kept = ["fp8", ("int", 4), "none"]
    dense = [("int", 8), "fp8", "mxfp4"]
    a = S.predict_R(x, kept, dense)
    b = S.predict_R(x, kept, dense)
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))
    want = O.predict_R(raw, dtype, [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense])
    rel_close(raw_np(a), want)
    got = S.predict_R_pairs48(x, ["fp8", "none"], [("int", 8), "nvfp4"])
    want = O.predict_R(raw, dtype, [O.QSpec("fp8"), O.QSpec("none")],
                       [O.QSpec("int", 8), O.QSpec("nvfp4")], pattern="pairs4:8")
    rel_close(raw_np(got), want)


def test_col_l2norm_within_one_ulp():
    import workloads as W
    raw = W.activation_x(3, 512, 1024)
    x = to_dev(raw, "bf16")
    got = raw_np(S.col_l2norm(x))
    want = O.col_l2norm(raw, "bf16")
    assert np.all(np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64)) <= 1)


def test_copy_kernel():
    a = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    S.copy(a, b)
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# transposed operands (V along seq) through every call
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("shape", [(2, 160, 72), (3, 1056, 128), (1, 4128, 24)])
def test_transposed_quantize_prune_quantize_and_energy(shape):
    rng = np.random.default_rng(shape[1])
    raw = random_raw(rng, shape, "bf16")
    x = to_dev(raw, "bf16")
    rows = np.ascontiguousarray(np.swapaxes(raw, 1, 2)).reshape(-1, shape[1])
    nr, k = rows.shape
    for fmt, bits in (("fp8", 0), ("int", 8)):
        c, s = S.quantize(x, (fmt, bits), axis=1)
        wc, ws = O.quantize_rows(rows, "bf16", O.QSpec(fmt, bits))
        assert_same(raw_np(s).reshape(nr), ws, "scales")
        assert_same(raw_np(c).reshape(nr, k), wc, "codes")
        pc, pm, ps = S.prune_quantize(x, (fmt, bits), axis=1)
        wc, wm, ws = O.prune_quantize(rows, "bf16", O.QSpec(fmt, bits))
        assert_same(raw_np(pm).reshape(nr, k // 8), wm, "meta")
        assert_same(raw_np(ps).reshape(nr), ws, "scales")
        assert_same(raw_np(pc).reshape(nr, k // 2), wc, "codes")
    c, sc = S.quantize(x, "mxfp4", axis=1)
    wc, wsc = O.quantize_mxfp4(rows, "bf16")
    assert_same(raw_np(c).reshape(nr, k // 2), wc, "mx codes")
    assert_same(raw_np(sc).reshape(nr, k // 32), wsc, "mx scales")
    c, sc, ts = S.quantize(x, "nvfp4", axis=1)
    wc, wsc, wts = O.quantize_nvfp4(rows, "bf16")
    assert raw_np(ts)[0] == wts
    assert_same(raw_np(c).reshape(nr, k // 2), wc, "nv codes")
    kept, dense = ["none", "none", "fp8"], ["fp8", ("int", 8), "nvfp4"]
    got = S.predict_R(x, kept, dense, axis=1, rows_per_block=shape[2])
    want = O.predict_R(rows, "bf16", [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                       rows_per_block=shape[2])
    rel_close(raw_np(got), want)


# ---------------------------------------------------------------------------
# pairwise 4:8 ([PD §6])
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [16, 48, 1024, 4096, 4112])
def test_prune_compress_pairs48(dtype, k):
    for kind in ("normal", "ties"):
        raw = inputs(k + 5, 19, k, dtype, kind)
        x = to_dev(raw, dtype)
        v, m = S.prune_compress_pairs48(x)
        wv, wm = O.prune_compress_pairs48(raw, dtype)
        assert_same(raw_np(m), wm, "meta")
        assert_same(raw_np(v), wv, "values")


def test_prune_compress_pairs48_strided_rows():
    rng = np.random.default_rng(48)
    full = random_raw(rng, (21, 2048 + 32), "bf16")
    x = to_dev(full, "bf16")[:, 16:16 + 2048]
    v, m = S.prune_compress_pairs48(x)
    wv, wm = O.prune_compress_pairs48(np.ascontiguousarray(full[:, 16:16 + 2048]), "bf16")
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(v), wv, "values")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [16, 128, 4096])
def test_predict_R_pairs48(dtype, k):
    raw = inputs(k + 9, 37, k, dtype, "normal")
    x = to_dev(raw, dtype)
    kept = ["none", "fp8", ("int", 4), "fp8"]
    dense = ["fp8", ("int", 8), ("int", 3), "nvfp4"]
    got = S.predict_R_pairs48(x, kept, dense, rows_per_block=8)
    want = O.predict_R(raw, dtype, [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                       rows_per_block=8, pattern="pairs4:8")
    rel_close(raw_np(got), want)
    if k % 32 == 0:
        got = S.predict_R_pairs48(x, ["none"], ["mxfp4"])
        want = O.predict_R(raw, dtype, [O.QSpec("none")], [O.QSpec("mxfp4")], pattern="pairs4:8")
        rel_close(raw_np(got), want)


# ---------------------------------------------------------------------------
# Block formats on kept values and the sparse FP4 operand ([PD §3], [PD §6])
# ---------------------------------------------------------------------------


def check_pq(got, want, what):
    names = ("codes", "meta", "scales", "tensor scale")
    assert len(got) == len(want), (what, len(got), len(want))
    for g, w, n in zip(got, want, names):
        g = raw_np(g)
        w = np.asarray(w)
        if n == "tensor scale":
            g, w = g.reshape(-1)[:1], np.asarray([w], dtype=np.float32)
        assert_same(g, w, f"{what} {n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [64, 128, 1088, 4096])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_prune_quantize_block_kept(dtype, k, fmt):
    for kind in ("normal", "ties"):
        raw = inputs(k + 17, 23, k, dtype, kind)
        x = to_dev(raw, dtype)
        check_pq(S.prune_quantize(x, fmt), O.prune_quantize(raw, dtype, O.QSpec(fmt)),
                 f"2:4 {fmt} {kind}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_prune_quantize_block_kept_wanda(fmt):
    rng = np.random.default_rng(61)
    k = 1024
    raw = inputs(62, 31, k, "bf16", "ties")
    norm = (rng.integers(0, 4, size=k) * 0.5 + rng.random(k) * (rng.random(k) < 0.5)).astype(np.float32)
    x = to_dev(raw, "bf16")
    n = torch.from_numpy(norm).cuda()
    got = S.prune_quantize(x, fmt, score="wanda", col_norm=n)
    check_pq(got, O.prune_quantize(raw, "bf16", O.QSpec(fmt), "wanda", norm), f"wanda {fmt}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [16, 48, 1024, 4096, 4112, 8192])
def test_prune_quantize_pairs48_rows(dtype, k):
    rows = 19 if k <= 4112 else 5
    for kind in ("normal", "ties"):
        raw = inputs(k + 29, rows, k, dtype, kind)
        x = to_dev(raw, dtype)
        for fmt, bits in (("fp8", 0), ("int", 8), ("int", 4), ("int", 12)):
            got = S.prune_quantize_pairs48(x, (fmt, bits))
            check_pq(got, O.prune_quantize_pairs48(raw, dtype, O.QSpec(fmt, bits)),
                     f"4:8 {fmt}{bits} {kind}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [32, 64, 1024, 4096, 4160])
def test_prune_quantize_pairs48_fp4(dtype, k):
    for kind in ("normal", "ties"):
        raw = inputs(k + 31, 27, k, dtype, kind)
        x = to_dev(raw, dtype)
        fmts = ["nvfp4"] + (["mxfp4"] if k % 64 == 0 else [])
        for fmt in fmts:
            got = S.prune_quantize_pairs48(x, fmt)
            check_pq(got, O.prune_quantize_pairs48(raw, dtype, O.QSpec(fmt)), f"4:8 {fmt} {kind}")


def test_prune_quantize_pairs48_kept_max_below_row_max():
    # rows where a dropped pair holds the row's largest element: the INT/FP8
    # row scale and the NVFP4 tensor maximum come from the kept values
    rng = np.random.default_rng(77)
    k = 256
    x = rng.standard_normal((16, k)).astype(np.float32)
    g = x.reshape(16, k // 8, 4, 2)
    g[:, :, 0, :] = [5.0, 0.0]
    g[:, :, 1:3, :] = 4.0
    g[:, :, 3, :] = 0.0
    for fmt, bits in (("int", 4), ("fp8", 0), ("nvfp4", 0)):
        got = S.prune_quantize_pairs48(to_dev(x, "f32"), (fmt, bits))
        want = O.prune_quantize_pairs48(x, "f32", O.QSpec(fmt, bits))
        check_pq(got, want, f"kept max {fmt}")


def test_prune_quantize_nv_given_tensor_amax():
    raw = inputs(90, 33, 512, "bf16", "normal")
    x = to_dev(raw, "bf16")
    T = np.float32(7.5)
    t = torch.tensor([T], dtype=torch.float32, device="cuda")
    for pq, opq in ((S.prune_quantize, O.prune_quantize),
                    (S.prune_quantize_pairs48, O.prune_quantize_pairs48)):
        got = pq(x, "nvfp4", tensor_amax=t)
        check_pq(got, opq(raw, "bf16", O.QSpec("nvfp4", tensor_amax=float(T))), "given T")


def test_prune_quantize_pairs48_transposed():
    rng = np.random.default_rng(5)
    shape = (2, 256, 40)
    raw = random_raw(rng, shape, "bf16")
    x = to_dev(raw, "bf16")
    rows = np.ascontiguousarray(np.swapaxes(raw, 1, 2)).reshape(-1, shape[1])
    for q in (("fp8", 0), ("nvfp4", 0)):
        got = S.prune_quantize_pairs48(x, q, axis=1)
        want = O.prune_quantize_pairs48(rows, "bf16", O.QSpec(*q))
        flat = [g.reshape(rows.shape[0], -1) if g.numel() > 1 else g for g in got]
        if q[0] == "fp8":
            flat[2] = got[2].reshape(-1)
        check_pq(flat, want, f"transposed {q[0]}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [64, 1024, 4096])
def test_predict_R_block_kept(dtype, k):
    raw = inputs(k + 41, 37, k, dtype, "normal")
    x = to_dev(raw, dtype)
    kept = ["nvfp4", "mxfp4", "nvfp4", "fp8"]
    dense = ["nvfp4", "mxfp4", ("int", 4), "nvfp4"]
    okept = [qs_oracle(q) for q in kept]
    odense = [qs_oracle(q) for q in dense]
    got = S.predict_R(x, kept, dense, rows_per_block=8)
    rel_close(raw_np(got), O.predict_R(raw, dtype, okept, odense, rows_per_block=8))
    got = S.predict_R_pairs48(x, kept, dense, rows_per_block=8)
    rel_close(raw_np(got), O.predict_R(raw, dtype, okept, odense, rows_per_block=8,
                                       pattern="pairs4:8"))


def test_predict_R_block_kept_wanda():
    rng = np.random.default_rng(12)
    k = 512
    raw = inputs(13, 40, k, "bf16", "normal")
    norm = (rng.random(k) * 2).astype(np.float32)
    x = to_dev(raw, "bf16")
    n = torch.from_numpy(norm).cuda()
    got = S.predict_R(x, ["nvfp4", "mxfp4"], ["nvfp4", "fp8"], score="wanda", col_norm=n)
    want = O.predict_R(raw, "bf16", [O.QSpec("nvfp4"), O.QSpec("mxfp4")],
                       [O.QSpec("nvfp4"), O.QSpec("fp8")], "wanda", norm)
    rel_close(raw_np(got), want)


# ---------------------------------------------------------------------------
# the hand-worked rows with inexact fp32 scales, through the library
# ---------------------------------------------------------------------------


def test_hand_rows_inexact_scales():
    import json
    import os
    from conftest import GOLDEN
    hand = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))

    def f32hex(xs):
        return np.array([int(h, 16) for h in xs], dtype=np.uint32).view(np.float32)

    for key, q in (("fp8_row_inexact_scale", "fp8"), ("int8_row_inexact_scale", ("int", 8))):
        ex = hand[key]
        x = to_dev(f32hex(ex["row_hex"])[None, :], "f32")
        c, s = S.quantize(x, q)
        assert int(raw_np(s).view(np.uint32)[0]) == int(ex["scale_hex"], 16), key
        want = [int(h, 16) for h in ex["codes"]] if q == "fp8" else ex["codes"]
        assert raw_np(c)[0].astype(np.int64).tolist() == want, key
    ex = hand["nvfp4_inexact_tensor_scale"]
    x = to_dev(np.stack([f32hex(r) for r in ex["rows_hex"]]), "f32")
    c, bs, ts = S.quantize(x, "nvfp4")
    assert int(raw_np(ts).view(np.uint32)[0]) == int(ex["tensor_scale_hex"], 16)
    assert raw_np(bs)[:, 0].tolist() == [int(h, 16) for h in ex["block_scales"]]
    assert raw_np(c).tolist() == [[int(h, 16) for h in r] for r in ex["packed"]]
