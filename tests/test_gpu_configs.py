"""GPU parity at the full sizes of the five benchmark workloads, in the launch
configuration the benchmark uses.  The oracle recomputes whole outputs where
it finishes in seconds and sampled rows / row blocks otherwise (every row and
block is independent, so a sample is checked exactly).

Workloads (synthetic, seeded; see the design notes for the recipe):
  tiny      fp32 256x1024 N(0,1)
  act       bf16 4096x4096 activation, 4 outlier channels x50
  weight    bf16 14336x4096 weight, Wanda with the activation's channel norms
  attn      Q [32,16384,128], K/V [8,16384,128], P [32,4096,4096]
  heavy     bf16 16384x4096 Student-t(4)
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import pruning_quantization_amd as S  # noqa: E402
from gpu_util import raw_np, to_dev  # noqa: E402
from test_gpu_parity import assert_same, qs_oracle, rel_close  # noqa: E402


def sample_rows(n, k=24, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=k, replace=False)]))


def test_tiny_fp32():
    raw = W.gaussian_f32(0, 256, 1024)
    x = to_dev(raw, "f32")
    v, m = S.prune_compress(x)
    wv, wm = O.prune_compress(raw, "f32")
    assert_same(raw_np(v), wv, "kept values")
    assert_same(raw_np(m), wm, "meta")
    c, s = S.quantize(x, ("int", 8))
    wc, ws = O.quantize_rows(raw, "f32", O.QSpec("int", 8))
    assert_same(raw_np(c), wc, "int8 codes")
    assert_same(raw_np(s), ws, "int8 scales")
    got = raw_np(S.predict_R(x, ["none"], [("int", 8)]))
    want = O.predict_R(raw, "f32", [O.QSpec("none")], [O.QSpec("int", 8)])
    rel_close(got, want)
    assert 0.1309 < got[0, 0, 0] < 0.1339          # the pages' Gaussian 13.2% energy loss


@pytest.fixture(scope="module")
def act():
    bits = W.activation_x(1, 4096, 4096)
    return bits, to_dev(bits, "bf16")


def test_act_fused_fp8_and_dense(act):
    bits, x = act
    c, m, s = S.prune_quantize(x, "fp8")
    wc, wm, ws = O.prune_quantize(bits, "bf16", O.QSpec("fp8"))
    assert_same(raw_np(c), wc, "codes")
    assert_same(raw_np(m), wm, "meta")
    assert_same(raw_np(s), ws, "scales")
    for q in ("fp8", ("int", 8)):
        c, s = S.quantize(x, q)
        wc, ws = O.quantize_rows(bits, "bf16", qs_oracle(q))
        assert_same(raw_np(c), wc, f"dense {q}")
        assert_same(raw_np(s), ws, f"dense {q} scales")


def test_act_predict_R(act):
    bits, x = act
    kept, dense = ["fp8", "fp8"], ["fp8", ("int", 8)]
    got = raw_np(S.predict_R(x, kept, dense))
    want = O.predict_R(bits, "bf16", [O.QSpec("fp8")] * 2, [O.QSpec("fp8"), O.QSpec("int", 8)])
    rel_close(got, want)


def test_act_col_norms(act):
    bits, x = act
    got = raw_np(S.col_l2norm(x))
    want = O.col_l2norm(bits, "bf16")
    d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert d.max() <= 1


def test_weight_wanda_and_sweep(act):
    xbits, _ = act
    norms = O.col_l2norm(xbits, "bf16")               # oracle norms feed both sides
    wbits = W.weight_w(2, 14336, 4096)
    w = to_dev(wbits, "bf16")
    n = torch.from_numpy(norms).cuda()
    v, m = S.prune_compress(w, score="wanda", col_norm=n)
    rows = sample_rows(14336, seed=2)
    wv, wm = O.prune_compress(wbits[rows], "bf16", "wanda", norms)
    assert_same(raw_np(v)[rows], wv, "kept values")
    assert_same(raw_np(m)[rows], wm, "meta")
    kept = [("int", 2 * m_) for m_ in range(2, 9)]
    dense = [("int", m_ + 1) for m_ in range(2, 9)]
    got = raw_np(S.predict_R(w, kept, dense, score="wanda", col_norm=n, rows_per_block=128))
    assert got.shape == (112, 7, 5)
    for blk in (0, 57, 111):
        sub = wbits[blk * 128:(blk + 1) * 128]
        want = O.predict_R(sub, "bf16", [qs_oracle(q) for q in kept], [qs_oracle(q) for q in dense],
                           "wanda", norms)
        rel_close(got[blk:blk + 1], want)


def test_attention_q_k_v():
    for name, heads, seed in (("Q", 32, 3), ("K", 8, 4)):
        bits = W.attention_qkv(seed, heads, 16384, 128)
        x = to_dev(bits.reshape(-1, 128), "bf16")
        v, m = S.prune_compress(x)
        rows = sample_rows(heads * 16384, seed=seed)
        flat = bits.reshape(-1, 128)
        wv, wm = O.prune_compress(flat[rows], "bf16")
        assert_same(raw_np(v)[rows], wv, f"{name} kept")
        assert_same(raw_np(m)[rows], wm, f"{name} meta")
        got = raw_np(S.predict_R(x, ["none", "none"], ["fp8", ("int", 8)], rows_per_block=16384))
        for h in (0, heads - 1):
            want = O.predict_R(flat[h * 16384:(h + 1) * 16384], "bf16", [O.QSpec("none")] * 2,
                               [O.QSpec("fp8"), O.QSpec("int", 8)])
            rel_close(got[h:h + 1], want)
    # V [8, 16384, 128] pruned along seq: rows are (head, dim), K = seq
    bits = W.attention_qkv(5, 8, 16384, 128)
    x = to_dev(bits, "bf16")
    v, m = S.prune_compress(x, axis=1)
    rowsT = np.ascontiguousarray(np.swapaxes(bits, 1, 2)).reshape(-1, 16384)
    pick = sample_rows(8 * 128, seed=5)
    wv, wm = O.prune_compress(rowsT[pick], "bf16")
    assert_same(raw_np(v).reshape(-1, 8192)[pick], wv, "V kept")
    assert_same(raw_np(m).reshape(-1, 2048)[pick], wm, "V meta")
    c, s = S.quantize(x, "fp8", axis=1)
    wc, ws = O.quantize_rows(rowsT[pick], "bf16", O.QSpec("fp8"))
    assert_same(raw_np(c).reshape(-1, 16384)[pick], wc, "V fp8 codes")
    assert_same(raw_np(s).reshape(-1)[pick], ws, "V fp8 scales")
    got = raw_np(S.predict_R(x, ["none", "none"], ["fp8", ("int", 8)], axis=1, rows_per_block=128))
    for h in (0, 7):
        want = O.predict_R(rowsT[h * 128:(h + 1) * 128], "bf16", [O.QSpec("none")] * 2,
                           [O.QSpec("fp8"), O.QSpec("int", 8)])
        rel_close(got[h:h + 1], want)


def test_attention_probabilities():
    bits = W.attention_p(6, 32, 4096, 4096)
    x = to_dev(bits.reshape(-1, 4096), "bf16")
    v, m = S.prune_compress(x)
    flat = bits.reshape(-1, 4096)
    rows = sample_rows(32 * 4096, seed=6)
    wv, wm = O.prune_compress(flat[rows], "bf16")
    assert_same(raw_np(v)[rows], wv, "P kept")
    assert_same(raw_np(m)[rows], wm, "P meta")
    got = raw_np(S.predict_R(x, ["none", "none"], ["fp8", ("int", 8)], rows_per_block=4096))
    for h in (0, 31):
        want = O.predict_R(flat[h * 4096:(h + 1) * 4096], "bf16", [O.QSpec("none")] * 2,
                           [O.QSpec("fp8"), O.QSpec("int", 8)])
        rel_close(got[h:h + 1], want)


def test_heavy_tailed_4x_tier():
    bits = W.student_t_x(7, 16384, 4096)
    x = to_dev(bits, "bf16")
    T = float(O.tensor_absmax(bits, "bf16"))
    rows = sample_rows(16384, seed=7)
    c, m, s = S.prune_quantize(x, "fp8")
    wc, wm, ws = O.prune_quantize(bits[rows], "bf16", O.QSpec("fp8"))
    assert_same(raw_np(c)[rows], wc, "fused codes")
    assert_same(raw_np(m)[rows], wm, "fused meta")
    assert_same(raw_np(s)[rows], ws, "fused scales")
    c, sc = S.quantize(x, "mxfp4")
    wc, wsc = O.quantize_mxfp4(bits[rows], "bf16")
    assert_same(raw_np(c)[rows], wc, "mx codes")
    assert_same(raw_np(sc)[rows], wsc, "mx scales")
    c, sc, ts = S.quantize(x, "nvfp4")
    wc, wsc, wts = O.quantize_nvfp4(bits[rows], "bf16", tensor_amax=T)
    assert raw_np(ts)[0] == wts
    assert_same(raw_np(c)[rows], wc, "nv codes")
    assert_same(raw_np(sc)[rows], wsc, "nv scales")
    got = raw_np(S.predict_R(x, ["fp8", "fp8"], ["mxfp4", "nvfp4"], rows_per_block=128))
    assert got.shape == (128, 2, 5)
    for blk in (0, 77, 127):
        sub = bits[blk * 128:(blk + 1) * 128]
        want = O.predict_R(sub, "bf16", [O.QSpec("fp8")] * 2,
                           [O.QSpec("mxfp4"), O.QSpec("nvfp4", tensor_amax=T)])
        rel_close(got[blk:blk + 1], want)


# ---------------------------------------------------------------------------
# Full-size checks of the rows beyond the fused path: the sparse FP4 operand
# (pairwise 4:8 + NVFP4) on the heavy-tailed tier, the rotated activation,
# the operator-level error and the GEMMs on the prepared operands
# ---------------------------------------------------------------------------


def test_heavy_sparse_fp4():
    bits = W.student_t_x(7, 16384, 4096)
    x = to_dev(bits, "bf16")
    kv, _ = O.prune_compress_pairs48(bits, "bf16")              # whole-tensor kept maximum
    Tk = float(np.max(np.abs(O.decode_input(kv, "bf16"))))
    del kv
    rows = sample_rows(16384, seed=17)
    c, m, sc, ts = S.prune_quantize_pairs48(x, "nvfp4")
    wc, wm, wsc, wts = O.prune_quantize_pairs48(bits[rows], "bf16", O.QSpec("nvfp4", tensor_amax=Tk))
    assert raw_np(ts)[0] == wts
    assert_same(raw_np(c)[rows], wc, "sparse fp4 codes")
    assert_same(raw_np(m)[rows], wm, "sparse fp4 meta")
    assert_same(raw_np(sc)[rows], wsc, "sparse fp4 scales")
    got = raw_np(S.predict_R_pairs48(x, ["nvfp4"], ["nvfp4"], rows_per_block=128))
    T = float(O.tensor_absmax(bits, "bf16"))
    for blk in (0, 99):
        sub = bits[blk * 128:(blk + 1) * 128]
        want = O.predict_R(sub, "bf16", [O.QSpec("nvfp4", tensor_amax=Tk)],
                           [O.QSpec("nvfp4", tensor_amax=T)], pattern="pairs4:8")
        rel_close(got[blk:blk + 1], want)


def test_act_rotated(act):
    bits, x = act
    assert O.rotation_exact(bits, "bf16", 128).all()
    rot = O.rotate(bits, "bf16", 128)
    c, m, s = S.prune_quantize_rot(x, 128, "fp8")
    wc, wm, ws = O.prune_quantize(rot, "bf16", O.QSpec("fp8"))
    assert_same(raw_np(c), wc, "rotated codes")
    assert_same(raw_np(m), wm, "rotated meta")
    assert_same(raw_np(s), ws, "rotated scales")
    kept, dense = ["fp8", "fp8"], ["fp8", ("int", 8)]
    got = raw_np(S.predict_R_rot(x, 128, kept, dense))
    want = O.predict_R(rot, "bf16", [O.QSpec("fp8")] * 2, [O.QSpec("fp8"), O.QSpec("int", 8)])
    rel_close(got, want)


def test_act_rotated_whole_row(act):
    # one 4096-element Hadamard block per token (the whole hidden dimension)
    bits, x = act
    assert O.rotation_exact(bits, "bf16", 4096).all()
    rot = O.rotate(bits, "bf16", 4096)
    c, m, s = S.prune_quantize_rot(x, 4096, "fp8")
    wc, wm, ws = O.prune_quantize(rot, "bf16", O.QSpec("fp8"))
    assert_same(raw_np(c), wc, "rotated codes")
    assert_same(raw_np(m), wm, "rotated meta")
    assert_same(raw_np(s), ws, "rotated scales")
    kept, dense = ["fp8", "fp8"], ["fp8", ("int", 8)]
    got = raw_np(S.predict_R_rot(x, 4096, kept, dense))
    want = O.predict_R(rot, "bf16", [O.QSpec("fp8")] * 2, [O.QSpec("fp8"), O.QSpec("int", 8)])
    rel_close(got, want)


@pytest.fixture(scope="module")
def weight():
    bits = W.weight_w(2, 14336, 4096)
    return bits, to_dev(bits, "bf16")


def test_act_operator_error(act, weight):
    bits, x = act
    wbits, w = weight
    sides = [("2:4", ("fp8", 0)), ("dense", ("fp8", 0)), ("dense", ("int", 8))]
    got = raw_np(S.operator_error(x, w, sides))
    rows = sample_rows(4096, k=12, seed=21)
    want = O.operator_error(bits[rows], "bf16", wbits, "bf16",
                            [O.Side(p, O.QSpec(*q)) for p, q in sides])
    rel_close(got[rows], want, rtol=1e-3)


def test_act_gemms(act, weight):
    bits, x = act
    wbits, w = weight
    rows = sample_rows(4096, k=8, seed=22)
    b64 = O.decode_input(wbits, "bf16")
    k = 4096

    def check(got, a64, bnd_scale=1.0, extra=0.0):
        ref = a64 @ b64.T
        bound = bnd_scale * (k - 1) * 2.0 ** -24 * (np.abs(a64) @ np.abs(b64).T) + extra * np.abs(ref) + 1e-300
        assert (np.abs(got.astype(np.float64) - ref) <= bound).all()

    vals, meta = S.prune_compress(x)
    check(raw_np(S.sparse_gemm(vals, meta, w))[rows],
          O.reconstruct(bits[rows], "bf16", O.Side("2:4", O.QSpec("none"))))
    check(raw_np(S.dense_gemm(x, w))[rows], O.decode_input(bits[rows], "bf16"))
    ca, sa = S.quantize(x, "fp8")
    cb, sb = S.quantize(w, "fp8")
    wcb, wsb = O.quantize_rows(wbits, "bf16", O.QSpec("fp8"))
    b64 = O.dequantize_rows(wcb, O.QSpec("fp8"), wsb)
    check(raw_np(S.fp8_gemm(ca, sa, cb, sb))[rows],
          O.reconstruct(bits[rows], "bf16", O.Side("dense", O.QSpec("fp8"))), 2.0, 3 * 2.0 ** -24)
