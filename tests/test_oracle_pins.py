"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, not against the oracle itself.

Sources: Qin, "Is 2:4 Sparsity Still Worth It?" — paper-daily.com English
summary §2 (equal bits), §3 (formats), §4 (energy loss, additivity, predicted
R), §6 (pairwise 4:8). Hand-worked examples live in tests/golden/.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W
from conftest import GOLDEN

HAND = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))
PAGES = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))


def bf16(vals):
    """bf16 bit patterns of exactly representable values (sign of zero kept)."""
    a = np.asarray(vals, dtype=np.float64)
    bits = W.to_bf16_bits(a)
    back = W.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.array_equal(back, a), "hand example must be bf16-exact"
    bits[(a == 0) & np.signbit(a)] = 0x8000
    return bits


def hexs(xs):
    return np.array([int(h, 16) for h in xs], dtype=np.uint8)


# ---------------------------------------------------------------------------
# Hand-worked layouts and codes
# ---------------------------------------------------------------------------


def test_meta_layout_hand_example():
    ex = HAND["meta_layout"]
    raw = bf16([ex["row"]])
    vals, meta = O.prune_compress(raw, O.BF16)
    assert np.array_equal(O.decode_input(vals, O.BF16)[0], ex["kept"])
    assert np.array_equal(meta[0], hexs(ex["meta_bytes"]))


def test_tie_groups_hand_example():
    ex = HAND["tie_groups"]
    raw = bf16([sum(ex["groups"], [])])
    idx = O.select_2of4(O.score_values(O.decode_input(raw, O.BF16)))
    assert idx[0].tolist() == ex["kept_positions"]


def test_int4_row_hand_example():
    ex = HAND["int4_row"]
    codes, s = O.quantize_rows(bf16([ex["row"]]), O.BF16, O.QSpec("int", ex["bits"]))
    assert codes[0].tolist() == ex["codes"]
    assert int(s.view(np.uint32)[0]) == int(ex["scale_hex"], 16)


def test_fp8_row_hand_example():
    ex = HAND["fp8_row"]
    raw = bf16([ex["row"]])
    codes, s = O.quantize_rows(raw, O.BF16, O.QSpec("fp8"))
    assert np.array_equal(codes[0], hexs(ex["dense_codes"]))
    assert s[0] == ex["dense_scale"]
    pc, meta, ps = O.prune_quantize(raw, O.BF16, O.QSpec("fp8"))
    assert np.array_equal(meta[0], hexs(ex["pruned_meta_bytes"]))
    assert np.array_equal(pc[0], hexs(ex["pruned_codes"]))
    assert ps[0] == ex["pruned_scale"]


def test_mxfp4_hand_example():
    ex = HAND["mxfp4_row"]
    row = np.zeros(128)
    exp_codes = np.zeros(128, dtype=np.int64)
    for b, (vals, cods) in enumerate(zip(ex["row_blocks"], ex["block_codes"])):
        row[b * 32:b * 32 + len(vals)] = vals
        exp_codes[b * 32:b * 32 + len(cods)] = cods
    raw = bf16([row.tolist()])
    packed, sc = O.quantize_mxfp4(raw, O.BF16)
    assert sc[0].tolist() == ex["scale_codes"]
    got = np.empty(128, dtype=np.int64)
    got[0::2] = packed[0] & 0xF
    got[1::2] = packed[0] >> 4
    assert got.tolist() == exp_codes.tolist()


def test_nvfp4_hand_example():
    ex = HAND["nvfp4_tensor"]
    raw = bf16(ex["rows"])
    packed, bs, s_t = O.quantize_nvfp4(raw, O.BF16)
    assert float(s_t) == ex["tensor_scale"]
    assert np.array_equal(bs[:, 0], hexs(ex["block_scales"]))
    for r in range(2):
        assert np.array_equal(packed[r], hexs(ex["packed"][r]))


def f32hex(xs):
    return np.array([int(h, 16) for h in xs], dtype=np.uint32).view(np.float32)


def test_fp8_row_inexact_scale_hand_example():
    # [PD §3]: FP8 with one scale per row; the scale 448/amax is inexact in fp32
    ex = HAND["fp8_row_inexact_scale"]
    raw = f32hex(ex["row_hex"])[None, :]
    codes, s = O.quantize_rows(raw, O.F32, O.QSpec("fp8"))
    assert int(s.view(np.uint32)[0]) == int(ex["scale_hex"], 16)
    assert np.array_equal(codes[0], hexs(ex["codes"]))


def test_int8_row_inexact_scale_hand_example():
    # [PD §3]: INT8 with one scale per row; qmax/amax inexact in fp32
    ex = HAND["int8_row_inexact_scale"]
    raw = f32hex(ex["row_hex"])[None, :]
    codes, s = O.quantize_rows(raw, O.F32, O.QSpec("int", ex["bits"]))
    assert int(s.view(np.uint32)[0]) == int(ex["scale_hex"], 16)
    assert codes[0].tolist() == ex["codes"]


def test_nvfp4_inexact_tensor_scale_hand_example():
    # [PD §3]: NVFP4 = an FP8 scale per 16 elements plus one fp32 scale per
    # tensor; here T/2688 is inexact, and so are 448/T, the block scale times
    # s_t and its reciprocal
    ex = HAND["nvfp4_inexact_tensor_scale"]
    raw = np.stack([f32hex(r) for r in ex["rows_hex"]])
    packed, bs, s_t = O.quantize_nvfp4(raw, O.F32)
    assert int(np.float32(s_t).view(np.uint32)) == int(ex["tensor_scale_hex"], 16)
    assert np.array_equal(bs[:, 0], hexs(ex["block_scales"]))
    for r in range(2):
        assert np.array_equal(packed[r], hexs(ex["packed"][r]))
        got = np.empty(16, dtype=np.int64)
        got[0::2] = packed[r] & 0xF
        got[1::2] = packed[r] >> 4
        assert got.tolist() == ex["codes"][r]


def _e2m1_nearest(y):
    """E2M1 code of each y: nearest of the 8 magnitudes, ties to the even code,
    saturating, sign copied (a second, independent encoder for the check below)."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    a = np.minimum(np.abs(y).astype(np.float64), 6.0)
    d = np.abs(a[..., None] - grid)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    return code | np.where(np.signbit(y), 8, 0)


def test_inexact_scale_examples_catch_precision_mistakes():
    # The rows above are sensitive: forming any one fp32 step of the NVFP4
    # chain in fp64 instead (or replacing a division by a reciprocal
    # multiply) changes a stored value.  Each variant below plants one such
    # mistake in a plain numpy rendering of the chain and must disagree with
    # the hand-worked result.
    ex = HAND["nvfp4_inexact_tensor_scale"]
    x = np.stack([f32hex(r) for r in ex["rows_hex"]]).astype(np.float32)
    T = np.float32(np.abs(x).max())
    want_codes = np.array(ex["codes"])
    want_bs = hexs(ex["block_scales"])
    want_st = int(ex["tensor_scale_hex"], 16)

    def chain(st_mode="ok", g_mode="ok", d_mode="ok", inv_mode="ok", y_mode="ok"):
        st32 = np.float32(T / np.float32(2688.0))
        st = {"ok": st32, "recip": np.float32(T * np.float32(1.0 / 2688.0))}[st_mode]
        g = np.float32(448.0) / T if g_mode == "ok" else 448.0 / np.float64(T)
        amax = np.abs(x).max(axis=1)
        bs = O.e4m3_encode(np.float32(amax * g) if g_mode == "ok" else np.float32(amax.astype(np.float64) * g))
        bval = O.e4m3_decode(bs)
        if d_mode == "ok":
            d = (bval.astype(np.float32) * st).astype(np.float32)
        elif d_mode == "fp64":
            d = bval * np.float64(st)                          # product left unrounded
        else:                                                  # s_t unrounded inside d
            d = np.float32(bval * (np.float64(T) / 2688.0))
        if inv_mode == "ok":
            y = np.float32(x * np.float32(1.0 / np.float64(np.float32(d))[:, None]).astype(np.float32)) \
                if d_mode == "ok" else np.float32(x * np.float32(1.0 / d)[:, None])
        else:                                                  # one rounding of x / d
            y = np.float32(x.astype(np.float64) / np.float64(d)[:, None])
        if y_mode == "fp64":
            y = x.astype(np.float64) * np.float64(np.float32(1.0 / np.float64(np.float32(d))))[:, None]
        return int(np.float32(st).view(np.uint32)), bs, _e2m1_nearest(y)

    st, bs, codes = chain()
    assert st == want_st and np.array_equal(bs, want_bs) and np.array_equal(codes, want_codes)
    for variant in ({"st_mode": "recip"}, {"g_mode": "fp64"}, {"d_mode": "fp64"},
                    {"d_mode": "st_fp64"}, {"inv_mode": "div"}, {"y_mode": "fp64"}):
        st, bs, codes = chain(**variant)
        assert (st != want_st or not np.array_equal(bs, want_bs)
                or not np.array_equal(codes, want_codes)), variant


def test_row_scale_examples_catch_precision_mistakes():
    # Same for the per-row FP8 and INT8 examples: s = fp32(amax/qmax),
    # inv = fp32(qmax/amax), y = fp32(x * inv); each variant plants one
    # mistake (s from a reciprocal multiply, inv = 1/s, x / s, an unrounded
    # inv or an unrounded y) and must change the scale bits or a code.
    for key, q, enc in (("fp8_row_inexact_scale", 448.0, lambda y: O.e4m3_encode(y)),
                        ("int8_row_inexact_scale", 127.0, lambda y: np.clip(np.rint(y), -127, 127))):
        ex = HAND[key]
        x = f32hex(ex["row_hex"]).astype(np.float32)
        want_s = int(ex["scale_hex"], 16)
        want = hexs(ex["codes"]) if key.startswith("fp8") else np.array(ex["codes"])
        amax = np.float32(np.abs(x).max())

        def chain(mode):
            s = np.float32(amax / np.float32(q))
            if mode == "s_recip":
                s = np.float32(amax * np.float32(1.0 / q))
            inv = np.float32(np.float32(q) / amax)
            if mode == "inv_from_s":
                y = np.float32(x * np.float32(np.float32(1.0) / s))
            elif mode == "div":
                y = np.float32(x / s)
            elif mode == "inv_fp64":
                y = np.float32(x.astype(np.float64) * (q / np.float64(amax)))
            elif mode == "y_fp64":
                y = x.astype(np.float64) * np.float64(inv)
            else:
                y = np.float32(x * inv)
            return int(np.float32(s).view(np.uint32)), np.asarray(enc(y)).astype(np.int64)

        s, c = chain("ok")
        assert s == want_s and np.array_equal(c, want.astype(np.int64)), key
        for mode in ("s_recip", "inv_from_s", "div", "inv_fp64", "y_fp64"):
            s, c = chain(mode)
            assert s != want_s or not np.array_equal(c, want.astype(np.int64)), (key, mode)


def test_predict_R_hand_example():
    ex = HAND["predict_R_row"]
    raw = bf16([ex["row"]])
    e = O.error_energy(raw, O.BF16, O.QSpec("none"), O.QSpec("int", 4))
    assert e[0, 0] == ex["sum_x2"] and e[0, 1] == ex["sum_dropped"] and e[0, 2] == 0.0
    r = O.predict_R(raw, O.BF16, [O.QSpec("none")], [O.QSpec("int", 4)])[0, 0]
    assert r[0] == pytest.approx(ex["E_prune"], rel=1e-15)
    assert r[1] == 0.0
    assert r[2] == pytest.approx(ex["E_prune"], rel=1e-15)
    assert r[3] == pytest.approx(ex["E_dense_approx"], rel=1e-6)
    assert r[4] == pytest.approx(ex["R_approx"], rel=1e-6)
    ek = O.error_energy(raw, O.BF16, O.QSpec("int", 4), O.QSpec("int", 4))
    assert ek[0, 2] == pytest.approx(ex["kept_int4_sum_err2_approx"], rel=1e-6)


# ---------------------------------------------------------------------------
# P2: brute force over all six masks of a group
# ---------------------------------------------------------------------------

PAIRS = list(itertools.combinations(range(4), 2))   # lexicographic order


def brute_keep(scores):
    """Pair with the largest kept score sum; among equal sums the
    lexicographically smallest pair (exact rational arithmetic)."""
    best = None
    for p in PAIRS:
        v = scores[p[0]] + scores[p[1]]
        if best is None or v > best[0]:
            best = (v, p)
    return list(best[1])


def test_all_tie_patterns_small_alphabet():
    alphabet = [0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0]
    groups = list(itertools.product(alphabet, repeat=4))
    raw = bf16([sum((list(g) for g in groups), [])])
    idx = O.select_2of4(O.score_values(O.decode_input(raw, O.BF16)))[0]
    for g, got in zip(groups, idx.tolist()):
        want = brute_keep([Fraction(abs(v)) ** 2 for v in g])
        assert got == want, (g, got, want)


def test_bruteforce_random_magnitude_and_wanda():
    rng = np.random.default_rng(7)
    rows, k = 64, 64
    # small integer values make ties frequent; scaling keeps them exact
    w = rng.integers(-4, 5, size=(rows, k)) * 0.25
    raw = bf16(w)
    norm = (rng.integers(0, 4, size=k) * 0.5).astype(np.float32)
    x = O.decode_input(raw, O.BF16)
    for score in ("magnitude", "wanda"):
        idx = O.select_2of4(O.score_values(x, score, norm))
        for r in range(rows):
            for g in range(k // 4):
                vals = [Fraction(float(v)) for v in x[r, 4 * g:4 * g + 4]]
                if score == "magnitude":
                    sc = [v * v for v in vals]
                else:
                    sc = [abs(v) * Fraction(float(norm[4 * g + i])) for i, v in enumerate(vals)]
                assert idx[r, g].tolist() == brute_keep(sc)


# ---------------------------------------------------------------------------
# P3: additivity of prune and kept-quantization error ([PD §4])
# ---------------------------------------------------------------------------


def test_additivity_exact_rational():
    rng = np.random.default_rng(3)
    raw = W.to_bf16_bits(rng.standard_normal((8, 32)))
    x = O.decode_input(raw, O.BF16)
    for q in (O.QSpec("int", 4), O.QSpec("int", 8), O.QSpec("fp8")):
        codes, meta, s = O.prune_quantize(raw, O.BF16, q)
        xhat = O.dequantize_pruned(codes, meta, q, s)
        mask = O.decompress(np.ones_like(codes, dtype=np.uint8), meta).astype(bool)
        e = O.error_energy(raw, O.BF16, q, O.QSpec("int", 8))
        total = Fraction(0)
        dropped = Fraction(0)
        kept = Fraction(0)
        for r in range(x.shape[0]):
            for j in range(x.shape[1]):
                xv = Fraction(float(x[r, j]))
                hv = Fraction(float(xhat[r, j]))
                total += (xv - hv) ** 2
                if mask[r, j]:
                    kept += (xv - hv) ** 2
                else:
                    dropped += xv ** 2
        assert total == dropped + kept                      # exact
        assert float(dropped) == pytest.approx(e[0, 1], rel=1e-12)
        assert float(kept) == pytest.approx(e[0, 2], rel=1e-12)


def test_additivity_full_size_fp64():
    raw = W.gaussian_f32(11, 256, 1024)
    q = O.QSpec("int", 6)
    codes, meta, s = O.prune_quantize(raw, O.F32, q)
    xhat = O.dequantize_pruned(codes, meta, q, s)
    x = O.decode_input(raw, O.F32)
    e = O.error_energy(raw, O.F32, q, O.QSpec("int", 4))
    assert np.sum((x - xhat) ** 2) == pytest.approx(e[0, 1] + e[0, 2], rel=1e-12)


# ---------------------------------------------------------------------------
# P1 / P7: the pages' Gaussian figures ([PD §4])
# ---------------------------------------------------------------------------


def gaussian_energy_loss_closed_form():
    """E[Y(1)^2 + Y(2)^2] / 4 for the two smallest of four iid |N(0,1)|,
    from the order-statistic densities (numerical integration)."""
    from scipy import integrate, stats

    def moment(k):
        f = lambda y: y * y * 4 * math.comb(3, k - 1) * (stats.halfnorm.cdf(y) ** (k - 1)) * \
            (stats.halfnorm.sf(y) ** (4 - k)) * stats.halfnorm.pdf(y)
        return integrate.quad(f, 0, np.inf, epsabs=1e-13)[0]
    return (moment(1) + moment(2)) / 4


def test_gaussian_energy_loss_closed_form_matches_pages():
    cf = gaussian_energy_loss_closed_form()
    assert cf == pytest.approx(0.1324474, abs=2e-7)
    assert round(cf, 3) == PAGES["gaussian_24_energy_loss"]["value"]


def test_gaussian_energy_loss_of_oracle():
    cf = gaussian_energy_loss_closed_form()
    raw = W.gaussian_f32(0, 256, 1024)
    e = O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", 8))
    loss = e[0, 1] / e[0, 0]
    assert 0.1309 < loss < 0.1339                 # 3 sd of the seed spread at this shape
    big = W.gaussian_f32(1, 2048, 2048)
    e = O.error_energy(big, O.F32, O.QSpec("none"), O.QSpec("int", 8))
    # sd of the estimate at 4M elements is about 1.3e-4
    assert abs(e[0, 1] / e[0, 0] - cf) < 6e-4


def test_gaussian_relative_errors_match_pages():
    raw = W.gaussian_f32(5, 4096, 128)            # 128-element scale vectors
    dense = {b: O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", b)) for b in (3, 8)}
    rel = {b: math.sqrt(d[0, 3] / d[0, 0]) for b, d in dense.items()}
    assert rel[3] == pytest.approx(PAGES["gaussian_dense_int3_relative_error"]["value"], abs=0.004)
    assert rel[8] == pytest.approx(PAGES["gaussian_dense_int8_relative_error"]["value"], abs=0.001)
    lo, hi = (PAGES["gaussian_24_side_relative_error"][k] for k in ("low", "high"))
    for m in (3, 4, 6, 8):
        r = O.predict_R(raw, O.F32, [O.QSpec("int", 2 * m)], [O.QSpec("int", m + 1)])[0, 0]
        assert lo - 0.005 <= math.sqrt(r[2]) <= hi + 0.01
    # the curves cross only below 3 bits: R > 1 at m = 2 (INT4 kept vs INT3)
    r = O.predict_R(raw, O.F32, [O.QSpec("int", 4)], [O.QSpec("int", 3)])[0, 0]
    assert r[4] > 1.0


def test_each_added_bit_quarters_dense_error_energy():
    raw = W.gaussian_f32(9, 1024, 256)
    # the uniform-noise picture holds once the grid is fine (from about 5 bits)
    e = [O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", b))[0, 3] for b in range(5, 13)]
    ratios = np.array(e[:-1]) / np.array(e[1:])
    assert np.all((ratios > 3.6) & (ratios < 4.4))
    # E_2:4 tends to the energy loss as kept bits grow ([PD §4])
    r = O.predict_R(raw, O.F32, [O.QSpec("int", 16)], [O.QSpec("int", 9)])[0, 0]
    assert r[1] < 1e-8 and r[2] == pytest.approx(r[0], rel=1e-6)


# ---------------------------------------------------------------------------
# P4: the equal-bits accounting ([PD §2])
# ---------------------------------------------------------------------------


def test_equal_bits_accounting():
    for m in range(1, 9):
        assert O.bits_per_element(O.QSpec("int", 2 * m), sparse24=True, row_len=4096) == \
            O.bits_per_element(O.QSpec("int", m + 1), row_len=4096)
    for a, ab, b, bb in PAGES["equal_bits"]["pairs"]:
        assert O.bits_per_element(O.QSpec(a, ab), sparse24=True) == O.bits_per_element(O.QSpec(b, bb))
    assert O.bits_per_element(O.QSpec("none"), sparse24=True, value_bits=16) > \
        O.bits_per_element(O.QSpec("fp8"))
    m = PAGES["equal_bits"]["eight_bit_budget_kept_bits"] // 2
    assert O.bits_per_element(O.QSpec("int", 2 * m), sparse24=True) == 8.0
    assert O.bits_per_element(O.QSpec("mxfp4")) == 4.25
    assert O.bits_per_element(O.QSpec("nvfp4")) == 4.5


# ---------------------------------------------------------------------------
# P5: invariants
# ---------------------------------------------------------------------------


def test_mask_invariants_and_roundtrip():
    rng = np.random.default_rng(12)
    raw = W.to_bf16_bits(rng.standard_normal((33, 72)) * np.exp(rng.standard_normal((33, 1))))
    vals, meta = O.prune_compress(raw, O.BF16)
    idx = O.indices_from_meta(meta)
    assert np.all(idx[..., 0] < idx[..., 1])
    dense = O.decompress(vals, meta)
    x = O.decode_input(raw, O.BF16)
    mask = O.decompress(np.ones_like(vals), meta).astype(bool)
    assert np.array_equal(O.decode_input(dense, O.BF16), np.where(mask, x, 0.0))
    assert np.all(mask.reshape(33, -1, 4).sum(-1) == 2)
    # magnitude keeps every group's maximum, so kept amax == row amax
    assert np.array_equal(np.abs(O.decode_input(vals, O.BF16)).max(1), np.abs(x).max(1))


def test_energy_loss_bounds():
    # at most two non-zeros per group -> nothing dropped
    x = np.zeros((4, 16))
    x[:, 0::4] = 1.0
    x[:, 2::4] = -3.0
    e = O.error_energy(bf16(x), O.BF16, O.QSpec("none"), O.QSpec("int", 8))
    assert e[0, 1] == 0.0
    # all magnitudes equal in every group -> exactly half dropped
    y = np.where(np.arange(16) % 3 == 0, 2.0, -2.0) * np.ones((4, 1))
    e = O.error_energy(bf16(y), O.BF16, O.QSpec("none"), O.QSpec("int", 8))
    assert e[0, 1] / e[0, 0] == 0.5


def test_energy_loss_independent_of_bits():
    raw = W.activation_x(2, 64, 512)
    el = {O.error_energy(raw, O.BF16, O.QSpec("int", b), O.QSpec("int", b))[0, 1] for b in (2, 5, 8, 16)}
    assert len(el) == 1


def test_blocks_partition_the_sums():
    raw = W.student_t_x(4, 384, 256)
    whole = O.error_energy(raw, O.BF16, O.QSpec("fp8"), O.QSpec("nvfp4"))
    blk = O.error_energy(raw, O.BF16, O.QSpec("fp8"), O.QSpec("nvfp4"), rows_per_block=128)
    assert blk.shape == (3, 4)
    assert np.allclose(blk.sum(0), whole[0], rtol=1e-12)


def test_degenerate_R():
    z = np.zeros((1, 8), dtype=np.uint16)
    r = O.predict_R(z, O.BF16, [O.QSpec("fp8")], [O.QSpec("int", 8)])[0, 0]
    assert np.all(np.isnan(r))
    # exactly representable row: dense error 0, 2:4 error > 0 -> R = inf
    raw = bf16([[1, 3, -1, 3, 2, 1, 3, -3]])          # amax 3 = qmax of INT3: scale 1
    r = O.predict_R(raw, O.BF16, [O.QSpec("none")], [O.QSpec("int", 3)])[0, 0]
    assert r[3] == 0.0 and r[4] == np.inf


# ---------------------------------------------------------------------------
# P6: encoders against library routines and exact brute force
# ---------------------------------------------------------------------------


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = W.bf16_bits_to_f32(bits)
    return v[np.isfinite(v)]


def test_e4m3_matches_torch_cast_on_all_bf16_and_random_fp32():
    import torch

    v = all_finite_bf16().astype(np.float32)
    rng = np.random.default_rng(0)
    r = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 10, 200000))).astype(np.float32)
    for y in (v, r):
        clamped = np.clip(y, -448.0, 448.0)
        want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = O.e4m3_encode(y)
        # torch keeps the sign of -0 as 0x80 as well
        assert np.array_equal(got, want)


def exact_nearest(grid, a):
    """Brute force over a grid with Fractions; ties go to the even index."""
    a = Fraction(a)
    best = None
    for i, g in enumerate(grid):
        d = abs(a - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_e2m1_brute_force_on_all_bf16_in_range():
    v = all_finite_bf16()
    v = v[np.abs(v) <= 8.0]
    got = O.e2m1_encode(v)
    for x, c in zip(v.tolist(), got.tolist()):
        assert c & 7 == exact_nearest([0, 0.5, 1, 1.5, 2, 3, 4, 6], abs(x))
        assert (c >> 3) == (1 if math.copysign(1.0, x) < 0 else 0)
    assert np.all(O.e2m1_encode(np.array([7.0, 100.0, -1e30])) & 7 == 7)


def test_e2m1_midpoints_from_definition():
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, c in mids.items():
        assert O.e2m1_encode(np.array([y]))[0] == c
        assert O.e2m1_encode(np.array([-y]))[0] == c | 8


def test_e4m3_grid_definition():
    g = O.E4M3_GRID
    assert g[0x7E] == 448.0 and g[0x08] == 2.0 ** -6 and g[0x01] == 2.0 ** -9 and g[0x38] == 1.0
    assert np.all(np.diff(g) > 0)
    codes = np.arange(0x7F)
    assert np.array_equal(O.e4m3_encode(g), codes)              # idempotent on the grid
    assert np.array_equal(O.e4m3_encode(-g), codes | 0x80)


def test_int_rtn_brute_force():
    rng = np.random.default_rng(1)
    y = np.concatenate([np.arange(-20, 20.5, 0.5), rng.standard_normal(2000) * 10])
    for b in (2, 3, 4, 8):
        qmax = 2 ** (b - 1) - 1
        got = O.int_rtn_codes(y, b)
        for yy, c in zip(y.tolist(), got.tolist()):
            grid = list(range(-qmax, qmax + 1))
            # nearest integer in range, ties to the even integer
            f = Fraction(yy)
            best = min(grid, key=lambda q: (abs(f - q), q % 2))
            assert c == best


def test_mxfp4_scale_rule():
    # power-of-two scale: amax in [2^(e+2), 2^(e+3)) gives code e + 127
    for e in (-10, -1, 0, 3, 20):
        for frac in (1.0, 1.5, 1.9921875):
            row = np.zeros(32)
            row[5] = frac * 2.0 ** (e + 2)
            _, sc = O.quantize_mxfp4(bf16([row.tolist()]), O.BF16)
            assert sc[0, 0] == e + 127


def test_tiny_rows_zero_coded():
    t = 2.0 ** -130                                    # subnormal bf16, amax < 2^-64
    raw = bf16([[t, -t, 0, 0, 0, 0, 0, 2.0 ** -70]])
    c, s = O.quantize_rows(raw, O.BF16, O.QSpec("int", 8))
    assert np.all(c == 0) and s[0] == 0.0
    c, s = O.quantize_rows(raw, O.BF16, O.QSpec("fp8"))
    assert np.array_equal(c[0], hexs(["0x00", "0x80", "0x00", "0x00", "0x00", "0x00", "0x00", "0x00"]))


def test_col_l2norm_closed_form():
    # columns built so the norm is known exactly: 3-4-5 and constant columns
    x = np.zeros((16, 8))
    x[0, 0], x[1, 0] = 3.0, 4.0
    x[:, 1] = 0.5
    x[:, 2] = -2.0
    x[::2, 3] = 1.0
    raw = bf16(x)
    n = O.col_l2norm(raw, O.BF16)
    assert n.dtype == np.float32
    assert n[0] == 5.0 and n[1] == 2.0 and n[2] == 8.0 and n[4] == 0.0
    assert n[3] == np.float32(math.sqrt(8.0))


# ---------------------------------------------------------------------------
# Pairwise 4:8 ([PD §6])
# ---------------------------------------------------------------------------


def test_pairs48_hand_example():
    ex = HAND["pairs48_row"]
    raw = bf16([ex["row"]])
    vals, meta = O.prune_compress_pairs48(raw, O.BF16)
    assert O.decode_input(vals, O.BF16)[0].tolist() == ex["kept"]
    assert np.array_equal(meta[0], hexs(ex["meta_bytes"]))


def exp_order_stat_mean(k, n, mean):
    """E[X_(k)] of n iid exponentials: mean * sum_{i<k} 1/(n-i) (exact)."""
    return Fraction(mean) * sum(Fraction(1, n - i) for i in range(k))


def test_pairs48_gaussian_loss_closed_form_and_pages():
    # a pair's energy a^2 + b^2 of iid N(0,1) is exponential with mean 2;
    # dropping the two smallest of four loses (E[X(1)] + E[X(2)]) / 8
    cf = (exp_order_stat_mean(1, 4, 2) + exp_order_stat_mean(2, 4, 2)) / 8
    assert cf == Fraction(5, 24)
    assert round(float(cf), 3) == PAGES["pairwise_48_energy_loss"]["value"]
    raw = W.gaussian_f32(21, 2048, 2048)
    e = O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", 8), pattern="pairs4:8")
    loss = e[0, 1] / e[0, 0]
    assert abs(loss - float(cf)) < 6e-4
    # ranking pairs by |a| + |b| instead would lose about 21.35%: excluded
    x = O.decode_input(raw, O.F32)
    l1 = np.abs(x[:, 0::2]) + np.abs(x[:, 1::2])
    sel = O.select_pairs48(l1)
    g = (x * x).reshape(2048, 256, 4, 2).sum(-1)
    kept = np.take_along_axis(g, sel, axis=-1).sum()
    assert 1 - kept / (x * x).sum() > float(cf) + 3e-3


def test_pairs48_bruteforce_ties():
    rng = np.random.default_rng(8)
    w = rng.integers(-2, 3, size=(32, 64)) * 0.5          # many equal pair energies
    raw = bf16(w)
    x = O.decode_input(raw, O.BF16)
    sel = O.select_pairs48(O.pair_scores(x))
    for r in range(32):
        for gi in range(8):
            e = [Fraction(float(x[r, 8 * gi + 2 * p])) ** 2 + Fraction(float(x[r, 8 * gi + 2 * p + 1])) ** 2
                 for p in range(4)]
            assert sel[r, gi].tolist() == brute_keep(e)


def test_pairs48_energy_loss_exceeds_24():
    raw = W.gaussian_f32(22, 512, 1024)
    e24 = O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", 8))
    e48 = O.error_energy(raw, O.F32, O.QSpec("none"), O.QSpec("int", 8), pattern="pairs4:8")
    assert e48[0, 1] > e24[0, 1]            # pairs cannot each be chosen by size ([PD §6])
    assert e48[0, 0] == e24[0, 0]


# ---------------------------------------------------------------------------
# Sparse FP4 and block formats on kept values ([PD §6]: pairwise 4:8 with
# NVFP4 values; [PD §3]: MXFP4)
# ---------------------------------------------------------------------------


def test_pairs48_nvfp4_hand_example():
    ex = HAND["pairs48_nvfp4"]
    raw = bf16(ex["rows"])
    codes, meta, bs, st = O.prune_quantize_pairs48(raw, O.BF16, O.QSpec("nvfp4"))
    assert np.array_equal(meta, np.stack([hexs(m) for m in ex["meta_bytes"]]))
    assert np.array_equal(codes, np.stack([hexs(p) for p in ex["packed"]]))
    assert np.array_equal(bs[:, 0], hexs(ex["block_scales"]))
    assert float(st) == ex["tensor_scale"]
    vals, _ = O.prune_compress_pairs48(raw, O.BF16)
    assert np.array_equal(O.decode_input(vals, O.BF16), np.array(ex["kept"], dtype=np.float64))


def test_pairs48_kept_amax_hand_example():
    ex = HAND["pairs48_kept_amax"]
    raw = bf16([ex["row"]])
    codes, meta, s = O.prune_quantize_pairs48(raw, O.BF16, O.QSpec("int", ex["bits"]))
    assert np.array_equal(meta[0], hexs(ex["meta_bytes"]))
    assert codes[0].tolist() == ex["codes"]
    assert int(np.float32(s[0]).view(np.uint32)) == int(ex["scale_hex"], 16)
    r = O.predict_R(raw, O.BF16, [O.QSpec("int", ex["bits"])], [O.QSpec("int", 8)],
                    pattern="pairs4:8")
    assert r[0, 0, 0] == ex["sum_dropped"] / ex["sum_x2"]
    # each kept 4 comes back as 7 * s with s = fp32(4/7): error energy 4 (7s - 4)^2
    sc = float(np.uint32(int(ex["scale_hex"], 16)).view(np.float32))
    assert r[0, 0, 1] == pytest.approx(4 * (7 * sc - 4) ** 2 / ex["sum_x2"], rel=1e-12)


def test_sparse24_mxfp4_hand_example():
    ex = HAND["sparse24_mxfp4"]
    raw = bf16([ex["row"]])
    assert raw.shape == (1, 64)
    codes, meta, sc = O.prune_quantize(raw, O.BF16, O.QSpec("mxfp4"))
    assert np.array_equal(meta[0], hexs(ex["meta_bytes"]))
    assert sc[0].tolist() == ex["scale_codes"]
    assert np.array_equal(codes[0], hexs(ex["packed"]))
    vals, _ = O.prune_compress(raw, O.BF16)
    assert O.decode_input(vals, O.BF16)[0, :16].tolist() == ex["kept_first16"]


def test_decompress_pairs48_places_kept_pairs():
    rng = np.random.default_rng(7)
    x = rng.integers(-3, 4, size=(5, 64)).astype(np.float64)
    raw = bf16(x)
    vals, meta = O.prune_compress_pairs48(raw, O.BF16)
    dense = O.decompress_pairs48(O.decode_input(vals, O.BF16), meta)
    g = x.reshape(5, 8, 4, 2)
    d = dense.reshape(5, 8, 4, 2)
    for r in range(5):
        for q in range(8):
            kept = [p for p in range(4) if np.any(d[r, q, p] != 0) or False]
            e = (g[r, q] ** 2).sum(axis=1)
            nib = (meta[r, q // 2] >> (4 * (q % 2))) & 0xF
            want = sorted({nib & 3, nib >> 2})
            assert len(want) == 2
            for p in range(4):
                if p in want:
                    assert np.array_equal(d[r, q, p], g[r, q, p])
                else:
                    assert np.all(d[r, q, p] == 0)
            # the kept pairs carry the two largest energies
            assert min(e[want]) >= max(e[[p for p in range(4) if p not in want]])
            assert set(kept) <= set(want)


def test_block_scaled_kept_reconstruction_is_exact_on_grid():
    # kept values already on the E2M1 grid under a power-of-two MX scale come
    # back unchanged: 2:4 prune then MXFP4 loses only the dropped elements
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(grid, size=(4, 128)) * rng.choice([-1, 1], size=(4, 128))
    x[:, ::32] = 6.0  # every MX block of kept values reaches 6 -> scale 2^0
    raw = bf16(x)
    codes, meta, sc = O.prune_quantize(raw, O.BF16, O.QSpec("mxfp4"))
    xhat = O.dequantize_pruned(codes, meta, O.QSpec("mxfp4"), sc)
    vals, _ = O.prune_compress(raw, O.BF16)
    assert np.array_equal(xhat, O.decompress(O.decode_input(vals, O.BF16), meta))


def test_sparse_bits_accounting():
    # 2:4: v/2 + 1 index bit; pairwise 4:8: v/2 + 1/2; block scales cover kept values
    assert O.bits_per_element(O.QSpec("nvfp4"), pattern="pairs4:8") == 2 + 0.5 + 0.25
    assert O.bits_per_element(O.QSpec("mxfp4"), pattern="2:4") == 2 + 1 + 0.125
    assert O.bits_per_element(O.QSpec("int", 8), pattern="pairs4:8") == 4.5
    assert O.bits_per_element(O.QSpec("int", 8), pattern="2:4") == \
        O.bits_per_element(O.QSpec("int", 8), sparse24=True) == 5.0
    n = 1 << 20
    assert O.bits_per_element(O.QSpec("nvfp4"), pattern="pairs4:8", tensor_elems=n) == 2.75 + 32 / n


# ---------------------------------------------------------------------------
# Hadamard rotation ([PD §4]: a rescaled orthogonal +-1 matrix mixes values and
# spreads outliers; the pages measure R about twice as large after rotation on
# Q, K and linear-layer inputs)
# ---------------------------------------------------------------------------


def test_hadamard_matrix_is_sylvester_and_orthogonal():
    for n in (1, 2, 8, 64, 512):
        h = O.hadamard_matrix(n)
        i = np.arange(n)
        pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
        assert np.array_equal(h, (-1.0) ** pc)
        assert np.array_equal(h @ h.T, n * np.eye(n))
    for k in range(0, 13):
        n = 1 << k
        c = O.hadamard_scale(n)
        assert abs(c * c * n - 1.0) <= 4e-16
        if k % 2 == 0:
            assert c == 2.0 ** (-k // 2)


def test_hadamard8_hand_example():
    ex = HAND["hadamard8"]
    raw = bf16(ex["rows"])
    y = O.rotate(raw, O.BF16, ex["n"])
    want = np.stack([hexs(r).astype(np.uint16) if False else
                     np.array([int(h, 16) for h in r], dtype=np.uint16) for r in ex["rotated_bf16"]])
    assert np.array_equal(y, want)


def test_rotation_one_hot_columns():
    # e_j rotates to column j of H scaled by 1/sqrt(n); n = 64 has an exact scale 1/8
    n = 64
    x = np.eye(n, dtype=np.float32)
    y = O.rotate(x, O.F32, n).astype(np.float64)
    assert np.array_equal(y, O.hadamard_matrix(n).T / 8.0)


def test_rotation_involution_and_energy():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    for n in (8, 128, 512):
        y = O.rotate(x, O.F32, n)
        z = O.rotate(y, O.F32, n)
        assert np.allclose(z, x, rtol=0, atol=1e-5)
        e0 = (x.astype(np.float64) ** 2).sum(axis=1)
        e1 = (y.astype(np.float64) ** 2).sum(axis=1)
        assert np.allclose(e1, e0, rtol=2e-6)
    raw = W.to_bf16_bits(x)
    yb = O.decode_input(O.rotate(raw, O.BF16, 128), O.BF16)
    xb = O.decode_input(raw, O.BF16)
    assert np.allclose((yb ** 2).sum(axis=1), (xb ** 2).sum(axis=1), rtol=1e-2)


def test_rotation_exactness_predicate():
    raw = W.activation_x(3, 64, 1024)
    assert O.rotation_exact(raw, O.BF16, 128).all()
    x = np.zeros((1, 8), dtype=np.float32)
    x[0, 0], x[0, 1] = 2.0 ** 40, 1.0 + 2.0 ** -23
    assert not O.rotation_exact(x, O.F32, 8).all()
    x[0, 1] = 1.0
    assert O.rotation_exact(x, O.F32, 8).all()


def test_rotation_flattens_outliers_and_raises_R():
    # [PD §4]: rotation spreads the outlier channels, so 2:4 drops more energy
    # while the dense quantizer's range narrows; the pages measure R about twice
    # as large on linear-layer inputs
    raw = W.activation_x(0, 256, 4096)
    rot = O.rotate(raw, O.BF16, 128)
    assert O.rotation_exact(raw, O.BF16, 128).all()
    ks, ds = [O.QSpec("fp8"), O.QSpec("fp8")], [O.QSpec("fp8"), O.QSpec("int", 8)]
    r0 = O.predict_R(raw, O.BF16, ks, ds)[0]
    r1 = O.predict_R(rot, O.BF16, ks, ds)[0]
    assert r1[0, 0] > 2 * r0[0, 0]               # energy loss grows (outliers were always kept)
    assert r1[1, 3] < r0[1, 3]                   # dense INT8 error shrinks
    for p in range(2):
        assert r1[p, 4] > 1.3 * r0[p, 4]         # R grows


def test_rotation_leaves_gaussian_loss_unchanged():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((256, 1024)).astype(np.float32)
    y = O.rotate(x, O.F32, 128)
    e = O.error_energy(y, O.F32, O.QSpec("none"), O.QSpec("int", 8))[0]
    assert 0.1309 <= e[1] / e[0] <= 0.1339         # still the Gaussian 13.2% [PD §4]


# ---------------------------------------------------------------------------
# Operator-level error ([PD §2]: relative error of the operator output; [PD §4]:
# the energy criterion predicts it)
# ---------------------------------------------------------------------------


def test_operator_error_with_orthogonal_b_equals_energy():
    # B = H / sqrt(K) is orthogonal, so ||(Ahat - A) B^T||^2 = ||Ahat - A||^2:
    # the operator-level error energy is exactly the tensor's error energy
    rng = np.random.default_rng(21)
    k = 256
    raw = W.to_bf16_bits(rng.standard_normal((12, k)))
    b = (O.hadamard_matrix(k) / 16.0).astype(np.float32)       # exact in fp32
    sides = [O.Side("2:4", O.QSpec("fp8")), O.Side("dense", O.QSpec("int", 4)),
             O.Side("pairs4:8", O.QSpec("nvfp4")), O.Side("dense", O.QSpec("mxfp4"))]
    op = O.operator_error(raw, O.BF16, b, O.F32, sides)
    e24 = O.error_energy(raw, O.BF16, O.QSpec("fp8"), O.QSpec("int", 4))[0]
    e48 = O.error_energy(raw, O.BF16, O.QSpec("nvfp4"), O.QSpec("mxfp4"), pattern="pairs4:8")[0]
    tot = op[:, 0].sum()
    assert tot == pytest.approx(e24[0], rel=1e-12)
    assert op[:, 1].sum() == pytest.approx(e24[1] + e24[2], rel=1e-9)
    assert op[:, 2].sum() == pytest.approx(e24[3], rel=1e-9)
    assert op[:, 3].sum() == pytest.approx(e48[1] + e48[2], rel=1e-9)
    assert op[:, 4].sum() == pytest.approx(e48[3], rel=1e-9)


def test_operator_error_exact_quantizer_is_zero():
    # integer rows with amax 127: INT8 reproduces them, so the output is exact
    rng = np.random.default_rng(5)
    a = rng.integers(-127, 128, size=(6, 64)).astype(np.float32)
    a[:, 0] = 127
    b = rng.standard_normal((10, 64)).astype(np.float32)
    op = O.operator_error(a, O.F32, b, O.F32, [O.Side("dense", O.QSpec("int", 8)),
                                               O.Side("2:4", O.QSpec("none"))])
    assert np.all(op[:, 1] == 0.0)
    assert np.all(op[:, 2] > 0.0)


def test_operator_error_random_b_tracks_energy():
    # with an iid Gaussian B, E ||D B^T||^2 = N ||D||^2: the measured and the
    # predicted error energies agree to a few percent, so measured and
    # predicted R agree
    rng = np.random.default_rng(9)
    raw = W.activation_x(2, 64, 1024)
    b = rng.standard_normal((2048, 1024)).astype(np.float32)
    sides = [O.Side("2:4", O.QSpec("fp8")), O.Side("dense", O.QSpec("fp8")),
             O.Side("dense", O.QSpec("int", 8))]
    op = O.operator_error(raw, O.BF16, b, O.F32, sides).sum(axis=0)
    r = O.predict_R(raw, O.BF16, [O.QSpec("fp8"), O.QSpec("fp8")],
                    [O.QSpec("fp8"), O.QSpec("int", 8)])[0]
    meas = [np.sqrt(op[1] / op[2]), np.sqrt(op[1] / op[3])]
    assert meas[0] == pytest.approx(r[0, 4], rel=0.1)
    assert meas[1] == pytest.approx(r[1, 4], rel=0.1)
