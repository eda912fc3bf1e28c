"""GPU parity of the GEMMs that consume the pruned operand ([PD §3]): the
sparse-MFMA GEMM on the compressed 2:4 layout and the dense GEMM of the
same tile, against the oracle's fp64 product of the decompressed operand.

Bound: bf16 x bf16 products are exact in fp32 and any order of K fp32
additions is within (K - 1) 2^-24 sum_k |a_k b_k| of the exact sum, so each
output must lie within that of the fp64 reference (plus one fp64 rounding)."""
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


def check(got, a64, b64, k):
    ref = a64 @ b64.T
    bound = (k - 1) * 2.0 ** -24 * (np.abs(a64) @ np.abs(b64).T) + 1e-300
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs outside the bound; worst ratio {(err / bound).max()}"


@pytest.mark.parametrize("m,n,k", [(16, 16, 64), (256, 256, 128), (300, 200, 64), (513, 777, 1024), (64, 1024, 4096)])
def test_sparse_gemm(m, n, k):
    rng = np.random.default_rng(m * 7 + n + k)
    a = W.to_bf16_bits(rng.standard_normal((m, k)))
    b = W.to_bf16_bits(rng.standard_normal((n, k)))
    vals, meta = S.prune_compress(to_dev(a, "bf16"))
    got = raw_np(S.sparse_gemm(vals, meta, to_dev(b, "bf16")))
    wv, wm = O.prune_compress(a, "bf16")
    a64 = O.decompress(O.decode_input(wv, "bf16"), wm)
    check(got, a64, O.decode_input(b, "bf16"), k)


def test_sparse_gemm_ties_and_zeros():
    rng = np.random.default_rng(3)
    m, n, k = 128, 96, 256
    a = W.adversarial_groups_bf16(5, m, k)
    b = W.to_bf16_bits(rng.standard_normal((n, k)))
    vals, meta = S.prune_compress(to_dev(a, "bf16"))
    got = raw_np(S.sparse_gemm(vals, meta, to_dev(b, "bf16")))
    wv, wm = O.prune_compress(a, "bf16")
    check(got, O.decompress(O.decode_input(wv, "bf16"), wm), O.decode_input(b, "bf16"), k)


@pytest.mark.parametrize("m,n,k", [(16, 16, 64), (300, 200, 128), (513, 777, 1024)])
def test_dense_gemm(m, n, k):
    rng = np.random.default_rng(m + n * 3 + k)
    a = W.to_bf16_bits(rng.standard_normal((m, k)))
    b = W.to_bf16_bits(rng.standard_normal((n, k)))
    got = raw_np(S.dense_gemm(to_dev(a, "bf16"), to_dev(b, "bf16")))
    check(got, O.decode_input(a, "bf16"), O.decode_input(b, "bf16"), k)


@pytest.mark.parametrize("m,n,k", [(16, 16, 128), (300, 200, 256), (513, 777, 1024)])
def test_fp8_gemm(m, n, k):
    # the dense FP8 rival: codes and row scales from quantize(), product on the
    # e4m3 MFMA, against the fp64 product of the dequantized operands
    rng = np.random.default_rng(m + 5 * n + k)
    a = W.to_bf16_bits(rng.standard_normal((m, k)))
    b = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.05)
    ca, sa = S.quantize(to_dev(a, "bf16"), "fp8")
    cb, sb = S.quantize(to_dev(b, "bf16"), "fp8")
    got = raw_np(S.fp8_gemm(ca, sa, cb, sb))
    wa, wsa = O.quantize_rows(a, "bf16", O.QSpec("fp8"))
    wb, wsb = O.quantize_rows(b, "bf16", O.QSpec("fp8"))
    a64 = O.dequantize_rows(wa, O.QSpec("fp8"), wsa)
    b64 = O.dequantize_rows(wb, O.QSpec("fp8"), wsb)
    ref = a64 @ b64.T
    # sum in fp32 over the code products, then two fp32 scale multiplies.  The
    # e4m3 MFMA's internal summation was measured up to 8% past the
    # round-to-nearest bound on single outputs, so it gets twice that bound.
    bound = 2 * (k - 1) * 2.0 ** -24 * (np.abs(a64) @ np.abs(b64).T) + 3 * 2.0 ** -24 * np.abs(ref) + 1e-300
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= bound).all(), f"{(err > bound).sum()} outside; worst {(err / bound).max()}"
