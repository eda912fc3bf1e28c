"""GPU parity of the operator-level output error ([PD §2]) against the
oracle's fp64 products.

Tolerance: per-row energies within 1e-3 relative.  The GPU forms each
residual with one fp32 FMA (2^-24) and splits it into bf16 hi + lo (2^-17);
products accumulate in fp32 over up to 2K terms, which bounds each output's
relative error by about 2K * 2^-24 (2.4e-4 at K = 2048, before the random
signs of the rounding errors average it down); a per-row energy sums squares
of 128-column tiles in fp32 (127 * 2^-24) and the tiles in fp64."""
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
from test_gpu_parity import rel_close  # noqa: E402

SIDES = [("2:4", ("fp8", 0)), ("dense", ("fp8", 0)), ("dense", ("int", 8)),
         ("2:4", ("none", 0)), ("pairs4:8", ("nvfp4", 0)), ("dense", ("nvfp4", 0)),
         ("dense", ("mxfp4", 0)), ("2:4", ("int", 4)), ("2:4", ("mxfp4", 0))]


def osides(sides):
    return [O.Side(p, O.QSpec(*q)) for p, q in sides]


@pytest.mark.parametrize("m,n,k", [(64, 128, 64), (200, 300, 256), (128, 512, 1024), (37, 1000, 2048)])
def test_operator_error(m, n, k):
    rng = np.random.default_rng(m + n + k)
    a = W.activation_x(m, m, k)
    b = W.to_bf16_bits(rng.standard_normal((n, k)))
    got = raw_np(S.operator_error(to_dev(a, "bf16"), to_dev(b, "bf16"), SIDES))
    want = O.operator_error(a, "bf16", b, "bf16", osides(SIDES))
    rel_close(got, want, rtol=1e-3)


def test_operator_error_row_layout():
    # rows of very different size: a transposed or mixed-up epilogue fails here
    rng = np.random.default_rng(1)
    m, n, k = 48, 256, 512
    scale = 2.0 ** np.arange(m)[:, None] / 2.0 ** 20
    a = W.to_bf16_bits(rng.standard_normal((m, k)) * scale)
    b = W.to_bf16_bits(rng.standard_normal((n, k)) * (1 + np.arange(n)[:, None] % 7))
    sides = [("dense", ("int", 8))]
    got = raw_np(S.operator_error(to_dev(a, "bf16"), to_dev(b, "bf16"), sides))
    want = O.operator_error(a, "bf16", b, "bf16", osides(sides))
    rel_close(got, want, rtol=1e-3)


def test_operator_error_orthogonal_b_matches_energies():
    # with B = H / sqrt(K) the output errors equal the tensor error energies
    k = 256
    a = W.activation_x(4, 96, k)
    b = W.to_bf16_bits(O.hadamard_matrix(k) / 16.0)
    got = raw_np(S.operator_error(to_dev(a, "bf16"), to_dev(b, "bf16"),
                                  [("2:4", ("fp8", 0)), ("dense", ("int", 8))])).sum(axis=0)
    e = raw_np(S.error_energy(to_dev(a, "bf16"), "fp8", ("int", 8)))[0]
    rel_close(got, [e[0], e[1] + e[2], e[3]], rtol=1e-3)
