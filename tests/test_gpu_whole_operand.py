"""GPU parity of whole-operand energies (one block of rows) when a team sums
more than one row into its partial slot.

The energy kernels run on a persistent grid of at most 4 workgroups per CU;
with more rows than resident teams, each team walks several rows, every lane
adds its share of each row into its own fp64 slot in LDS, and each
workgroup adds its slots in a fixed order at the end.  These cases use more
rows than the teams a 256-CU MI355X holds, in the launch shapes the calls use
at those sizes, and compare with the fp64 oracle to 1e-6 relative
("Is 2:4 Sparsity Still Worth It?", paper-daily.com English summary, §4:
energies over the tensor's total sum of squares).
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
from gpu_util import raw_np, random_raw, to_dev  # noqa: E402
from test_gpu_parity import qs_oracle, rel_close  # noqa: E402


def oracle_whole(raw, dtype, kept, dense, score="magnitude", norms=None, chunk=2048):
    """Oracle predict_R of the whole operand from sums over row chunks (every
    sum is additive over rows; chunks keep the fp64 temporaries small)."""
    out = []
    for kq, dq in zip(kept, dense):
        tot = np.zeros((1, 4))
        for r0 in range(0, raw.shape[0], chunk):
            tot += O.error_energy(raw[r0:r0 + chunk], dtype, qs_oracle(kq), qs_oracle(dq), score,
                                  norms)
        out.append(O.energies_to_R(tot))
    return np.stack(out, axis=1)


def resident_teams(team):
    """Teams the energy kernel's grid can hold at once: 4 workgroups of 256
    lanes per CU at most."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return cus * 4 * (256 // team)


@pytest.mark.parametrize("dtype,rows,k,team", [("bf16", 9000, 4096, 64), ("f32", 2500, 4096, 128),
                                               ("f16", 2500, 4096, 128), ("bf16", 1500, 16384, 256)])
def test_whole_operand_several_rows_per_team(dtype, rows, k, team):
    assert rows > resident_teams(team)
    raw = random_raw(np.random.default_rng(rows + k), (rows, k), dtype)
    x = to_dev(raw, dtype)
    kept, dense = ["fp8", ("int", 4)], [("int", 8), "fp8"]
    if k > 4096:
        kept, dense = ["fp8"], [("int", 8)]
    print(f"whole operand {dtype} [{rows}, {k}] pairs {list(zip(kept, dense))}", flush=True)
    a = S.predict_R(x, kept, dense)
    b = S.predict_R(x, kept, dense)
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))      # fixed order: repeatable
    rel_close(raw_np(a), oracle_whole(raw, dtype, kept, dense))


def test_whole_weight_wanda_sweep():
    """The weight W [14336, 4096] with Wanda 2:4 (channel norms of the
    activation X [4096, 4096]) over the equal-bits sweep 2:4 + INT-2m against
    dense INT-(m+1), m = 2..8, as one block: the benchmark's call."""
    xbits = W.activation_x(1, 4096, 4096)
    norms = O.col_l2norm(xbits, "bf16")
    wbits = W.weight_w(2, 14336, 4096)
    w = to_dev(wbits, "bf16")
    n = torch.from_numpy(norms).cuda()
    kept = [("int", 2 * m) for m in range(2, 9)]
    dense = [("int", m + 1) for m in range(2, 9)]
    print("Wanda sweep, whole W [14336, 4096], 7 pairs", flush=True)
    got = raw_np(S.predict_R(w, kept, dense, score="wanda", col_norm=n))
    assert got.shape == (1, 7, 5)
    rel_close(got, oracle_whole(wbits, "bf16", kept, dense, "wanda", norms))
    # the blocked path (already compared per block) sums to the same totals
    raw_blocks = np.stack([raw_np(S.error_energy(w, kq, dq, score="wanda", col_norm=n,
                                                 rows_per_block=128)).sum(axis=0)
                           for kq, dq in zip(kept, dense)])
    whole = np.stack([raw_np(S.error_energy(w, kq, dq, score="wanda", col_norm=n))[0]
                      for kq, dq in zip(kept, dense)])
    rel_close(whole, raw_blocks, rtol=1e-12)


@pytest.mark.parametrize("dtype,rows,k,team,kept,dense,rpb", [
    ("bf16", 50000, 128, 16, "fp8", ("int", 8), 7),          # held rows, 4 teams per wave
    ("bf16", 9000, 4096, 64, ("int", 4), "fp8", 100),        # held rows, one-wave teams
    ("bf16", 9000, 4096, 64, "fp8", "mxfp4", 100),           # packed rows (block format)
    ("f32", 20000, 256, 32, "fp8", ("int", 8), 33),          # fp32 operand
])
def test_blocked_sums_segments_straddle_blocks(dtype, rows, k, team, kept, dense, rpb):
    """Blocked energies when each team walks several contiguous rows whose
    blocks do not line up with the team's rows: a team's rows then fall in
    two blocks, and each block's sums gather rows of several teams.  Every
    block is compared with the fp64 oracle to 1e-6 relative, and the output
    repeats bit for bit."""
    assert rows > resident_teams(team)
    raw = random_raw(np.random.default_rng(rows + k + rpb), (rows, k), dtype)
    x = to_dev(raw, dtype)
    print(f"blocked {dtype} [{rows}, {k}] rows_per_block {rpb} {kept} vs {dense}", flush=True)
    a = S.predict_R(x, [kept], [dense], rows_per_block=rpb)
    b = S.predict_R(x, [kept], [dense], rows_per_block=rpb)
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))
    want = O.predict_R(raw, dtype, [qs_oracle(kept)], [qs_oracle(dense)], rows_per_block=rpb)
    rel_close(raw_np(a), want)
