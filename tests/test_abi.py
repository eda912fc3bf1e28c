"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments on the host before any HIP call, and
reports the missing device.  Pointers passed here are never dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from conftest import ROOT

B = pytest.importorskip("pruning_quantization_amd.binding")

HEADER = os.path.join(ROOT, "include", "sparq24.h")
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced on the host
OK, INVALID, UNSUPPORTED, SHAPE, ALIGN, WORKSPACE, DEVICE = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def L():
    try:
        return B.lib()
    except ImportError as e:
        pytest.skip(str(e))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparq24_[a-zA-Z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.SYMBOLS)


def tensor(dtype=B.BF16, batch=1, rows=4, k=64, bs=None, rs=None, ks=1, data=FAKE):
    c = B.CTensor()
    c.data, c.dtype, c.batch, c.rows, c.k = data, dtype, batch, rows, k
    c.row_stride = k if rs is None else rs
    c.batch_stride = rows * c.row_stride if bs is None else bs
    c.k_stride = ks
    return c


def pc(L, t, score=0, norm=None, vals=FAKE, meta=FAKE):
    return L.sparq24_prune_compress(ctypes.byref(t), score, norm, vals, meta, None)


def test_prune_compress_validation(L):
    assert pc(L, tensor(k=12)) == SHAPE
    assert pc(L, tensor(dtype=7)) == INVALID
    assert pc(L, tensor(rows=-1)) == INVALID
    assert pc(L, tensor(data=None)) == INVALID
    assert pc(L, tensor(data=FAKE + 8)) == ALIGN
    assert pc(L, tensor(), vals=None) == INVALID
    assert pc(L, tensor(), meta=FAKE + 4) == ALIGN
    assert pc(L, tensor(), score=5) == INVALID
    assert pc(L, tensor(), score=1, norm=None) == INVALID
    assert pc(L, tensor(rows=4, k=64, rs=68)) == ALIGN                     # 136-byte rows
    assert pc(L, tensor(rows=4, k=64, rs=32)) == UNSUPPORTED               # overlapping rows
    assert pc(L, tensor(rows=4, k=64, rs=2, ks=4)) == UNSUPPORTED          # neither layout
    # transposed rows are tiled by 64 on grid.y: 65535 tiles at most
    big = 65535 * 64
    assert pc(L, tensor(rows=big + 8, k=64, rs=1, ks=big + 8, bs=0)) == UNSUPPORTED
    # empty operands are a no-op, even with null outputs
    assert pc(L, tensor(rows=0), vals=None, meta=None) == OK
    assert pc(L, tensor(k=0), vals=None, meta=None) == OK


def test_valid_call_reports_missing_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert pc(L, tensor()) == DEVICE
    t = tensor(rows=8, k=128, rs=1, ks=8)          # transposed layout accepted
    assert pc(L, t) == DEVICE


def q(fmt, bits=0):
    s = B.CQSpec()
    s.fmt, s.bits, s.tensor_amax_in = fmt, bits, None
    return s


def test_quantize_validation_and_workspace_query(L):
    t = tensor(k=48)
    n = ctypes.c_size_t(123)
    f = L.sparq24_quantize
    assert f(ctypes.byref(t), ctypes.byref(q(B.Q_MXFP4)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == SHAPE
    assert f(ctypes.byref(t), ctypes.byref(q(B.Q_INT, 1)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == UNSUPPORTED
    assert f(ctypes.byref(t), ctypes.byref(q(B.Q_INT, 17)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == UNSUPPORTED
    assert f(ctypes.byref(t), ctypes.byref(q(9)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == INVALID
    assert f(ctypes.byref(t), ctypes.byref(q(B.Q_NONE)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == UNSUPPORTED
    assert f(ctypes.byref(t), None, FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == INVALID
    t64 = tensor(k=64)
    assert f(ctypes.byref(t64), ctypes.byref(q(B.Q_NVFP4)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value > 0                                       # NVFP4 needs partial maxima
    small = ctypes.c_size_t(n.value - 1)
    assert f(ctypes.byref(t64), ctypes.byref(q(B.Q_NVFP4)), FAKE, FAKE, FAKE, FAKE, ctypes.byref(small), None) == WORKSPACE
    assert f(ctypes.byref(t64), ctypes.byref(q(B.Q_NVFP4)), FAKE, FAKE, FAKE, FAKE, None, None) == WORKSPACE
    assert f(ctypes.byref(t64), ctypes.byref(q(B.Q_INT, 8)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value == 0
    big = tensor(k=32768 + 8)
    assert f(ctypes.byref(big), ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == SHAPE
    # transposed operand: staged through the workspace (8 x 128 bf16 = 2 KiB)
    tt = tensor(rows=8, k=128, rs=1, ks=8)
    assert f(ctypes.byref(tt), ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value >= 8 * 128 * 2
    assert L.sparq24_col_l2norm(ctypes.byref(tt), FAKE, None, ctypes.byref(n), None) == UNSUPPORTED


def test_energy_validation(L):
    t = tensor(k=64)
    n = ctypes.c_size_t(0)
    arr = (B.CQSpec * 2)(q(B.Q_FP8), q(B.Q_INT, 4))
    darr = (B.CQSpec * 2)(q(B.Q_FP8), q(B.Q_INT, 3))
    f = L.sparq24_predict_R
    assert f(ctypes.byref(t), 0, None, arr, darr, 0, 0, FAKE, None, ctypes.byref(n), None) == INVALID
    assert f(ctypes.byref(t), 0, None, arr, darr, 17, 0, FAKE, None, ctypes.byref(n), None) == INVALID
    assert f(ctypes.byref(t), 0, None, arr, darr, 2, -1, FAKE, None, ctypes.byref(n), None) == INVALID
    assert f(ctypes.byref(t), 0, None, arr, darr, 2, 0, FAKE, None, ctypes.byref(n), None) == OK
    # 4 rows x (2 + 2 kept + 2 dense) doubles + one block of sums, rounded to 256 B
    assert n.value >= 4 * 6 * 8 + 6 * 8
    # block formats on kept values block the compressed row: K % 64 (MX), K % 32 (NV)
    kept_mx = (B.CQSpec * 1)(q(B.Q_MXFP4))
    kept_nv = (B.CQSpec * 1)(q(B.Q_NVFP4))
    assert f(ctypes.byref(t), 0, None, kept_mx, darr, 1, 0, FAKE, None, ctypes.byref(n), None) == OK
    assert f(ctypes.byref(tensor(k=32)), 0, None, kept_mx, darr, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    assert f(ctypes.byref(tensor(k=48)), 0, None, kept_nv, darr, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    n0 = n.value
    assert f(ctypes.byref(t), 0, None, kept_nv, darr, 1, 0, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value > n0 - 1                    # kept NVFP4 adds the kept-maximum partials
    none = (B.CQSpec * 1)(q(B.Q_NONE))
    assert f(ctypes.byref(t), 0, None, none, none, 1, 0, FAKE, None, ctypes.byref(n), None) == UNSUPPORTED
    t48 = tensor(k=48)
    mx = (B.CQSpec * 1)(q(B.Q_MXFP4))
    assert f(ctypes.byref(t48), 0, None, arr, mx, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    empty = tensor(rows=0)
    assert f(ctypes.byref(empty), 0, None, arr, darr, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    g = L.sparq24_error_energy
    assert g(ctypes.byref(t), 0, None, None, ctypes.byref(q(B.Q_FP8)), 0, FAKE, None, ctypes.byref(n), None) == INVALID


def test_predict_R_noalloc_size_limit(L):
    # the static scratch holds SPARQ24_NOALLOC_SCRATCH_BYTES (8 MiB); a plan past
    # it is rejected on the host, before the device is touched
    arr = (B.CQSpec * 2)(q(B.Q_FP8), q(B.Q_INT, 4))
    f = L.sparq24_predict_R_noalloc
    assert f(ctypes.byref(tensor(rows=1 << 20, k=64)), 0, None, arr, arr, 2, 0, FAKE, None) == WORKSPACE
    assert f(ctypes.byref(tensor(rows=4, k=64)), 0, None, arr, arr, 0, 0, FAKE, None) == INVALID
    assert f(ctypes.byref(tensor(rows=4, k=64)), 0, None, arr, arr, 2, 0, None, None) == INVALID
    assert f(ctypes.byref(tensor(rows=4, k=64)), 0, None, arr, arr, 2, 0, FAKE, None) == DEVICE


def test_pairs48_validation(L):
    f = L.sparq24_prune_compress_pairs48
    assert f(ctypes.byref(tensor(k=24)), FAKE, FAKE, None) == SHAPE        # K % 16
    assert f(ctypes.byref(tensor(k=32)), None, FAKE, None) == INVALID
    assert f(ctypes.byref(tensor(rows=8, k=128, rs=1, ks=8)), FAKE, FAKE, None) == UNSUPPORTED
    n = ctypes.c_size_t(0)
    g = L.sparq24_predict_R_pairs48
    arr = (B.CQSpec * 1)(q(B.Q_FP8))
    assert g(ctypes.byref(tensor(k=24)), arr, arr, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    assert g(ctypes.byref(tensor(k=32)), arr, arr, 1, 0, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value > 0


def test_prune_quantize_validation(L):
    n = ctypes.c_size_t(7)
    f = L.sparq24_prune_quantize
    g = L.sparq24_prune_quantize_pairs48

    def pq(t, qq, ws=None, nb=None, ts=FAKE, score=0, norm=None):
        return f(ctypes.byref(t), score, norm, ctypes.byref(qq), FAKE, FAKE, FAKE, ts, ws, nb, None)

    def pq48(t, qq, ws=None, nb=None, ts=FAKE):
        return g(ctypes.byref(t), ctypes.byref(qq), FAKE, FAKE, FAKE, ts, ws, nb, None)

    assert pq(tensor(k=32), q(B.Q_MXFP4), nb=ctypes.byref(n)) == SHAPE      # 32 kept per block
    assert pq(tensor(k=64), q(B.Q_MXFP4), nb=ctypes.byref(n)) == OK and n.value == 0
    assert pq(tensor(k=48), q(B.Q_NVFP4), nb=ctypes.byref(n)) == SHAPE      # 16 kept per block
    assert pq(tensor(k=64), q(B.Q_NVFP4), nb=ctypes.byref(n)) == OK and n.value > 0
    assert pq(tensor(k=64), q(B.Q_NONE), nb=ctypes.byref(n)) == UNSUPPORTED
    assert pq(tensor(k=64), q(B.Q_NVFP4), ws=FAKE, nb=ctypes.byref(n), ts=None) == INVALID
    assert pq(tensor(k=64), q(B.Q_NVFP4), ws=FAKE, nb=ctypes.byref(n), ts=FAKE + 2) == ALIGN
    assert pq(tensor(k=64), q(B.Q_FP8), nb=ctypes.byref(n), score=1) == INVALID  # Wanda without norms
    assert pq48(tensor(k=24), q(B.Q_FP8), nb=ctypes.byref(n)) == SHAPE
    assert pq48(tensor(k=16), q(B.Q_FP8), nb=ctypes.byref(n)) == OK and n.value == 0
    assert pq48(tensor(k=32), q(B.Q_MXFP4), nb=ctypes.byref(n)) == SHAPE
    assert pq48(tensor(k=32), q(B.Q_NVFP4), nb=ctypes.byref(n)) == OK and n.value > 0
    # transposed operands are staged through the workspace
    assert pq48(tensor(rows=8, k=128, rs=1, ks=8), q(B.Q_FP8), nb=ctypes.byref(n)) == OK
    assert n.value >= 8 * 128 * 2


def test_rotation_validation(L):
    n = ctypes.c_size_t(5)
    h = L.sparq24_hadamard
    for blk in (0, 4, 12, 1536, 8192):
        assert h(ctypes.byref(tensor(k=8192)), blk, FAKE, None, ctypes.byref(n), None) == INVALID
    assert h(ctypes.byref(tensor(k=192)), 128, FAKE, None, ctypes.byref(n), None) == SHAPE
    assert h(ctypes.byref(tensor(k=256)), 128, FAKE, None, ctypes.byref(n), None) == OK and n.value == 0
    assert h(ctypes.byref(tensor(rows=8, k=128, rs=1, ks=8)), 64, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value >= 8 * 128 * 2
    fq = L.sparq24_quantize_rot
    assert fq(ctypes.byref(tensor(k=256)), 0, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == INVALID
    assert fq(ctypes.byref(tensor(k=256)), 64, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == OK
    fp = L.sparq24_prune_quantize_rot
    for pat, want in ((0, OK), (1, OK), (2, INVALID)):
        assert fp(ctypes.byref(tensor(k=256)), 64, pat, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE,
                  FAKE, None, ctypes.byref(n), None) == want
    fr = L.sparq24_predict_R_rot
    arr = (B.CQSpec * 1)(q(B.Q_FP8))
    assert fr(ctypes.byref(tensor(k=256)), 128, 1, arr, arr, 1, 0, FAKE, None, ctypes.byref(n), None) == OK
    assert n.value > 0
    assert fr(ctypes.byref(tensor(k=256)), 512, 0, arr, arr, 1, 0, FAKE, None, ctypes.byref(n), None) == SHAPE
    # whole-row blocks up to 4096 elements, rotated by a 256-lane workgroup per row
    # (at most four 8-element units per lane: rows of up to 8192 elements)
    assert fq(ctypes.byref(tensor(k=4096)), 4096, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == OK
    assert fq(ctypes.byref(tensor(k=8192)), 8192, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == INVALID
    assert fq(ctypes.byref(tensor(k=16384)), 1024, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == UNSUPPORTED
    assert fq(ctypes.byref(tensor(k=16384)), 512, ctypes.byref(q(B.Q_FP8)), FAKE, FAKE, FAKE, None,
              ctypes.byref(n), None) == OK


def test_copy_validation(L):
    assert L.sparq24_copy(FAKE, FAKE, 0, None) == OK
    assert L.sparq24_copy(FAKE, FAKE, 24, None) == ALIGN
    assert L.sparq24_copy(None, FAKE, 32, None) == INVALID


def test_bits_per_element_matches_oracle(L):
    cases = [(("int", 8), True, 4096), (("int", 5), False, 4096), (("int", 14), True, 0),
             (("fp8", 0), False, 4096), (("mxfp4", 0), False, 0), (("nvfp4", 0), False, 0)]
    for (fmt, bits), sp, rl in cases:
        got = B.bits_per_element((fmt, bits), sparse24=sp, row_len=rl)
        want = O.bits_per_element(O.QSpec(fmt, bits), sparse24=sp, row_len=rl or None)
        assert got == want
    assert B.bits_per_element("none", sparse24=True, value_bits=16) == 9.0
    for fmt in ("mxfp4", "nvfp4", ("int", 8), "fp8"):
        for pat in ("dense", "2:4", "pairs4:8"):
            qq = fmt if isinstance(fmt, tuple) else (fmt, 0)
            got = B.bits_per_element(qq, row_len=4096, tensor_elems=1 << 20, pattern=pat)
            want = O.bits_per_element(O.QSpec(*qq), row_len=4096, tensor_elems=1 << 20, pattern=pat)
            assert got == want, (fmt, pat)
    assert B.bits_per_element(("int", 1)) < 0


def test_status_strings(L):
    for s in range(8):
        assert L.sparq24_status_string(s)
    assert B.version().count(".") == 2
