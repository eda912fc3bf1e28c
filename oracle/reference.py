"""Step-by-step reference definitions (numpy, fp64; fp32 steps emulated exactly).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the CPU baseline
of the benchmark; never by the product path.

Operands are 2-D arrays ``[rows, K]`` whose last axis is the GEMM reduction
axis along which the hardware forms its groups of four
([PD intro], [PD §1]: the hardware fixes which operand is sparse and along
which axis). A 3-D operand is passed with its leading dims flattened into
rows, and a strided operand (V pruned along the sequence) is passed already
transposed so that the reduction axis is last.

Storage encodings: ``"bf16"`` = uint16 bit patterns, ``"f16"`` = numpy
float16, ``"f32"`` = numpy float32.

Readings of steps the pages leave open (each is also listed in the design
notes):

* Groups are aligned runs of four along K starting at k = 0; K % 8 == 0 so
  that the 4-bit group metadata fills whole bytes.
* Ties between equal scores keep the lower position.
* The 2:4 side quantizes its kept values with one symmetric scale per row
  taken from the absolute maximum of the kept values.
* INT-b is symmetric round-to-nearest-even with qmax = 2^(b-1) - 1.
* FP8 is OCP e4m3 (max 448, no infinities), round-to-nearest-even,
  saturating, with the sign copied from the scaled value.
* MXFP4 uses the OCP MX rule for the shared power-of-two scale; NVFP4 uses an
  fp32 tensor scale T/(448*6) and e4m3 block scales.
* A row (or NVFP4 tensor) whose absolute maximum is below 2^-64 is encoded
  as zeros with a zero scale; this keeps every reciprocal finite in fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

BF16, F16, F32 = "bf16", "f16", "f32"

#: Rows (or an NVFP4 tensor) with absolute maximum below this are zero-coded.
TINY_AMAX = 2.0 ** -64

# ---------------------------------------------------------------------------
# Input
# ---------------------------------------------------------------------------


def decode_input(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored operand elements."""
    if dtype == BF16:
        r = np.asarray(raw, dtype=np.uint16)
        return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F16:
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == F32:
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_rows(raw: np.ndarray) -> None:
    if raw.ndim != 2:
        raise ValueError("oracle operands are 2-D [rows, K]")
    if raw.shape[1] % 8 != 0:
        raise ValueError("K must be a multiple of 8")


# ---------------------------------------------------------------------------
# 2:4 selection and compression  ([PD intro], [PD §2], [PD §3 Q&A on pruners])
# ---------------------------------------------------------------------------


def score_values(x: np.ndarray, score: str = "magnitude",
                 col_norm: Optional[np.ndarray] = None) -> np.ndarray:
    """Pruning score of every element.

    Magnitude pruning ranks by |x|; Wanda ranks a weight by its magnitude times
    the size of the activation on its input channel, taken here as the L2
    norm of that input column ([PD §2], the three pruners of the 2:4 side).
    The product of an fp32 norm and a (<= fp32) element is exact in fp64.
    """
    a = np.abs(x)
    if score == "magnitude":
        return a
    if score == "wanda":
        if col_norm is None:
            raise ValueError("wanda needs col_norm")
        n = np.asarray(col_norm, dtype=np.float32).astype(np.float64)
        if n.shape != (x.shape[-1],):
            raise ValueError("col_norm must have K entries")
        return a * n[None, :]
    raise ValueError(f"unknown score {score!r}")


def select_2of4(s: np.ndarray) -> np.ndarray:
    """Positions kept in every group of four: the two largest scores.

    Returns int64 ``[rows, K/4, 2]`` with i0 < i1. Equal scores are ordered
    by position, lower first ([PD intro]: two non-zeros kept in every four
    along the reduction axis; tie rule is a reading).
    """
    rows, k = s.shape
    g = s.reshape(rows, k // 4, 4)
    # descending score; a stable sort keeps equal scores in ascending position
    order = np.argsort(-g, axis=-1, kind="stable")
    return np.sort(order[..., :2], axis=-1).astype(np.int64)


def meta_from_indices(idx: np.ndarray) -> np.ndarray:
    """Pack kept positions into metadata bytes.

    Group g uses the nibble (i0 | i1 << 2); groups 2j and 2j+1 share byte j,
    the even group in the low nibble. This is 2 bits per kept value, i.e. the
    1 bit per original element that the equal-bits accounting charges ([PD §2]).
    """
    rows, ng, _ = idx.shape
    nib = (idx[..., 0] | (idx[..., 1] << 2)).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def indices_from_meta(meta: np.ndarray) -> np.ndarray:
    """Inverse of :func:`meta_from_indices`."""
    rows, nb = meta.shape
    nib = np.empty((rows, nb * 2), dtype=np.int64)
    nib[:, 0::2] = meta & 0xF
    nib[:, 1::2] = meta >> 4
    return np.stack([nib & 3, nib >> 2], axis=-1)


def _mask_from_indices(idx: np.ndarray, k: int) -> np.ndarray:
    rows, ng, _ = idx.shape
    m = np.zeros((rows, ng, 4), dtype=bool)
    np.put_along_axis(m, idx, True, axis=-1)
    return m.reshape(rows, k)


def _kept_from_indices(arr: np.ndarray, idx: np.ndarray) -> np.ndarray:
    rows, k = arr.shape
    g = arr.reshape(rows, k // 4, 4)
    return np.take_along_axis(g, idx, axis=-1).reshape(rows, k // 2)


def prune_compress(raw: np.ndarray, dtype: str, score: str = "magnitude",
                   col_norm: Optional[np.ndarray] = None):
    """Online 2:4 prune-and-compress of one operand ([PD §3], fused kernel).

    Returns ``(values, meta)``: the kept elements in their storage encoding,
    in ascending position order, ``[rows, K/2]``; and metadata bytes
    ``[rows, K/8]``.
    """
    _check_rows(raw)
    x = decode_input(raw, dtype)
    idx = select_2of4(score_values(x, score, col_norm))
    return _kept_from_indices(np.asarray(raw), idx), meta_from_indices(idx)


def decompress(values: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """Scatter kept values back to their positions; dropped slots are zero
    (all-zero bits in the storage encoding)."""
    rows, kh = values.shape
    k = kh * 2
    idx = indices_from_meta(meta)
    out = np.zeros((rows, k // 4, 4), dtype=values.dtype)
    np.put_along_axis(out, idx, values.reshape(rows, k // 4, 2), axis=-1)
    return out.reshape(rows, k)


# ---------------------------------------------------------------------------
# Pairwise 4:8 ([PD §6]: Blackwell's sparse FP4 splits each group of eight
# into four adjacent pairs and keeps two pairs)
# ---------------------------------------------------------------------------


def pair_scores(x: np.ndarray) -> np.ndarray:
    """Energy of each adjacent pair, fp64(a^2 + b^2) (the squares are exact,
    the sum is rounded once).  Returns [rows, K/2]."""
    a = x[:, 0::2]
    b = x[:, 1::2]
    return a * a + b * b


def select_pairs48(ps: np.ndarray) -> np.ndarray:
    """Pairs kept in every group of four pairs (eight elements): the two
    largest pair energies, ties to the lower pair.  Keeping pairs by their
    energy is the reading under which i.i.d. Gaussian data lose exactly 5/24
    of their energy, the pages' 20.8%.  Returns [rows, K/8, 2], p0 < p1."""
    rows, npair = ps.shape
    g = ps.reshape(rows, npair // 4, 4)
    order = np.argsort(-g, axis=-1, kind="stable")
    return np.sort(order[..., :2], axis=-1).astype(np.int64)


def prune_compress_pairs48(raw: np.ndarray, dtype: str):
    """Pairwise 4:8 prune-and-compress.

    Returns ``(values [rows, K/2], meta [rows, K/16])``: the two kept pairs of
    each group in pair order, and per group the nibble (p0 | p1 << 2), two
    groups per byte with the even group in the low nibble."""
    rows, k = raw.shape
    if k % 16:
        raise ValueError("pairwise 4:8 needs K % 16 == 0")
    x = decode_input(raw, dtype)
    sel = select_pairs48(pair_scores(x))                         # [rows, K/8, 2]
    pairs = np.asarray(raw).reshape(rows, k // 8, 4, 2)
    kept = np.take_along_axis(pairs, sel[..., None], axis=2)    # [rows, K/8, 2, 2]
    nib = (sel[..., 0] | (sel[..., 1] << 2)).astype(np.uint8)
    meta = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return kept.reshape(rows, k // 2), meta


def _mask_pairs48(x: np.ndarray) -> np.ndarray:
    rows, k = x.shape
    sel = select_pairs48(pair_scores(x))
    m = np.zeros((rows, k // 8, 4), dtype=bool)
    np.put_along_axis(m, sel, True, axis=-1)
    return np.repeat(m.reshape(rows, k // 2), 2, axis=1)


def decompress_pairs48(values: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """Dense [rows, K] from pairwise 4:8 values [rows, K/2] and meta
    [rows, K/16]; dropped pairs are zero."""
    rows, half = values.shape
    k = 2 * half
    nib = np.empty((rows, k // 8), dtype=np.int64)
    nib[:, 0::2] = meta & 0xF
    nib[:, 1::2] = meta >> 4
    out = np.zeros((rows, k // 8, 4, 2), dtype=values.dtype)
    v = values.reshape(rows, k // 8, 2, 2)
    g = np.arange(k // 8)
    for r in range(rows):
        out[r, g, nib[r] & 3] = v[r, :, 0]
        out[r, g, nib[r] >> 2] = v[r, :, 1]
    return out.reshape(rows, k)


# ---------------------------------------------------------------------------
# Hadamard rotation along K ([PD §4]: before low-bit quantization the tensor
# is multiplied by a rescaled +-1 orthogonal Hadamard matrix, which spreads
# outliers over many elements)
# ---------------------------------------------------------------------------


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1:
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_scale(n: int) -> float:
    """fp64 1/sqrt(n) for n = 2^k: 2^-(k/2) for even k, and for odd k
    2^-((k-1)/2) times the correctly rounded sqrt(1/2)."""
    k = n.bit_length() - 1
    c = 1.0 if k % 2 == 0 else math.sqrt(0.5)
    return math.ldexp(c, -(k // 2))


def _f32_to_bf16_bits(y32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of finite fp32 values to bf16 bit patterns."""
    u = np.asarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def rotate(raw: np.ndarray, dtype: str, n: int) -> np.ndarray:
    """Block Hadamard rotation along K: every aligned block b of n elements
    becomes y = H_n x_b / sqrt(n), returned in the input's storage type.

    The sums S = H_n x_b are formed in fp64 (a matrix product; exact whenever
    :func:`rotation_exact` holds, so the summation order does not matter), a
    zero sum is taken as +0, then fp64(S * hadamard_scale(n)) is rounded to
    fp32 and, for 16-bit storage, from fp32 to the storage type (each step
    round-to-nearest-even).  Applying it twice gives back the input up to
    those roundings (H_n H_n = n I)."""
    rows, k = raw.shape
    if k % n:
        raise ValueError("K must be a multiple of the block size")
    x = decode_input(raw, dtype).reshape(rows * (k // n), n)
    S = x @ hadamard_matrix(n).T + 0.0
    y32 = (S * hadamard_scale(n)).astype(np.float32).reshape(rows, k)
    if dtype == BF16:
        return _f32_to_bf16_bits(y32)
    if dtype == F16:
        return y32.astype(np.float16)
    return y32


def rotation_exact(raw: np.ndarray, dtype: str, n: int) -> np.ndarray:
    """Per block: True when every partial sum of any +-1 combination of the
    block's values is exact in fp64, so that every summation order gives the
    exact S of :func:`rotate`.  All values are multiples of 2^L (L the lowest
    set bit over the block) and every partial sum is below n * 2^E (|x| <
    2^E), so E + log2(n) - L <= 53 bits suffice."""
    rows, k = raw.shape
    x = np.abs(decode_input(raw, dtype).reshape(rows * (k // n), n))
    f, e = np.frexp(x)                                   # x = f * 2^e, 0.5 <= f < 1
    m = (f * 2.0 ** 53).astype(np.int64)                 # exact: <= 53 significant bits
    lsb = np.where(m > 0, m & -m, 1).astype(np.float64)  # lowest set bit (1 for zeros)
    low = np.where(m > 0, e - 53 + np.log2(lsb).astype(np.int64), 10 ** 6)
    hi = np.where(m > 0, e, -10 ** 6).max(axis=1)
    lo = low.min(axis=1)
    need = np.where((m > 0).any(axis=1), hi + int(math.log2(n)) - lo, 0)
    return (need <= 53).reshape(rows, k // n)


# ---------------------------------------------------------------------------
# Element encoders ([PD §3]: FP8, MXFP4 and NVFP4 as the dense rivals; a
# reading fixes OCP e4m3 and E2M1 with round-to-nearest-even, saturating)
# ---------------------------------------------------------------------------


def _e4m3_grid() -> np.ndarray:
    codes = np.arange(0x7F)                    # 0x7F is NaN in e4m3 (no Inf)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))


#: Non-negative e4m3 values indexed by their 7-bit code (0 .. 0x7E = 448).
E4M3_GRID = _e4m3_grid()
#: Non-negative E2M1 values indexed by their 3-bit code.
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_code(grid: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each a >= 0; on an exact tie the
    even index. Values beyond the last point map to the last point, which is
    what saturation means for a finite grid."""
    a = np.asarray(a, dtype=np.float64)
    j = np.clip(np.searchsorted(grid, a, side="left"), 1, grid.size - 1)
    lo = grid[j - 1]
    hi = grid[j]
    dlo = a - lo
    dhi = hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (j % 2 == 0))
    return np.where(pick_hi, j, j - 1).astype(np.int64)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """OCP e4m3 code (uint8) of each finite y: nearest of the 127 finite
    magnitudes, ties to the even code, saturating at 448; sign bit copied
    from y (so -0 gives 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    mag = _nearest_code(E4M3_GRID, np.abs(y))
    return (mag | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("NaN code")
    v = E4M3_GRID[c & 0x7F]
    return np.where(c & 0x80, -v, v)


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """E2M1 code (4 bits, in uint8) of each finite y: nearest of
    {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6;
    sign bit (bit 3) copied from y."""
    y = np.asarray(y, dtype=np.float64)
    mag = _nearest_code(E2M1_GRID, np.abs(y))
    return (mag | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    v = E2M1_GRID[c & 7]
    return np.where(c & 8, -v, v)


def int_rtn_codes(y: np.ndarray, bits: int) -> np.ndarray:
    """Symmetric b-bit round-to-nearest ([PD §2], plain RTN): round half to
    even, clip to [-(2^(b-1)-1), 2^(b-1)-1]."""
    qmax = 2 ** (bits - 1) - 1
    return np.clip(np.rint(np.asarray(y, dtype=np.float64)), -qmax, qmax).astype(np.int64)


# ---------------------------------------------------------------------------
# Quantizer specs
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class QSpec:
    """A quantizer: fmt in {"none", "int", "fp8", "mxfp4", "nvfp4"}.

    ``bits`` is used by "int" (2..16). ``tensor_amax`` optionally fixes the
    NVFP4 tensor maximum (otherwise it is the operand's own maximum).
    """
    fmt: str
    bits: int = 0
    tensor_amax: Optional[float] = None


def _qmax(q: QSpec) -> float:
    if q.fmt == "int":
        if not 2 <= q.bits <= 16:
            raise ValueError("int bits must be in [2, 16]")
        return float(2 ** (q.bits - 1) - 1)
    if q.fmt == "fp8":
        return 448.0
    raise ValueError(f"{q.fmt} has no per-row qmax")


# ---------------------------------------------------------------------------
# Per-row quantization ([PD §3]: "INT8 with one scale per row"; FP8)
# ---------------------------------------------------------------------------


def row_scale(amax: np.ndarray, qmax: float):
    """Per-row scale s = fp32(amax / qmax) and reciprocal inv = fp32(qmax / amax).

    Both are single IEEE fp32 divisions. Rows with amax below 2^-64 get
    s = inv = 0 (their codes are then zero)."""
    a = np.asarray(amax, dtype=np.float32)
    q = np.float32(qmax)
    s = np.zeros_like(a)
    inv = np.zeros_like(a)
    big = a.astype(np.float64) >= TINY_AMAX
    s[big] = a[big] / q
    inv[big] = q / a[big]
    return s, inv


def _encode_scaled(v: np.ndarray, inv: np.ndarray, q: QSpec) -> np.ndarray:
    """Codes of fp32-valued v [rows, n] scaled by the per-row fp32 inv."""
    y = np.asarray(v, dtype=np.float32) * inv.astype(np.float32)[:, None]   # fp32 product
    if q.fmt == "int":
        c = int_rtn_codes(y, q.bits)
        return c.astype(np.int8 if q.bits <= 8 else np.int16)
    if q.fmt == "fp8":
        return e4m3_encode(y)
    raise ValueError(q.fmt)


def dequantize_rows(codes: np.ndarray, q: QSpec, scales: np.ndarray) -> np.ndarray:
    """x_hat = value(code) * s in fp64 (the product is exact)."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]
    if q.fmt == "int":
        return codes.astype(np.float64) * s
    if q.fmt == "fp8":
        return e4m3_decode(codes) * s
    raise ValueError(q.fmt)


def quantize_rows(raw: np.ndarray, dtype: str, q: QSpec):
    """Dense per-row INT-b or FP8 quantization of every element.

    Returns ``(codes [rows, K], scales fp32 [rows])``."""
    _check_rows(raw)
    x = decode_input(raw, dtype).astype(np.float32)     # exact
    amax = np.max(np.abs(x), axis=1)
    s, inv = row_scale(amax, _qmax(q))
    return _encode_scaled(x, inv, q), s


# ---------------------------------------------------------------------------
# Block-scaled 4-bit formats ([PD §3]: MXFP4 with one power-of-two scale per
# 32 elements; NVFP4 with an FP8 scale per 16 elements plus one per tensor)
# ---------------------------------------------------------------------------


def _pack_nibbles(c: np.ndarray) -> np.ndarray:
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(p: np.ndarray) -> np.ndarray:
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize_mxfp4(raw: np.ndarray, dtype: str):
    """MXFP4: per 32-element block along K, an E8M0 scale 2^e with
    e = floor(log2(block amax)) - 2 clamped to [-127, 127] (the OCP MX rule,
    2 being the largest E2M1 exponent), then E2M1 codes of x / 2^e.

    Returns ``(codes packed two per byte [rows, K/2], e8m0 [rows, K/32])``;
    element 2j sits in the low nibble of byte j. All-zero blocks get scale
    code 0."""
    _check_rows(raw)
    rows, k = raw.shape
    if k % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    x = decode_input(raw, dtype).reshape(rows, k // 32, 32)
    amax = np.max(np.abs(x), axis=-1)
    _, ex = np.frexp(amax)                 # amax = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1 - 2, -127, 127)
    e = np.where(amax > 0, e, -127)
    y = x / np.exp2(e)[..., None]          # division by a power of two
    codes = e2m1_encode(y).reshape(rows, k)
    return _pack_nibbles(codes), (e + 127).astype(np.uint8)


def dequantize_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = _unpack_nibbles(packed)
    rows, k = c.shape
    v = e2m1_decode(c).reshape(rows, k // 32, 32)
    return (v * np.exp2(scales.astype(np.float64) - 127)[..., None]).reshape(rows, k)


def tensor_absmax(raw: np.ndarray, dtype: str) -> np.float32:
    return np.float32(np.max(np.abs(decode_input(raw, dtype))))


def quantize_nvfp4(raw: np.ndarray, dtype: str, tensor_amax: Optional[float] = None):
    """NVFP4-style: fp32 tensor scale s_t = T / 2688 (2688 = 448 * 6) with T
    the tensor's absolute maximum; per 16-element block an e4m3 scale
    b = e4m3(amax_blk * 448 / T); elements are E2M1 codes of x / (b * s_t).
    Each listed product and quotient is one fp32 operation.

    Returns ``(codes packed [rows, K/2], block scales e4m3 [rows, K/16],
    s_t fp32)``. T below 2^-64 zero-codes the whole tensor."""
    _check_rows(raw)
    rows, k = raw.shape
    if k % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    x = decode_input(raw, dtype).astype(np.float32).reshape(rows, k // 16, 16)
    t = np.float32(tensor_absmax(raw, dtype) if tensor_amax is None else tensor_amax)
    if float(t) < TINY_AMAX:
        s_t = np.float32(0.0)
        g = np.float32(0.0)
    else:
        s_t = t / np.float32(2688.0)
        g = np.float32(448.0) / t
    amax = np.max(np.abs(x), axis=-1)                     # fp32, exact
    b = e4m3_encode(amax * g)                              # fp32 product
    bval = e4m3_decode(b).astype(np.float32)
    d = bval * s_t                                         # fp32 product
    inv = np.zeros_like(d)
    nz = d > 0
    inv[nz] = np.float32(1.0) / d[nz]                      # fp32 reciprocal
    y = x * inv[..., None]                                 # fp32 product
    codes = e2m1_encode(y).reshape(rows, k)
    return _pack_nibbles(codes), b, np.float32(s_t)


def dequantize_nvfp4(packed: np.ndarray, bscales: np.ndarray, s_t) -> np.ndarray:
    """x_hat = e2m1 * block scale * s_t, exact in fp64."""
    c = _unpack_nibbles(packed)
    rows, k = c.shape
    v = e2m1_decode(c).reshape(rows, k // 16, 16)
    bv = e4m3_decode(bscales)[..., None]
    return (v * bv * float(np.float32(s_t))).reshape(rows, k)


# ---------------------------------------------------------------------------
# Fused prune + quantize of the kept values ([PD §4]: the 2:4 side quantizes
# the kept values to 2m bits; [PD §5]: 2:4 stacked on FP8)
# ---------------------------------------------------------------------------


def quantize_kept(kept_raw: np.ndarray, dtype: str, q: QSpec):
    """Quantize compressed kept values ``[rows, K/2]`` (stored in ``dtype``).

    INT / FP8: one scale per row from the kept values' absolute maximum,
    returns ``(codes [rows, K/2], scales fp32 [rows])``.  MXFP4 / NVFP4: the
    block format applied to the compressed row, so a block covers 32 / 16
    consecutive kept values; returns what :func:`quantize_mxfp4` /
    :func:`quantize_nvfp4` return, with the NVFP4 tensor maximum taken over
    the kept values unless ``q.tensor_amax`` is given (the sparse FP4 format
    of [PD §6] scales what it stores)."""
    if q.fmt in ("int", "fp8"):
        kept = decode_input(kept_raw, dtype).astype(np.float32)
        amax = np.max(np.abs(kept), axis=1)
        s, inv = row_scale(amax, _qmax(q))
        return _encode_scaled(kept, inv, q), s
    if q.fmt == "mxfp4":
        return quantize_mxfp4(kept_raw, dtype)
    if q.fmt == "nvfp4":
        return quantize_nvfp4(kept_raw, dtype, q.tensor_amax)
    raise ValueError(q.fmt)


def prune_quantize(raw: np.ndarray, dtype: str, q: QSpec, score: str = "magnitude",
                   col_norm: Optional[np.ndarray] = None):
    """Prune 2:4, then quantize the kept values (:func:`quantize_kept`).

    Returns ``(codes, meta [rows, K/8], *scales)``: INT/FP8 codes [rows, K/2]
    with fp32 row scales; MXFP4 packed codes [rows, K/4] with E8M0 scales
    [rows, K/64]; NVFP4 packed codes [rows, K/4], e4m3 scales [rows, K/32]
    and the fp32 tensor scale."""
    vals, meta = prune_compress(raw, dtype, score, col_norm)
    qc = quantize_kept(vals, dtype, q)
    return (qc[0], meta) + tuple(qc[1:])


def prune_quantize_pairs48(raw: np.ndarray, dtype: str, q: QSpec):
    """Pairwise 4:8 prune, then quantize the kept values
    (:func:`quantize_kept`); with NVFP4 this is the sparse FP4 operand of
    [PD §6].  Returns ``(codes, meta [rows, K/16], *scales)`` as
    :func:`prune_quantize`."""
    vals, meta = prune_compress_pairs48(raw, dtype)
    qc = quantize_kept(vals, dtype, q)
    return (qc[0], meta) + tuple(qc[1:])


def dequantize_kept(codes: np.ndarray, q: QSpec, *scales) -> np.ndarray:
    """fp64 kept values [rows, K/2] from :func:`quantize_kept`'s output."""
    if q.fmt in ("int", "fp8"):
        return dequantize_rows(codes, q, scales[0])
    if q.fmt == "mxfp4":
        return dequantize_mxfp4(codes, scales[0])
    if q.fmt == "nvfp4":
        return dequantize_nvfp4(codes, scales[0], scales[1])
    raise ValueError(q.fmt)


def dequantize_pruned(codes: np.ndarray, meta: np.ndarray, q: QSpec, *scales,
                      pattern: str = "2:4") -> np.ndarray:
    """Dense fp64 reconstruction of a pruned-and-quantized operand."""
    kept = dequantize_kept(codes, q, *scales)
    return decompress(kept, meta) if pattern == "2:4" else decompress_pairs48(kept, meta)


# ---------------------------------------------------------------------------
# Energy reductions and predicted R ([PD §4])
# ---------------------------------------------------------------------------


def _reconstruct_kept(kept_raw: np.ndarray, dtype: str, q: QSpec) -> np.ndarray:
    """Kept values after the sparse side's quantizer, fp64 [rows, K/2]."""
    if q.fmt == "none":
        return decode_input(kept_raw, dtype)
    codes, *scales = quantize_kept(kept_raw, dtype, q)
    return dequantize_kept(codes, q, *scales)


def _reconstruct_dense(raw: np.ndarray, dtype: str, q: QSpec,
                       tensor_amax: Optional[float]) -> np.ndarray:
    """Every element after a dense quantizer, fp64 [rows, K]."""
    if q.fmt == "none":
        return decode_input(raw, dtype)
    if q.fmt in ("int", "fp8"):
        c, s = quantize_rows(raw, dtype, q)
        return dequantize_rows(c, q, s)
    if q.fmt == "mxfp4":
        return dequantize_mxfp4(*quantize_mxfp4(raw, dtype))
    if q.fmt == "nvfp4":
        t = q.tensor_amax if q.tensor_amax is not None else tensor_amax
        return dequantize_nvfp4(*quantize_nvfp4(raw, dtype, t))
    raise ValueError(q.fmt)


def _block_sums(per_row: np.ndarray, rows_per_block: int) -> np.ndarray:
    rows = per_row.shape[0]
    rpb = rows if rows_per_block in (0, None) else rows_per_block
    nblk = -(-rows // rpb)
    return np.array([per_row[b * rpb:(b + 1) * rpb].sum(axis=0) for b in range(nblk)])


def error_energy(raw: np.ndarray, dtype: str, kept_q: QSpec, dense_q: QSpec,
                 score: str = "magnitude", col_norm: Optional[np.ndarray] = None,
                 rows_per_block: int = 0, pattern: str = "2:4") -> np.ndarray:
    """Absolute error energies per block of rows ([PD §4]).

    Returns fp64 ``[nblk, 4]`` = (sum x^2, sum of dropped x^2, sum over kept
    elements of (x - x_hat)^2 under ``kept_q``, sum over all elements of
    (x - x_hat)^2 under ``dense_q``). Blocks are runs of ``rows_per_block``
    rows (0 = the whole operand); the NVFP4 tensor maximum is always taken
    over the whole operand.  ``pattern`` "pairs4:8" uses the pairwise 4:8
    selection (magnitude only) in place of element-wise 2:4.
    """
    _check_rows(raw)
    rows, k = raw.shape
    x = decode_input(raw, dtype)
    if pattern == "2:4":
        idx = select_2of4(score_values(x, score, col_norm))
        mask = _mask_from_indices(idx, k)
        kept_raw = _kept_from_indices(np.asarray(raw), idx)
    elif pattern == "pairs4:8":
        if score != "magnitude":
            raise ValueError("pairwise 4:8 ranks pairs by energy only")
        kept_raw, _ = prune_compress_pairs48(raw, dtype)
        mask = _mask_pairs48(x)
    else:
        raise ValueError(pattern)
    x2 = x * x                     # exact: inputs carry at most 24 significant bits
    kept_x = decode_input(kept_raw, dtype)
    kept_hat = _reconstruct_kept(kept_raw, dtype, kept_q)
    t = float(tensor_absmax(raw, dtype))
    dense_hat = _reconstruct_dense(raw, dtype, dense_q, t)
    per_row = np.stack([
        x2.sum(axis=1),
        np.where(mask, 0.0, x2).sum(axis=1),
        ((kept_x - kept_hat) ** 2).sum(axis=1),
        ((x - dense_hat) ** 2).sum(axis=1),
    ], axis=1)
    return _block_sums(per_row, rows_per_block)


def predict_R(raw: np.ndarray, dtype: str, kept_qs: Sequence[QSpec],
              dense_qs: Sequence[QSpec], score: str = "magnitude",
              col_norm: Optional[np.ndarray] = None, rows_per_block: int = 0,
              pattern: str = "2:4") -> np.ndarray:
    """Predicted R per block and quantizer pair ([PD §4]).

    For pair p: E_prune = dropped energy / total energy (the "2:4 energy
    loss"); E_qkept = kept-side quantization error energy / total;
    E_2:4 = E_prune + E_qkept (the two errors sit on disjoint elements once
    the mask is fixed, so they add); E_dense = dense error energy / total;
    R = sqrt(E_2:4 / E_dense). Division follows IEEE fp64 (0/0 = NaN,
    x/0 = inf).

    Returns fp64 ``[nblk, npairs, 5]`` = (E_prune, E_qkept, E_2:4, E_dense, R).
    """
    if len(kept_qs) != len(dense_qs):
        raise ValueError("kept_qs and dense_qs must pair up")
    outs = []
    for kq, dq in zip(kept_qs, dense_qs):
        s = error_energy(raw, dtype, kq, dq, score, col_norm, rows_per_block, pattern)
        outs.append(energies_to_R(s))
    return np.stack(outs, axis=1)


def energies_to_R(s: np.ndarray) -> np.ndarray:
    """The five outputs of one quantizer pair from the four absolute sums of
    :func:`error_energy` ([PD §4]): fp64 ``[nblk, 4]`` -> ``[nblk, 5]`` =
    (E_prune, E_qkept, E_2:4 = E_prune + E_qkept, E_dense, R), each energy
    over the block's total sum of squares, R = sqrt(E_2:4 / E_dense)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        tot = s[:, 0]
        e_prune = s[:, 1] / tot
        e_qk = s[:, 2] / tot
        e24 = e_prune + e_qk
        e_d = s[:, 3] / tot
        r = np.sqrt(e24 / e_d)
    return np.stack([e_prune, e_qk, e24, e_d, r], axis=1)


# ---------------------------------------------------------------------------
# Operator-level error ([PD §2]: accuracy is the relative error of the
# operator's output against a full-precision reference output)
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Side:
    """One side of a comparison: ``pattern`` "dense", "2:4" or "pairs4:8"
    (magnitude selection) and the quantizer of the values it keeps (fmt
    "none" keeps the sparse side's values in the input's storage type)."""
    pattern: str
    q: QSpec


def reconstruct(raw: np.ndarray, dtype: str, side: Side) -> np.ndarray:
    """The operand the GEMM consumes on that side, fp64 [rows, K]: pruned
    elements are zero, kept or dense values are dequantized (NVFP4's tensor
    maximum over what is quantized: all values, or the kept ones)."""
    if side.pattern == "dense":
        if side.q.fmt == "none":
            raise ValueError("a dense side needs a quantizer")
        return _reconstruct_dense(raw, dtype, side.q, float(tensor_absmax(raw, dtype)))
    if side.pattern == "2:4":
        vals, meta = prune_compress(raw, dtype)
        return decompress(_reconstruct_kept(vals, dtype, side.q), meta)
    if side.pattern == "pairs4:8":
        vals, meta = prune_compress_pairs48(raw, dtype)
        return decompress_pairs48(_reconstruct_kept(vals, dtype, side.q), meta)
    raise ValueError(side.pattern)


def operator_error(a_raw: np.ndarray, a_dtype: str, b_raw: np.ndarray, b_dtype: str,
                   sides: Sequence[Side]) -> np.ndarray:
    """Squared output errors of Y = A B^T per row of A ([PD §2]).

    A [M, K] is the operand under test, B [N, K] the unmodified second
    operand (both with the reduction axis last).  Returns fp64 [M, 1 + S]:
    column 0 is sum_n Y[m, n]^2 of the reference output (the exact product of
    the stored values, formed in fp64), column 1 + s is sum_n (Yhat - Y)^2
    where Yhat uses side s's reconstruction of A.  Since Yhat - Y =
    (Ahat - A) B^T, the relative error energy of side s is column 1 + s
    summed over rows divided by column 0 summed over rows; the measured R of
    two sides is the square root of the ratio of their error energies."""
    A = decode_input(a_raw, a_dtype)
    B = decode_input(b_raw, b_dtype)
    out = np.empty((A.shape[0], 1 + len(sides)))
    out[:, 0] = ((A @ B.T) ** 2).sum(axis=1)
    for i, side in enumerate(sides):
        D = reconstruct(a_raw, a_dtype, side) - A
        out[:, 1 + i] = ((D @ B.T) ** 2).sum(axis=1)
    return out


# ---------------------------------------------------------------------------
# Wanda input-channel norms and the equal-bits accounting
# ---------------------------------------------------------------------------


def col_l2norm(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Per-column L2 norm of an activation X [tokens, channels]: the
    "activation size" Wanda multiplies a weight's magnitude by ([PD §2]).
    The sum of squares is exactly rounded (math.fsum), its square root taken
    in fp64 and rounded once to fp32."""
    x = decode_input(raw, dtype)
    out = np.empty(x.shape[1], dtype=np.float32)
    for j in range(x.shape[1]):
        col = x[:, j]
        out[j] = np.float32(math.sqrt(math.fsum((col * col).tolist())))
    return out


def bits_per_element(q: QSpec, sparse24: bool = False, row_len: Optional[int] = None,
                     value_bits: Optional[int] = None,
                     tensor_elems: Optional[int] = None, pattern: Optional[str] = None) -> float:
    """Storage bits charged per original element ([PD §2]: values, indices
    and scales all count).

    Dense: value bits + scale bits amortised over the elements they cover
    (one fp32 per row of ``row_len`` for INT/FP8 rows; 8 bits per 32 for
    MXFP4; 8 bits per 16 plus one fp32 per tensor for NVFP4).
    Sparse (``pattern`` "2:4", or ``sparse24=True``, or "pairs4:8"): half the
    elements at the kept value width, plus the position bits (2:4: 2 bits per
    kept value, 1 per original element; pairwise 4:8: 2 bits per kept pair,
    1/2 per original element), plus the scales: the per-row scale as on the
    dense side, block scales over kept values (so half as many per original
    element), the NVFP4 tensor scale once. ``value_bits`` gives the width for
    fmt "none" (e.g. 16 for bf16).
    """
    if pattern is None:
        pattern = "2:4" if sparse24 else "dense"
    block = 0.0
    row = 0.0
    tensor = 0.0
    if q.fmt == "int":
        v, row = q.bits, (32.0 / row_len if row_len else 0.0)
    elif q.fmt == "fp8":
        v, row = 8, (32.0 / row_len if row_len else 0.0)
    elif q.fmt == "none":
        if value_bits is None:
            raise ValueError("fmt none needs value_bits")
        v = value_bits
    elif q.fmt == "mxfp4":
        v, block = 4, 8.0 / 32.0
    elif q.fmt == "nvfp4":
        v, block, tensor = 4, 8.0 / 16.0, (32.0 / tensor_elems if tensor_elems else 0.0)
    else:
        raise ValueError(q.fmt)
    if pattern == "dense":
        return float(v) + row + block + tensor
    index = {"2:4": 1.0, "pairs4:8": 0.5}[pattern]
    return v / 2.0 + index + row + block / 2.0 + tensor
