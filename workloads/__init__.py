"""Seeded synthetic operands for the 2:4-vs-quantization hot path.

This module only draws random numbers and stores them in the operand's storage
type. It holds none of the method's arithmetic (no scores, masks, scales or
codes), so the CPU oracle and the HIP library can both consume its bytes
without sharing any code with each other.

The operand families and their value structure follow the paper's setting
(Qin, "Is 2:4 Sparsity Still Worth It?", paper-daily (en) summary, intro and
§1: linear-layer weights W and inputs X, attention Q, K, V and probabilities P)
and its Gaussian analysis (§4). Sizes are those of an 8B-class transformer
layer at long prefill lengths. No dataset or trained weight is used: every
tensor is synthetic.

Every generator returns a numpy array in the operand's storage encoding:
``uint16`` bit patterns for bf16, ``float32`` for fp32. bf16 values are drawn
in fp64, rounded to fp32 and then to bf16 with round-to-nearest-even (via the
torch CPU cast), so both sides of a parity check see identical bytes.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "gaussian_f32",
    "activation_x",
    "weight_w",
    "attention_qkv",
    "attention_p",
    "student_t_x",
    "adversarial_groups_bf16",
]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round an fp64/fp32 array to bf16 (RNE, via fp32) and return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian_f32(seed: int, rows: int = 256, k: int = 1024) -> np.ndarray:
    """iid N(0, 1) stored as fp32, shape [rows, k]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, k)).astype(np.float32)


def activation_x(seed: int, tokens: int = 4096, hidden: int = 4096,
                 outlier_frac: float = 0.001, outlier_scale: float = 50.0,
                 return_channels: bool = False):
    """Linear-layer input X [tokens, hidden] in bf16.

    Rows are N(0, 1); round(outlier_frac * hidden) hidden channels (at least
    one), fixed per seed and drawn without replacement, are multiplied by
    ``outlier_scale`` in every token.
    """
    rng = np.random.default_rng(seed)
    n_out = max(1, int(round(outlier_frac * hidden)))
    chans = np.sort(rng.choice(hidden, size=n_out, replace=False))
    x = rng.standard_normal((tokens, hidden))
    x[:, chans] *= outlier_scale
    bits = to_bf16_bits(x)
    return (bits, chans) if return_channels else bits


def weight_w(seed: int, rows: int = 14336, k: int = 4096,
             std: float = 0.02, row_sigma: float = 0.5) -> np.ndarray:
    """Weight W [rows, k] in bf16: N(0, std^2) times a per-row lognormal(0, row_sigma) factor."""
    rng = np.random.default_rng(seed)
    row_scale = np.exp(rng.normal(0.0, row_sigma, size=(rows, 1)))
    w = rng.normal(0.0, std, size=(rows, k)) * row_scale
    return to_bf16_bits(w)


def attention_qkv(seed: int, heads: int, seq: int, dim: int = 128,
                  outlier_dims: int = 4, outlier_scale: float = 8.0) -> np.ndarray:
    """Q, K or V [heads, seq, dim] in bf16: N(0, 1) with ``outlier_dims``
    head dimensions per head (drawn independently per head) scaled by
    ``outlier_scale``."""
    rng = np.random.default_rng(seed)
    out = np.empty((heads, seq, dim), dtype=np.uint16)
    for h in range(heads):
        dims = rng.choice(dim, size=outlier_dims, replace=False)
        a = rng.standard_normal((seq, dim))
        a[:, dims] *= outlier_scale
        out[h] = to_bf16_bits(a)
    return out


def attention_p(seed: int, heads: int = 32, q: int = 4096, k: int = 4096,
                logit_std: float = 3.0) -> np.ndarray:
    """Attention probabilities P [heads, q, k] in bf16: a row softmax over keys
    of iid N(0, logit_std^2) logits, evaluated in fp64 and rounded once to bf16.
    No causal mask."""
    rng = np.random.default_rng(seed)
    out = np.empty((heads, q, k), dtype=np.uint16)
    for h in range(heads):
        z = rng.standard_normal((q, k)) * logit_std
        z -= z.max(axis=1, keepdims=True)
        np.exp(z, out=z)
        z /= z.sum(axis=1, keepdims=True)
        out[h] = to_bf16_bits(z)
    return out


def student_t_x(seed: int, rows: int = 16384, k: int = 4096, nu: float = 4.0) -> np.ndarray:
    """Heavy-tailed activation [rows, k] in bf16: standard Student-t(nu), unscaled."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_t(nu, size=(rows, k)))


def adversarial_groups_bf16(seed: int, rows: int, k: int) -> np.ndarray:
    """bf16 rows built to stress tie-breaking and encoder edge cases.

    Values are drawn from a small alphabet (so groups of four often tie in
    magnitude, including +0/-0), mixed with subnormals, values near the fp8
    and fp4 saturation points after scaling, and some all-zero rows.
    """
    rng = np.random.default_rng(seed)
    alphabet = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 1.5, -3.0,
                         448.0, -448.0, 6.0, -6.0, 1e-40, -1e-40, 3e-39, 0.25, 0.75, 5.0],
                        dtype=np.float64)
    a = alphabet[rng.integers(0, alphabet.size, size=(rows, k))]
    # scatter some continuous values so scales are not always powers of two
    cont = rng.random((rows, k)) < 0.3
    a = np.where(cont, rng.standard_normal((rows, k)) * 3.0, a)
    bits = to_bf16_bits(a)
    # sign of zero survives the cast only through the bit pattern: force -0 where asked
    negz = (a == 0.0) & np.signbit(a)
    bits[negz] = np.uint16(0x8000)
    if rows >= 4:
        bits[rng.integers(0, rows)] = 0          # an all-(+0) row
        bits[rng.integers(0, rows)] = 0x8000     # an all-(-0) row
    return bits
