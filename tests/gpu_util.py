"""Helpers for GPU parity tests: move the same seeded bytes to the device and
back.  No method arithmetic lives here."""
import numpy as np
import torch

DEV = "cuda:0"


def t_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def t_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(DEV)


def t_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_dev(raw: np.ndarray, dtype: str) -> torch.Tensor:
    return {"bf16": t_bf16, "f16": t_f16, "f32": t_f32}[dtype](raw)


def raw_np(t: torch.Tensor) -> np.ndarray:
    """Storage bits / values of a device tensor in the oracle's encoding."""
    c = t.detach().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def random_raw(rng, shape, dtype: str, scale=1.0) -> np.ndarray:
    import workloads as W
    a = rng.standard_normal(shape) * scale
    if dtype == "bf16":
        return W.to_bf16_bits(a)
    if dtype == "f16":
        return a.astype(np.float16)
    return a.astype(np.float32)


def tie_heavy_raw(rng, shape, dtype: str) -> np.ndarray:
    """Small-alphabet values (many equal magnitudes, signed zeros, subnormals)."""
    import workloads as W
    bits = W.adversarial_groups_bf16(int(rng.integers(1 << 30)), *shape)
    if dtype == "bf16":
        return bits
    v = W.bf16_bits_to_f32(bits)
    if dtype == "f16":
        return v.astype(np.float16)
    return v.astype(np.float32)
