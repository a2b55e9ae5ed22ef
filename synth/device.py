"""Seeded inputs on the device: float64 values that are exact in the storage
dtype become contiguous torch device tensors of that dtype, bit for bit.
Plumbing only (a copy of the rounded bits); no arithmetic of the method."""
import numpy as np


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(values64: np.ndarray, dtype: str, device="cuda"):
    """float64 values exact in `dtype` -> contiguous device tensor of that dtype."""
    import torch
    from .draw import storage_bits
    bits = storage_bits(np.ascontiguousarray(values64), dtype)
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(bits)
    return t.to(device).contiguous()


def device_inputs(inp, A=None, b1=None, B=None, device="cuda"):
    """X, A, b1, B, dY of `inp` on the device (weights may be overridden, e.g. by a shard slice)."""
    d = inp.dtype
    return (to_device(inp.X, d, device), to_device(inp.A if A is None else A, d, device),
            to_device(inp.b1 if b1 is None else b1, d, device), to_device(inp.B if B is None else B, d, device),
            to_device(inp.dY, d, device))
