"""Helpers shared by the GPU tests: move seeded inputs to the device, run one
rank's forward + backward through the C ABI, bring results back as float64.
Torch is plumbing here (device memory, copies, the stream)."""
import numpy as np

TOL = {"f32": 1e-4, "f16": 5e-3, "bf16": 2e-2}


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(values64: np.ndarray, dtype: str):
    """float64 values exact in `dtype` -> contiguous device tensor of that dtype."""
    import torch
    from synth import storage_bits
    bits = storage_bits(np.ascontiguousarray(values64), dtype)
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(bits)
    return t.to("cuda").contiguous()


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def device_inputs(inp, A=None, b1=None, B=None):
    """X, A, b1, B, dY of `inp` on the device (weights may be overridden, e.g. by a shard slice)."""
    d = inp.dtype
    return (to_device(inp.X, d), to_device(inp.A if A is None else A, d), to_device(inp.b1 if b1 is None else b1, d),
            to_device(inp.B if B is None else B, d), to_device(inp.dY, d))


def run_shard(tpmlp, X, A, b1, B, dY, keep_h=True, keep_dz=True, staged=True):
    """Forward then backward of one rank; returns the device outputs.
    staged=False gives the library the minimal workspaces (operands read in
    place instead of through k-contiguous copies)."""
    import torch
    Z, H, Yp = tpmlp.fwd(X, A, b1, B, keep_h=keep_h, staged=staged)
    g = tpmlp.bwd(dY, X, A, B, Z, H, keep_dz=keep_dz, staged=staged)
    torch.cuda.synchronize()
    out = {"Z": Z, "Yp": Yp, **g}
    if H is not None:
        out["H"] = H
    return out


def compare(got: dict, ref: dict, tol: float, keys=None):
    """Per-tensor max|got - ref| / max|ref|; returns {key: err} and asserts each <= tol."""
    from oracle import rel_err
    errs = {}
    for k in keys or ref:
        if k not in got or got[k] is None:
            continue
        g = got[k] if isinstance(got[k], np.ndarray) else to_host(got[k])
        errs[k] = rel_err(g, ref[k])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"parity failed (tol {tol}): {bad}; all: {errs}"
    return errs
