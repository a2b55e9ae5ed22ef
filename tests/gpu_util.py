"""Helpers shared by the GPU tests: move seeded inputs to the device, run one
rank's forward + backward through the C ABI, bring results back as float64.
Torch is plumbing here (device memory, copies, the stream)."""
import numpy as np

from synth.device import device_inputs, to_device, torch_dtype  # noqa: F401  (re-exported for the tests)

TOL = {"f32": 1e-4, "f16": 5e-3, "bf16": 2e-2}


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


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


def tile_complete_samples(n, seed, band=64):
    """One random index in every `band`-wide band of [0, n), plus 0, n-1 and
    the two indices on each side of every multiple of 256 and 320 (tile
    edges of the planner's largest tiles)."""
    rng = np.random.default_rng(seed)
    idx = {0, n - 1}
    for b0 in range(0, n, band):
        idx.add(int(rng.integers(b0, min(n, b0 + band))))
    for t in (256, 320):
        for e in range(t, n, t):
            idx.update((e - 1, e))
    return np.array(sorted(i for i in idx if 0 <= i < n))
