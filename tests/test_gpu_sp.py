"""Sequence-parallel forward (tp_mlp_fwd_sp) on the GPU.

X is held as equal token-row slices in separate device buffers, one per
rank ("Training GPT-2 with Megatron-LM", section 5.1, --sequence-parallel);
the first GEMM reads every token row from the slice that holds it instead of
an all-gathered copy ("Understanding the Megatron-LM architecture: how 3D
parallelism assigns roles", section 1, the row-split item).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, device_inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def _slices(X, n):
    """n separate device buffers holding X's token rows in n equal blocks."""
    rows = X.shape[0] // n
    return [X[i * rows:(i + 1) * rows].clone() for i in range(n)]


def _bits(t):
    import torch
    return t.view(torch.int16)


# (T, h, f, slices, forced tile): slices of whole 256-row tiles on the
# direct-load engines (planned, or forced on small shapes), slices that split
# a 256-row tile (the planner falls back to the register-staged engines,
# which map each row to its slice), ragged and single slices
SHAPES = [(8192, 1024, 2560, 4, None), (7800, 1024, 2560, 2, None), (1024, 264, 392, 4, "dma256"),
          (1024, 264, 392, 2, "dma320"), (1024, 264, 392, 2, "dma320m32"), (520, 264, 392, 4, None), (264, 136, 200, 3, None),
          (96, 64, 128, 1, None), (4096, 512, 768, 16, 256)]


@pytest.mark.parametrize("staged", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T,h,f,n,tile", SHAPES)
def test_sliced_forward_is_bitwise_the_gathered_forward(gpu_lib, T, h, f, n, tile, dtype, staged):
    import torch
    print(f"case fwd_sp T={T} h={h} f={f} slices={n} tile={tile} {dtype} staged={staged}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + n, sigma_dy=1.0)
    X, A, b1, B, _ = device_inputs(inp)
    gpu_lib.tp_mlp_debug_plan(tile, 0)
    try:
        Z0, H0, Y0 = gpu_lib.fwd(X, A, b1, B, staged=staged)
        e = lambda *s: torch.full(s, float("nan"), dtype=X.dtype, device="cuda")
        Z, H, Yp = e(T, f), e(T, f), e(T, h)
        code = gpu_lib.TPMLP_BF16 if dtype == "bf16" else gpu_lib.TPMLP_F16
        nws = gpu_lib.tp_mlp_fwd_workspace_bytes(T, h, f, code)
        ws = torch.empty((nws,), dtype=torch.uint8, device="cuda") if (staged and nws) else None
        gpu_lib.tp_mlp_fwd_sp(_slices(X, n), A, b1, B, Z, H, Yp, ws)
        torch.cuda.synchronize()
    finally:
        gpu_lib.tp_mlp_debug_plan(None, 0)
    for got, want, k in ((Z, Z0, "Z"), (H, H0, "H"), (Yp, Y0, "Yp")):
        assert torch.equal(_bits(got), _bits(want)), k


@pytest.mark.parametrize("T,h,F,P,dtype", [(8192, 2560, 10240, 4, "bf16"), (520, 264, 1568, 4, "f16"),
                                           (384, 128, 512, 2, "bf16")])
def test_sequence_parallel_emulation_matches_the_unsharded_mlp(gpu_lib, T, h, F, P, dtype):
    """P ranks with tensor and sequence parallelism, emulated one after the
    other on the one GPU: rank r holds token slice r of X and its weight
    shard; its forward reads all P slices (the all-gather) and yields Z_r,
    H_r and the partial Yp_r over all tokens; rank r's reduce-scatter sums
    the P partials (plus b2) over its own token rows. The slices of Y
    stacked, and each rank's Z_r and H_r, must match the unsharded MLP."""
    import torch
    print(f"case sp emulation T={T} h={h} F={F} P={P} {dtype}", flush=True)
    inp = synth.draw_inputs(T, h, F, dtype, seed=17, sigma_dy=1.0, full=True, tp=P)
    b2 = synth.round_to_storage(np.random.default_rng(18).normal(0.0, 0.01, h), dtype)
    X = to_device(inp.X, dtype)
    xs = _slices(X, P)
    del X
    parts, zs, hs = [], [], []
    for r in range(P):
        A_r, b1_r, B_r = oracle.shard_weights(inp.A, inp.b1, inp.B, P, r)
        _, A_d, b1_d, B_d, _ = device_inputs(inp, A=A_r, b1=b1_r, B=B_r)
        f = A_r.shape[1]
        e = lambda *s: torch.empty(s, dtype=xs[0].dtype, device="cuda")
        Z, H, Yp = e(T, f), e(T, f), e(T, h)
        code = gpu_lib.TPMLP_BF16 if dtype == "bf16" else gpu_lib.TPMLP_F16
        nws = gpu_lib.tp_mlp_fwd_workspace_bytes(T, h, f, code)
        ws = torch.empty((nws,), dtype=torch.uint8, device="cuda") if nws else None
        gpu_lib.tp_mlp_fwd_sp(xs, A_d, b1_d, B_d, Z, H, Yp, ws)
        parts.append(Yp)
        zs.append(Z)
        hs.append(H)
    b2_d = to_device(b2, dtype)
    rows = T // P
    Y = []
    for r in range(P):
        out = torch.empty((rows, h), dtype=xs[0].dtype, device="cuda")
        gpu_lib.tp_mlp_reduce_partials(parts, b2_d, out, r * rows, (r + 1) * rows)
        Y.append(out)
    torch.cuda.synchronize()
    ref = oracle.mlp_forward(inp.X, inp.A, inp.b1, inp.B, b2)
    tol = TOL[dtype]
    errs = {"Y": oracle.rel_err(np.concatenate([to_host(y) for y in Y], axis=0), ref["Y"]),
            "Z": oracle.rel_err(np.concatenate([to_host(z) for z in zs], axis=1), ref["Z"]),
            "H": oracle.rel_err(np.concatenate([to_host(x) for x in hs], axis=1), ref["H"])}
    print("errors", errs, flush=True)
    assert all(v <= tol for v in errs.values()), errs
