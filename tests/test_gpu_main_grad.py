"""Parity of tp_mlp_bwd_main_grad (weight gradients added to fp32 main
gradients, beta = 1) against the float64 oracle, through the C ABI.

main_new - main_old must match the oracle's dA, dB and db1 to the per-tensor
tolerance of the storage dtype (the operands, dZ included, are rounded to
storage like in tp_mlp_bwd). Starting from zero, rounding the main gradients
to the storage dtype must reproduce tp_mlp_bwd's outputs bit for bit: both
paths run the same kernels up to the epilogue.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, device_inputs, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture
def tile(request, gpu_lib):
    """Force one 16-bit tile engine through tp_mlp_debug_plan (None = the
    planner's choice); the default plan is restored afterwards."""
    value = getattr(request, "param", None)
    gpu_lib.tp_mlp_debug_plan(value, 0)
    yield value
    gpu_lib.tp_mlp_debug_plan(None, 0)


def _main_grad_step(tpmlp, X, A, b1, B, dY, mains, keep_h=True, keep_dz=True, staged=True):
    import torch
    Z, H, _ = tpmlp.fwd(X, A, b1, B, keep_h=keep_h, staged=staged)
    T, f, h = X.shape[0], A.shape[1], X.shape[1]
    dZ = torch.empty((T, f), dtype=X.dtype, device=X.device) if keep_dz else None
    dXp = torch.empty((T, h), dtype=X.dtype, device=X.device)
    flags = (0 if keep_dz else tpmlp.TPMLP_WS_DZ) | (0 if staged else tpmlp.TPMLP_WS_MINIMAL)
    code = {torch.float32: tpmlp.TPMLP_F32, torch.float16: tpmlp.TPMLP_F16, torch.bfloat16: tpmlp.TPMLP_BF16}[X.dtype]
    nws = tpmlp.tp_mlp_workspace_bytes(T, h, f, code, flags)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=X.device) if nws else None
    tpmlp.tp_mlp_bwd_main_grad(dY, X, A, B, Z, H, dZ, dXp, mains["dA"], mains["dB"], mains["db1"], ws)
    torch.cuda.synchronize()
    return dXp


def _mains(h, f, rng, scale):
    import torch
    m = {"dA": rng.standard_normal((h, f)) * scale, "dB": rng.standard_normal((f, h)) * scale,
         "db1": rng.standard_normal((f,)) * scale}
    return m, {k: torch.as_tensor(v, dtype=torch.float32, device="cuda") for k, v in m.items()}


def _err(new, old, ref):
    return float(np.max(np.abs(new - old - ref)) / max(np.max(np.abs(ref)), 1e-30))


@pytest.mark.parametrize("tile", [128, 256, "dma256", "dma320"], indirect=True)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f", [(200, 136, 264), (520, 264, 392), (8, 8, 8), (2048, 1024, 1024)])
def test_main_grad_accumulates(gpu_lib, tile, dtype, T, h, f):
    # 2048 x 1024 x 1024 (f = h): dB and dA as one paired launch on the direct-load tiles
    print(f"case main-grad tile={tile} dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + 2 * h + f, sigma_dy=1.0)
    ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    rng = np.random.default_rng(T + h)
    scale = float(np.max(np.abs(ref["dA"])))
    old, mains = _mains(h, f, rng, scale)
    X, A, b1, B, dY = device_inputs(inp)
    dXp = _main_grad_step(gpu_lib, X, A, b1, B, dY, mains)
    got = {k: to_host(v) for k, v in mains.items()}
    for k in ("dA", "dB", "db1"):
        assert _err(got[k], old[k], ref[k]) <= TOL[dtype], k
    assert oracle.rel_err(to_host(dXp), ref["dXp"]) <= TOL[dtype]
    # a second micro-batch with the same data adds the same gradients again
    _main_grad_step(gpu_lib, X, A, b1, B, dY, mains)
    for k in ("dA", "dB", "db1"):
        assert _err(to_host(mains[k]), old[k], 2.0 * ref[k]) <= TOL[dtype], k


@pytest.mark.parametrize("tile", [128, "dma256", "dma320"], indirect=True)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_main_grad_from_zero_rounds_to_the_plain_backward(gpu_lib, tile, dtype):
    import torch
    T, h, f = 520, 264, 392
    inp = synth.draw_inputs(T, h, f, dtype, seed=5, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    Z, H, _ = gpu_lib.fwd(X, A, b1, B)
    plain = gpu_lib.bwd(dY, X, A, B, Z, H)
    mains = {"dA": torch.zeros((h, f), dtype=torch.float32, device="cuda"),
             "dB": torch.zeros((f, h), dtype=torch.float32, device="cuda"),
             "db1": torch.zeros((f,), dtype=torch.float32, device="cuda")}
    _main_grad_step(gpu_lib, X, A, b1, B, dY, mains)
    for k in ("dA", "dB", "db1"):
        assert torch.equal(mains[k].to(X.dtype).view(torch.int16), plain[k].view(torch.int16)), k


@pytest.mark.parametrize("keep_h,keep_dz,staged", [(False, True, True), (True, False, True), (True, True, False),
                                                   (False, False, False)])
def test_main_grad_variants(gpu_lib, keep_h, keep_dz, staged):
    """H recomputed from Z, dZ kept in the workspace, operands read in place."""
    T, h, f = 520, 264, 392
    inp = synth.draw_inputs(T, h, f, "bf16", seed=17, sigma_dy=1.0)
    ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    old, mains = _mains(h, f, np.random.default_rng(3), 1.0)
    _main_grad_step(gpu_lib, *device_inputs(inp), mains, keep_h=keep_h, keep_dz=keep_dz, staged=staged)
    for k in ("dA", "dB", "db1"):
        assert _err(to_host(mains[k]), old[k], ref[k]) <= TOL["bf16"], k


@pytest.mark.parametrize("T,h,f", [(64, 128, 256), (200, 132, 268)])
def test_main_grad_fp32_storage(gpu_lib, T, h, f):
    inp = synth.draw_inputs(T, h, f, "f32", seed=23, sigma_dy=1.0)
    ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    old, mains = _mains(h, f, np.random.default_rng(4), 0.1)
    _main_grad_step(gpu_lib, *device_inputs(inp), mains)
    for k in ("dA", "dB", "db1"):
        assert _err(to_host(mains[k]), old[k], ref[k]) <= TOL["f32"], k


@pytest.mark.slow
def test_main_grad_full_size_sampled(gpu_lib):
    """The h=10240 shard in bench.py's launch configuration (256 x 320 tiles,
    staged operands): tile-complete samples of FFN columns (one in every
    64-wide band) give columns of dA and rows of dB over their whole other
    dimension, so every output tile of both; checked with db1 against the
    oracle, from zero-started main gradients."""
    import torch
    cfg = synth.get_config("gpt_h10240")
    T, h, f = cfg.tokens, cfg.hidden, cfg.ffn_shard
    print(f"case main-grad full size T={T} h={h} f={f}", flush=True)
    inp = synth.draw_config(cfg)
    mains = {"dA": torch.zeros((h, f), dtype=torch.float32, device="cuda"),
             "dB": torch.zeros((f, h), dtype=torch.float32, device="cuda"),
             "db1": torch.zeros((f,), dtype=torch.float32, device="cuda")}
    _main_grad_step(gpu_lib, *device_inputs(inp), mains)
    from tests.gpu_util import tile_complete_samples
    cols = tile_complete_samples(f, 8)
    rc = oracle.sampled_cols(inp.X, inp.A, inp.b1, inp.B, inp.dY, cols)
    ci = torch.as_tensor(cols, device="cuda")
    assert oracle.rel_err(to_host(mains["dA"].index_select(1, ci)), rc["dA"]) <= TOL[cfg.dtype]
    assert oracle.rel_err(to_host(mains["dB"].index_select(0, ci)), rc["dB"]) <= TOL[cfg.dtype]
    assert oracle.rel_err(to_host(mains["db1"].index_select(0, ci)), rc["db1"]) <= TOL[cfg.dtype]
