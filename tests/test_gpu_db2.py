"""Parity of tp_mlp_db2 (db2 = sum over tokens of dY) against the oracle's
bias2_grad, through the C ABI: storage-dtype output and fp32 main-gradient
accumulation (two micro-batches add twice), ragged and empty shapes, the
h=10240 workload's dY, and bitwise run-to-run determinism."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, to_device, to_host

pytestmark = pytest.mark.gpu


def _dy(T, h, dtype, seed, sigma=1.0):
    inp = synth.draw_inputs(T, h, 8 if dtype != "f32" else 4, dtype, seed=seed, sigma_dy=sigma)
    return inp.dY


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("T,h", [(200, 136), (520, 264), (8, 8), (256, 64), (1000, 1032)])
def test_db2_matches_oracle(gpu_lib, dtype, T, h):
    import torch
    print(f"case db2 dtype={dtype} T={T} h={h}", flush=True)
    dY = _dy(T, h, dtype, seed=T + h)
    d = to_device(dY, dtype)
    got = gpu_lib.db2(d)
    torch.cuda.synchronize()
    ref = oracle.bias2_grad(dY)
    err = oracle.rel_err(to_host(got), ref)
    assert err <= TOL[dtype], err
    again = gpu_lib.db2(d)
    torch.cuda.synchronize()
    assert torch.equal(got, again)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_db2_accumulates_into_fp32(gpu_lib, dtype):
    import torch
    T, h = 520, 264
    dY = _dy(T, h, dtype, seed=3)
    d = to_device(dY, dtype)
    rng = np.random.default_rng(1)
    start = rng.standard_normal(h)
    main = torch.as_tensor(start, dtype=torch.float32, device="cuda")
    n = gpu_lib.tp_mlp_db2_workspace_bytes(T, h, {"f32": 0, "f16": 1, "bf16": 2}[dtype])
    ws = torch.empty((n,), dtype=torch.uint8, device="cuda") if n else None
    ref = oracle.bias2_grad(dY)
    old = to_host(main)
    for step in range(2):
        gpu_lib.tp_mlp_db2(d, main, ws, accumulate=True)
        torch.cuda.synchronize()
        new = to_host(main)
        err = float(np.max(np.abs(new - old - ref)) / np.max(np.abs(ref)))
        assert err <= 1e-5, (step, err)  # fp32 sums of exact inputs, no rounding to storage
        old = new


def test_db2_of_no_tokens_is_zero(gpu_lib):
    import torch
    d = torch.empty((0, 136), dtype=torch.bfloat16, device="cuda")
    out = torch.full((136,), 7.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.tp_mlp_db2(d, out, None)
    torch.cuda.synchronize()
    assert bool((out == 0).all())


@pytest.mark.slow
def test_db2_full_size_h10240(gpu_lib):
    """dY of the h=10240 workload (16384 x 10240 bf16, N(0, 0.01^2))."""
    import torch
    cfg = synth.get_config("gpt_h10240")
    print("case db2 full-size h10240", flush=True)
    inp = synth.draw_config(cfg)
    got = gpu_lib.db2(to_device(inp.dY, cfg.dtype))
    torch.cuda.synchronize()
    err = oracle.rel_err(to_host(got), oracle.bias2_grad(inp.dY))
    assert err <= TOL[cfg.dtype], err
