"""Parity of tp_mlp_bwd_recompute (Z_i recomputed from X inside the backward,
H_i taken as gelu(Z_i)) against the float64 oracle, through the C ABI, and
bit for bit against tp_mlp_fwd (H not kept) followed by tp_mlp_bwd with
H = NULL, which runs the same kernels on the same values."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, device_inputs

pytestmark = pytest.mark.gpu

GRADS = ("dZ", "dXp", "dA", "dB", "db1")


@pytest.fixture
def tile(request, gpu_lib):
    """Force one 16-bit tile engine through tp_mlp_debug_plan (None = the
    planner's choice); the default plan is restored afterwards."""
    value = getattr(request, "param", None)
    gpu_lib.tp_mlp_debug_plan(value, 0)
    yield value
    gpu_lib.tp_mlp_debug_plan(None, 0)


CASES = ([(None, "f32")] + [(t, d) for t in (None, 128, 256, "dma256", "dma320") for d in ("f16", "bf16")])


@pytest.mark.parametrize("tile,dtype", CASES, indirect=["tile"])
@pytest.mark.parametrize("T,h,f", [(200, 136, 264), (520, 264, 392)])
def test_recompute_matches_oracle_and_plain_backward(gpu_lib, tile, dtype, T, h, f):
    import torch
    print(f"case recompute tile={tile} dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + 5 * f, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    got = gpu_lib.bwd_recompute(dY, X, A, b1, B)
    torch.cuda.synchronize()
    ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    compare(got, ref, TOL[dtype], keys=GRADS)
    Z, _, _ = gpu_lib.fwd(X, A, b1, B, keep_h=False)
    plain = gpu_lib.bwd(dY, X, A, B, Z, None)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(got[k], plain[k]), k


@pytest.mark.parametrize("keep_dz,staged", [(False, True), (True, False), (False, False)])
def test_recompute_workspace_variants(gpu_lib, keep_dz, staged):
    import torch
    T, h, f = 520, 264, 392
    inp = synth.draw_inputs(T, h, f, "bf16", seed=31, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    got = gpu_lib.bwd_recompute(dY, X, A, b1, B, keep_dz=keep_dz, staged=staged)
    torch.cuda.synchronize()
    ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    compare(got, ref, TOL["bf16"], keys=[k for k in GRADS if got[k] is not None])


def test_recompute_events_bracket_each_step(gpu_lib):
    import torch
    T, h, f = 520, 264, 392
    inp = synth.draw_inputs(T, h, f, "bf16", seed=2, sigma_dy=1.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(gpu_lib.RECOMPUTE_EVENTS) + 1)]
    X, A, b1, B, dY = device_inputs(inp)
    gpu_lib.bwd_recompute(dY, X, A, b1, B, events=ev)
    torch.cuda.synchronize()
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    assert len(times) == 11 and all(t >= 0.0 for t in times)
    assert times[1] > 0.0  # the recomputing GEMM
    assert ev[0].elapsed_time(ev[-1]) == pytest.approx(sum(times), rel=1e-3, abs=1e-3)


@pytest.mark.slow
def test_recompute_full_size_sampled(gpu_lib):
    """The h=10240 shard (staged operands, 256 x 320 tiles): tile-complete
    samples of rows and columns (one in every 64-wide band) against the
    oracle."""
    import torch
    from tests.gpu_util import tile_complete_samples
    cfg = synth.get_config("gpt_h10240")
    print(f"case recompute full size T={cfg.tokens} h={cfg.hidden} f={cfg.ffn_shard}", flush=True)
    inp = synth.draw_config(cfg)
    X, A, b1, B, dY = device_inputs(inp)
    got = gpu_lib.bwd_recompute(dY, X, A, b1, B)
    torch.cuda.synchronize()
    rows = tile_complete_samples(cfg.tokens, 1)
    cols = tile_complete_samples(cfg.ffn_shard, 2)
    rr = oracle.sampled_rows(inp.X, inp.A, inp.b1, inp.B, inp.dY, rows)
    rc = oracle.sampled_cols(inp.X, inp.A, inp.b1, inp.B, inp.dY, cols)
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    tol = TOL[cfg.dtype]
    from tests.gpu_util import to_host
    assert oracle.rel_err(to_host(got["dZ"].index_select(0, ri)), rr["dZ"]) <= tol
    assert oracle.rel_err(to_host(got["dXp"].index_select(0, ri)), rr["dXp"]) <= tol
    assert oracle.rel_err(to_host(got["dA"].index_select(1, ci)), rc["dA"]) <= tol
    assert oracle.rel_err(to_host(got["dB"].index_select(0, ci)), rc["dB"]) <= tol
    assert oracle.rel_err(to_host(got["db1"].index_select(0, ci)), rc["db1"]) <= tol
