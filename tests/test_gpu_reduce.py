"""Parity of tp_mlp_reduce_partials (sum over ranks of the row-parallel
partials, plus b2; all rows or one rank's slice of rows) against the float64
oracle, through the C ABI.

Partials are seeded N(0,1) values rounded to the storage dtype, the bias
N(0, 0.1^2). The bar is the per-tensor tolerance of the other outputs. The
kernel sums in fp32 and rounds once, so nearly every element must also equal
the correctly rounded exact sum bit for bit; a kernel that rounded after each
rank would miss that in a large fraction of elements.
"""
import numpy as np
import pytest

import oracle
from synth import round_to_storage
from tests.gpu_util import TOL, to_device, to_host, torch_dtype

pytestmark = pytest.mark.gpu


def _draw(rng, shape, sigma, dtype):
    return round_to_storage(rng.standard_normal(shape) * sigma, dtype)


def _run(gpu_lib, parts_d, bias_d, rb, re_, dtype, h):
    import torch
    out = torch.full((re_ - rb, h), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    gpu_lib.tp_mlp_reduce_partials(parts_d, bias_d, out, rb, re_)
    torch.cuda.synchronize()
    return out


def _check(got, ref, dtype):
    assert got.shape == ref.shape
    assert oracle.rel_err(got, ref) <= TOL[dtype]
    if got.size and dtype != "f32":
        miss = np.mean(got != round_to_storage(ref, dtype))
        assert miss <= 1e-3, f"{miss:.4f} of the elements differ from the rounded exact sum"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("P", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("T,h", [(8, 8), (200, 136), (520, 264)])
def test_reduce_partials_all_rows_and_slices(gpu_lib, dtype, P, T, h):
    print(f"case reduce dtype={dtype} P={P} T={T} h={h}", flush=True)
    rng = np.random.default_rng(1000 + 7 * P + T + h)
    parts = [_draw(rng, (T, h), 1.0, dtype) for _ in range(P)]
    bias = _draw(rng, (h,), 0.1, dtype)
    parts_d = [to_device(p, dtype) for p in parts]
    bias_d = to_device(bias, dtype)
    # the all-reduce (forward form, with b2, and backward form, without)
    full = to_host(_run(gpu_lib, parts_d, bias_d, 0, T, dtype, h))
    _check(full, oracle.reduce_partials(parts, bias), dtype)
    _check(to_host(_run(gpu_lib, parts_d, None, 0, T, dtype, h)), oracle.reduce_partials(parts), dtype)
    # the reduce-scatter: P slices of rows (the last one ragged when P does
    # not divide T), which stack to the all-reduce bit for bit
    cuts = [T * r // P for r in range(P + 1)]
    slices = []
    for r in range(P):
        got = to_host(_run(gpu_lib, parts_d, bias_d, cuts[r], cuts[r + 1], dtype, h))
        _check(got, oracle.reduce_partials(parts, bias, cuts[r], cuts[r + 1]), dtype)
        slices.append(got)
    assert np.array_equal(np.concatenate(slices, axis=0), full)


def test_reduce_partials_single_row_and_empty_range(gpu_lib):
    import torch
    rng = np.random.default_rng(7)
    T, h = 64, 128
    parts = [_draw(rng, (T, h), 1.0, "bf16") for _ in range(4)]
    parts_d = [to_device(p, "bf16") for p in parts]
    got = to_host(_run(gpu_lib, parts_d, None, 63, 64, "bf16", h))
    _check(got, oracle.reduce_partials(parts, None, 63, 64), "bf16")
    # an empty range writes nothing
    guard = torch.full((2, h), -7.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.tp_mlp_reduce_partials(parts_d, None, guard[:0], 5, 5)
    torch.cuda.synchronize()
    assert torch.all(guard == -7.0)


def test_reduce_partials_leaves_neighbouring_memory_untouched(gpu_lib):
    import torch
    rng = np.random.default_rng(9)
    T, h, G = 200, 136, 4096
    parts = [_draw(rng, (T, h), 1.0, "bf16") for _ in range(3)]
    parts_d = [to_device(p, "bf16") for p in parts]
    raw = torch.full(((120 - 40) * h + 2 * G,), -4096.0, dtype=torch.bfloat16, device="cuda")
    out = raw[G:G + (120 - 40) * h].view(120 - 40, h)
    gpu_lib.tp_mlp_reduce_partials(parts_d, None, out, 40, 120)
    torch.cuda.synchronize()
    assert torch.all(raw[:G] == -4096.0) and torch.all(raw[G + (120 - 40) * h:] == -4096.0)
    _check(to_host(out), oracle.reduce_partials(parts, None, 40, 120), "bf16")


def test_reduce_partials_of_four_shards_give_the_unsharded_mlp(gpu_lib):
    """Four TP shards of a small bf16 MLP run one after the other; the
    library's own reduction of their Yp (+ b2) and dXp matches the unsharded
    oracle, and its reduce-scatter slices stack to the same result."""
    import synth
    from tests.gpu_util import device_inputs, run_shard
    T, h, F, P = 256, 128, 1024, 4
    inp = synth.draw_inputs(T, h, F, "bf16", seed=13, sigma_dy=1.0, full=True, tp=P)
    rng = np.random.default_rng(14)
    b2 = _draw(rng, (h,), 0.1, "bf16")
    outs = []
    for r in range(P):
        A_i, b1_i, B_i = oracle.shard_weights(inp.A, inp.b1, inp.B, P, r)
        outs.append(run_shard(gpu_lib, *device_inputs(inp, A=A_i, b1=b1_i, B=B_i)))
    b2_d = to_device(b2, "bf16")
    Y = to_host(_run(gpu_lib, [o["Yp"] for o in outs], b2_d, 0, T, "bf16", h))
    dX = to_host(_run(gpu_lib, [o["dXp"] for o in outs], None, 0, T, "bf16", h))
    fw = oracle.mlp_forward(inp.X, inp.A, inp.b1, inp.B, b2)
    bw = oracle.mlp_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    assert oracle.rel_err(Y, fw["Y"]) <= TOL["bf16"]
    assert oracle.rel_err(dX, bw["dX"]) <= TOL["bf16"]
    rows = T // P
    ys = [to_host(_run(gpu_lib, [o["Yp"] for o in outs], b2_d, r * rows, (r + 1) * rows, "bf16", h))
          for r in range(P)]
    assert np.array_equal(np.concatenate(ys, axis=0), Y)
