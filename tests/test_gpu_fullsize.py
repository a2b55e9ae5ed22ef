"""Full-size parity in the launch configuration that bench.py times
(automatic tile choice, staged workspaces, H and dZ kept).

The 2.4B, 7B and h=10240 shards are compared element by element: every
element of Z, H, Yp, dZ, dXp, dA, dB and db1 against the float64 oracle run
on the whole shard (about 0.6, 1.6 and 21 TFLOP of float64 work), so every
output tile of every GEMM is checked, in the launches' full-wave work-item
order. The four TP shards of the 2.4B MLP are checked the same way against
the unsharded MLP. The error bound is the per-tensor max|err| / max|ref|.

One case has operands too large for a full float64 oracle on the host (2 GiB
X and dY); it is checked on tile-complete samples: at least one token row
in every 64-row band and one column in every 64-column band (so in every
output tile of every tile size the planner uses), plus the first and last
rows and columns.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, device_inputs, run_shard, tile_complete_samples, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(*a):
    print(*a, flush=True)


def _check(name, got, ref, tol, errs):
    e = oracle.rel_err(got, ref)
    errs[name] = e
    assert e <= tol, f"{name}: {e} > {tol}"


def _full_parity(inp, out, tol):
    """Every element of every output against the float64 oracle of the shard."""
    errs = {}
    _log("oracle forward ...")
    fw = oracle.shard_forward(inp.X, inp.A, inp.b1, inp.B)
    for k in ("Z", "H", "Yp"):
        _check(k, to_host(out[k]), fw[k], tol, errs)
    _log("oracle backward ...")
    bw = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY, Z_i=fw["Z"])
    del fw
    for k in ("dZ", "dXp", "dA", "dB", "db1"):
        _check(k, to_host(out[k]), bw[k], tol, errs)
    return errs


@pytest.mark.parametrize("name", ["gpt_2p4b", "gpt_7b", "gpt_h10240"])
def test_full_size_shard_every_element(gpu_lib, name):
    cfg = synth.get_config(name)
    _log(f"case full-size {name} T={cfg.tokens} h={cfg.hidden} f={cfg.ffn_shard} {cfg.dtype}")
    inp = synth.draw_config(cfg)
    out = run_shard(gpu_lib, *device_inputs(inp))
    out = {k: v for k, v in out.items()}
    errs = _full_parity(inp, out, TOL[cfg.dtype])
    _log("errors", errs)


def test_four_shards_of_the_2p4b_mlp_sum_to_the_unsharded_result(gpu_lib):
    """All four TP shards of the 2.4B-shaped MLP (h=2560, F=10240), run one
    after the other on the one GPU, partials summed locally on the device;
    every element checked against the unsharded oracle: Y and dX from the
    summed partials, Z, H, dZ, dA and db1 from the shards' column blocks
    side by side, dB from their row blocks stacked ("Understanding the
    Megatron-LM architecture: how 3D parallelism assigns roles", section 1,
    the column-split and row-split items)."""
    import torch
    cfg = synth.get_config("gpt_2p4b")
    T, h, F, P = cfg.tokens, cfg.hidden, cfg.ffn, cfg.tp
    _log(f"case 4-shard emulation T={T} h={h} F={F}")
    inp = synth.draw_inputs(T, h, F, cfg.dtype, seed=11, full=True, tp=P)
    outs = []
    for r in range(P):
        A_i, b1_i, B_i = oracle.shard_weights(inp.A, inp.b1, inp.B, P, r)
        outs.append(run_shard(gpu_lib, *device_inputs(inp, A=A_i, b1=b1_i, B=B_i)))
    Y = sum(o["Yp"].to(torch.float32) for o in outs)
    dX = sum(o["dXp"].to(torch.float32) for o in outs)
    tol = TOL[cfg.dtype]
    errs = {}
    _log("oracle forward (unsharded) ...")
    fw = oracle.mlp_forward(inp.X, inp.A, inp.b1, inp.B)
    _check("Y", to_host(Y), fw["Y"], tol, errs)
    for k in ("Z", "H"):
        _check(k, np.concatenate([to_host(o[k]) for o in outs], axis=1), fw[k], tol, errs)
    _log("oracle backward (unsharded) ...")
    bw = oracle.mlp_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY, Z=fw["Z"])
    del fw
    _check("dX", to_host(dX), bw["dX"], tol, errs)
    for k in ("dZ", "dA"):
        _check(k, np.concatenate([to_host(o[k]) for o in outs], axis=1), bw[k], tol, errs)
    _check("db1", np.concatenate([to_host(o["db1"]) for o in outs]), bw["db1"], tol, errs)
    _check("dB", np.concatenate([to_host(o["dB"]) for o in outs], axis=0), bw["dB"], tol, errs)
    _log("errors", errs)


def test_operands_beyond_the_direct_load_offset_range(gpu_lib):
    """X and dY of 131072 x 8192 bf16 (2 GiB each, more than 2^30 elements):
    the first GEMM and the dZ GEMM (512 tiles of 256 x 256 each) exceed the
    32-bit byte offsets of the direct-load engine and run on the
    register-staged 256 x 256 engine with 64-bit addressing; Yp and dXp still
    use direct loads, and the weight gradients (32 tiles each) the 128 x 128
    engine. Checked on tile-complete samples of token rows and on every one
    of the f = 256 FFN columns."""
    import torch
    T, h, f = 131072, 8192, 256
    _log(f"case large operands T={T} h={h} f={f} bf16")
    inp = synth.draw_inputs(T, h, f, "bf16", seed=21, sigma_dy=1.0)
    out = run_shard(gpu_lib, *device_inputs(inp))
    rows = tile_complete_samples(T, 3)
    cols = np.arange(f)
    tol = TOL["bf16"]
    errs = {}
    _log(f"oracle on {len(rows)} rows and {len(cols)} of {f} columns ...")
    rr = oracle.sampled_rows(inp.X, inp.A, inp.b1, inp.B, inp.dY, rows)
    rc = oracle.sampled_cols(inp.X, inp.A, inp.b1, inp.B, inp.dY, cols)
    ri = torch.as_tensor(rows, device="cuda")
    ci = torch.as_tensor(cols, device="cuda")
    for k in ("Z", "H", "Yp", "dZ", "dXp"):
        _check(f"{k}[rows]", to_host(out[k].index_select(0, ri)), rr[k], tol, errs)
    for k in ("Z", "H", "dZ", "dA"):
        _check(f"{k}[:,cols]", to_host(out[k].index_select(1, ci)), rc[k], tol, errs)
    _check("db1[cols]", to_host(out["db1"].index_select(0, ci)), rc["db1"], tol, errs)
    _check("dB[cols,:]", to_host(out["dB"].index_select(0, ci)), rc["dB"], tol, errs)
    _log("errors", errs)
