"""Full-size parity on sampled outputs, in the launch configuration that
bench.py times (automatic tile choice, H and dZ kept).

At full size the oracle evaluates the definitions only on sampled token rows
(Z, H, Yp, dZ, dXp of those tokens) and sampled FFN columns (Z, H, dZ over
all tokens, and from them dA, db1, dB of those columns); the samples include
the first and last rows/columns and every 128 / 256 tile boundary they hit.
The error bound is the same per-tensor max|err| / max|ref|, taken over the
sampled elements.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, device_inputs, run_shard, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _samples(n, n_random, seed):
    fixed = {0, 1, 127, 128, 255, 256, n // 2, n - 257, n - 256, n - 129, n - 128, n - 2, n - 1}
    rng = np.random.default_rng(seed)
    extra = set(rng.choice(n, size=min(n_random, n), replace=False).tolist())
    return np.array(sorted(i for i in fixed | extra if 0 <= i < n))


def _check(name, got, ref, tol, errs):
    e = oracle.rel_err(got, ref)
    errs[name] = e
    assert e <= tol, f"{name}: {e} > {tol}"


def _sampled_parity(inp, out, A, b1, B, tol, seed=0):
    T, f = inp.X.shape[0], A.shape[1]
    rows = _samples(T, 40, seed)
    cols = _samples(f, 16, seed + 1)
    rr = oracle.sampled_rows(inp.X, A, b1, B, inp.dY, rows)
    rc = oracle.sampled_cols(inp.X, A, b1, B, inp.dY, cols)
    import torch
    ri = torch.as_tensor(rows, device="cuda")
    ci = torch.as_tensor(cols, device="cuda")
    errs = {}
    for k in ("Z", "H", "Yp", "dZ", "dXp"):
        _check(f"{k}[rows]", to_host(out[k].index_select(0, ri)), rr[k], tol, errs)
    for k in ("Z", "H", "dZ", "dA"):
        _check(f"{k}[:,cols]", to_host(out[k].index_select(1, ci)), rc[k], tol, errs)
    _check("db1[cols]", to_host(out["db1"].index_select(0, ci)), rc["db1"], tol, errs)
    _check("dB[cols,:]", to_host(out["dB"].index_select(0, ci)), rc["dB"], tol, errs)
    for k, v in out.items():
        assert bool(torch.isfinite(v).all()), k
    return errs


@pytest.mark.parametrize("name", ["gpt_2p4b", "gpt_7b", "gpt_h10240"])
def test_full_size_shard_sampled(gpu_lib, name):
    cfg = synth.get_config(name)
    print(f"case full-size {name} T={cfg.tokens} h={cfg.hidden} f={cfg.ffn_shard} {cfg.dtype}", flush=True)
    inp = synth.draw_config(cfg)
    out = run_shard(gpu_lib, *device_inputs(inp))
    errs = _sampled_parity(inp, out, inp.A, inp.b1, inp.B, TOL[cfg.dtype])
    print("errors", errs, flush=True)


def test_four_shards_of_the_2p4b_mlp_sum_to_the_unsharded_result(gpu_lib):
    """All four TP shards of the 2.4B-shaped MLP (h=2560, F=10240), run one
    after the other on the one GPU, partials summed locally on the device;
    checked on sampled rows and columns against the unsharded oracle."""
    import torch
    cfg = synth.get_config("gpt_2p4b")
    T, h, F, P = cfg.tokens, cfg.hidden, cfg.ffn, cfg.tp
    print(f"case 4-shard emulation T={T} h={h} F={F}", flush=True)
    inp = synth.draw_inputs(T, h, F, cfg.dtype, seed=11, full=True, tp=P)
    outs = []
    for r in range(P):
        A_i, b1_i, B_i = oracle.shard_weights(inp.A, inp.b1, inp.B, P, r)
        o = run_shard(gpu_lib, *device_inputs(inp, A=A_i, b1=b1_i, B=B_i))
        outs.append({k: v for k, v in o.items()})
    Y = sum(o["Yp"].to(torch.float32) for o in outs)
    dX = sum(o["dXp"].to(torch.float32) for o in outs)
    rows = _samples(T, 40, 5)
    cols = _samples(F, 24, 6)
    fw = oracle.mlp_forward(inp.X[rows], inp.A, inp.b1, inp.B)
    bw = oracle.mlp_backward(inp.X[rows], inp.A, inp.b1, inp.B, inp.dY[rows])
    tol = TOL[cfg.dtype]
    ri = torch.as_tensor(rows, device="cuda")
    errs = {}
    _check("Y[rows]", to_host(Y.index_select(0, ri)), fw["Y"], tol, errs)
    _check("dX[rows]", to_host(dX.index_select(0, ri)), bw["dX"], tol, errs)
    rc = oracle.sampled_cols(inp.X, inp.A, inp.b1, inp.B, inp.dY, cols)
    f = F // P
    dA = np.stack([to_host(outs[c // f]["dA"][:, c % f]) for c in cols], axis=1)
    db1 = np.array([to_host(outs[c // f]["db1"][c % f]) for c in cols])
    dB = np.stack([to_host(outs[c // f]["dB"][c % f, :]) for c in cols], axis=0)
    _check("dA[:,cols]", dA, rc["dA"], tol, errs)
    _check("db1[cols]", db1, rc["db1"], tol, errs)
    _check("dB[cols,:]", dB, rc["dB"], tol, errs)
    print("errors", errs, flush=True)


def test_operands_beyond_the_direct_load_offset_range(gpu_lib):
    """X and dY of 131072 x 8192 bf16 (2 GiB each, more than 2^30 elements):
    the first GEMM and the dZ GEMM (512 tiles of 256 x 256 each) exceed the
    32-bit byte offsets of the direct-load engine and run on the
    register-staged 256 x 256 engine with 64-bit addressing; Yp and dXp still
    use direct loads, and the weight gradients (32 tiles each) the 128 x 128
    engine. Checked on sampled rows and columns."""
    T, h, f = 131072, 8192, 256
    print(f"case large operands T={T} h={h} f={f} bf16", flush=True)
    inp = synth.draw_inputs(T, h, f, "bf16", seed=21, sigma_dy=1.0)
    out = run_shard(gpu_lib, *device_inputs(inp))
    errs = _sampled_parity(inp, out, inp.A, inp.b1, inp.B, TOL["bf16"], seed=3)
    print("errors", errs, flush=True)
