"""Parity of the HIP path against the float64 oracle, element by element.

Tolerances are the per-tensor bounds max|gpu - ref| / max|ref| <= 1e-4
(fp32), 5e-3 (fp16), 2e-2 (bf16). Every call goes through the C ABI
(tp_mlp_fwd / tp_mlp_bwd); the oracle sees the same seeded, storage-rounded
inputs.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, device_inputs, run_shard, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture
def tile(request, gpu_lib):
    """Force one 16-bit tile engine through tp_mlp_debug_plan (None = the
    planner's choice); the default plan is restored afterwards."""
    value = getattr(request, "param", None)
    gpu_lib.tp_mlp_debug_plan(value, 0)
    yield value
    gpu_lib.tp_mlp_debug_plan(None, 0)


def _oracle_shard(inp):
    fw = oracle.shard_forward(inp.X, inp.A, inp.b1, inp.B)
    bw = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    return {**fw, **bw}


# ------------------------------------------------------------ small ----

RAGGED = [
    (8, 8, 8),          # one partial tile everywhere
    (200, 136, 264),    # several tiles, ragged M / N / K tails
    (520, 264, 392),
    (128, 128, 128),    # exactly one tile
    (264, 64, 328),     # K shorter than one 64-wide step
]


@pytest.mark.parametrize("tile", [128, 256, "dma256", "dma320", "dma320m32"], indirect=True)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f", RAGGED)
def test_ragged_shapes_16bit(gpu_lib, tile, dtype, T, h, f):
    print(f"case ragged dtype={dtype} tile={tile} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + h + f, sigma_dy=1.0)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp))
    compare(got, ref, TOL[dtype])


@pytest.mark.parametrize("tile", ["dma256"], indirect=True)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f", [(200, 136, 264), (520, 264, 392), (4352, 5440, 5440)])
def test_operands_read_in_place(gpu_lib, tile, dtype, T, h, f):
    """Minimal workspaces: the large-tile engine reads the mn-contiguous
    operands in place (transposing LDS reads) instead of staged copies. The
    last shape has more than one wave of 256 x 256 tiles, where those
    launches run on the 16x16x32 MFMA form."""
    print(f"case in-place dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + 3 * f, sigma_dy=1.0)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp), staged=False)
    compare(got, ref, TOL[dtype])


@pytest.mark.parametrize("tile", ["dma256", "dma320", "dma320m32"], indirect=True)
@pytest.mark.parametrize("cus", [3, 4, 5])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f", [(520, 264, 392), (1000, 264, 392)])
def test_k_split_last_wave(gpu_lib, tile, cus, dtype, T, h, f):
    """Tail tiles computed as k-ranges plus an ordered fp32 sum, planned as
    if the chip had `cus` CUs so that small shapes split (3 CUs: dB and dA
    split their one leftover tile into 3 ranges; 4 and 5: Yp and dXp split
    ragged K = 392 into 2 or 3)."""
    gpu_lib.tp_mlp_debug_plan(tile, cus)
    print(f"case k-split cus={cus} dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + cus, sigma_dy=1.0)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp))
    compare(got, ref, TOL[dtype])
    again = run_shard(gpu_lib, *device_inputs(inp))
    import torch
    for k in got:
        assert torch.equal(got[k].view(torch.int16), again[k].view(torch.int16)), k


@pytest.mark.parametrize("T,h,f", [(4, 4, 4), (200, 132, 268), (64, 128, 256)])
def test_ragged_shapes_fp32(gpu_lib, T, h, f):
    print(f"case ragged dtype=f32 T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, "f32", seed=7, sigma_dy=1.0)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp))
    compare(got, ref, TOL["f32"])


@pytest.mark.parametrize("tile", [128, 256, "dma256", "dma320"], indirect=True)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_without_h_and_dz_buffers(gpu_lib, tile, dtype):
    """H not kept (GeLU applied to Z on load) and dZ kept in the workspace."""
    T, h, f = 264, 200, 328
    print(f"case no-H/no-dZ dtype={dtype} tile={tile}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=5, sigma_dy=1.0)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp), keep_h=False, keep_dz=False)
    assert got["dZ"] is None and "H" not in got
    compare(got, ref, TOL[dtype])


def test_tiny_fp32_two_shards_sum_to_the_full_mlp(gpu_lib):
    """Both TP=2 shards of the fp32 workload, run one after the other on the
    one GPU; partials summed locally and columns concatenated must match
    the unsharded MLP ("Understanding the Megatron-LM architecture: how 3D
    parallelism assigns roles", section 1)."""
    import torch
    cfg = synth.get_config("tiny")
    inp = synth.draw_config(cfg)
    full_f = oracle.mlp_forward(inp.X, inp.A, inp.b1, inp.B)
    full_b = oracle.mlp_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
    outs = []
    for r in range(cfg.tp):
        A_i, b1_i, B_i = oracle.shard_weights(inp.A, inp.b1, inp.B, cfg.tp, r)
        outs.append(run_shard(gpu_lib, *device_inputs(inp, A=A_i, b1=b1_i, B=B_i)))
    got = {
        "Y": to_host(sum(o["Yp"].to(torch.float32) for o in outs)),
        "dX": to_host(sum(o["dXp"].to(torch.float32) for o in outs)),
        "Z": np.concatenate([to_host(o["Z"]) for o in outs], axis=1),
        "H": np.concatenate([to_host(o["H"]) for o in outs], axis=1),
        "dZ": np.concatenate([to_host(o["dZ"]) for o in outs], axis=1),
        "dA": np.concatenate([to_host(o["dA"]) for o in outs], axis=1),
        "db1": np.concatenate([to_host(o["db1"]) for o in outs]),
        "dB": np.concatenate([to_host(o["dB"]) for o in outs], axis=0),
    }
    ref = {"Y": full_f["Y"], "Z": full_f["Z"], "H": full_f["H"], "dX": full_b["dX"], "dZ": full_b["dZ"],
           "dA": full_b["dA"], "db1": full_b["db1"], "dB": full_b["dB"]}
    compare(got, ref, TOL["f32"])
    # one shard alone is not the answer
    assert oracle.rel_err(to_host(outs[0]["Yp"]), full_f["Y"]) > 0.1


def test_gpt2_small_fp16_against_full_oracle(gpu_lib):
    cfg = synth.get_config("gpt2_small")
    print("case gpt2_small fp16 full", flush=True)
    inp = synth.draw_config(cfg)
    ref = _oracle_shard(inp)
    got = run_shard(gpu_lib, *device_inputs(inp))
    errs = compare(got, ref, TOL["f16"])
    print("errors", errs, flush=True)
    # adjoint invariants on the GPU outputs (fp64 on the host)
    ip = lambda u, v: float(np.sum(u * v))
    g = {k: to_host(v) for k, v in got.items()}
    assert ip(g["dB"], inp.B) == pytest.approx(ip(inp.dY, g["Yp"]), rel=2e-2)
    assert ip(g["dA"], inp.A) == pytest.approx(ip(g["dXp"], inp.X), rel=2e-2)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_empty_dimensions(gpu_lib, dtype):
    """T = 0: dA, dB, db1 are sums over no tokens (zeros); f = 0: Yp and dXp
    are products over an empty dimension (zeros); h = 0: Z = b1."""
    import torch
    from tests.gpu_util import torch_dtype
    td = torch_dtype(dtype)
    nan = float("nan")
    # T = 0
    inp = synth.draw_inputs(0, 16, 24, dtype, seed=1)
    X, A, b1, B, dY = device_inputs(inp)
    Z, H, Yp = gpu_lib.fwd(X, A, b1, B)
    dZ = torch.empty((0, 24), dtype=td, device="cuda")
    dXp = torch.empty((0, 16), dtype=td, device="cuda")
    dA = torch.full((16, 24), nan, dtype=td, device="cuda")
    dB = torch.full((24, 16), nan, dtype=td, device="cuda")
    db1 = torch.full((24,), nan, dtype=td, device="cuda")
    gpu_lib.tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, None)
    torch.cuda.synchronize()
    for t in (dA, dB, db1):
        assert torch.all(t == 0)
    # f = 0
    inp = synth.draw_inputs(16, 16, 0, dtype, seed=2)
    X, A, b1, B, dY = device_inputs(inp)
    Yp = torch.full((16, 16), nan, dtype=td, device="cuda")
    Z = torch.empty((16, 0), dtype=td, device="cuda")
    gpu_lib.tp_mlp_fwd(X, A, b1, B, Z, None, Yp)
    dXp = torch.full((16, 16), nan, dtype=td, device="cuda")
    e = lambda *s: torch.empty(s, dtype=td, device="cuda")
    gpu_lib.tp_mlp_bwd(dY, X, A, B, Z, None, e(16, 0), dXp, e(16, 0), e(0, 16), e(0), None)
    torch.cuda.synchronize()
    assert torch.all(Yp == 0) and torch.all(dXp == 0)
    # h = 0
    inp = synth.draw_inputs(16, 0, 24, dtype, seed=3)
    X, A, b1, B, dY = device_inputs(inp)
    got = run_shard(gpu_lib, X, A, b1, B, dY)
    assert np.array_equal(to_host(got["Z"]), np.broadcast_to(inp.b1, (16, 24)))
    assert torch.all(got["dZ"] == 0) and torch.all(got["db1"] == 0)


def test_deterministic_bitwise(gpu_lib):
    import torch
    inp = synth.draw_inputs(520, 264, 392, "bf16", seed=9, sigma_dy=1.0)
    a = run_shard(gpu_lib, *device_inputs(inp))
    b = run_shard(gpu_lib, *device_inputs(inp))
    for k in a:
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16)), k


# A shape whose every GEMM has more than one full wave of work items (256
# CUs): 17 x 17 tiles of 256 x 320 (or 17 x 22 of 256 x 256) for the token
# GEMMs, 22 x 17 for the weight gradients, with a partial last wave that
# the planner splits into k-ranges. It runs the XCD renumbering of full
# waves (map_work) as well as the plain order of the last wave.
FULL_WAVE = (4352, 5440, 5440)
# f = h with few tiles and a long reduction: dB and dA run as one paired
# launch (16 + 16 or 25 + 25 tiles of 256 x 256), unsplit
PAIRED, PAIRED_RAGGED = (2048, 1024, 1024), (2056, 1032, 1032)


@pytest.mark.parametrize("tile,cus,shape", [(128, None, None), (256, None, None), ("dma256", None, None),
                                            ("dma256", 4, None), ("dma320", None, None), ("dma320", 2, None),
                                            (None, None, FULL_WAVE), ("dma256", None, FULL_WAVE),
                                            ("dma320", None, FULL_WAVE), ("dma320m32", None, FULL_WAVE),
                                            ("dma320m32", 2, None), (None, None, PAIRED),
                                            (None, None, PAIRED_RAGGED), ("dma256", None, PAIRED)],
                         indirect=["tile"])
def test_outputs_leave_neighbouring_memory_untouched(gpu_lib, tile, cus, shape):
    """Each output lives between two poisoned guard regions, which must
    survive forward + backward unchanged, and every element of every output
    must be overwritten (the poison value may not remain) and match the
    oracle (cus: k-split tails planned as if the chip had that many CUs, so
    that the partials use the workspace; FULL_WAVE: launches of more than
    one full wave of work items; PAIRED: dB and dA from one launch)."""
    import torch
    if cus is not None:
        gpu_lib.tp_mlp_debug_plan(tile, cus)
    T, h, f = shape if shape else (520, 264, 392) if cus else (200, 136, 264)
    print(f"case guard bands tile={tile} cus={cus} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, "bf16", seed=4, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    G = 4096  # guard elements on each side (keeps 16-byte alignment)
    bufs = {}

    def guarded(*shape):
        n = int(np.prod(shape))
        raw = torch.full((n + 2 * G,), -4096.0, dtype=torch.bfloat16, device="cuda")
        bufs[len(bufs)] = (raw, n)
        return raw[G:G + n].view(*shape)

    Z, H, Yp = guarded(T, f), guarded(T, f), guarded(T, h)
    nfws = gpu_lib.tp_mlp_fwd_workspace_bytes(T, h, f, gpu_lib.TPMLP_BF16)
    fws_raw = torch.full((nfws + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
    gpu_lib.tp_mlp_fwd(X, A, b1, B, Z, H, Yp, fws_raw[G:G + nfws] if nfws else None)
    dZ, dXp, dA, dB, db1 = guarded(T, f), guarded(T, h), guarded(h, f), guarded(f, h), guarded(f)
    nws = gpu_lib.tp_mlp_workspace_bytes(T, h, f, gpu_lib.TPMLP_BF16)
    ws_raw = torch.full((nws + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = ws_raw[G:G + nws]
    gpu_lib.tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, ws)
    torch.cuda.synchronize()
    for raw, n in bufs.values():
        assert torch.all(raw[:G] == -4096.0) and torch.all(raw[G + n:] == -4096.0)
        assert not torch.any(raw[G:G + n] == -4096.0)
    assert torch.all(ws_raw[:G] == 0x5A) and torch.all(ws_raw[G + nws:] == 0x5A)
    assert torch.all(fws_raw[:G] == 0x5A) and torch.all(fws_raw[G + nfws:] == 0x5A)
    ref = _oracle_shard(inp)
    compare({"Z": Z, "H": H, "Yp": Yp, "dZ": dZ, "dXp": dXp, "dA": dA, "dB": dB, "db1": db1}, ref, TOL["bf16"])


def test_events_bracket_each_step(gpu_lib):
    import torch
    inp = synth.draw_inputs(512, 256, 512, "f16", seed=6)
    X, A, b1, B, dY = device_inputs(inp)
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    be = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
    Z, H, Yp = gpu_lib.fwd(X, A, b1, B, events=fe)
    gpu_lib.bwd(dY, X, A, B, Z, H, events=be)
    torch.cuda.synchronize()
    for ev in (fe, be):
        for a, b in zip(ev[:-1], ev[1:]):
            assert a.elapsed_time(b) >= 0.0


def test_null_event_entries_are_skipped(gpu_lib):
    """Only the non-NULL entries are recorded: here B1's two boundaries and
    F1's, the way bench.py brackets one GEMM per step."""
    import torch
    inp = synth.draw_inputs(512, 256, 512, "bf16", seed=7)
    X, A, b1, B, dY = device_inputs(inp)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    fe, be = [None, mk(), mk(), None, None], [mk(), mk()] + [None] * 8
    Z, H, Yp = gpu_lib.fwd(X, A, b1, B, events=fe)
    got = gpu_lib.bwd(dY, X, A, B, Z, H, events=be)
    torch.cuda.synchronize()
    assert fe[1].elapsed_time(fe[2]) > 0.0 and be[0].elapsed_time(be[1]) > 0.0
    compare({"Z": Z, "H": H, "Yp": Yp, **got}, _oracle_shard(inp), TOL["bf16"])


# ----------------------------------------------- GeLU epilogue grids ----

def _grid_inputs(dtype, n):
    """X[:, 0] = grid, A[0, :] = 1 and B[:, 0] = 1, dY[:, 0] = 1 (zeros elsewhere):
    Z = grid + b1 exactly in fp32, and dH = dY B^T = 1, so dZ = gelu'(Z)."""
    from synth import Inputs, round_to_storage
    T, h, f = n, 8, 8
    grid = round_to_storage(np.linspace(-8.0, 8.0, T), dtype)
    X = np.zeros((T, h)); X[:, 0] = grid
    A = np.zeros((h, f)); A[0, :] = 1.0
    b1 = round_to_storage(np.linspace(-0.03, 0.05, f), dtype)
    B = np.zeros((f, h)); B[:, 0] = 1.0
    dY = np.zeros((T, h)); dY[:, 0] = 1.0
    return Inputs(dtype, X, A, b1, B, dY)


def test_gelu_epilogues_fp32_grid(gpu_lib):
    """fp32 storage: GeLU and gelu' of the epilogues within 1e-5 (abs) of the
    float64 formulas on a grid over [-8, 8]."""
    inp = _grid_inputs("f32", 4004)
    got = run_shard(gpu_lib, *device_inputs(inp))
    z = inp.X[:, :1] + inp.b1[None, :]
    assert np.array_equal(to_host(got["Z"]), z.astype(np.float32).astype(np.float64))
    assert np.max(np.abs(to_host(got["H"]) - oracle.gelu(to_host(got["Z"])))) <= 1e-5
    assert np.max(np.abs(to_host(got["dZ"]) - oracle.gelu_grad(to_host(got["Z"])))) <= 1e-5


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_epilogue_rounding_is_nearest_even(gpu_lib, dtype):
    """Z = grid + b1 is exact in fp32, so its 16-bit store must equal the
    correctly rounded value bit for bit. H = gelu(z) from the fp32 sum and
    dZ = gelu'(stored Z), both computed in fp32, must be within one 16-bit
    ulp of the exact float64 value, plus the fp32 evaluation's own error,
    and equal to the correctly rounded value almost everywhere on z >= -3."""
    from synth import round_to_storage
    inp = _grid_inputs(dtype, 4000)
    got = run_shard(gpu_lib, *device_inputs(inp))
    z = inp.X[:, :1] + inp.b1[None, :]
    zs = round_to_storage(z, dtype)  # the backward reads the stored Z
    assert np.array_equal(to_host(got["Z"]), zs)
    for name, exact in (("H", oracle.gelu(z)), ("dZ", oracle.gelu_grad(zs))):
        g = to_host(got[name])
        r = round_to_storage(exact, dtype)
        ulp = np.abs(np.nextafter(r.astype(np.float32), np.float32(np.inf)).astype(np.float64) - r)
        ulp16 = ulp * (2 ** (23 - (10 if dtype == "f16" else 7)))
        # fp32 evaluation error: a few ulp of each term; the gelu' term
        # 1 - tanh^2 is scaled by |x| sqrt(2/pi) (1 + 3c x^2)
        floor = 1e-6 if name == "H" else 2.0 ** -22 * (1 + np.abs(z) * 0.8 * (1 + 0.134 * z * z))
        bad = np.abs(g - exact) > ulp16 + floor
        assert not bad.any(), (name, list(zip(z[bad][:5], g[bad][:5], exact[bad][:5])))
        well = z >= -3.0
        assert np.mean(g[well] == r[well]) > 0.99, name


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f,keep_dz", [(2048, 1024, 1040, True), (2056, 1032, 1048, False)])
def test_sub_wave_k_split(gpu_lib, dtype, T, h, f, keep_dz):
    """Weight gradients with few output tiles and a long reduction (T >= 2048
    tokens): 20-25 tiles of 256 x 256, every tile split into 4 k-ranges
    whose fp32 partials are summed in a fixed order (the ragged case ends in
    a short last range). f != h, so dB and dA are not paired. Against the
    oracle, and bitwise run to run."""
    import torch
    print(f"case sub-wave k-split dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + f, sigma_dy=1.0)
    dev = device_inputs(inp)
    out = run_shard(gpu_lib, *dev, keep_dz=keep_dz)
    compare(out, _oracle_shard(inp), TOL[dtype])
    again = run_shard(gpu_lib, *dev, keep_dz=keep_dz)
    for k in ("dA", "dB", "dXp", "db1"):
        assert torch.equal(out[k], again[k]), k


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,h,f,keep_dz", [PAIRED + (True,), PAIRED_RAGGED + (False,)])
@pytest.mark.parametrize("tile", [None, "dma256"], indirect=True)
def test_paired_weight_gradients(gpu_lib, tile, dtype, T, h, f, keep_dz):
    """f = h, few output tiles, a long reduction: dB = H^T dY and dA = X^T dZ
    run as one launch of 2 x 16 (or 2 x 25, ragged) tiles of 256 x 256, each
    tile over the whole reduction. Against the oracle, bitwise run to run,
    and with H not kept (gelu(Z) applied on load: not paired) against the
    same oracle."""
    import torch
    print(f"case paired dB/dA tile={tile} dtype={dtype} T={T} h={h} f={f}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + 3 * f, sigma_dy=1.0)
    dev = device_inputs(inp)
    ref = _oracle_shard(inp)
    out = run_shard(gpu_lib, *dev, keep_dz=keep_dz)
    compare(out, ref, TOL[dtype])
    again = run_shard(gpu_lib, *dev, keep_dz=keep_dz)
    for k in ("dA", "dB", "dXp", "db1"):
        assert torch.equal(out[k], again[k]), k
    compare(run_shard(gpu_lib, *dev, keep_h=False, keep_dz=keep_dz), ref, TOL[dtype])
