"""Parity of the transposed-B layout (TPMLP_LAYOUT_B_T: the second weight
passed as B_i^T [hidden, ffn_shard], its gradient returned in that order)
against the float64 oracle, through the C ABI, on every tile engine, with
and without H kept, staged and minimal workspaces, the fp32 main-gradient
and the recomputing backward. Z and H do not depend on B and must equal the
default layout's bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, device_inputs, to_host

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


def _ref(inp):
    ref = {**oracle.shard_forward(inp.X, inp.A, inp.b1, inp.B),
           **oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)}
    ref["dB"] = ref["dB"].T.copy()   # returned as [h, f] in this layout
    return ref


@pytest.mark.parametrize("tile,dtype", CASES, indirect=["tile"])
@pytest.mark.parametrize("T,h,f", [(200, 136, 264), (520, 264, 392)])
@pytest.mark.parametrize("keep_h,staged", [(True, True), (False, True), (True, False), (False, False)])
def test_b_transposed_matches_oracle(gpu_lib, tile, dtype, T, h, f, keep_h, staged):
    import torch
    print(f"case layout_b_t tile={tile} dtype={dtype} T={T} h={h} f={f} keep_h={keep_h} staged={staged}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=3 * T + f, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    Bt = B.t().contiguous()
    Z, H, Yp = gpu_lib.fwd(X, A, b1, Bt, keep_h=keep_h, staged=staged, b_transposed=True)
    g = gpu_lib.bwd(dY, X, A, Bt, Z, H, staged=staged, b_transposed=True)
    torch.cuda.synchronize()
    assert tuple(g["dB"].shape) == (h, f)
    got = {"Z": Z, "Yp": Yp, **g}
    if H is not None:
        got["H"] = H
    compare(got, _ref(inp), TOL[dtype])
    Z0, H0, _ = gpu_lib.fwd(X, A, b1, B, keep_h=keep_h, staged=staged)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z0)
    if keep_h:
        assert torch.equal(H, H0)


@pytest.mark.parametrize("tile", [None, 128, "dma256", "dma320"], indirect=True)
@pytest.mark.parametrize("staged", [True, False])
def test_b_transposed_main_grad_accumulates(gpu_lib, tile, staged):
    """Two micro-batches add twice into the fp32 main gradients, dB_main in
    [h, f] order; each addition matches the oracle's weight gradients."""
    import torch
    T, h, f, dtype = 520, 264, 392, "bf16"
    inp = synth.draw_inputs(T, h, f, dtype, seed=77, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    Bt = B.t().contiguous()
    rng = np.random.default_rng(5)
    start = {"dA": rng.standard_normal((h, f)) * 1e-2, "dB": rng.standard_normal((h, f)) * 1e-2,
             "db1": rng.standard_normal((f,)) * 1e-2}
    mains = {k: torch.as_tensor(v, dtype=torch.float32, device="cuda") for k, v in start.items()}
    ref = _ref(inp)
    code = gpu_lib.TPMLP_BF16
    flags = 0 if staged else gpu_lib.TPMLP_WS_MINIMAL
    nws = gpu_lib.tp_mlp_workspace_bytes(T, h, f, code, flags, gpu_lib.TPMLP_LAYOUT_B_T)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device="cuda")
    old = {k: v.copy() for k, v in start.items()}
    for step in range(2):
        Z, H, _ = gpu_lib.fwd(X, A, b1, Bt, staged=staged, b_transposed=True)
        dZ = torch.empty((T, f), dtype=X.dtype, device="cuda")
        dXp = torch.empty((T, h), dtype=X.dtype, device="cuda")
        gpu_lib.tp_mlp_bwd_main_grad(dY, X, A, Bt, Z, H, dZ, dXp, mains["dA"], mains["dB"], mains["db1"], ws,
                                     b_transposed=True)
        torch.cuda.synchronize()
        new = {k: to_host(v) for k, v in mains.items()}
        for k in ("dA", "dB", "db1"):
            err = float(np.max(np.abs(new[k] - old[k] - ref[k])) / np.max(np.abs(ref[k])))
            assert err <= TOL[dtype], (step, k, err)
        old = new


@pytest.mark.parametrize("tile,dtype", [(None, "f32"), (None, "bf16"), (128, "f16"), ("dma256", "bf16"),
                                        ("dma320", "f16")], indirect=["tile"])
@pytest.mark.parametrize("staged", [True, False])
def test_b_transposed_recompute(gpu_lib, tile, dtype, staged):
    """The recomputing backward in this layout equals the plain backward
    (H = NULL) in this layout bit for bit, and the oracle to tolerance."""
    import torch
    T, h, f = 520, 264, 392
    inp = synth.draw_inputs(T, h, f, dtype, seed=91, sigma_dy=1.0)
    X, A, b1, B, dY = device_inputs(inp)
    Bt = B.t().contiguous()
    got = gpu_lib.bwd_recompute(dY, X, A, b1, Bt, staged=staged, b_transposed=True)
    torch.cuda.synchronize()
    compare(got, _ref(inp), TOL[dtype], keys=GRADS)
    Z, _, _ = gpu_lib.fwd(X, A, b1, Bt, keep_h=False, staged=staged, b_transposed=True)
    plain = gpu_lib.bwd(dY, X, A, Bt, Z, None, staged=staged, b_transposed=True)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(got[k], plain[k]), k


@pytest.mark.slow
def test_b_transposed_full_size_h10240_sampled(gpu_lib):
    """The h=10240 TP=4 shard (bf16) in this layout, in bench.py's launch
    configuration (staged workspaces, H and dZ kept), on tile-complete
    samples of rows and columns (one in every 64-wide band, so in every
    output tile) against the oracle's restricted definitions."""
    import torch
    from tests.gpu_util import tile_complete_samples

    def _check(name, got, ref, tol, errs):
        errs[name] = oracle.rel_err(got, ref)
        assert errs[name] <= tol, f"{name}: {errs[name]} > {tol}"
    cfg = synth.get_config("gpt_h10240")
    print(f"case full-size layout_b_t {cfg.name}", flush=True)
    inp = synth.draw_config(cfg)
    X, A, b1, B, dY = device_inputs(inp)
    Bt = B.t().contiguous()
    del B
    Z, H, Yp = gpu_lib.fwd(X, A, b1, Bt, b_transposed=True)
    g = gpu_lib.bwd(dY, X, A, Bt, Z, H, b_transposed=True)
    torch.cuda.synchronize()
    out = {"Z": Z, "H": H, "Yp": Yp, **g}
    T, f = cfg.tokens, cfg.ffn_shard
    rows, cols = tile_complete_samples(T, 0), tile_complete_samples(f, 1)
    rr = oracle.sampled_rows(inp.X, inp.A, inp.b1, inp.B, inp.dY, rows)
    rc = oracle.sampled_cols(inp.X, inp.A, inp.b1, inp.B, inp.dY, cols)
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    tol, errs = TOL[cfg.dtype], {}
    for k in ("Z", "H", "Yp", "dZ", "dXp"):
        _check(f"{k}[rows]", to_host(out[k].index_select(0, ri)), rr[k], tol, errs)
    for k in ("Z", "H", "dZ", "dA"):
        _check(f"{k}[:,cols]", to_host(out[k].index_select(1, ci)), rc[k], tol, errs)
    _check("db1[cols]", to_host(out["db1"].index_select(0, ci)), rc["db1"], tol, errs)
    _check("dB^T[:,cols]", to_host(out["dB"].index_select(1, ci)).T, rc["dB"], tol, errs)
    print("errors", errs, flush=True)


@pytest.mark.parametrize("dtype,T,h,f,b_transposed,b_staged", [
    ("bf16", 8192, 2560, 2560, False, True),    # 2.4B shard: A_i^T and B_i^T copied
    ("bf16", 8192, 2560, 2560, True, False),    # B_i^T passed: only A_i^T copied
    ("f16", 4096, 768, 3072, False, False),     # GPT-2-small: A_i^T copied, the second GEMM reads B_i in place
])
def test_weights_staged_reuses_the_copies(gpu_lib, dtype, T, h, f, b_transposed, b_staged):
    """TPMLP_LAYOUT_WEIGHTS_STAGED: a forward over new tokens that reuses the
    weight copies an earlier forward left in its workspace equals a plain
    forward bit for bit (also with X given as row slices); and with other
    weights passed, the copied ones are used: the copies are really skipped."""
    import torch
    print(f"case weights staged dtype={dtype} T={T} h={h} f={f} b_t={b_transposed}", flush=True)
    first = synth.draw_inputs(T, h, f, dtype, seed=31)
    second = synth.draw_inputs(T, h, f, dtype, seed=32)
    X, A, b1, B, _ = device_inputs(first)
    X2 = device_inputs(second)[0]
    if b_transposed:
        B = B.t().contiguous()
    nfws = gpu_lib.tp_mlp_fwd_workspace_bytes(T, h, f, gpu_lib.TPMLP_F16 if dtype == "f16" else gpu_lib.TPMLP_BF16,
                                              gpu_lib.TPMLP_LAYOUT_B_T if b_transposed else 0)
    assert nfws > 0
    ws, fresh = (torch.empty((nfws,), dtype=torch.uint8, device="cuda") for _ in range(2))
    new = lambda: tuple(torch.empty((T, n), dtype=X.dtype, device="cuda") for n in (f, f, h))

    def fwd(x, a, b, w, staged, out):
        gpu_lib.tp_mlp_fwd(x, a, b1, b, *out, w, b_transposed=b_transposed, weights_staged=staged)
        torch.cuda.synchronize()
        return out

    fwd(X, A, B, ws, False, new())                      # writes the copies into ws
    ref = fwd(X2, A, B, fresh, False, new())
    got = fwd(X2, A, B, ws, True, new())
    for name, r, g in zip(("Z", "H", "Yp"), ref, got):
        assert torch.equal(r.view(torch.int16), g.view(torch.int16)), name
    sliced = new()
    gpu_lib.tp_mlp_fwd_sp(list(X2.chunk(4)), A, b1, B, *sliced, ws, b_transposed=b_transposed, weights_staged=True)
    torch.cuda.synchronize()
    for name, r, g in zip(("Z", "H", "Yp"), ref, sliced):
        assert torch.equal(r.view(torch.int16), g.view(torch.int16)), name
    # zero weights passed with the flag: the copies of A_i (and B_i where it is copied) still hold the first ones
    Z0, H0, Yp0 = fwd(X2, torch.zeros_like(A), torch.zeros_like(B), ws, True, new())
    assert torch.equal(Z0.view(torch.int16), ref[0].view(torch.int16))
    if b_staged:
        assert torch.equal(Yp0.view(torch.int16), ref[2].view(torch.int16))
    else:
        assert not torch.any(Yp0)
