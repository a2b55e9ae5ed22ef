"""The hot path captured in a HIP graph: the library's calls launch kernels
on the caller's stream only (no allocation, copy, fill or synchronization),
so a captured forward + backward replays to the eager results. Each replay
follows eager work on the same buffers (they are refilled with NaN first),
and every replay's outputs must equal the eager run bit for bit (the kernels
are deterministic)."""
import pytest

import synth
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_and_compare(step, outs):
    import torch
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    # capture: torch.cuda.graph makes its capture stream current, and the
    # binding launches on the current stream
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up off the default stream, as torch's capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for v in outs.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.int16) if v.element_size() == 2 else v.view(torch.int32),
                               eager[k].view(torch.int16) if v.element_size() == 2 else eager[k].view(torch.int32)), (r, k)


@pytest.mark.parametrize("T,h,f,dtype", [(4096, 768, 3072, "f16"), (1024, 512, 768, "bf16")])
def test_mlp_step_replays_from_a_graph(gpu_lib, T, h, f, dtype):
    """tp_mlp_fwd + tp_mlp_bwd with full workspaces. The first shape runs
    the direct-load engine (192 tiles of 256 x 256) with k-split tails, the
    second the register-staged one."""
    import torch
    print(f"case graph mlp T={T} h={h} f={f} {dtype}", flush=True)
    inp = synth.draw_inputs(T, h, f, dtype, seed=T + f)
    X, A, b1, B, dY = device_inputs(inp)
    dev, td = X.device, X.dtype
    e = lambda *s: torch.empty(s, dtype=td, device=dev)
    outs = {"Z": e(T, f), "H": e(T, f), "Yp": e(T, h), "dZ": e(T, f), "dXp": e(T, h), "dA": e(h, f), "dB": e(f, h),
            "db1": e(f)}
    code = gpu_lib.TPMLP_F16 if dtype == "f16" else gpu_lib.TPMLP_BF16
    nfws = gpu_lib.tp_mlp_fwd_workspace_bytes(T, h, f, code)
    nws = gpu_lib.tp_mlp_workspace_bytes(T, h, f, code)
    fws = torch.empty((max(nfws, 1),), dtype=torch.uint8, device=dev)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)
    o = outs

    def step():
        gpu_lib.tp_mlp_fwd(X, A, b1, B, o["Z"], o["H"], o["Yp"], fws)
        gpu_lib.tp_mlp_bwd(dY, X, A, B, o["Z"], o["H"], o["dZ"], o["dXp"], o["dA"], o["dB"], o["db1"], ws)

    _replay_and_compare(step, outs)


def test_flash_attention_replays_from_a_graph(gpu_lib):
    """tp_attn_flash_fwd + tp_attn_flash_bwd (causal, head width 80)."""
    import torch
    from synth.device import to_device
    b, s, h, n, d = 2, 320, 256, 2, 80
    print(f"case graph attention b={b} s={s} h={h} heads={n} d={d}", flush=True)
    inp = synth.draw_attn_inputs(b, s, h, n, d, "bf16", seed=5, sigma_dy=1.0)
    X, Wqkv, bqkv, Wo, dY = (to_device(getattr(inp, k), "bf16") for k in ("X", "Wqkv", "bqkv", "Wo", "dY"))
    T, q, dev = b * s, n * d, X.device
    e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=dev)
    outs = {"QKV": e(T, 3 * q), "O": e(T, q), "Yp": e(T, h), "LSE": torch.empty((b * n, s), dtype=torch.float32,
                                                                                device=dev),
            "dQKV": e(T, 3 * q), "dXp": e(T, h), "dWqkv": e(h, 3 * q), "dbqkv": e(3 * q), "dWo": e(q, h)}
    code = gpu_lib.TPMLP_BF16
    fws = torch.empty((gpu_lib.tp_attn_flash_fwd_workspace_bytes(b, s, h, n, d, code, True),), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty((gpu_lib.tp_attn_flash_bwd_workspace_bytes(b, s, h, n, d, code, True),), dtype=torch.uint8,
                      device=dev)
    o = outs
    kw = dict(batch=b, heads=n, causal=True)

    def step():
        gpu_lib.tp_attn_flash_fwd(X, Wqkv, bqkv, Wo, o["QKV"], o["LSE"], o["O"], o["Yp"], fws, **kw)
        gpu_lib.tp_attn_flash_bwd(dY, X, Wqkv, Wo, o["QKV"], o["LSE"], o["O"], o["dQKV"], o["dXp"], o["dWqkv"],
                                  o["dbqkv"], o["dWo"], bws, **kw)

    _replay_and_compare(step, outs)
