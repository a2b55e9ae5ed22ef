"""Parity of the fused attention path (tp_attn_flash_fwd / tp_attn_flash_bwd)
against the float64 oracle, through the C ABI: QKV, the rows' log-sum-exp
LSE, O and the partial Yp of the forward, every gradient of the backward,
per-tensor max|err| / max|ref| within the storage dtype's tolerance. The
head widths cover every kernel variant (d / 16 rounded up = 1 .. 8), the
sequence lengths ragged ends against the 128-row workgroups and the 64-row
blocks of the inner loops; sharp softmax rows (large scores) exercise the
running maximum's rescaling; a sequence of 8200 tokens is longer than the
materialized path admits; the 2.4B-shaped shard runs in full."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, to_device

pytestmark = pytest.mark.gpu

FWD = ("QKV", "LSE", "O", "Yp")
BWD = ("dQKV", "dXp", "dWqkv", "dbqkv", "dWo")


def _dev(inp):
    d = inp.dtype
    return tuple(to_device(getattr(inp, k), d) for k in ("X", "Wqkv", "bqkv", "Wo", "dY"))


def _run(tp, X, Wqkv, bqkv, Wo, dY, batch, heads, causal):
    import torch
    fw = tp.attn_flash_fwd(X, Wqkv, bqkv, Wo, batch, heads, causal)
    bw = tp.attn_flash_bwd(dY, X, Wqkv, Wo, fw["QKV"], fw["LSE"], fw["O"], batch, heads, causal)
    torch.cuda.synchronize()
    return {**fw, **bw}


def _ref(inp, causal):
    fw = oracle.attn_shard_forward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, inp.batch, inp.heads, causal)
    bw = oracle.attn_shard_backward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, inp.dY, inp.batch, inp.heads, causal)
    fw["LSE"] = fw.pop("L").reshape(inp.batch * inp.heads, inp.seq)
    fw.pop("P")
    return {**fw, **bw}


SHAPES = [(2, 64, 128, 2, 32), (2, 136, 72, 3, 24), (1, 200, 96, 2, 80), (3, 8, 16, 1, 8), (1, 264, 136, 4, 40),
          (2, 72, 64, 1, 128), (1, 136, 64, 2, 56), (1, 192, 96, 1, 96), (2, 328, 64, 1, 104)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("batch,seq,hidden,heads,d", SHAPES)
def test_flash_attention_matches_oracle(gpu_lib, dtype, causal, batch, seq, hidden, heads, d):
    print(f"case flash dtype={dtype} causal={causal} b={batch} s={seq} h={hidden} n={heads} d={d}", flush=True)
    inp = synth.draw_attn_inputs(batch, seq, hidden, heads, d, dtype, seed=seq + 7 * d, sigma_w=0.1,
                                 sigma_dy=1.0)
    got = _run(gpu_lib, *_dev(inp), batch, heads, causal)
    errs = compare(got, _ref(inp, causal), TOL[dtype], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


@pytest.mark.parametrize("causal", [True, False])
def test_flash_sharp_rows(gpu_lib, causal):
    """Scores of magnitude ~10-30: the running maximum of a row moves by
    many units between key blocks and the rescaling of O and of the sum
    carries the result."""
    print(f"case flash sharp causal={causal}", flush=True)
    inp = synth.draw_attn_inputs(2, 520, 64, 2, 64, "f16", seed=31, sigma_w=0.35, sigma_dy=1.0)
    got = _run(gpu_lib, *_dev(inp), 2, 2, causal)
    errs = compare(got, _ref(inp, causal), TOL["f16"], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


def test_flash_agrees_with_the_materialized_path(gpu_lib):
    """Both paths on the same device inputs: QKV bitwise (the same GEMM),
    O, Yp and the gradients within the dtype's tolerance of each other, and
    exp(S - LSE) reproduces the materialized path's P."""
    import torch
    inp = synth.draw_attn_inputs(2, 200, 96, 2, 80, "bf16", seed=5, sigma_w=0.1, sigma_dy=1.0)
    X, Wqkv, bqkv, Wo, dY = _dev(inp)
    f = _run(gpu_lib, X, Wqkv, bqkv, Wo, dY, 2, 2, True)
    m = gpu_lib.attn_fwd(X, Wqkv, bqkv, Wo, 2, 2, True)
    m.update(gpu_lib.attn_bwd(dY, X, Wqkv, Wo, m["QKV"], m["P"], m["O"], 2, 2, True))
    torch.cuda.synchronize()
    assert torch.equal(f["QKV"], m["QKV"])
    compare({k: f[k] for k in ("O", "Yp") + BWD}, {k: m[k].float().cpu().numpy() for k in ("O", "Yp") + BWD},
            TOL["bf16"])
    qkv = f["QKV"].float().cpu().reshape(2, 200, 3, 2, 80)
    Q, K = qkv[:, :, 0].transpose(1, 2), qkv[:, :, 1].transpose(1, 2)
    S = (Q @ K.transpose(-1, -2)).reshape(4, 200, 200) / np.sqrt(80)
    P = torch.exp(S - f["LSE"].cpu()[..., None]).tril()
    assert float((P - m["P"].float().cpu()).abs().max()) <= 2e-2


def test_flash_is_deterministic(gpu_lib):
    import torch
    inp = synth.draw_attn_inputs(2, 136, 72, 3, 24, "bf16", seed=1, sigma_w=0.1, sigma_dy=1.0)
    dev = _dev(inp)
    a = _run(gpu_lib, *dev, 2, 3, True)
    b = _run(gpu_lib, *dev, 2, 3, True)
    for k in FWD + BWD:
        assert torch.equal(a[k], b[k]), k


def test_flash_rejects_bad_arguments(gpu_lib):
    import torch
    inp = synth.draw_attn_inputs(1, 16, 16, 1, 8, "bf16", seed=2)
    X, Wqkv, bqkv, Wo, dY = _dev(inp)
    with pytest.raises(gpu_lib.TpMlpError) as e:
        gpu_lib.attn_flash_fwd(X.float(), Wqkv.float(), bqkv.float(), Wo.float(), 1, 1)
    assert e.value.status == 4  # fp32 is not an attention storage dtype
    small = torch.empty((16,), dtype=torch.uint8, device="cuda")
    fw = gpu_lib.attn_flash_fwd(X, Wqkv, bqkv, Wo, 1, 1)
    with pytest.raises(gpu_lib.TpMlpError) as e:
        gpu_lib.attn_flash_bwd(dY, X, Wqkv, Wo, fw["QKV"], fw["LSE"], fw["O"], 1, 1, ws=small)
    assert e.value.status == 5
    wide = synth.draw_attn_inputs(1, 16, 16, 1, 136, "bf16", seed=3)
    Xw, Ww, bw, Wow, _ = _dev(wide)
    with pytest.raises(gpu_lib.TpMlpError) as e:
        gpu_lib.attn_flash_fwd(Xw, Ww, bw, Wow, 1, 1)
    assert e.value.status == 2  # TPMLP_ERR_SHAPE: head_dim > 128
    torch.cuda.synchronize()


@pytest.mark.slow
@pytest.mark.parametrize("causal", [True, False])
def test_flash_longer_than_the_materialized_cap(gpu_lib, causal):
    """One sequence of 8200 tokens (the materialized path stops at 4096),
    one head of width 64, fp16, every output against the oracle."""
    print(f"case flash seq=8200 causal={causal}", flush=True)
    inp = synth.draw_attn_inputs(1, 8200, 64, 1, 64, "f16", seed=8200, sigma_w=0.1, sigma_dy=1.0)
    got = _run(gpu_lib, *_dev(inp), 1, 1, causal)
    errs = compare(got, _ref(inp, causal), TOL["f16"], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f16", False)])
def test_flash_2p4b_shard_full(gpu_lib, dtype, causal):
    """One TP=4 rank of the 2.4B model's attention (8 of 32 heads, width
    80, 4 sequences of 2048 tokens), every output against the full float64
    oracle."""
    cfg = synth.get_attn_config("attn_2p4b")
    print(f"case flash full-size {cfg.name} {dtype} causal={causal}", flush=True)
    inp = synth.draw_attn_inputs(cfg.micro_batch, cfg.seq_len, cfg.hidden, cfg.heads_shard, cfg.head_dim, dtype,
                                 seed=cfg.seed, sigma_dy=cfg.sigma_dy)
    got = _run(gpu_lib, *_dev(inp), cfg.micro_batch, cfg.heads_shard, causal)
    errs = compare(got, _ref(inp, causal), TOL[dtype], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
