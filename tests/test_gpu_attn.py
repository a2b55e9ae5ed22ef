"""Parity of the attention shard (tp_attn_fwd / tp_attn_bwd) against the
float64 oracle, through the C ABI: every output of the forward (QKV, the
softmax probabilities P, O, the partial Yp) and of the backward (dQKV, dXp,
dWqkv, dbqkv, dWo), per-tensor max|err| / max|ref| within the storage
dtype's tolerance; causal and unmasked; ragged shapes against the 128 x 128
tiles; all heads of a layer split over two ranks and summed on the device;
and the 2.4B-shaped shard (8 of 32 heads of width 80, seq 2048) in full."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, to_device, to_host

pytestmark = pytest.mark.gpu

FWD = ("QKV", "P", "O", "Yp")
BWD = ("dQKV", "dXp", "dWqkv", "dbqkv", "dWo")


def _dev(inp):
    d = inp.dtype
    return tuple(to_device(getattr(inp, k), d) for k in ("X", "Wqkv", "bqkv", "Wo", "dY"))


def _run(tp, X, Wqkv, bqkv, Wo, dY, batch, heads, causal):
    import torch
    fw = tp.attn_fwd(X, Wqkv, bqkv, Wo, batch, heads, causal)
    bw = tp.attn_bwd(dY, X, Wqkv, Wo, fw["QKV"], fw["P"], fw["O"], batch, heads, causal)
    torch.cuda.synchronize()
    return {**fw, **bw}


def _ref(inp, causal):
    fw = oracle.attn_shard_forward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, inp.batch, inp.heads, causal)
    bw = oracle.attn_shard_backward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, inp.dY, inp.batch, inp.heads, causal)
    fw["P"] = fw["P"].reshape(inp.batch * inp.heads, inp.seq, inp.seq)
    return {**fw, **bw}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("batch,seq,hidden,heads,d", [(2, 64, 128, 2, 32), (2, 136, 72, 3, 24), (1, 200, 96, 2, 80),
                                                      (3, 8, 16, 1, 8), (1, 264, 136, 4, 40), (2, 72, 64, 1, 128),
                                                      (1, 136, 48, 2, 136)])
def test_attention_shard_matches_oracle(gpu_lib, dtype, causal, batch, seq, hidden, heads, d):
    print(f"case attn dtype={dtype} causal={causal} b={batch} s={seq} h={hidden} n={heads} d={d}", flush=True)
    inp = synth.draw_attn_inputs(batch, seq, hidden, heads, d, dtype, seed=seq + 7 * d, sigma_w=0.1,
                                 sigma_dy=1.0)
    got = _run(gpu_lib, *_dev(inp), batch, heads, causal)
    errs = compare(got, _ref(inp, causal), TOL[dtype], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    if causal:  # masked probabilities are exactly zero
        import torch
        P = got["P"].float().cpu()
        upper = torch.triu(torch.ones(seq, seq, dtype=torch.bool), diagonal=1)
        assert bool((P[:, upper] == 0).all())


def test_attention_is_deterministic(gpu_lib):
    import torch
    inp = synth.draw_attn_inputs(2, 136, 72, 3, 24, "bf16", seed=1, sigma_w=0.1, sigma_dy=1.0)
    dev = _dev(inp)
    a = _run(gpu_lib, *dev, 2, 3, True)
    b = _run(gpu_lib, *dev, 2, 3, True)
    for k in FWD + BWD:
        assert torch.equal(a[k], b[k]), k


def test_two_ranks_sum_to_the_unsharded_attention(gpu_lib):
    """All four heads of a small layer (hidden 128) split over TP = 2 ranks,
    each rank run through the library, partials summed on the device: the
    sums must match the unsharded oracle's Y and dX, and each rank's weight
    gradients the matching blocks of the unsharded ones."""
    import torch
    cfg = synth.get_attn_config("attn_small")
    n, d, P = cfg.heads, cfg.head_dim, cfg.tp
    full = synth.draw_attn_inputs(cfg.micro_batch, cfg.seq_len, cfg.hidden, n, d, cfg.dtype, seed=cfg.seed,
                                  sigma_dy=cfg.sigma_dy, full=True)
    fw = oracle.attn_forward(full.X, full.Wqkv, full.bqkv, full.Wo, full.batch, n, cfg.causal)
    bw = oracle.attn_backward(full.X, full.Wqkv, full.bqkv, full.Wo, full.dY, full.batch, n, cfg.causal)
    X, dY = to_device(full.X, cfg.dtype), to_device(full.dY, cfg.dtype)
    Y = dX = 0
    tol = TOL[cfg.dtype]
    for r in range(P):
        Wi, bi, Woi = oracle.attn_shard_weights(full.Wqkv, full.bqkv, full.Wo, n, P, r)
        cols, rows = oracle.attn_shard_columns(n, d, P, r)
        o = _run(gpu_lib, X, to_device(Wi, cfg.dtype), to_device(bi, cfg.dtype), to_device(Woi, cfg.dtype), dY,
                 full.batch, n // P, cfg.causal)
        Y = Y + o["Yp"].float()
        dX = dX + o["dXp"].float()
        compare({"dWqkv": o["dWqkv"], "dbqkv": o["dbqkv"], "dWo": o["dWo"]},
                {"dWqkv": bw["dWqkv"][:, cols], "dbqkv": bw["dbqkv"][cols], "dWo": bw["dWo"][rows, :]}, tol)
    torch.cuda.synchronize()
    compare({"Y": to_host(Y), "dX": to_host(dX)}, {"Y": fw["Y"], "dX": bw["dX"]}, tol)


def test_attention_rejects_bad_arguments(gpu_lib):
    import torch
    inp = synth.draw_attn_inputs(1, 16, 16, 1, 8, "bf16", seed=2)
    X, Wqkv, bqkv, Wo, dY = _dev(inp)
    with pytest.raises(gpu_lib.TpMlpError) as e:
        gpu_lib.attn_fwd(X.float(), Wqkv.float(), bqkv.float(), Wo.float(), 1, 1)
    assert e.value.status == 4  # fp32 is not an attention storage dtype
    small = torch.empty((16,), dtype=torch.uint8, device="cuda")
    fw = gpu_lib.attn_fwd(X, Wqkv, bqkv, Wo, 1, 1)
    with pytest.raises(gpu_lib.TpMlpError) as e:
        gpu_lib.attn_bwd(dY, X, Wqkv, Wo, fw["QKV"], fw["P"], fw["O"], 1, 1, ws=small)
    assert e.value.status == 5


@pytest.mark.slow
def test_attention_2p4b_shard_full(gpu_lib):
    """One TP=4 rank of the 2.4B model's attention (8 of 32 heads, width
    80, 4 sequences of 2048 tokens, bf16, causal), every output against the
    full float64 oracle."""
    cfg = synth.get_attn_config("attn_2p4b")
    print(f"case attn full-size {cfg.name}", flush=True)
    inp = synth.draw_attn_inputs(cfg.micro_batch, cfg.seq_len, cfg.hidden, cfg.heads_shard, cfg.head_dim, cfg.dtype,
                                 seed=cfg.seed, sigma_dy=cfg.sigma_dy)
    got = _run(gpu_lib, *_dev(inp), cfg.micro_batch, cfg.heads_shard, cfg.causal)
    errs = compare(got, _ref(inp, cfg.causal), TOL[cfg.dtype], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)



@pytest.mark.slow
@pytest.mark.parametrize("dtype,causal,batch", [("f16", True, 4), ("bf16", False, 2)])
def test_attention_2p4b_shape_other_dtype_and_mask(gpu_lib, dtype, causal, batch):
    """The 2.4B shard's heads (8 of width 80, seq 2048) in fp16 with the
    causal mask, and unmasked in bf16, every output against the oracle."""
    cfg = synth.get_attn_config("attn_2p4b")
    print(f"case attn 2p4b-shaped dtype={dtype} causal={causal} batch={batch}", flush=True)
    inp = synth.draw_attn_inputs(batch, cfg.seq_len, cfg.hidden, cfg.heads_shard, cfg.head_dim, dtype,
                                 seed=7, sigma_dy=cfg.sigma_dy)
    got = _run(gpu_lib, *_dev(inp), batch, cfg.heads_shard, causal)
    errs = compare(got, _ref(inp, causal), TOL[dtype], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("seq", [1024, 4096, 3000])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_long_rows(gpu_lib, seq, causal):
    """Sequences whose softmax rows take 4 (seq 1024) and 16 (seq 3000 and
    4096, the longest the shape check admits) fp32 values per lane, one
    sequence of two heads of width 40, fp16, causal and unmasked, every
    output against the oracle."""
    print(f"case attn long rows seq={seq} causal={causal}", flush=True)
    inp = synth.draw_attn_inputs(1, seq, 64, 2, 40, "f16", seed=seq, sigma_w=0.1, sigma_dy=1.0)
    got = _run(gpu_lib, *_dev(inp), 1, 2, causal)
    errs = compare(got, _ref(inp, causal), TOL["f16"], keys=FWD + BWD)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    if causal:
        import torch
        P = got["P"].float().cpu()
        upper = torch.triu(torch.ones(seq, seq, dtype=torch.bool), diagonal=1)
        assert bool((P[:, upper] == 0).all())

