"""Pins for the seeded input generator and for the workload shapes.

The rounding is checked against the IEEE-754 definition (nearest value of
the format, ties to even), against NumPy's own fp16 conversion and torch's
fp32 -> bf16 conversion; the workload shapes are checked against the sizes
printed on the pages (tests/golden/page_configs.txt).
"""
import os

import numpy as np
import pytest

import synth
from synth import round_to_storage, storage_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_configs.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = int(v)
    return out


def test_workloads_follow_the_pages():
    g = _golden()
    c3 = synth.get_config("gpt_2p4b")
    assert (c3.hidden, c3.seq_len, c3.micro_batch) == (g["p2_2p4b_hidden"], g["p2_2p4b_seq"], g["p2_2p4b_micro_batch"])
    c4 = synth.get_config("gpt_7b")
    assert c4.tp == g["p2_7b_tp"] and c4.hidden == g["p2_ffn_split_dim"]
    assert g["p2_7b_world"] == 4 * 2 * 4
    c5 = synth.get_config("gpt_h10240")
    assert (c5.hidden, c5.tp, c5.micro_batch) == (g["p3_hidden"], g["p3_tp"], g["p3_micro_batch"])
    assert g["p3_world"] == 8 * 4 * 4
    c2 = synth.get_config("gpt2_small")
    assert c2.seq_len == g["p2_context_length"]


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_shard_holds_one_tp_th_of_the_ffn_weights(name):
    # "Training GPT-2 with Megatron-LM", section 1: a 4-way split leaves 1/4
    # of the FFN weights on each GPU.
    c = synth.get_config(name)
    per_rank = c.hidden * c.ffn_shard + c.ffn_shard * c.hidden
    assert per_rank * c.tp == 2 * c.hidden * c.ffn


def _neighbours(r, dtype):
    np_t = {"f16": np.float16, "f32": np.float32}[dtype]
    v = np.array(r, dtype=np_t)
    return (np.nextafter(v, np_t(-np.inf)).astype(np.float64), np.nextafter(v, np_t(np.inf)).astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_rounding_is_nearest_even_by_definition(dtype):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(2000) * s for s in (1e-6, 1e-3, 1.0, 1e3)])
    r = round_to_storage(x, dtype)
    lo, hi = _neighbours(r, dtype)
    # r is a value of the format and no other value of the format is nearer
    assert np.all(np.abs(x - r) <= np.abs(x - lo))
    assert np.all(np.abs(x - r) <= np.abs(x - hi))


def test_rounding_matches_numpy_fp16_and_fp32():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(200000) * 4.0
    assert np.array_equal(round_to_storage(x, "f16"), x.astype(np.float16).astype(np.float64))
    assert np.array_equal(round_to_storage(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_bf16_rounding_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(200000) * 3.0).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_storage(x32.astype(np.float64), "bf16"), ref)


def test_ties_overflow_and_subnormals():
    # bf16 has 7 stored mantissa bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    assert round_to_storage(np.array([1 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert round_to_storage(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 1 + 2.0 ** -6
    assert round_to_storage(np.array([-(1 + 3 * 2.0 ** -8)]), "bf16")[0] == -(1 + 2.0 ** -6)
    # fp16: largest finite 65504; 65520 is the tie with 2^16 and goes to inf
    assert round_to_storage(np.array([65519.0]), "f16")[0] == 65504.0
    assert np.isinf(round_to_storage(np.array([65520.0]), "f16")[0])
    # fp16 subnormals are spaced 2^-24: 2^-25 ties to 0, 3*2^-25 ties to 2^-23
    assert round_to_storage(np.array([2.0 ** -25]), "f16")[0] == 0.0
    assert round_to_storage(np.array([3 * 2.0 ** -25]), "f16")[0] == 2.0 ** -23
    # bf16 subnormals are spaced 2^-133
    assert round_to_storage(np.array([1.4 * 2.0 ** -133]), "bf16")[0] == 2.0 ** -133
    assert round_to_storage(np.array([0.0, -0.0]), "bf16").tolist() == [0.0, 0.0]


def test_storage_bits_roundtrip():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    for dtype, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        r = round_to_storage(rng.standard_normal(1000), dtype)
        b = storage_bits(r, dtype)
        t = torch.from_numpy(b.view(np.int16) if dtype == "bf16" else b)
        if dtype == "bf16":
            t = t.view(torch.bfloat16)
        assert np.array_equal(t.to(torch.float64).numpy(), r)


def test_draws_are_seeded_and_ordered():
    a = synth.draw_inputs(16, 8, 24, "bf16", seed=0)
    b = synth.draw_inputs(16, 8, 24, "bf16", seed=0)
    c = synth.draw_inputs(16, 8, 24, "bf16", seed=1)
    for k in ("X", "A", "b1", "B", "dY"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert not np.array_equal(a.X, c.X)
    # each tensor chunk comes from its own PCG64 stream keyed (seed, tensor, chunk)
    X = np.random.Generator(np.random.PCG64([0, 0, 0])).standard_normal((16, 8))
    A = np.random.Generator(np.random.PCG64([0, 1, 0])).standard_normal((8, 24)) * 0.02
    assert np.array_equal(a.X, round_to_storage(X, "bf16"))
    assert np.array_equal(a.A, round_to_storage(A, "bf16"))
    assert a.X.std() > 0.5 and a.A.std() < 0.05


def test_chunked_draws_do_not_depend_on_threads(monkeypatch):
    from synth import draw as d
    monkeypatch.setattr(d, "DRAW_CHUNK", 64)
    a = synth.draw_inputs(40, 16, 24, "f16", seed=3)
    monkeypatch.setattr(d, "_threads", lambda: 1)
    b = synth.draw_inputs(40, 16, 24, "f16", seed=3)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.dY, b.dY)
    # chunk 1 of X is the second stream of the X tensor
    x1 = np.random.Generator(np.random.PCG64([3, 0, 1])).standard_normal(64)
    assert np.array_equal(a.X.reshape(-1)[64:128], round_to_storage(x1, "f16"))


def test_attention_workload_matches_the_pages():
    """The attention shard's workload is the 2.4B run's printed attention
    shape (hidden, heads, seq, micro-batch), one rank of TP 4 like its MLP."""
    g = _golden()
    a = synth.get_attn_config("attn_2p4b")
    c3 = synth.get_config("gpt_2p4b")
    assert (a.hidden, a.heads, a.seq_len, a.micro_batch) == (g["p2_2p4b_hidden"], g["p2_2p4b_heads"],
                                                             g["p2_2p4b_seq"], g["p2_2p4b_micro_batch"])
    assert a.tp == c3.tp and a.head_dim * a.heads == a.hidden and a.heads_shard * a.tp == a.heads
    x = synth.draw_attn_inputs(1, 8, 16, 2, 8, "bf16", seed=3)
    y = synth.draw_attn_inputs(1, 8, 16, 2, 8, "bf16", seed=3)
    assert all(np.array_equal(getattr(x, k), getattr(y, k)) for k in ("X", "Wqkv", "bqkv", "Wo", "dY"))
    assert x.Wqkv.shape == (16, 48) and x.Wo.shape == (16, 16) and x.seq == 8 and x.head_dim == 8
