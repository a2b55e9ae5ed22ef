"""The allocation-free backward (tp_mlp_bwd_static) through the C ABI.

It must give bitwise the results of tp_mlp_bwd with a minimal workspace
(the same plan: in-place operands, no staged copies, no k-split), and match
the float64 oracle within the dtype's tolerance, on two calls in a row, the
second with a smaller input: the static scratch then still holds the first
call's column partials, which the second call must not read. Outputs start
as NaN, so an element left unwritten cannot pass the bitwise check.
"""
import pytest

import oracle
import synth
from tests.gpu_util import TOL, compare, device_inputs

pytestmark = pytest.mark.gpu

GRADS = ("dZ", "dXp", "dA", "dB", "db1")

# (dtype, first shape, second shape, keep H): the 2.4B shard (large tiles)
# then a ragged small shape, and small shapes for the other engines
CASES = [
    ("bf16", (8192, 2560, 2560), (520, 264, 392), True),
    ("f16", (1040, 264, 392), (264, 136, 200), False),
    ("bf16", (520, 136, 264), (200, 64, 128), True),
    ("f32", (200, 132, 268), (64, 128, 256), True),
]


def _bits(t):
    import torch
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("dtype,first,second,keep_h", CASES)
def test_static_backward_matches_the_workspace_backward(gpu_lib, dtype, first, second, keep_h):
    import torch
    for (T, h, f), seed in ((first, 31), (second, 32)):
        print(f"case bwd_static dtype={dtype} T={T} h={h} f={f} keep_h={keep_h}", flush=True)
        inp = synth.draw_inputs(T, h, f, dtype, seed=seed, sigma_dy=1.0)
        X, A, b1, B, dY = device_inputs(inp)
        Z, H, _ = gpu_lib.fwd(X, A, b1, B, keep_h=keep_h)
        want = gpu_lib.bwd(dY, X, A, B, Z, H, staged=False)
        nan = lambda *s: torch.full(s, float("nan"), dtype=X.dtype, device="cuda")
        got = {"dZ": nan(T, f), "dXp": nan(T, h), "dA": nan(h, f), "dB": nan(f, h), "db1": nan(f)}
        gpu_lib.tp_mlp_bwd_static(dY, X, A, B, Z, H, got["dZ"], got["dXp"], got["dA"], got["dB"], got["db1"])
        torch.cuda.synchronize()
        for k in GRADS:
            assert torch.equal(_bits(got[k]), _bits(want[k])), k
        ref = oracle.shard_backward(inp.X, inp.A, inp.b1, inp.B, inp.dY)
        compare(got, ref, TOL[dtype], keys=GRADS)


def test_static_backward_rejects_a_shape_beyond_the_scratch(gpu_lib):
    """A shape whose column partials exceed the static scratch fails with
    TPMLP_ERR_SCRATCH before anything is enqueued (outputs untouched)."""
    import torch
    # 4096 tiles of 256 tokens x 2056 columns of fp32 partials: 32.1 MiB
    T, h, f = 1 << 20, 8, 2056
    assert gpu_lib.tp_mlp_workspace_bytes(T, h, f, gpu_lib.TPMLP_BF16, gpu_lib.TPMLP_WS_MINIMAL) > \
        gpu_lib.TPMLP_STATIC_SCRATCH_BYTES
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    dY, X, A, B, Z = e(T, h), e(T, h), e(h, f), e(f, h), e(T, f)
    dZ, dXp, dA, dB, db1 = e(T, f), e(T, h), e(h, f), e(f, h), e(f)
    dA.fill_(3.0)
    with pytest.raises(gpu_lib.TpMlpError) as exc:
        gpu_lib.tp_mlp_bwd_static(dY, X, A, B, Z, None, dZ, dXp, dA, dB, db1)
    assert exc.value.status == 8
    torch.cuda.synchronize()
    assert bool((dA == 3.0).all())
