"""Pins for the float64 oracle: closed forms, brute force, finite differences,
a library cross-check, and the tensor-parallel split identities.

None of these re-types the oracle's matrix code: each check is a fact that
holds independently of it (an identity of the GeLU, a derivative taken
numerically, torch's own tanh-GeLU and autograd, loops over scalars, or the
column/row split of "Understanding the Megatron-LM architecture: how 3D
parallelism assigns roles", section 1).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import gelu, gelu_grad


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- GeLU ----

GRID = np.linspace(-8.0, 8.0, 4001)


def test_gelu_odd_part_is_identity():
    # tanh is odd, so gelu(x) - gelu(-x) = x/2 (1+t) + x/2 (1-t) = x exactly.
    assert np.max(np.abs(gelu(GRID) - gelu(-GRID) - GRID)) <= 1e-14


def test_gelu_grad_symmetry():
    # differentiating the identity above: gelu'(x) + gelu'(-x) = 1.
    assert np.max(np.abs(gelu_grad(GRID) + gelu_grad(-GRID) - 1.0)) <= 1e-14


def test_gelu_special_values():
    assert gelu(0.0) == 0.0
    assert gelu_grad(0.0) == 0.5
    # far tails: gelu -> x on the right, -> 0 on the left; gelu' -> 1 and 0.
    assert gelu(30.0) == 30.0
    assert abs(gelu(-30.0)) < 1e-300
    assert gelu_grad(30.0) == 1.0
    assert abs(gelu_grad(-30.0)) < 1e-300


def test_gelu_grad_matches_central_differences():
    h = 1e-5
    fd = (gelu(GRID + h) - gelu(GRID - h)) / (2 * h)
    assert np.max(np.abs(fd - gelu_grad(GRID))) <= 1e-9


def test_gelu_matches_torch_tanh_gelu():
    torch = pytest.importorskip("torch")
    x = torch.from_numpy(GRID)
    ref = torch.nn.functional.gelu(x, approximate="tanh").numpy()
    assert np.max(np.abs(gelu(GRID) - ref)) <= 4e-15
    # torch's derivative of its own tanh GeLU, through autograd
    xg = x.clone().requires_grad_(True)
    torch.nn.functional.gelu(xg, approximate="tanh").sum().backward()
    assert np.max(np.abs(gelu_grad(GRID) - xg.grad.numpy())) <= 2e-14


def test_gelu_is_the_tanh_form_not_erf():
    # x * Phi(x) (the exact GeLU) stays within 5e-4 of the tanh approximation
    # everywhere, but differs by more than 1e-4 somewhere: the approximation
    # is present and its constants are the right ones to within its error.
    exact = np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in GRID])
    d = np.abs(gelu(GRID) - exact)
    assert d.max() <= 5e-4
    assert d.max() >= 1e-4


# ------------------------------------------------------- brute force ----

def _brute_forward(X, A, b1, B):
    T, h, F = len(X), len(X[0]), len(A[0])
    Z = [[b1[j] + sum(X[t][k] * A[k][j] for k in range(h)) for j in range(F)] for t in range(T)]
    H = [[float(gelu(Z[t][j])) for j in range(F)] for t in range(T)]
    Y = [[sum(H[t][j] * B[j][c] for j in range(F)) for c in range(h)] for t in range(T)]
    return np.array(Z), np.array(H), np.array(Y)


def _brute_backward(X, A, b1, B, dY):
    T, h, F = len(X), len(X[0]), len(A[0])
    Z, H, _ = _brute_forward(X, A, b1, B)
    dB = [[sum(H[t][j] * dY[t][c] for t in range(T)) for c in range(h)] for j in range(F)]
    dH = [[sum(dY[t][c] * B[j][c] for c in range(h)) for j in range(F)] for t in range(T)]
    dZ = [[dH[t][j] * float(gelu_grad(Z[t][j])) for j in range(F)] for t in range(T)]
    dA = [[sum(X[t][k] * dZ[t][j] for t in range(T)) for j in range(F)] for k in range(h)]
    db1 = [sum(dZ[t][j] for t in range(T)) for j in range(F)]
    dX = [[sum(dZ[t][j] * A[k][j] for j in range(F)) for k in range(h)] for t in range(T)]
    return {k: np.array(v) for k, v in
            dict(dZ=dZ, dA=dA, db1=db1, dB=dB, dX=dX).items()}


@pytest.mark.parametrize("T,h,F", [(1, 4, 8), (3, 4, 8), (8, 8, 16), (5, 3, 7)])
def test_forward_and_backward_match_scalar_loops(T, h, F):
    rng = np.random.default_rng(100 + T)
    X, A, b1, B, dY = (_rand(rng, T, h), _rand(rng, h, F, scale=0.3), _rand(rng, F, scale=0.1),
                       _rand(rng, F, h, scale=0.3), _rand(rng, T, h))
    fw = oracle.mlp_forward(X, A, b1, B)
    Z, H, Y = _brute_forward(X.tolist(), A.tolist(), b1.tolist(), B.tolist())
    for got, ref in ((fw["Z"], Z), (fw["H"], H), (fw["Y"], Y)):
        assert oracle.rel_err(got, ref) <= 1e-12
    bw = oracle.mlp_backward(X, A, b1, B, dY)
    ref = _brute_backward(X.tolist(), A.tolist(), b1.tolist(), B.tolist(), dY.tolist())
    for k in ("dZ", "dA", "db1", "dB", "dX"):
        assert oracle.rel_err(bw[k], ref[k]) <= 1e-12, k


# ---------------------------------------------------- finite differences ----

def test_backward_matches_directional_finite_differences():
    rng = np.random.default_rng(7)
    T, h, F = 5, 6, 7
    P = dict(X=_rand(rng, T, h), A=_rand(rng, h, F, scale=0.4), b1=_rand(rng, F, scale=0.2),
             B=_rand(rng, F, h, scale=0.4))
    dY = _rand(rng, T, h)
    g = oracle.mlp_backward(P["X"], P["A"], P["b1"], P["B"], dY)
    grads = dict(X=g["dX"], A=g["dA"], b1=g["db1"], B=g["dB"])

    def loss(Q):
        return float(np.sum(dY * oracle.mlp_forward(Q["X"], Q["A"], Q["b1"], Q["B"])["Y"]))

    eps = 1e-6
    for name in P:
        V = _rand(rng, *P[name].shape)
        Qp = dict(P); Qp[name] = P[name] + eps * V
        Qm = dict(P); Qm[name] = P[name] - eps * V
        fd = (loss(Qp) - loss(Qm)) / (2 * eps)
        an = float(np.sum(grads[name] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), name


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    T, h, F = 9, 8, 12
    X, A, b1, B, dY = (_rand(rng, T, h), _rand(rng, h, F, scale=0.3), _rand(rng, F, scale=0.1),
                       _rand(rng, F, h, scale=0.3), _rand(rng, T, h))
    tX, tA, tb1, tB = (torch.tensor(v, dtype=torch.float64, requires_grad=True) for v in (X, A, b1, B))
    tY = torch.nn.functional.gelu(tX @ tA + tb1, approximate="tanh") @ tB
    tY.backward(torch.tensor(dY))
    g = oracle.mlp_backward(X, A, b1, B, dY)
    assert oracle.rel_err(oracle.mlp_forward(X, A, b1, B)["Y"], tY.detach().numpy()) <= 1e-13
    for ours, t in (("dX", tX), ("dA", tA), ("db1", tb1), ("dB", tB)):
        assert oracle.rel_err(g[ours], t.grad.numpy()) <= 1e-13, ours


# -------------------------------------------- tensor-parallel split ----

@pytest.mark.parametrize("tp", [1, 2, 4])
def test_split_identities(tp):
    rng = np.random.default_rng(20 + tp)
    T, h, F = 6, 8, 16
    X, A, b1, B, dY, b2 = (_rand(rng, T, h), _rand(rng, h, F, scale=0.3), _rand(rng, F, scale=0.1),
                           _rand(rng, F, h, scale=0.3), _rand(rng, T, h), _rand(rng, h, scale=0.1))
    full = oracle.mlp_forward(X, A, b1, B, b2)
    g = oracle.mlp_backward(X, A, b1, B, dY)
    fw = [oracle.shard_forward(X, *oracle.shard_weights(A, b1, B, tp, r)) for r in range(tp)]
    bw = [oracle.shard_backward(X, *oracle.shard_weights(A, b1, B, tp, r), dY) for r in range(tp)]
    # column split: concatenating the shards' columns gives X A + b1 and its GeLU
    assert oracle.rel_err(np.concatenate([s["Z"] for s in fw], axis=1), full["Z"]) <= 1e-12
    assert oracle.rel_err(np.concatenate([s["H"] for s in fw], axis=1), full["H"]) <= 1e-12
    # row split: the partials sum (all-reduce) to the full output
    assert oracle.rel_err(sum(s["Yp"] for s in fw) + b2[None, :], full["Y"]) <= 1e-12
    assert oracle.rel_err(sum(s["dXp"] for s in bw), g["dX"]) <= 1e-12
    assert oracle.rel_err(np.concatenate([s["dA"] for s in bw], axis=1), g["dA"]) <= 1e-12
    assert oracle.rel_err(np.concatenate([s["db1"] for s in bw]), g["db1"]) <= 1e-12
    assert oracle.rel_err(np.concatenate([s["dB"] for s in bw], axis=0), g["dB"]) <= 1e-12
    if tp > 1:
        # a single shard is not the whole answer
        assert oracle.rel_err(fw[0]["Yp"] + b2[None, :], full["Y"]) > 1e-3


# ------------------------------------- reduction of the row-split partials ----

def test_reduce_partials_matches_scalar_loops():
    rng = np.random.default_rng(51)
    P, T, h = 3, 5, 4
    parts = [_rand(rng, T, h) for _ in range(P)]
    bias = _rand(rng, h)
    for rb, re_ in ((0, T), (1, 4), (2, 2)):
        got = oracle.reduce_partials(parts, bias, rb, re_)
        assert got.shape == (re_ - rb, h)
        for r in range(rb, re_):
            for c in range(h):
                s = 0.0
                for i in range(P):
                    s += parts[i][r][c]
                s += bias[c]
                assert got[r - rb][c] == pytest.approx(s, rel=1e-15, abs=1e-15)
    # without a bias: the plain sum
    got = oracle.reduce_partials(parts)
    assert got[4][3] == pytest.approx(parts[0][4][3] + parts[1][4][3] + parts[2][4][3], rel=1e-15)


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_reduced_partials_give_the_unsharded_mlp(tp):
    """The all-reduce of the shards' partials (plus b2) is the unsharded
    output and input gradient; the reduce-scatter slices, stacked, are the
    same sum."""
    rng = np.random.default_rng(60 + tp)
    T, h, F = 8, 8, 16
    X, A, b1, B, dY, b2 = (_rand(rng, T, h), _rand(rng, h, F, scale=0.3), _rand(rng, F, scale=0.1),
                           _rand(rng, F, h, scale=0.3), _rand(rng, T, h), _rand(rng, h, scale=0.1))
    full = oracle.mlp_forward(X, A, b1, B, b2)
    g = oracle.mlp_backward(X, A, b1, B, dY)
    yps = [oracle.shard_forward(X, *oracle.shard_weights(A, b1, B, tp, r))["Yp"] for r in range(tp)]
    dxps = [oracle.shard_backward(X, *oracle.shard_weights(A, b1, B, tp, r), dY)["dXp"] for r in range(tp)]
    assert oracle.rel_err(oracle.reduce_partials(yps, b2), full["Y"]) <= 1e-12
    assert oracle.rel_err(oracle.reduce_partials(dxps), g["dX"]) <= 1e-12
    rows = T // tp
    scattered = [oracle.reduce_partials(yps, b2, r * rows, (r + 1) * rows) for r in range(tp)]
    assert oracle.rel_err(np.concatenate(scattered, axis=0), full["Y"]) <= 1e-12
    if tp > 1:
        # leaving out a rank, or the bias, gives a different answer
        assert oracle.rel_err(oracle.reduce_partials(yps[1:], b2), full["Y"]) > 1e-3
        assert oracle.rel_err(oracle.reduce_partials(yps), full["Y"]) > 1e-3


def test_adjoint_invariants():
    rng = np.random.default_rng(31)
    T, h, f = 7, 8, 12
    X, A, b1, B, dY = (_rand(rng, T, h), _rand(rng, h, f, scale=0.3), _rand(rng, f, scale=0.1),
                       _rand(rng, f, h, scale=0.3), _rand(rng, T, h))
    fw = oracle.shard_forward(X, A, b1, B)
    bw = oracle.shard_backward(X, A, b1, B, dY)

    def ip(u, v):
        return float(np.sum(u * v))

    assert ip(bw["dB"], B) == pytest.approx(ip(dY, fw["Yp"]), rel=1e-12)
    assert ip(bw["dA"], A) == pytest.approx(ip(bw["dXp"], X), rel=1e-12)
    assert ip(bw["dA"], A) == pytest.approx(ip(bw["dZ"], fw["Z"] - b1[None, :]), rel=1e-12)
    assert ip(bw["db1"], b1) == pytest.approx(ip(bw["dZ"], np.broadcast_to(b1, fw["Z"].shape)), rel=1e-12)


def test_sampled_restrictions_match_full_shard():
    rng = np.random.default_rng(41)
    T, h, f = 20, 16, 24
    X, A, b1, B, dY = (_rand(rng, T, h), _rand(rng, h, f, scale=0.3), _rand(rng, f, scale=0.1),
                       _rand(rng, f, h, scale=0.3), _rand(rng, T, h))
    fw = oracle.shard_forward(X, A, b1, B)
    bw = oracle.shard_backward(X, A, b1, B, dY)
    rows = [0, 5, 19]
    cols = [1, 7, 23]
    r = oracle.sampled_rows(X, A, b1, B, dY, rows)
    for k, full in (("Z", fw["Z"]), ("H", fw["H"]), ("Yp", fw["Yp"]), ("dZ", bw["dZ"]), ("dXp", bw["dXp"])):
        assert oracle.rel_err(r[k], full[rows]) <= 1e-13, k
    c = oracle.sampled_cols(X, A, b1, B, dY, cols)
    for k, full in (("Z", fw["Z"][:, cols]), ("H", fw["H"][:, cols]), ("dZ", bw["dZ"][:, cols]),
                    ("dA", bw["dA"][:, cols]), ("db1", bw["db1"][cols]), ("dB", bw["dB"][cols, :])):
        assert oracle.rel_err(c[k], full) <= 1e-13, k


def test_rel_err_definition():
    assert oracle.rel_err(np.array([1.0, 2.0]), np.array([1.0, 4.0])) == 0.5
    assert oracle.rel_err(np.zeros(0), np.zeros(0)) == 0.0
    assert oracle.rel_err(np.array([0.5]), np.array([0.0])) == 0.5


def test_second_bias_gradient():
    """db2 of the full MLP (with b2): against torch float64 autograd, a
    directional finite difference of <dY, Y> along b2, and a scalar loop."""
    import torch
    rng = np.random.default_rng(17)
    T, h, F = 6, 5, 7
    X, A, b1, B, dY = (rng.standard_normal(s) for s in ((T, h), (h, F), (F,), (F, h), (T, h)))
    b2 = rng.standard_normal(h)
    g = oracle.mlp_backward(X, A, b1, B, dY)["db2"]
    assert np.array_equal(g, oracle.bias2_grad(dY))
    tb2 = torch.tensor(b2, requires_grad=True)
    Y = torch.nn.functional.gelu(torch.tensor(X) @ torch.tensor(A) + torch.tensor(b1), approximate="tanh") \
        @ torch.tensor(B) + tb2
    (Y * torch.tensor(dY)).sum().backward()
    assert np.max(np.abs(tb2.grad.numpy() - g)) <= 1e-12
    D, eps = rng.standard_normal(h), 1e-6
    L = lambda bb: float(np.sum(dY * oracle.mlp_forward(X, A, b1, B, b2=bb)["Y"]))
    fd = (L(b2 + eps * D) - L(b2 - eps * D)) / (2 * eps)
    assert abs(fd - float(g @ D)) <= 1e-7 * max(1.0, abs(fd))
    loop = [sum(dY[t][c] for t in range(T)) for c in range(h)]
    assert np.max(np.abs(np.array(loop) - g)) <= 1e-12
