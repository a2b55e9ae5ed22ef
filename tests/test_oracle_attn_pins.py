"""Pins of the attention oracle (oracle/attn.py) to things other than itself.

The pages print no tensor values for attention, so the pins are:
  * scalar loops written from the definitions (math.exp, explicit sums) on
    tiny shapes, for the forward and the backward;
  * closed forms: the first query of a causal row sees only itself
    (P = 1, O = V); all-zero queries give uniform weights over the visible
    keys, so O is the running mean of V; shift invariance of softmax;
  * invariants: rows of P sum to 1, the causal upper triangle is exactly 0;
  * torch's scaled_dot_product_attention and autograd in float64 on the
    CPU (the special case reduces to a library routine);
  * directional finite differences of <dY, Y>;
  * the tensor-parallel split identities (heads split over ranks): the
    partials sum to the unsharded output and input gradient, the shards'
    weight gradients are the unsharded ones' column / row blocks.
A plausible mistake (a missing 1/sqrt(d), a transposed mask, a wrong head
slice, a dropped softmax term in the backward) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle


def _draw(batch, seq, hidden, heads, d, seed, w=0.3):
    rng = np.random.default_rng(seed)
    T, q = batch * seq, heads * d
    return (rng.standard_normal((T, hidden)), rng.standard_normal((hidden, 3 * q)) * w,
            rng.standard_normal(3 * q) * 0.1, rng.standard_normal((q, hidden)) * w,
            rng.standard_normal((T, hidden)))


def _loops_forward(X, Wqkv, bqkv, Wo, batch, heads, causal):
    T, h = X.shape
    q = Wqkv.shape[1] // 3
    d, s = q // heads, T // batch
    qkv = [[bqkv[c] + sum(X[t][k] * Wqkv[k][c] for k in range(h)) for c in range(3 * q)] for t in range(T)]
    O = [[0.0] * q for _ in range(T)]
    for b in range(batch):
        for j in range(heads):
            for i in range(s):
                ti = b * s + i
                keys = range(i + 1) if causal else range(s)
                sc = {}
                for k in keys:
                    tk = b * s + k
                    sc[k] = sum(qkv[ti][j * d + e] * qkv[tk][q + j * d + e] for e in range(d)) / math.sqrt(d)
                m = max(sc.values())
                z = sum(math.exp(v - m) for v in sc.values())
                for e in range(d):
                    O[ti][j * d + e] = sum(math.exp(sc[k] - m) / z * qkv[b * s + k][2 * q + j * d + e] for k in keys)
    Y = [[sum(O[t][c] * Wo[c][n] for c in range(q)) for n in range(h)] for t in range(T)]
    return np.array(qkv), np.array(O), np.array(Y)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("batch,seq,hidden,heads,d", [(1, 3, 4, 1, 2), (2, 4, 6, 2, 3), (2, 5, 4, 3, 2)])
def test_forward_matches_scalar_loops(causal, batch, seq, hidden, heads, d):
    X, Wqkv, bqkv, Wo, _ = _draw(batch, seq, hidden, heads, d, seed=batch * 7 + seq)
    fw = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)
    qkv, O, Y = _loops_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)
    for got, ref in ((fw["QKV"], qkv), (fw["O"], O), (fw["Y"], Y)):
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_softmax_invariants_and_causal_zeros():
    X, Wqkv, bqkv, Wo, _ = _draw(2, 9, 8, 2, 4, seed=3)
    P = oracle.attn_forward(X, Wqkv, bqkv, Wo, 2, 2, causal=True)["P"]
    assert np.allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    upper = np.triu(np.ones((9, 9), dtype=bool), k=1)
    assert np.all(P[..., upper] == 0.0) and np.all(P[..., ~upper] > 0.0)
    # the first query of every sequence sees only itself
    assert np.all(P[..., 0, 0] == 1.0)
    S = np.random.default_rng(1).standard_normal((3, 5, 5))
    assert np.allclose(oracle.softmax_rows(S + 7.5, False), oracle.softmax_rows(S, False), atol=1e-15)
    # the first output row of a causal sequence is V's first row
    fw = oracle.attn_forward(X, Wqkv, bqkv, Wo, 2, 2, causal=True)
    q = Wqkv.shape[1] // 3
    for b in range(2):
        assert np.allclose(fw["O"][b * 9], fw["QKV"][b * 9, 2 * q:], atol=1e-14)


def test_zero_queries_give_running_means_of_v():
    """Q = 0 (zero Q weights and bias): every visible key gets the same
    weight, so O[t] is the mean of V over positions 0..t (causal) or over
    the whole sequence (not causal)."""
    batch, seq, hidden, heads, d = 2, 6, 5, 2, 3
    X, Wqkv, bqkv, Wo, _ = _draw(batch, seq, hidden, heads, d, seed=4)
    q = heads * d
    Wqkv[:, :q] = 0.0
    bqkv[:q] = 0.0
    for causal in (True, False):
        fw = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)
        V = fw["QKV"][:, 2 * q:].reshape(batch, seq, q)
        if causal:
            ref = np.cumsum(V, axis=1) / np.arange(1, seq + 1)[None, :, None]
        else:
            ref = np.repeat(V.mean(axis=1, keepdims=True), seq, axis=1)
        assert np.allclose(fw["O"], ref.reshape(batch * seq, q), atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_sdpa_and_autograd_fp64(causal):
    import torch
    batch, seq, hidden, heads, d = 2, 7, 12, 3, 4
    X, Wqkv, bqkv, Wo, dY = _draw(batch, seq, hidden, heads, d, seed=5)
    fw = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)
    bw = oracle.attn_backward(X, Wqkv, bqkv, Wo, dY, batch, heads, causal)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(X=X, Wqkv=Wqkv, bqkv=bqkv, Wo=Wo).items()}
    qkv = t["X"] @ t["Wqkv"] + t["bqkv"]
    q = heads * d
    sp = lambda m: m.reshape(batch, seq, heads, d).transpose(1, 2)
    Q, K, V = sp(qkv[:, :q]), sp(qkv[:, q:2 * q]), sp(qkv[:, 2 * q:])
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal)
    O = O.transpose(1, 2).reshape(batch * seq, q)
    Y = O @ t["Wo"]
    (Y * torch.tensor(dY)).sum().backward()
    assert np.max(np.abs(Y.detach().numpy() - fw["Y"])) <= 1e-12
    assert np.max(np.abs(O.detach().numpy() - fw["O"])) <= 1e-12
    for k, g in (("X", "dX"), ("Wqkv", "dWqkv"), ("bqkv", "dbqkv"), ("Wo", "dWo")):
        ref = t[k].grad.numpy()
        assert np.max(np.abs(bw[g] - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref))), k


def test_backward_finite_differences():
    batch, seq, hidden, heads, d = 2, 5, 6, 2, 3
    X, Wqkv, bqkv, Wo, dY = _draw(batch, seq, hidden, heads, d, seed=6)
    bw = oracle.attn_backward(X, Wqkv, bqkv, Wo, dY, batch, heads, True)
    L = lambda X_, W_, b_, O_: float(np.sum(dY * oracle.attn_forward(X_, W_, b_, O_, batch, heads, True)["Y"]))
    rng = np.random.default_rng(7)
    eps = 1e-6
    args = [X, Wqkv, bqkv, Wo]
    for idx, g in enumerate(("dX", "dWqkv", "dbqkv", "dWo")):
        D = rng.standard_normal(args[idx].shape)
        plus = [a + eps * D if i == idx else a for i, a in enumerate(args)]
        minus = [a - eps * D if i == idx else a for i, a in enumerate(args)]
        fd = (L(*plus) - L(*minus)) / (2 * eps)
        an = float(np.sum(bw[g] * D))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (g, fd, an)


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_tensor_parallel_split_identities(tp):
    batch, seq, hidden, heads, d = 2, 6, 8, 4, 3
    X, Wqkv, bqkv, Wo, dY = _draw(batch, seq, hidden, heads, d, seed=8 + tp)
    bo = np.random.default_rng(9).standard_normal(hidden)
    full_f = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, True, bo=bo)
    full_b = oracle.attn_backward(X, Wqkv, bqkv, Wo, dY, batch, heads, True)
    Y = np.zeros_like(full_f["Y"]) + bo[None, :]
    dX = np.zeros_like(X)
    hp = heads // tp
    for r in range(tp):
        Wi, bi, Woi = oracle.attn_shard_weights(Wqkv, bqkv, Wo, heads, tp, r)
        assert Wi.shape == (hidden, 3 * hp * d) and Woi.shape == (hp * d, hidden)
        sf = oracle.attn_shard_forward(X, Wi, bi, Woi, batch, hp)
        sb = oracle.attn_shard_backward(X, Wi, bi, Woi, dY, batch, hp)
        Y += sf["Yp"]
        dX += sb["dXp"]
        cols, rows = oracle.attn_shard_columns(heads, d, tp, r)
        assert np.allclose(sf["QKV"], full_f["QKV"][:, cols], atol=1e-13)
        assert np.allclose(sf["O"], full_f["O"][:, rows], atol=1e-13)
        assert np.allclose(sf["P"], full_f["P"][:, r * hp:(r + 1) * hp], atol=1e-14)
        assert np.allclose(sb["dQKV"], full_b["dQKV"][:, cols], atol=1e-12)
        assert np.allclose(sb["dWqkv"], full_b["dWqkv"][:, cols], atol=1e-12)
        assert np.allclose(sb["dbqkv"], full_b["dbqkv"][cols], atol=1e-12)
        assert np.allclose(sb["dWo"], full_b["dWo"][rows, :], atol=1e-12)
        # adjoint of the row-parallel projection: <dWo_i, Wo_i> = <dY, Yp_i>
        assert math.isclose(float(np.sum(sb["dWo"] * Woi)), float(np.sum(dY * sf["Yp"])), rel_tol=1e-12)
    assert np.allclose(Y, full_f["Y"], atol=1e-12)
    assert np.allclose(dX, full_b["dX"], atol=1e-12)


def _loops_logsumexp(X, Wqkv, bqkv, batch, heads, causal):
    """L[b][j][i] = log(sum over the visible keys k of exp(q_i . k_k / sqrt(d))),
    written from the definition with scalar loops (no maximum taken out:
    the tiny draws keep every exponential in range)."""
    T, h = X.shape
    q = Wqkv.shape[1] // 3
    d, s = q // heads, T // batch
    qkv = [[bqkv[c] + sum(X[t][k] * Wqkv[k][c] for k in range(h)) for c in range(3 * q)] for t in range(T)]
    L = np.zeros((batch, heads, s))
    for b in range(batch):
        for j in range(heads):
            for i in range(s):
                keys = range(i + 1) if causal else range(s)
                tot = math.fsum(math.exp(sum(qkv[b * s + i][j * d + e] * qkv[b * s + k][q + j * d + e]
                                             for e in range(d)) / math.sqrt(d)) for k in keys)
                L[b, j, i] = math.log(tot)
    return L


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("batch,seq,hidden,heads,d", [(1, 3, 4, 1, 2), (2, 5, 4, 3, 2)])
def test_logsumexp_matches_scalar_loops(causal, batch, seq, hidden, heads, d):
    X, Wqkv, bqkv, Wo, _ = _draw(batch, seq, hidden, heads, d, seed=batch * 5 + seq)
    L = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)["L"]
    ref = _loops_logsumexp(X, Wqkv, bqkv, batch, heads, causal)
    assert np.max(np.abs(L - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_logsumexp_closed_forms_and_invariants():
    """Zero queries: every visible score is 0, so L[t] = log(t + 1) (causal)
    or log(seq); exp(S - L) is the softmax P; a shift of every score by c
    shifts L by c, also where exp(S) alone would overflow; the first causal
    query's L is its own score."""
    batch, seq, hidden, heads, d = 2, 6, 5, 2, 3
    X, Wqkv, bqkv, Wo, _ = _draw(batch, seq, hidden, heads, d, seed=11)
    q = heads * d
    Z = Wqkv.copy()
    Z[:, :q] = 0.0
    bz = bqkv.copy()
    bz[:q] = 0.0
    for causal, ref in ((True, np.log(np.arange(1, seq + 1))), (False, np.full(seq, np.log(seq)))):
        L = oracle.attn_forward(X, Z, bz, Wo, batch, heads, causal)["L"]
        assert np.allclose(L, np.broadcast_to(ref, L.shape), rtol=0, atol=1e-14)
    fw = oracle.attn_forward(X, Wqkv, bqkv, Wo, batch, heads, True)
    QKV = fw["QKV"]
    Q, K = (oracle.split_heads(QKV[:, i * q:(i + 1) * q], batch, heads) for i in range(2))
    S = Q @ K.transpose(0, 1, 3, 2) / math.sqrt(d)
    lower = np.tril(np.ones((seq, seq), dtype=bool))
    P = np.where(lower, np.exp(S - fw["L"][..., None]), 0.0)
    assert np.allclose(P, fw["P"], rtol=0, atol=1e-14)
    assert np.allclose(fw["L"][..., 0], S[..., 0, 0], rtol=0, atol=1e-14)
    rng = np.random.default_rng(12)
    S2 = rng.standard_normal((3, 7, 7))
    for causal in (True, False):
        base = oracle.row_logsumexp(S2, causal)
        shifted = oracle.row_logsumexp(S2 + 1000.0, causal)
        assert np.all(np.isfinite(shifted))
        assert np.allclose(shifted - 1000.0, base, rtol=0, atol=1e-11)
