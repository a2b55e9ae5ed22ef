"""Plain float64 oracle of causal self-attention and of one tensor-parallel shard.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it comes from:

* Tensor parallelism of the attention layer ("Megatron-LM overview",
  section 2.2: the Q, K and V computation is split across devices;
  "Understanding the Megatron-LM architecture: how 3D parallelism assigns
  roles", section 1: W_Q, W_K, W_V are split by output columns, the output
  projection by input rows). Rank i owns heads [i n_p, (i+1) n_p) of the
  n heads (n_p = n / P): the Q, K and V columns of those heads
  (Wqkv_i [h, 3 q], q = n_p d, laid out [Q heads | K heads | V heads], each
  head's d columns contiguous), their bias, and the rows of the output
  projection that read those heads (Wo_i [q, h]). Heads are independent, so
  the rank computes its heads' attention on its own and holds a partial sum
  Y_p,i = O_i Wo_i that is reduced over ranks (the output bias is added
  once after the reduction, by the caller).
* Per sequence and head: S = Q K^T / sqrt(d), keys after the query masked
  out (GPT's causal mask; the pages train GPT models), P = softmax(S) along
  the keys, O = P V. The pages enable a fused "scale + mask + softmax" step
  ("Training GPT-2 with Megatron-LM", section 6.2, the fused_softmax
  switch). Dropout is not applied (its random numbers are not on the pages).
* The log-sum-exp of each row of scaled, masked scores,
  L = log sum_{visible k} exp(S_k), is what the fused ("flash") form of
  attention keeps from its forward in place of P: P_k = exp(S_k - L).
  Written out as the definition, with the row maximum taken out first so
  that the exponentials cannot overflow.
* Backward by the chain rule (the pages give none): dO = dY Wo^T,
  dWo = O^T dY, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
  dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dWqkv = X^T dQKV,
  dbqkv = column sums of dQKV, dX = dQKV Wqkv^T (a partial on a shard).

All arithmetic is float64; matrix products use NumPy's matmul. Tokens are
rows b * seq + t of X (sequence b, position t).
"""
import math

import numpy as np


def _f64(*ts):
    return tuple(np.asarray(t, dtype=np.float64) for t in ts)


def split_heads(M, batch, heads):
    """[batch*seq, heads*d] -> [batch, heads, seq, d]."""
    T, c = M.shape
    s, d = T // batch, c // heads
    return M.reshape(batch, s, heads, d).transpose(0, 2, 1, 3)


def merge_heads(M):
    """[batch, heads, seq, d] -> [batch*seq, heads*d] (head j in columns j*d ... j*d + d - 1)."""
    b, n, s, d = M.shape
    return M.transpose(0, 2, 1, 3).reshape(b * s, n * d)


def softmax_rows(S, causal):
    """Row-wise softmax over the last axis; with `causal`, entries with key
    index > query index are excluded (their probability is exactly 0)."""
    S = np.array(S, dtype=np.float64, copy=True)
    s_q, s_k = S.shape[-2:]
    if causal:
        S[..., np.triu(np.ones((s_q, s_k), dtype=bool), k=1)] = -np.inf
    E = np.exp(S - S.max(axis=-1, keepdims=True))
    return E / E.sum(axis=-1, keepdims=True)


def row_logsumexp(S, causal):
    """L = log(sum over the visible keys of exp(S)) along the last axis, in
    natural log; with `causal`, keys after the query are not visible.
    Computed as m + log(sum exp(S - m)), m the row's largest visible score."""
    S = np.array(S, dtype=np.float64, copy=True)
    s_q, s_k = S.shape[-2:]
    if causal:
        S[..., np.triu(np.ones((s_q, s_k), dtype=bool), k=1)] = -np.inf
    m = S.max(axis=-1)
    return m + np.log(np.exp(S - m[..., None]).sum(axis=-1))


def attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal=True, bo=None):
    """Self-attention block (or one shard of it, with that shard's weights
    and its number of heads): returns QKV [T, 3q], P [batch, heads, s, s],
    L [batch, heads, s] (the rows' log-sum-exp), O [T, q] and
    Y [T, h] (= O Wo (+ bo))."""
    X, Wqkv, bqkv, Wo = _f64(X, Wqkv, bqkv, Wo)
    q = Wqkv.shape[1] // 3
    d = q // heads
    QKV = X @ Wqkv + bqkv[None, :]
    Q, K, V = (split_heads(QKV[:, i * q:(i + 1) * q], batch, heads) for i in range(3))
    S = (Q @ K.transpose(0, 1, 3, 2)) / math.sqrt(d)
    P = softmax_rows(S, causal)
    O = merge_heads(P @ V)
    Y = O @ Wo
    if bo is not None:
        Y = Y + np.asarray(bo, dtype=np.float64)[None, :]
    return {"QKV": QKV, "P": P, "L": row_logsumexp(S, causal), "O": O, "Y": Y}


def attn_backward(X, Wqkv, bqkv, Wo, dY, batch, heads, causal=True):
    """Gradients of the block for output gradient dY [T, h]: dQKV, dWqkv,
    dbqkv, dWo and dX (a partial over ranks on a shard)."""
    X, Wqkv, bqkv, Wo, dY = _f64(X, Wqkv, bqkv, Wo, dY)
    fw = attn_forward(X, Wqkv, bqkv, Wo, batch, heads, causal)
    q = Wqkv.shape[1] // 3
    d = q // heads
    QKV, P, O = fw["QKV"], fw["P"], fw["O"]
    Q, K, V = (split_heads(QKV[:, i * q:(i + 1) * q], batch, heads) for i in range(3))
    dO = dY @ Wo.T
    dWo = O.T @ dY
    dO4 = split_heads(dO, batch, heads)
    dV = P.transpose(0, 1, 3, 2) @ dO4
    dP = dO4 @ V.transpose(0, 1, 3, 2)
    dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
    c = 1.0 / math.sqrt(d)
    dQ = (dS @ K) * c
    dK = (dS.transpose(0, 1, 3, 2) @ Q) * c
    dQKV = np.concatenate([merge_heads(dQ), merge_heads(dK), merge_heads(dV)], axis=1)
    return {"dO": dO, "dQKV": dQKV, "dWqkv": X.T @ dQKV, "dbqkv": dQKV.sum(axis=0), "dWo": dWo,
            "dX": dQKV @ Wqkv.T}


def attn_shard_columns(heads, head_dim, tp, rank):
    """Column indices of the full [Q | K | V] projection owned by `rank`."""
    if heads % tp:
        raise ValueError("number of heads not divisible by the TP degree")
    n_p = heads // tp
    q_full = heads * head_dim
    own = np.arange(rank * n_p * head_dim, (rank + 1) * n_p * head_dim)
    return np.concatenate([own, q_full + own, 2 * q_full + own]), own


def attn_shard_weights(Wqkv, bqkv, Wo, heads, tp, rank):
    """Rank `rank` of `tp`: its heads' Q, K, V columns (and bias) and the
    rows of Wo that read them."""
    d = Wqkv.shape[1] // 3 // heads
    cols, rows = attn_shard_columns(heads, d, tp, rank)
    return Wqkv[:, cols], bqkv[cols], Wo[rows, :]


def attn_shard_forward(X, Wqkv_i, bqkv_i, Wo_i, batch, heads_i, causal=True):
    """One rank's forward: QKV_i, P_i, L_i, O_i and the partial Y_p,i (no bo)."""
    fw = attn_forward(X, Wqkv_i, bqkv_i, Wo_i, batch, heads_i, causal)
    return {"QKV": fw["QKV"], "P": fw["P"], "L": fw["L"], "O": fw["O"], "Yp": fw["Y"]}


def attn_shard_backward(X, Wqkv_i, bqkv_i, Wo_i, dY, batch, heads_i, causal=True):
    """One rank's backward: dQKV_i, dWqkv_i, dbqkv_i, dWo_i and the partial dX_p,i."""
    g = attn_backward(X, Wqkv_i, bqkv_i, Wo_i, dY, batch, heads_i, causal)
    return {"dQKV": g["dQKV"], "dWqkv": g["dWqkv"], "dbqkv": g["dbqkv"], "dWo": g["dWo"], "dXp": g["dX"]}
