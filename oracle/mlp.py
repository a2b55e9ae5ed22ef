"""Plain float64 oracle of the Transformer MLP and of one tensor-parallel shard.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it comes from:

* The MLP block is Y = GeLU(X A + b1) B (+ b2). The pages enable a fused
  "bias + GeLU" step in the model ("Training GPT-2 with Megatron-LM",
  section 6.2, the fused_bias_gelu switch); the bias is the first linear's.
* GeLU is the tanh approximation of Hendrycks & Gimpel, "Gaussian Error
  Linear Units" (2016): gelu(x) = x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715
  x^3))). The pages name GeLU but give no formula; this form is the one the
  library fixes.
* Tensor parallelism ("Understanding the Megatron-LM architecture: how 3D
  parallelism assigns roles", section 1; also "Megatron-LM overview",
  section 2.2): the first linear is split by output columns, so rank i holds
  A_i = A[:, c_i] and b1_i = b1[c_i] and computes its columns on its own; the
  second linear is split by input rows, B_i = B[c_i, :], so each rank holds a
  partial Y_p,i = H[:, c_i] B_i and the partials are summed (all-reduced).
  A shard is therefore exactly the unsharded MLP evaluated with weights
  (A_i, b1_i, B_i) and no second bias.
* Backward: the pages are silent; it follows by the chain rule from the
  forward. With dY given (the same on every rank, since the adjoint of a sum
  over ranks is a copy), dB = H^T dY, dH = dY B^T, dZ = dH * gelu'(Z),
  dA = X^T dZ, db1 = sum over tokens of dZ, dX = dZ A^T. On a shard dX is a
  partial that is summed over ranks like Y.

All arithmetic is float64. Matrix products use NumPy's matmul (a library
primitive); nothing is blocked, fused or reordered beyond the definitions.
"""
import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_C = 0.044715


def gelu(x):
    """tanh-approximate GeLU, x/2 (1 + tanh(u)), u = sqrt(2/pi)(x + c x^3)."""
    x = np.asarray(x, dtype=np.float64)
    u = SQRT_2_OVER_PI * (x + GELU_C * x ** 3)
    return 0.5 * x * (1.0 + np.tanh(u))


def gelu_grad(x):
    """d/dx of gelu: (1 + t)/2 + x/2 (1 - t^2) sqrt(2/pi) (1 + 3 c x^2), t = tanh(u)."""
    x = np.asarray(x, dtype=np.float64)
    t = np.tanh(SQRT_2_OVER_PI * (x + GELU_C * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_C * x * x)


def mlp_forward(X, A, b1, B, b2=None):
    """Forward of the MLP: Z = X A + b1, H = gelu(Z), Y = H B (+ b2).

    Shapes: X [T,h], A [h,F], b1 [F], B [F,h] (b2 [h] optional).
    Returns a dict with Z, H, Y (float64).
    """
    X, A, b1, B = (np.asarray(t, dtype=np.float64) for t in (X, A, b1, B))
    Z = X @ A + b1[None, :]
    H = gelu(Z)
    Y = H @ B
    if b2 is not None:
        Y = Y + np.asarray(b2, dtype=np.float64)[None, :]
    return {"Z": Z, "H": H, "Y": Y}


def bias2_grad(dY):
    """Gradient of the second bias: Y = H B + 1 b2^T, so dL/db2 = sum over
    tokens of dY (the same on every rank, since b2 is added once after the
    sum over ranks and dY is replicated)."""
    return np.asarray(dY, dtype=np.float64).sum(axis=0)


def mlp_backward(X, A, b1, B, dY, Z=None):
    """Backward of the MLP for a given output gradient dY [T,h].

    Returns dZ, dH, dA [h,F], db1 [F], dB [F,h], dX [T,h] and db2 [h]
    (the latter belongs to the unsharded block only). Z may be passed in to
    reuse the forward's pre-activation.
    """
    X, A, b1, B, dY = (np.asarray(t, dtype=np.float64) for t in (X, A, b1, B, dY))
    if Z is None:
        Z = X @ A + b1[None, :]
    H = gelu(Z)
    dB = H.T @ dY
    dH = dY @ B.T
    dZ = dH * gelu_grad(Z)
    dA = X.T @ dZ
    db1 = dZ.sum(axis=0)
    dX = dZ @ A.T
    db2 = bias2_grad(dY)
    return {"dZ": dZ, "dH": dH, "dA": dA, "db1": db1, "dB": dB, "dX": dX, "db2": db2}


def shard_weights(A, b1, B, tp: int, rank: int):
    """Rank `rank` of `tp`: column block of A and b1, row block of B."""
    F = A.shape[1]
    if F % tp:
        raise ValueError("FFN width not divisible by the TP degree")
    f = F // tp
    c = slice(rank * f, (rank + 1) * f)
    return A[:, c], b1[c], B[c, :]


def shard_forward(X, A_i, b1_i, B_i):
    """One rank's forward: Z_i, H_i and the partial Y_p,i = H_i B_i (no b2)."""
    out = mlp_forward(X, A_i, b1_i, B_i)
    return {"Z": out["Z"], "H": out["H"], "Yp": out["Y"]}


def shard_backward(X, A_i, b1_i, B_i, dY, Z_i=None):
    """One rank's backward: dZ_i, dA_i, db1_i, dB_i and the partial dX_p,i."""
    g = mlp_backward(X, A_i, b1_i, B_i, dY, Z=Z_i)
    return {"dZ": g["dZ"], "dA": g["dA"], "db1": g["db1"], "dB": g["dB"], "dXp": g["dX"]}


def reduce_partials(parts, bias=None, row_begin=0, row_end=None):
    """Sum over ranks of the row-parallel partials, plus the second bias.

    The result of a row split is all-reduced ("Understanding the Megatron-LM
    architecture: how 3D parallelism assigns roles", section 1, the
    row-split item): Y = sum_i Y_p,i + b2 forward, dX = sum_i dX_p,i
    backward. With the sequence dimension split as well ("Training GPT-2 with
    Megatron-LM", section 5.1, --sequence-parallel) the all-reduce becomes a
    reduce-scatter: rank r keeps only its slice of token rows of the same
    sum, here rows [row_begin, row_end). float64, exact up to rounding.
    """
    T = np.asarray(parts[0]).shape[0]
    row_end = T if row_end is None else row_end
    acc = np.zeros_like(np.asarray(parts[0][row_begin:row_end], dtype=np.float64))
    for p in parts:
        acc = acc + np.asarray(p[row_begin:row_end], dtype=np.float64)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)[None, :]
    return acc


def sampled_rows(X, A_i, b1_i, B_i, dY, rows):
    """Shard outputs restricted to token rows `rows`.

    The MLP is token-wise, so Z, H, Y_p, dZ and dX_p of a token depend only
    on that token's X and dY row: this is the shard forward/backward applied
    to the selected rows alone.
    """
    rows = np.asarray(rows)
    Xr = np.asarray(X[rows], dtype=np.float64)
    dYr = np.asarray(dY[rows], dtype=np.float64)
    fw = shard_forward(Xr, A_i, b1_i, B_i)
    dH = dYr @ np.asarray(B_i, dtype=np.float64).T
    dZ = dH * gelu_grad(fw["Z"])
    dXp = dZ @ np.asarray(A_i, dtype=np.float64).T
    return {"Z": fw["Z"], "H": fw["H"], "Yp": fw["Yp"], "dZ": dZ, "dXp": dXp}


def sampled_cols(X, A_i, b1_i, B_i, dY, cols):
    """Shard outputs restricted to FFN-shard columns `cols`.

    Column j of Z, H and dZ needs only column j of A_i, b1_i[j] and row j of
    B_i, over all tokens; from them dA_i[:, j] = X^T dZ[:, j],
    db1_i[j] = sum_t dZ[t, j] and dB_i[j, :] = H[:, j]^T dY.
    """
    cols = np.asarray(cols)
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    Ac = np.asarray(A_i[:, cols], dtype=np.float64)
    bc = np.asarray(b1_i[cols], dtype=np.float64)
    Bc = np.asarray(B_i[cols, :], dtype=np.float64)
    Z = X @ Ac + bc[None, :]
    H = gelu(Z)
    dZ = (dY @ Bc.T) * gelu_grad(Z)
    return {
        "Z": Z,
        "H": H,
        "dZ": dZ,
        "dA": X.T @ dZ,
        "db1": dZ.sum(axis=0),
        "dB": H.T @ dY,
    }


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over all elements of one tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)
