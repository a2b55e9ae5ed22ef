"""Seeded Gaussian draws, rounded to nearest-even into the storage dtype.

The rounding is written from the IEEE-754 definition: a finite x is snapped
to the nearest multiple of the unit in the last place of its binade (never
finer than the format's subnormal spacing), ties to the even multiple, and
results beyond the largest finite value become +-inf. It is carried out in
float64, where every step below is exact, so fp64 -> fp16 and fp64 -> bf16
are each rounded once (no double rounding through fp32).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import Config

# (stored mantissa bits, minimum normal exponent, largest finite value)
_FORMATS = {
    "f32": (23, -126, float(np.finfo(np.float32).max)),
    "f16": (10, -14, 65504.0),
    "bf16": (7, -126, float.fromhex("0x1.fep127")),
}

# NumPy container that holds the storage bits of each dtype.
STORAGE_NUMPY = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

_CHUNK = 1 << 22


def _round_chunk(x: np.ndarray, mant: int, emin: int, maxval: float) -> None:
    _, e = np.frexp(x)                      # x = m * 2**e with 0.5 <= |m| < 1
    q = np.maximum(e - 1, emin) - mant      # exponent of one ulp at x
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)   # np.rint rounds half to even
    over = np.abs(r) > maxval
    if over.any():
        r[over] = np.copysign(np.inf, x[over])
    x[...] = r


def round_to_storage(x, dtype: str, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Return float64 values of x rounded (RNE) to the storage dtype.

    `out` may be x itself for in-place rounding of a float64 array.
    """
    mant, emin, maxval = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    if out is None:
        out = np.array(x, dtype=np.float64, copy=True)
    elif out is not x:
        out[...] = x
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        _round_chunk(flat[s:s + _CHUNK], mant, emin, maxval)
    return out


def storage_bits(r: np.ndarray, dtype: str) -> np.ndarray:
    """Pack float64 values that are exact in `dtype` into its storage container.

    f32 -> float32, f16 -> float16, bf16 -> uint16 (the top half of the fp32
    bit pattern, which is exact for a bf16-representable value).
    """
    if dtype == "f32":
        return r.astype(np.float32)
    if dtype == "f16":
        return r.astype(np.float16)
    if dtype == "bf16":
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(f"unknown storage dtype {dtype!r}")


@dataclass
class Inputs:
    """One draw of the shard's operands, as float64 values exact in `dtype`.

    A, b1 and B are either the full FFN weights (all_shards) or one rank's
    blocks A_i [h, f], b1_i [f], B_i [f, h].
    """
    dtype: str
    X: np.ndarray
    A: np.ndarray
    b1: np.ndarray
    B: np.ndarray
    dY: np.ndarray
    tp: int = 1
    full: bool = False
    _bits: dict = field(default_factory=dict, repr=False)

    def bits(self, name: str) -> np.ndarray:
        if name not in self._bits:
            self._bits[name] = storage_bits(getattr(self, name), self.dtype)
        return self._bits[name]

    @property
    def tokens(self) -> int:
        return self.X.shape[0]

    @property
    def hidden(self) -> int:
        return self.X.shape[1]


# Draws are made in chunks of DRAW_CHUNK consecutive (row-major) elements;
# chunk c of tensor t comes from its own PCG64 stream seeded with the entropy
# (seed, t, c), so chunks can be drawn in parallel and the values do not
# depend on the number of threads.
DRAW_CHUNK = 1 << 22
TENSOR_IDS = {"X": 0, "A": 1, "b1": 2, "B": 3, "dY": 4, "Wqkv": 5, "bqkv": 6, "Wo": 7}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: int, tensor: str, shape, sigma: float, dtype: str) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    flat = out.reshape(-1)
    tid = TENSOR_IDS[tensor]

    def fill(c: int) -> None:
        seg = flat[c * DRAW_CHUNK:(c + 1) * DRAW_CHUNK]
        rng = np.random.Generator(np.random.PCG64([seed, tid, c]))
        rng.standard_normal(out=seg, dtype=np.float64)
        if sigma != 1.0:
            seg *= sigma
        round_to_storage(seg, dtype, out=seg)

    n_chunks = (flat.size + DRAW_CHUNK - 1) // DRAW_CHUNK
    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def draw_inputs(tokens: int, hidden: int, ffn: int, dtype: str, *, seed: int = 0,
                sigma_x: float = 1.0, sigma_w: float = 0.02, sigma_b: float = 0.01,
                sigma_dy: float = 0.01, tp: int = 1, full: bool = False) -> Inputs:
    """Draw X [T,h], A [h,ffn], b1 [ffn], B [ffn,h], dY [T,h].

    Every tensor is i.i.d. N(0, sigma^2), drawn in float64 from PCG64 streams
    keyed by (seed, tensor, chunk) and rounded to nearest-even into `dtype`.
    `ffn` is the width of what is drawn: the full FFN when full=True (shards
    are sliced later), otherwise the shard width f.
    """
    X = _normal(seed, "X", (tokens, hidden), sigma_x, dtype)
    A = _normal(seed, "A", (hidden, ffn), sigma_w, dtype)
    b1 = _normal(seed, "b1", (ffn,), sigma_b, dtype)
    B = _normal(seed, "B", (ffn, hidden), sigma_w, dtype)
    dY = _normal(seed, "dY", (tokens, hidden), sigma_dy, dtype)
    return Inputs(dtype, X, A, b1, B, dY, tp=tp, full=full)


def draw_config(cfg: Config) -> Inputs:
    width = cfg.ffn if cfg.all_shards else cfg.ffn_shard
    return draw_inputs(cfg.tokens, cfg.hidden, width, cfg.dtype, seed=cfg.seed,
                       sigma_x=cfg.sigma_x, sigma_w=cfg.sigma_w, sigma_b=cfg.sigma_b,
                       sigma_dy=cfg.sigma_dy, tp=cfg.tp, full=cfg.all_shards)


@dataclass
class AttnInputs:
    """One draw of the attention shard's operands (float64 values exact in
    `dtype`): X [T, h], Wqkv [h, 3q], bqkv [3q], Wo [q, h], dY [T, h], with
    q = heads * head_dim the width of the heads drawn (one rank's, or all of
    them when full=True)."""
    dtype: str
    batch: int
    heads: int
    X: np.ndarray
    Wqkv: np.ndarray
    bqkv: np.ndarray
    Wo: np.ndarray
    dY: np.ndarray
    full: bool = False

    @property
    def seq(self) -> int:
        return self.X.shape[0] // self.batch

    @property
    def head_dim(self) -> int:
        return self.Wo.shape[0] // self.heads


def draw_attn_inputs(batch: int, seq: int, hidden: int, heads: int, head_dim: int, dtype: str, *, seed: int = 0,
                     sigma_x: float = 1.0, sigma_w: float = 0.02, sigma_b: float = 0.01, sigma_dy: float = 0.01,
                     full: bool = False) -> AttnInputs:
    """Draw X, Wqkv, bqkv, Wo and dY for `heads` heads of width `head_dim`
    (i.i.d. N(0, sigma^2) like draw_inputs, from their own PCG64 streams)."""
    T, q = batch * seq, heads * head_dim
    X = _normal(seed, "X", (T, hidden), sigma_x, dtype)
    Wqkv = _normal(seed, "Wqkv", (hidden, 3 * q), sigma_w, dtype)
    bqkv = _normal(seed, "bqkv", (3 * q,), sigma_b, dtype)
    Wo = _normal(seed, "Wo", (q, hidden), sigma_w, dtype)
    dY = _normal(seed, "dY", (T, hidden), sigma_dy, dtype)
    return AttnInputs(dtype, batch, heads, X, Wqkv, bqkv, Wo, dY, full=full)
