"""ctypes binding of libtpmlp.so (include/tp_mlp.h), same names as the C ABI.

Argument marshalling only: tensors are torch device tensors whose data
pointers are handed to the library together with torch's current HIP
stream; every step of the computation runs in the library's kernels. There
is no fallback: if the library is missing or was not built, loading fails
with an error.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtpmlp.so")

TPMLP_F32, TPMLP_F16, TPMLP_BF16 = 0, 1, 2
STATUS = {
    0: "TPMLP_OK",
    1: "TPMLP_ERR_NULL",
    2: "TPMLP_ERR_SHAPE",
    3: "TPMLP_ERR_ALIGN",
    4: "TPMLP_ERR_DTYPE",
    5: "TPMLP_ERR_WORKSPACE",
    6: "TPMLP_ERR_HIP",
    7: "TPMLP_ERR_ALIAS",
    8: "TPMLP_ERR_SCRATCH",
}
EXPORTS = ("tp_mlp_abi_version", "tp_mlp_status_string", "tp_mlp_fwd_workspace_bytes", "tp_mlp_workspace_bytes",
           "tp_mlp_fwd", "tp_mlp_fwd_sp", "tp_mlp_bwd", "tp_mlp_bwd_static", "tp_mlp_bwd_recompute", "tp_mlp_bwd_main_grad", "tp_mlp_reduce_partials",
           "tp_mlp_db2_workspace_bytes", "tp_mlp_db2", "tp_mlp_debug_plan",
           "tp_attn_fwd_workspace_bytes", "tp_attn_bwd_workspace_bytes", "tp_attn_fwd", "tp_attn_bwd",
           "tp_attn_flash_fwd_workspace_bytes", "tp_attn_flash_bwd_workspace_bytes", "tp_attn_flash_fwd",
           "tp_attn_flash_bwd")
TPMLP_MAX_PARTS = 16
TPMLP_WS_DZ, TPMLP_WS_MINIMAL, TPMLP_WS_RECOMPUTE = 1, 2, 4
TPMLP_STATIC_SCRATCH_BYTES = 32 << 20   # device scratch of tp_mlp_bwd_static
FWD_EVENTS = ("TA", "F1", "TB", "F2")                                     # steps bracketed by the 5 events
BWD_EVENTS = ("B1", "B5", "TH", "TdY", "B2", "TX", "TdZ", "B3", "B4")    # ... by the 10 events
RECOMPUTE_EVENTS = ("TA", "F1") + BWD_EVENTS                              # ... by the 12 events


class TpMlpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


TPMLP_LAYOUT_B_T = 1   # B passed as B_i^T [hidden, ffn_shard] (dB returned in that order)
TPMLP_LAYOUT_WEIGHTS_STAGED = 2  # the forward workspace already holds the weight copies (tp_mlp_fwd*)


class tpmlp_shape(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("ffn_shard", ctypes.c_int64), ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32)]


class tpattn_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.tp_mlp_abi_version.restype = ctypes.c_int
    lib.tp_mlp_abi_version.argtypes = []
    lib.tp_mlp_status_string.restype = ctypes.c_char_p
    lib.tp_mlp_status_string.argtypes = [ctypes.c_int]
    lib.tp_mlp_fwd_workspace_bytes.restype = sz
    lib.tp_mlp_fwd_workspace_bytes.argtypes = [ctypes.POINTER(tpmlp_shape)]
    lib.tp_mlp_workspace_bytes.restype = sz
    lib.tp_mlp_workspace_bytes.argtypes = [ctypes.POINTER(tpmlp_shape), ctypes.c_uint]
    lib.tp_mlp_fwd.restype = ctypes.c_int
    lib.tp_mlp_fwd.argtypes = [ctypes.POINTER(tpmlp_shape)] + [vp] * 7 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_fwd_sp.restype = ctypes.c_int
    lib.tp_mlp_fwd_sp.argtypes = [ctypes.POINTER(tpmlp_shape), ctypes.c_int, ctypes.POINTER(vp)] + [vp] * 6 + \
        [vp, sz, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_bwd.restype = ctypes.c_int
    lib.tp_mlp_bwd.argtypes = [ctypes.POINTER(tpmlp_shape)] + [vp] * 11 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_bwd_static.restype = ctypes.c_int
    lib.tp_mlp_bwd_static.argtypes = [ctypes.POINTER(tpmlp_shape)] + [vp] * 11 + [vp, ctypes.POINTER(vp)]
    lib.tp_mlp_bwd_recompute.restype = ctypes.c_int
    lib.tp_mlp_bwd_recompute.argtypes = [ctypes.POINTER(tpmlp_shape)] + [vp] * 10 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_bwd_main_grad.restype = ctypes.c_int
    lib.tp_mlp_bwd_main_grad.argtypes = [ctypes.POINTER(tpmlp_shape)] + [vp] * 11 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_reduce_partials.restype = ctypes.c_int
    lib.tp_mlp_reduce_partials.argtypes = [ctypes.POINTER(tpmlp_shape), ctypes.c_int, ctypes.POINTER(vp), vp,
                                           ctypes.c_int64, ctypes.c_int64, vp, vp]
    lib.tp_mlp_db2_workspace_bytes.restype = sz
    lib.tp_mlp_db2_workspace_bytes.argtypes = [ctypes.POINTER(tpmlp_shape)]
    lib.tp_mlp_db2.restype = ctypes.c_int
    lib.tp_mlp_db2.argtypes = [ctypes.POINTER(tpmlp_shape), vp, vp, ctypes.c_int, vp, sz, vp]
    lib.tp_mlp_debug_plan.restype = ctypes.c_int
    lib.tp_mlp_debug_plan.argtypes = [ctypes.c_int, ctypes.c_int]
    ap = ctypes.POINTER(tpattn_shape)
    lib.tp_attn_fwd_workspace_bytes.restype = sz
    lib.tp_attn_fwd_workspace_bytes.argtypes = [ap]
    lib.tp_attn_bwd_workspace_bytes.restype = sz
    lib.tp_attn_bwd_workspace_bytes.argtypes = [ap]
    lib.tp_attn_fwd.restype = ctypes.c_int
    lib.tp_attn_fwd.argtypes = [ap] + [vp] * 8 + [vp, sz, vp]
    lib.tp_attn_bwd.restype = ctypes.c_int
    lib.tp_attn_bwd.argtypes = [ap] + [vp] * 12 + [vp, sz, vp]
    for name in ("tp_attn_flash_fwd_workspace_bytes", "tp_attn_flash_bwd_workspace_bytes"):
        getattr(lib, name).restype = sz
        getattr(lib, name).argtypes = [ap]
    lib.tp_attn_flash_fwd.restype = ctypes.c_int
    lib.tp_attn_flash_fwd.argtypes = [ap] + [vp] * 8 + [vp, sz, vp]
    lib.tp_attn_flash_bwd.restype = ctypes.c_int
    lib.tp_attn_flash_bwd.argtypes = [ap] + [vp] * 12 + [vp, sz, vp]
    _lib = lib
    return lib


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: TPMLP_F32, torch.float16: TPMLP_F16, torch.bfloat16: TPMLP_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous row-major")
    return t.data_ptr() or None


def _stream(stream):
    """hipStream_t handle of `stream` (a torch stream or a raw handle), or of
    torch's current stream when it is None."""
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _on_stream(stream):
    """Context for the wrappers that allocate with torch: inside it, torch's
    current stream is the launch stream `stream` (None: torch's current
    stream, nothing changes). Outputs and workspaces allocated there belong
    to the launch stream in torch's caching allocator, so a workspace freed
    when the wrapper returns is reused only by work ordered after the
    library's kernels on that stream, never by other streams' work that
    could overlap them."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    import torch
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _events(events):
    if events is None:
        return None
    arr = (ctypes.c_void_p * len(events))()
    for i, e in enumerate(events):
        if e is None:  # a NULL entry: that point is not recorded
            arr[i] = None
        elif hasattr(e, "cuda_event"):
            if not e.cuda_event:  # torch creates its HIP event on first record
                e.record()
            arr[i] = e.cuda_event
        else:
            arr[i] = int(e)
    return arr


def _check(status: int):
    if status != 0:
        raise TpMlpError(status, load().tp_mlp_status_string(status).decode())


def shape_of(tokens: int, hidden: int, ffn_shard: int, dtype: int, layout: int = 0) -> tpmlp_shape:
    return tpmlp_shape(tokens, hidden, ffn_shard, dtype, layout)


def _layout(b_transposed: bool, weights_staged: bool = False) -> int:
    return (TPMLP_LAYOUT_B_T if b_transposed else 0) | (TPMLP_LAYOUT_WEIGHTS_STAGED if weights_staged else 0)


# tile names of tp_mlp_debug_plan (TPMLP_PLAN_* in include/tp_mlp.h)
PLAN_TILES = {None: 0, "auto": 0, 128: 1, "128": 1, 256: 2, "256": 2, "dma256": 3, "dma320": 4, "dma320m32": 5}


def tp_mlp_debug_plan(tile=None, tail_cus: int = 0) -> None:
    """Force a GEMM engine and the k-split planner's CU count for the calls
    that follow (tests and tuning only; None / 0 restore the defaults)."""
    if tile not in PLAN_TILES:
        raise ValueError(f"unknown tile {tile!r}; one of {sorted(map(str, PLAN_TILES))}")
    _check(load().tp_mlp_debug_plan(PLAN_TILES[tile], int(tail_cus)))


class debug_plan:
    """Context manager around tp_mlp_debug_plan that restores the default
    plan on exit."""

    def __init__(self, tile=None, tail_cus: int = 0):
        self.tile, self.tail_cus = tile, tail_cus

    def __enter__(self):
        tp_mlp_debug_plan(self.tile, self.tail_cus)
        return self

    def __exit__(self, *exc):
        tp_mlp_debug_plan(None, 0)
        return False


def tp_mlp_abi_version() -> int:
    return load().tp_mlp_abi_version()


def tp_mlp_status_string(status: int) -> str:
    return load().tp_mlp_status_string(status).decode()


def tp_mlp_fwd_workspace_bytes(tokens: int, hidden: int, ffn_shard: int, dtype: int, layout: int = 0) -> int:
    s = shape_of(tokens, hidden, ffn_shard, dtype, layout)
    return load().tp_mlp_fwd_workspace_bytes(ctypes.byref(s))


def tp_mlp_workspace_bytes(tokens: int, hidden: int, ffn_shard: int, dtype: int, flags: int = 0,
                           layout: int = 0) -> int:
    s = shape_of(tokens, hidden, ffn_shard, dtype, layout)
    return load().tp_mlp_workspace_bytes(ctypes.byref(s), int(flags))


def _nbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def tp_mlp_fwd(X, A, b1, B, Z, H, Yp, ws=None, *, stream=None, events=None, b_transposed=False,
               weights_staged=False) -> None:
    """Forward of one TP rank into caller-allocated Z, H (or None) and Yp.
    weights_staged: `ws` already holds the weight copies of an earlier
    forward with the same weights and workspace (TPMLP_LAYOUT_WEIGHTS_STAGED)."""
    s = shape_of(X.shape[0], X.shape[1], A.shape[1], _dtype_code(X), _layout(b_transposed, weights_staged))
    ev = _events(events)
    _check(load().tp_mlp_fwd(ctypes.byref(s), _ptr(X), _ptr(A), _ptr(b1), _ptr(B), _ptr(Z), _ptr(H), _ptr(Yp),
                             _ptr(ws), _nbytes(ws), _stream(stream), ev))


def tp_mlp_fwd_sp(X_slices, A, b1, B, Z, H, Yp, ws=None, *, stream=None, events=None, b_transposed=False,
                  weights_staged=False) -> None:
    """Forward of one TP rank under sequence parallelism: X given as equal
    token-row slices (a list of [T/n, hidden] device tensors, one per rank),
    read in place by the first GEMM instead of an all-gathered copy."""
    n = len(X_slices)
    T = sum(x.shape[0] for x in X_slices)
    s = shape_of(T, X_slices[0].shape[1], A.shape[1], _dtype_code(X_slices[0]), _layout(b_transposed, weights_staged))
    arr = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in X_slices])
    ev = _events(events)
    _check(load().tp_mlp_fwd_sp(ctypes.byref(s), n, arr, _ptr(A), _ptr(b1), _ptr(B), _ptr(Z), _ptr(H), _ptr(Yp),
                                _ptr(ws), _nbytes(ws), _stream(stream), ev))


def tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, ws, *, stream=None, events=None, b_transposed=False) -> None:
    """Backward of one TP rank into caller-allocated gradients and workspace."""
    s = shape_of(X.shape[0], X.shape[1], A.shape[1], _dtype_code(X), _layout(b_transposed))
    nbytes = _nbytes(ws)
    ev = _events(events)
    _check(load().tp_mlp_bwd(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(A), _ptr(B), _ptr(Z), _ptr(H), _ptr(dZ),
                             _ptr(dXp), _ptr(dA), _ptr(dB), _ptr(db1), _ptr(ws), nbytes, _stream(stream), ev))


def tp_mlp_bwd_static(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, *, stream=None, events=None,
                      b_transposed=False) -> None:
    """Backward of one TP rank that allocates nothing and takes no workspace
    (its scratch is the library's static device array); dZ is required."""
    s = shape_of(X.shape[0], X.shape[1], A.shape[1], _dtype_code(X), _layout(b_transposed))
    ev = _events(events)
    _check(load().tp_mlp_bwd_static(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(A), _ptr(B), _ptr(Z), _ptr(H),
                                    _ptr(dZ), _ptr(dXp), _ptr(dA), _ptr(dB), _ptr(db1), _stream(stream), ev))


def tp_mlp_bwd_recompute(dY, X, A, b1, B, dZ, dXp, dA, dB, db1, ws, *, stream=None, events=None, b_transposed=False) -> None:
    """Backward of one TP rank that recomputes Z (and gelu(Z)) from X first."""
    s = shape_of(X.shape[0], X.shape[1], A.shape[1], _dtype_code(X), _layout(b_transposed))
    ev = _events(events)
    _check(load().tp_mlp_bwd_recompute(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(A), _ptr(b1), _ptr(B), _ptr(dZ),
                                       _ptr(dXp), _ptr(dA), _ptr(dB), _ptr(db1), _ptr(ws), _nbytes(ws),
                                       _stream(stream), ev))


def bwd_recompute(dY, X, A, b1, B, keep_dz: bool = True, staged: bool = True, stream=None, events=None,
                  b_transposed: bool = False):
    """Allocate the gradients and the workspace with torch and run
    tp_mlp_bwd_recompute."""
    import torch
    with _on_stream(stream):
        T, f, h = X.shape[0], A.shape[1], X.shape[1]
        dev, dt = X.device, X.dtype
        dZ = torch.empty((T, f), dtype=dt, device=dev) if keep_dz else None
        dXp = torch.empty((T, h), dtype=dt, device=dev)
        dA = torch.empty((h, f), dtype=dt, device=dev)
        dB = torch.empty((h, f) if b_transposed else (f, h), dtype=dt, device=dev)
        db1 = torch.empty((f,), dtype=dt, device=dev)
        flags = TPMLP_WS_RECOMPUTE | (0 if keep_dz else TPMLP_WS_DZ) | (0 if staged else TPMLP_WS_MINIMAL)
        nws = tp_mlp_workspace_bytes(T, h, f, _dtype_code(X), flags, _layout(b_transposed))
        ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev) if nws else None
        tp_mlp_bwd_recompute(dY, X, A, b1, B, dZ, dXp, dA, dB, db1, ws, stream=stream, events=events,
                             b_transposed=b_transposed)
        return {"dZ": dZ, "dXp": dXp, "dA": dA, "dB": dB, "db1": db1}


def tp_mlp_bwd_main_grad(dY, X, A, B, Z, H, dZ, dXp, dA_main, dB_main, db1_main, ws, *, stream=None,
                         events=None, b_transposed=False) -> None:
    """Backward of one TP rank that adds the weight gradients to fp32 main
    gradients (dA_main [h, f], dB_main [f, h], db1_main [f], float32)."""
    import torch
    for t in (dA_main, dB_main, db1_main):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("main gradients are float32")
    s = shape_of(X.shape[0], X.shape[1], A.shape[1], _dtype_code(X), _layout(b_transposed))
    ev = _events(events)
    _check(load().tp_mlp_bwd_main_grad(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(A), _ptr(B), _ptr(Z), _ptr(H),
                                       _ptr(dZ), _ptr(dXp), _ptr(dA_main), _ptr(dB_main), _ptr(db1_main), _ptr(ws),
                                       _nbytes(ws), _stream(stream), ev))


def tp_mlp_reduce_partials(parts, bias, out, row_begin: int = 0, row_end=None, *, stream=None) -> None:
    """out = sum of the [T, h] partials `parts` (one per rank, summed in list
    order in fp32) plus `bias` (or None), over rows [row_begin, row_end)."""
    T, h = parts[0].shape
    if row_end is None:
        row_end = T
    s = shape_of(T, h, 0, _dtype_code(parts[0]))
    arr = (ctypes.c_void_p * max(len(parts), 1))(*[_ptr(p) for p in parts])
    _check(load().tp_mlp_reduce_partials(ctypes.byref(s), len(parts), arr, _ptr(bias), int(row_begin), int(row_end),
                                         _ptr(out), _stream(stream)))


def tp_mlp_db2_workspace_bytes(tokens: int, hidden: int, dtype: int) -> int:
    s = shape_of(tokens, hidden, 8 if dtype != TPMLP_F32 else 4, dtype)
    return load().tp_mlp_db2_workspace_bytes(ctypes.byref(s))


def tp_mlp_db2(dY, db2, ws=None, *, accumulate: bool = False, stream=None) -> None:
    """db2 = column sums of dY [T, h] (storage dtype), or db2 += them when
    `accumulate` (db2 an fp32 main gradient)."""
    import torch
    if accumulate and db2.dtype != torch.float32:
        raise TypeError("an accumulated db2 is a float32 main gradient")
    T, h = dY.shape
    code = _dtype_code(dY)
    s = shape_of(T, h, 8 if code != TPMLP_F32 else 4, code)
    _check(load().tp_mlp_db2(ctypes.byref(s), _ptr(dY), _ptr(db2), 1 if accumulate else 0, _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def db2(dY, stream=None):
    """Allocate db2 (and the workspace) with torch and run tp_mlp_db2."""
    import torch
    with _on_stream(stream):
        T, h = dY.shape
        out = torch.empty((h,), dtype=dY.dtype, device=dY.device)
        n = tp_mlp_db2_workspace_bytes(T, h, _dtype_code(dY))
        ws = torch.empty((n,), dtype=torch.uint8, device=dY.device) if n else None
        tp_mlp_db2(dY, out, ws, stream=stream)
        return out


# ---- convenience wrappers that allocate the outputs with torch ----

def fwd(X, A, b1, B, keep_h: bool = True, staged: bool = True, stream=None, events=None, b_transposed: bool = False):
    """Allocate the outputs (and, if `staged`, the workspace) with torch and run tp_mlp_fwd."""
    import torch
    with _on_stream(stream):
        T, f, h = X.shape[0], A.shape[1], X.shape[1]
        Z = torch.empty((T, f), dtype=X.dtype, device=X.device)
        H = torch.empty((T, f), dtype=X.dtype, device=X.device) if keep_h else None
        Yp = torch.empty((T, h), dtype=X.dtype, device=X.device)
        nws = tp_mlp_fwd_workspace_bytes(T, h, f, _dtype_code(X), _layout(b_transposed)) if staged else 0
        ws = torch.empty((nws,), dtype=torch.uint8, device=X.device) if nws else None
        tp_mlp_fwd(X, A, b1, B, Z, H, Yp, ws, stream=stream, events=events, b_transposed=b_transposed)
        return Z, H, Yp


def bwd(dY, X, A, B, Z, H=None, keep_dz: bool = True, staged: bool = True, stream=None, events=None,
        b_transposed: bool = False):
    """Allocate the gradients and the workspace (the staged size, or the
    minimal one when `staged` is False) with torch and run tp_mlp_bwd."""
    import torch
    with _on_stream(stream):
        T, f, h = X.shape[0], A.shape[1], X.shape[1]
        dev, dt = X.device, X.dtype
        dZ = torch.empty((T, f), dtype=dt, device=dev) if keep_dz else None
        dXp = torch.empty((T, h), dtype=dt, device=dev)
        dA = torch.empty((h, f), dtype=dt, device=dev)
        dB = torch.empty((h, f) if b_transposed else (f, h), dtype=dt, device=dev)
        db1 = torch.empty((f,), dtype=dt, device=dev)
        flags = (0 if keep_dz else TPMLP_WS_DZ) | (0 if staged else TPMLP_WS_MINIMAL)
        nws = tp_mlp_workspace_bytes(T, h, f, _dtype_code(X), flags, _layout(b_transposed))
        ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev) if nws else None
        tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, ws, stream=stream, events=events, b_transposed=b_transposed)
        return {"dZ": dZ, "dXp": dXp, "dA": dA, "dB": dB, "db1": db1}


# ---- attention shard (include/tp_attn.h) ----

def attn_shape(batch: int, seq: int, hidden: int, heads: int, head_dim: int, dtype: int,
               causal: bool = True) -> tpattn_shape:
    return tpattn_shape(batch, seq, hidden, heads, head_dim, dtype, 1 if causal else 0)


def tp_attn_fwd_workspace_bytes(batch, seq, hidden, heads, head_dim, dtype, causal=True) -> int:
    s = attn_shape(batch, seq, hidden, heads, head_dim, dtype, causal)
    return load().tp_attn_fwd_workspace_bytes(ctypes.byref(s))


def tp_attn_bwd_workspace_bytes(batch, seq, hidden, heads, head_dim, dtype, causal=True) -> int:
    s = attn_shape(batch, seq, hidden, heads, head_dim, dtype, causal)
    return load().tp_attn_bwd_workspace_bytes(ctypes.byref(s))


def _attn_shape_of(X, Wo, batch, heads, causal):
    T, h = X.shape
    q = Wo.shape[0]
    if T % batch or q % heads:
        raise ValueError("tokens must split into `batch` sequences and Wo rows into `heads` heads")
    return attn_shape(batch, T // batch, h, heads, q // heads, _dtype_code(X), causal)


def tp_attn_fwd(X, Wqkv, bqkv, Wo, QKV, P, O, Yp, ws, *, batch, heads, causal=True, stream=None) -> None:
    """Forward of one rank's heads into caller-allocated QKV, P, O, Yp."""
    s = _attn_shape_of(X, Wo, batch, heads, causal)
    _check(load().tp_attn_fwd(ctypes.byref(s), _ptr(X), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo), _ptr(QKV), _ptr(P),
                              _ptr(O), _ptr(Yp), _ptr(ws), _nbytes(ws), _stream(stream)))


def tp_attn_bwd(dY, X, Wqkv, Wo, QKV, P, O, dQKV, dXp, dWqkv, dbqkv, dWo, ws, *, batch, heads, causal=True,
                stream=None) -> None:
    """Backward of one rank's heads into caller-allocated gradients."""
    s = _attn_shape_of(X, Wo, batch, heads, causal)
    _check(load().tp_attn_bwd(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(Wqkv), _ptr(Wo), _ptr(QKV), _ptr(P),
                              _ptr(O), _ptr(dQKV), _ptr(dXp), _ptr(dWqkv), _ptr(dbqkv), _ptr(dWo), _ptr(ws),
                              _nbytes(ws), _stream(stream)))


def attn_fwd(X, Wqkv, bqkv, Wo, batch, heads, causal=True, ws=None, stream=None):
    """Allocate the outputs (and the workspace unless given) with torch and run tp_attn_fwd."""
    import torch
    with _on_stream(stream):
        T, h = X.shape
        q = Wo.shape[0]
        s = T // batch
        e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=X.device)
        QKV, P, O, Yp = e(T, 3 * q), e(batch * heads, s, s), e(T, q), e(T, h)
        if ws is None:
            n = tp_attn_fwd_workspace_bytes(batch, s, h, heads, q // heads, _dtype_code(X), causal)
            ws = torch.empty((n,), dtype=torch.uint8, device=X.device)
        tp_attn_fwd(X, Wqkv, bqkv, Wo, QKV, P, O, Yp, ws, batch=batch, heads=heads, causal=causal, stream=stream)
        return {"QKV": QKV, "P": P, "O": O, "Yp": Yp}


def attn_bwd(dY, X, Wqkv, Wo, QKV, P, O, batch, heads, causal=True, ws=None, stream=None):
    """Allocate the gradients (and the workspace unless given) with torch and run tp_attn_bwd."""
    import torch
    with _on_stream(stream):
        T, h = X.shape
        q = Wo.shape[0]
        e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=X.device)
        dQKV, dXp, dWqkv, dbqkv, dWo = e(T, 3 * q), e(T, h), e(h, 3 * q), e(3 * q), e(q, h)
        if ws is None:
            n = tp_attn_bwd_workspace_bytes(batch, T // batch, h, heads, q // heads, _dtype_code(X), causal)
            ws = torch.empty((n,), dtype=torch.uint8, device=X.device)
        tp_attn_bwd(dY, X, Wqkv, Wo, QKV, P, O, dQKV, dXp, dWqkv, dbqkv, dWo, ws, batch=batch, heads=heads,
                    causal=causal, stream=stream)
        return {"dQKV": dQKV, "dXp": dXp, "dWqkv": dWqkv, "dbqkv": dbqkv, "dWo": dWo}


# ---- fused attention path (include/tp_attn.h, tp_attn_flash_*) ----

def tp_attn_flash_fwd_workspace_bytes(batch, seq, hidden, heads, head_dim, dtype, causal=True) -> int:
    s = attn_shape(batch, seq, hidden, heads, head_dim, dtype, causal)
    return load().tp_attn_flash_fwd_workspace_bytes(ctypes.byref(s))


def tp_attn_flash_bwd_workspace_bytes(batch, seq, hidden, heads, head_dim, dtype, causal=True) -> int:
    s = attn_shape(batch, seq, hidden, heads, head_dim, dtype, causal)
    return load().tp_attn_flash_bwd_workspace_bytes(ctypes.byref(s))


def tp_attn_flash_fwd(X, Wqkv, bqkv, Wo, QKV, LSE, O, Yp, ws, *, batch, heads, causal=True, stream=None) -> None:
    """Fused forward of one rank's heads into caller-allocated QKV, LSE (fp32), O, Yp."""
    s = _attn_shape_of(X, Wo, batch, heads, causal)
    _check(load().tp_attn_flash_fwd(ctypes.byref(s), _ptr(X), _ptr(Wqkv), _ptr(bqkv), _ptr(Wo), _ptr(QKV),
                                    _ptr(LSE), _ptr(O), _ptr(Yp), _ptr(ws), _nbytes(ws), _stream(stream)))


def tp_attn_flash_bwd(dY, X, Wqkv, Wo, QKV, LSE, O, dQKV, dXp, dWqkv, dbqkv, dWo, ws, *, batch, heads, causal=True,
                      stream=None) -> None:
    """Fused backward of one rank's heads into caller-allocated gradients."""
    s = _attn_shape_of(X, Wo, batch, heads, causal)
    _check(load().tp_attn_flash_bwd(ctypes.byref(s), _ptr(dY), _ptr(X), _ptr(Wqkv), _ptr(Wo), _ptr(QKV),
                                    _ptr(LSE), _ptr(O), _ptr(dQKV), _ptr(dXp), _ptr(dWqkv), _ptr(dbqkv), _ptr(dWo),
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def attn_flash_fwd(X, Wqkv, bqkv, Wo, batch, heads, causal=True, ws=None, stream=None):
    """Allocate the outputs (and the workspace unless given) with torch and run tp_attn_flash_fwd."""
    import torch
    with _on_stream(stream):
        T, h = X.shape
        q = Wo.shape[0]
        s = T // batch
        e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=X.device)
        QKV, O, Yp = e(T, 3 * q), e(T, q), e(T, h)
        LSE = torch.empty((batch * heads, s), dtype=torch.float32, device=X.device)
        if ws is None:
            n = tp_attn_flash_fwd_workspace_bytes(batch, s, h, heads, q // heads, _dtype_code(X), causal)
            ws = torch.empty((n,), dtype=torch.uint8, device=X.device)
        tp_attn_flash_fwd(X, Wqkv, bqkv, Wo, QKV, LSE, O, Yp, ws, batch=batch, heads=heads, causal=causal,
                          stream=stream)
        return {"QKV": QKV, "LSE": LSE, "O": O, "Yp": Yp}


def attn_flash_bwd(dY, X, Wqkv, Wo, QKV, LSE, O, batch, heads, causal=True, ws=None, stream=None):
    """Allocate the gradients (and the workspace unless given) with torch and run tp_attn_flash_bwd."""
    import torch
    with _on_stream(stream):
        T, h = X.shape
        q = Wo.shape[0]
        e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=X.device)
        dQKV, dXp, dWqkv, dbqkv, dWo = e(T, 3 * q), e(T, h), e(h, 3 * q), e(3 * q), e(q, h)
        if ws is None:
            n = tp_attn_flash_bwd_workspace_bytes(batch, T // batch, h, heads, q // heads, _dtype_code(X), causal)
            ws = torch.empty((n,), dtype=torch.uint8, device=X.device)
        tp_attn_flash_bwd(dY, X, Wqkv, Wo, QKV, LSE, O, dQKV, dXp, dWqkv, dbqkv, dWo, ws, batch=batch, heads=heads,
                          causal=causal, stream=stream)
        return {"dQKV": dQKV, "dXp": dXp, "dWqkv": dWqkv, "dbqkv": dbqkv, "dWo": dWo}
