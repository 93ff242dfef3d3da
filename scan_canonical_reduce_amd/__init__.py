"""Python binding of libcanon: canonical reduce and scan on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libcanon.so`` (built in-tree by ``scan_canonical_reduce_amd.build``);
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing or a tensor is not on the GPU the calls
raise.

The C ABI is declared in ``include/canon.h``; the functions here have the
same names without the ``canon_`` prefix:

    reduce(x, L, init)                 -> 0-d tensor, init + CR_L(x)
    scan(x, policy, param=0)           -> tensor of prefix values
    reduce_rows(X, L, init)            -> 1-d tensor, one value per row
    scan_rows(X, policy, param=0)      -> tensor shaped like X
    scan_with_init(x, policy, param, kind, init)
                                       -> init + each prefix value: "inclusive",
                                          "exclusive" or "include_initial"
                                          (len(x) + 1 outputs)
    scan_rows_with_init(X, policy, param, kind, init)
    reduce_op(x, L, op, init), reduce_rows_op(X, L, op, init),
    scan_op(x, policy, param, op, kind, init), scan_rows_op(...)
                                       -> the same with op in "add", "mul",
                                          "min", "max" (IEEE minimum/maximum)

``policy`` is "pairwise", "iterated_pairwise" (param = L) or "block_dyadic"
(param = B, a power of two).

The scans wait on values published by other workgroups with a bounded spin;
if a bound were ever exceeded the kernel records an error word in its
workspace.  The scan functions read that word (``check``): by default when
they allocated the workspace themselves (the call then synchronises), and
always when ``check=True``; a caller passing ``ws`` without ``check`` reads it
with ``workspace_error(ws)`` when convenient.  A nonzero word raises
CanonError.

    scan_tile_elems(policy, param, elem_size), scan_rows_tile_elems(...)
                                       -> elements per scan tile
    set_schedule(knob, value), schedule(grid=..., reduce_partials=..., spin_limit=...)
                                       -> the schedule override (tests)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcanon.so")

POLICIES = {"pairwise": 0, "iterated_pairwise": 1, "block_dyadic": 2}
SCAN_KINDS = {"inclusive": 0, "exclusive": 1, "include_initial": 2}
OPS = {"add": 0, "mul": 1, "min": 2, "max": 3}
# the absent value of each operator (its identity)
IDENTITY = {"add": -0.0, "mul": 1.0, "min": float("inf"), "max": float("-inf")}
STATUS = {0: "CANON_OK", 1: "CANON_EINVAL", 2: "CANON_EUNSUPPORTED", 3: "CANON_EWORKSPACE",
          4: "CANON_EHIP"}

EXPORTS = [
    "canon_abi_version", "canon_status_str", "canon_last_hip_error",
    "canon_reduce_workspace_bytes", "canon_reduce_f64", "canon_reduce_f32",
    "canon_reduce_rows_workspace_bytes", "canon_reduce_rows_f64", "canon_reduce_rows_f32",
    "canon_scan_workspace_bytes", "canon_scan_f64", "canon_scan_f32",
    "canon_scan_rows_workspace_bytes", "canon_scan_rows_f64", "canon_scan_rows_f32",
    "canon_scan_with_init_f64", "canon_scan_with_init_f32",
    "canon_scan_rows_with_init_f64", "canon_scan_rows_with_init_f32",
    "canon_reduce_op_f64", "canon_reduce_op_f32", "canon_reduce_rows_op_f64",
    "canon_reduce_rows_op_f32", "canon_scan_op_f64", "canon_scan_op_f32",
    "canon_scan_rows_op_f64", "canon_scan_rows_op_f32",
    "canon_workspace_error", "canon_scan_tile_elems", "canon_scan_rows_tile_elems",
    "canon_set_schedule", "canon_get_schedule", "canon_scan_noalloc_f64",
]

ABI_VERSION = 4
SCHED = {"grid": 0, "reduce_partials": 1, "spin_limit": 2}

_lib = None


class CanonError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded libcanon.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise CanonError(f"{LIB_PATH} is missing: build it with "
                         "`python -m scan_canonical_reduce_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, S, U, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
    D, F = ctypes.c_double, ctypes.c_float
    L.canon_abi_version.restype = I
    L.canon_status_str.argtypes = [I]
    L.canon_status_str.restype = ctypes.c_char_p
    L.canon_last_hip_error.restype = I
    L.canon_reduce_workspace_bytes.argtypes = [S, U, S]
    L.canon_reduce_workspace_bytes.restype = S
    L.canon_reduce_f64.argtypes = [P, S, U, D, P, P, S, P]
    L.canon_reduce_f32.argtypes = [P, S, U, F, P, P, S, P]
    L.canon_reduce_rows_workspace_bytes.argtypes = [S, S, U, S]
    L.canon_reduce_rows_workspace_bytes.restype = S
    L.canon_reduce_rows_f64.argtypes = [P, S, S, S, U, D, P, P, S, P]
    L.canon_reduce_rows_f32.argtypes = [P, S, S, S, U, F, P, P, S, P]
    L.canon_scan_workspace_bytes.argtypes = [S, I, U, S]
    L.canon_scan_workspace_bytes.restype = S
    L.canon_scan_f64.argtypes = [P, P, S, I, U, P, S, P]
    L.canon_scan_f32.argtypes = [P, P, S, I, U, P, S, P]
    L.canon_scan_rows_workspace_bytes.argtypes = [S, S, I, U, S]
    L.canon_scan_rows_workspace_bytes.restype = S
    L.canon_scan_rows_f64.argtypes = [P, S, P, S, S, S, I, U, P, S, P]
    L.canon_scan_rows_f32.argtypes = [P, S, P, S, S, S, I, U, P, S, P]
    L.canon_scan_with_init_f64.argtypes = [P, P, S, I, U, I, D, P, S, P]
    L.canon_scan_with_init_f32.argtypes = [P, P, S, I, U, I, F, P, S, P]
    L.canon_scan_rows_with_init_f64.argtypes = [P, S, P, S, S, S, I, U, I, D, P, S, P]
    L.canon_scan_rows_with_init_f32.argtypes = [P, S, P, S, S, S, I, U, I, F, P, S, P]
    L.canon_reduce_op_f64.argtypes = [P, S, U, I, D, P, P, S, P]
    L.canon_reduce_op_f32.argtypes = [P, S, U, I, F, P, P, S, P]
    L.canon_reduce_rows_op_f64.argtypes = [P, S, S, S, U, I, D, P, P, S, P]
    L.canon_reduce_rows_op_f32.argtypes = [P, S, S, S, U, I, F, P, P, S, P]
    L.canon_scan_op_f64.argtypes = [P, P, S, I, U, I, I, D, P, S, P]
    L.canon_scan_op_f32.argtypes = [P, P, S, I, U, I, I, F, P, S, P]
    L.canon_scan_rows_op_f64.argtypes = [P, S, P, S, S, S, I, U, I, I, D, P, S, P]
    L.canon_scan_rows_op_f32.argtypes = [P, S, P, S, S, S, I, U, I, I, F, P, S, P]
    L.canon_workspace_error.argtypes = [P, ctypes.POINTER(U), P]
    L.canon_scan_tile_elems.argtypes = [I, U, S]
    L.canon_scan_tile_elems.restype = S
    L.canon_scan_rows_tile_elems.argtypes = [I, U, S]
    L.canon_scan_rows_tile_elems.restype = S
    L.canon_set_schedule.argtypes = [I, ctypes.c_uint64]
    L.canon_get_schedule.argtypes = [I]
    L.canon_get_schedule.restype = ctypes.c_uint64
    L.canon_scan_noalloc_f64.argtypes = [P, P, S, I, U, P]
    for name in EXPORTS:
        if name not in ("canon_abi_version", "canon_status_str", "canon_last_hip_error",
                        "canon_scan_tile_elems", "canon_scan_rows_tile_elems",
                        "canon_get_schedule") and not name.endswith("workspace_bytes"):
            getattr(L, name).restype = I
    if L.canon_abi_version() != ABI_VERSION:
        raise CanonError("libcanon ABI version mismatch")
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status == 0:
        return
    msg = lib().canon_status_str(status).decode()
    if status == 4:
        msg += f" (hip error {lib().canon_last_hip_error()})"
    if status in (1, 2, 3):
        raise ValueError(f"{what}: {msg}")
    raise CanonError(f"{what}: {msg}")


def _sfx(t: torch.Tensor) -> str:
    if t.dtype == torch.float64:
        return "f64"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"canonical reduce/scan take float64 or float32, not {t.dtype}")


def _need_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU path)")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _policy(p) -> int:
    if isinstance(p, str):
        return POLICIES[p]
    return int(p)


def _kind(k) -> int:
    if isinstance(k, str):
        return SCAN_KINDS[k]
    return int(k)


def _ws(nbytes: int, device, ws: torch.Tensor | None) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _check_ws(w: torch.Tensor | None, ws: torch.Tensor | None, check, what: str) -> None:
    """Reads a scan's or reduce's error word: when check is True, or when
    check is None and the workspace is the binding's own (w is not the
    caller's ws)."""
    if w is None or check is False or (check is None and w is ws):
        return
    err = workspace_error(w)
    if err != 0:
        raise CanonError(f"{what}: a bounded wait gave up (error word {err:#x}); "
                         "the output is invalid")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def reduce_workspace_bytes(n: int, L: int, elem_size: int) -> int:
    return lib().canon_reduce_workspace_bytes(n, L, elem_size)


def scan_workspace_bytes(n: int, policy, param: int, elem_size: int) -> int:
    return lib().canon_scan_workspace_bytes(n, _policy(policy), param, elem_size)


def scan_rows_workspace_bytes(rows: int, cols: int, policy, param: int, elem_size: int) -> int:
    return lib().canon_scan_rows_workspace_bytes(rows, cols, _policy(policy), param, elem_size)


def reduce(x: torch.Tensor, L: int, init: float = 0.0, out: torch.Tensor | None = None,
           ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """init + CR_L(x) as a 0-d tensor on x's device (init when x is empty).
    check: read the workspace's error word (see scan)."""
    _need_gpu(x)
    if x.dim() != 1 or (x.numel() > 0 and x.stride(0) != 1):
        raise ValueError("reduce takes a contiguous 1-d tensor")
    sfx = _sfx(x)
    if out is None:
        out = torch.empty((), dtype=x.dtype, device=x.device)
    nb = lib().canon_reduce_workspace_bytes(x.numel(), L, x.element_size())
    w = _ws(nb, x.device, ws)
    st = getattr(lib(), f"canon_reduce_{sfx}")(
        _ptr(x), x.numel(), L, float(init), out.data_ptr(), _ptr(w), nb if w is None else w.numel(),
        _stream())
    _check(st, "reduce")
    _check_ws(w, ws, check, "reduce")
    return out


def scan(x: torch.Tensor, policy="pairwise", param: int = 0, out: torch.Tensor | None = None,
         ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """Prefix values of the policy's expression; out may be x (in place)."""
    _need_gpu(x)
    if x.dim() != 1 or (x.numel() > 0 and x.stride(0) != 1):
        raise ValueError("scan takes a contiguous 1-d tensor")
    sfx = _sfx(x)
    if out is None:
        out = torch.empty_like(x)
    p = _policy(policy)
    nb = lib().canon_scan_workspace_bytes(x.numel(), p, param, x.element_size())
    w = _ws(nb, x.device, ws)
    st = getattr(lib(), f"canon_scan_{sfx}")(
        _ptr(x), out.data_ptr(), x.numel(), p, param, _ptr(w), nb if w is None else w.numel(),
        _stream())
    _check(st, "scan")
    _check_ws(w, ws, check, "scan")
    return out


def _rows_view(X: torch.Tensor):
    if X.dim() != 2 or (X.numel() > 0 and X.stride(1) != 1):
        raise ValueError("row functions take a 2-d tensor with unit column stride")
    rows, cols = X.shape
    ld = X.stride(0) if rows > 1 else max(cols, 1)
    return rows, cols, ld


def reduce_rows(X: torch.Tensor, L: int, init: float = 0.0,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """One canonical reduce per row of a 2-d tensor."""
    _need_gpu(X)
    sfx = _sfx(X)
    rows, cols, ld = _rows_view(X)
    if out is None:
        out = torch.empty(rows, dtype=X.dtype, device=X.device)
    st = getattr(lib(), f"canon_reduce_rows_{sfx}")(
        _ptr(X), rows, cols, ld, L, float(init), out.data_ptr(), None, 0, _stream())
    _check(st, "reduce_rows")
    return out


def scan_rows(X: torch.Tensor, policy="pairwise", param: int = 0,
              out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
              check: bool | None = None) -> torch.Tensor:
    """One canonical scan per row of a 2-d tensor."""
    _need_gpu(X)
    sfx = _sfx(X)
    rows, cols, ldx = _rows_view(X)
    if out is None:
        out = torch.empty((rows, cols), dtype=X.dtype, device=X.device)
    _, _, ldy = _rows_view(out)
    p = _policy(policy)
    nb = lib().canon_scan_rows_workspace_bytes(rows, cols, p, param, X.element_size())
    w = _ws(nb, X.device, ws)
    st = getattr(lib(), f"canon_scan_rows_{sfx}")(
        _ptr(X), ldx, out.data_ptr(), ldy, rows, cols, p, param, _ptr(w),
        nb if w is None else w.numel(), _stream())
    _check(st, "scan_rows")
    _check_ws(w, ws, check, "scan_rows")
    return out


def scan_with_init(x: torch.Tensor, policy="pairwise", param: int = 0, kind="inclusive",
                   init: float = -0.0, out: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """Scan with an initial value: each output is init + the policy's value on
    the prefix it observes (x[0..i] for "inclusive", x[0..i-1] for
    "exclusive" and "include_initial", init alone for the empty prefix);
    "include_initial" has len(x) + 1 outputs.  out may be x (in place; for
    include_initial a buffer of len(x) + 1 whose head is x)."""
    _need_gpu(x)
    if x.dim() != 1 or (x.numel() > 0 and x.stride(0) != 1):
        raise ValueError("scan_with_init takes a contiguous 1-d tensor")
    sfx = _sfx(x)
    k = _kind(kind)
    m = x.numel() + (1 if k == 2 else 0)
    if out is None:
        out = torch.empty(m, dtype=x.dtype, device=x.device)
    if out.dim() != 1 or out.numel() < m or (m > 0 and out.stride(0) != 1) or out.dtype != x.dtype:
        raise ValueError(f"scan_with_init: out must be a contiguous {x.dtype} tensor of {m}")
    p = _policy(policy)
    nb = lib().canon_scan_workspace_bytes(x.numel(), p, param, x.element_size())
    w = _ws(nb, x.device, ws)
    st = getattr(lib(), f"canon_scan_with_init_{sfx}")(
        _ptr(x), out.data_ptr(), x.numel(), p, param, k, float(init), _ptr(w),
        nb if w is None else w.numel(), _stream())
    _check(st, "scan_with_init")
    _check_ws(w, ws, check, "scan_with_init")
    return out


def scan_rows_with_init(X: torch.Tensor, policy="pairwise", param: int = 0, kind="inclusive",
                        init: float = -0.0, out: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None,
                        check: bool | None = None) -> torch.Tensor:
    """scan_with_init of every row of a 2-d tensor; the result has one more
    column for include_initial."""
    _need_gpu(X)
    sfx = _sfx(X)
    rows, cols, ldx = _rows_view(X)
    k = _kind(kind)
    ycols = cols + (1 if k == 2 else 0)
    if out is None:
        out = torch.empty((rows, ycols), dtype=X.dtype, device=X.device)
    if out.dim() != 2 or out.shape[0] != rows or out.shape[1] < ycols or out.dtype != X.dtype:
        raise ValueError(f"scan_rows_with_init: out must be {X.dtype} of shape ({rows}, >= {ycols})")
    _, _, ldy = _rows_view(out)
    p = _policy(policy)
    nb = lib().canon_scan_rows_workspace_bytes(rows, cols, p, param, X.element_size())
    w = _ws(nb, X.device, ws)
    st = getattr(lib(), f"canon_scan_rows_with_init_{sfx}")(
        _ptr(X), ldx, out.data_ptr(), ldy, rows, cols, p, param, k, float(init), _ptr(w),
        nb if w is None else w.numel(), _stream())
    _check(st, "scan_rows_with_init")
    _check_ws(w, ws, check, "scan_rows_with_init")
    return out


def _op(op) -> int:
    if isinstance(op, str):
        return OPS[op]
    return int(op)


def _op_init(op, init):
    name = op if isinstance(op, str) else {v: k for k, v in OPS.items()}[int(op)]
    return IDENTITY[name] if init is None else init


def reduce_op(x: torch.Tensor, L: int, op="add", init=None, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """op(init, expression of x) with the operator op; init defaults to the
    operator's identity."""
    _need_gpu(x)
    if x.dim() != 1 or (x.numel() > 0 and x.stride(0) != 1):
        raise ValueError("reduce_op takes a contiguous 1-d tensor")
    sfx = _sfx(x)
    if out is None:
        out = torch.empty((), dtype=x.dtype, device=x.device)
    nb = lib().canon_reduce_workspace_bytes(x.numel(), L, x.element_size())
    w = _ws(nb, x.device, ws)
    st = getattr(lib(), f"canon_reduce_op_{sfx}")(
        _ptr(x), x.numel(), L, _op(op), float(_op_init(op, init)), out.data_ptr(), _ptr(w),
        nb if w is None else w.numel(), _stream())
    _check(st, "reduce_op")
    _check_ws(w, ws, check, "reduce_op")
    return out


def reduce_rows_op(X: torch.Tensor, L: int, op="add", init=None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """reduce_op of every row of a 2-d tensor."""
    _need_gpu(X)
    sfx = _sfx(X)
    rows, cols, ld = _rows_view(X)
    if out is None:
        out = torch.empty(rows, dtype=X.dtype, device=X.device)
    st = getattr(lib(), f"canon_reduce_rows_op_{sfx}")(
        _ptr(X), rows, cols, ld, L, _op(op), float(_op_init(op, init)), out.data_ptr(), None, 0,
        _stream())
    _check(st, "reduce_rows_op")
    return out


def scan_op(x: torch.Tensor, policy="pairwise", param: int = 0, op="add", kind="inclusive",
            init=None, out: torch.Tensor | None = None,
            ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """scan_with_init with the operator op; init defaults to the operator's
    identity (with kind "inclusive": the plain scan)."""
    _need_gpu(x)
    if x.dim() != 1 or (x.numel() > 0 and x.stride(0) != 1):
        raise ValueError("scan_op takes a contiguous 1-d tensor")
    sfx = _sfx(x)
    k = _kind(kind)
    m = x.numel() + (1 if k == 2 else 0)
    if out is None:
        out = torch.empty(m, dtype=x.dtype, device=x.device)
    if out.dim() != 1 or out.numel() < m or (m > 0 and out.stride(0) != 1) or out.dtype != x.dtype:
        raise ValueError(f"scan_op: out must be a contiguous {x.dtype} tensor of {m}")
    p = _policy(policy)
    nb = lib().canon_scan_workspace_bytes(x.numel(), p, param, x.element_size())
    w = _ws(nb, x.device, ws)
    st = getattr(lib(), f"canon_scan_op_{sfx}")(
        _ptr(x), out.data_ptr(), x.numel(), p, param, _op(op), k, float(_op_init(op, init)),
        _ptr(w), nb if w is None else w.numel(), _stream())
    _check(st, "scan_op")
    _check_ws(w, ws, check, "scan_op")
    return out


def scan_rows_op(X: torch.Tensor, policy="pairwise", param: int = 0, op="add", kind="inclusive",
                 init=None, out: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, check: bool | None = None) -> torch.Tensor:
    """scan_op of every row of a 2-d tensor (one more column for
    include_initial)."""
    _need_gpu(X)
    sfx = _sfx(X)
    rows, cols, ldx = _rows_view(X)
    k = _kind(kind)
    ycols = cols + (1 if k == 2 else 0)
    if out is None:
        out = torch.empty((rows, ycols), dtype=X.dtype, device=X.device)
    if out.dim() != 2 or out.shape[0] != rows or out.shape[1] < ycols or out.dtype != X.dtype:
        raise ValueError(f"scan_rows_op: out must be {X.dtype} of shape ({rows}, >= {ycols})")
    _, _, ldy = _rows_view(out)
    p = _policy(policy)
    nb = lib().canon_scan_rows_workspace_bytes(rows, cols, p, param, X.element_size())
    w = _ws(nb, X.device, ws)
    st = getattr(lib(), f"canon_scan_rows_op_{sfx}")(
        _ptr(X), ldx, out.data_ptr(), ldy, rows, cols, p, param, _op(op), k,
        float(_op_init(op, init)), _ptr(w), nb if w is None else w.numel(), _stream())
    _check(st, "scan_rows_op")
    _check_ws(w, ws, check, "scan_rows_op")
    return out


def workspace_error(ws: torch.Tensor) -> int:
    """The error word a single-pass scan left in its workspace (synchronises)."""
    v = ctypes.c_uint32(0)
    _check(lib().canon_workspace_error(ws.data_ptr(), ctypes.byref(v), _stream()),
           "workspace_error")
    return v.value


def scan_tile_elems(policy, param: int, elem_size: int) -> int:
    """Elements per tile of the 1-d scans (16-byte aligned data)."""
    return lib().canon_scan_tile_elems(_policy(policy), param, elem_size)


def scan_rows_tile_elems(policy, param: int, elem_size: int) -> int:
    """Elements per tile within a row of the row scans."""
    return lib().canon_scan_rows_tile_elems(_policy(policy), param, elem_size)


def set_schedule(knob, value: int) -> None:
    """The schedule override ("grid", "reduce_partials" or "spin_limit";
    0 = default)."""
    k = SCHED[knob] if isinstance(knob, str) else int(knob)
    _check(lib().canon_set_schedule(k, int(value)), "set_schedule")


def get_schedule(knob) -> int:
    k = SCHED[knob] if isinstance(knob, str) else int(knob)
    return int(lib().canon_get_schedule(k))


class schedule:
    """Context manager: the schedule override for the calls inside it, e.g.
    ``with schedule(grid=3): ...``; the previous values are restored."""

    def __init__(self, **knobs):
        self.knobs = knobs
        self.saved = {}

    def __enter__(self):
        for k, v in self.knobs.items():
            self.saved[k] = get_schedule(k)
            set_schedule(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_schedule(k, v)
        return False
