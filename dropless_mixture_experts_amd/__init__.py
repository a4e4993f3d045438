"""Dropless mixture-of-experts (dMoE) expert layer for MI355X (gfx950).

Thin Python binding of the C ABI in ``include/dmoe.h`` (``libdmoe.so``).
It only marshals arguments: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the HIP kernels.  There is
no CPU fallback: if the library is missing, importing works but every call
raises ``DMoELibraryMissing``.

Entry points mirror the C names::

    dmoe_max_tiles(dims)            -> int
    dmoe_workspace_bytes(dims)      -> int
    dmoe_schedule_bytes(dims)       -> int
    dmoe_metadata(dims, top_experts, meta, ws)
    dmoe_forward(dims, x, weights, w1, w3, w2, meta, saved, y)
    dmoe_backward(dims, dy, weights, w1, w3, w2, meta, saved, scratch,
                  dx, dw1, dw3, dw2, d_weights)
    dmoe_padded_gather(dims, x, meta, x_perm)
    dmoe_padded_scatter(dims, src_perm, weights_or_None, meta, out)

``allocate(dims, device)`` creates every caller-owned buffer with torch, and
``DMoELayer`` / ``dmoe_autograd`` wrap the three calls for convenience.
"""
from __future__ import annotations

import ctypes
import dataclasses
import functools
import os
from typing import Optional

import torch

__all__ = [
    "DMOE_F32", "DMOE_BF16", "DMoEError", "DMoELibraryMissing", "Dims",
    "Meta", "Saved", "GradScratch", "library_path", "load_library",
    "dmoe_max_tiles", "dmoe_workspace_bytes", "dmoe_schedule_bytes",
    "dmoe_metadata", "dmoe_metadata_noalloc", "dmoe_forward",
    "dmoe_backward", "dmoe_padded_gather", "dmoe_padded_scatter",
    "dmoe_router_forward", "dmoe_router_backward", "dmoe_token_round",
    "dmoe_token_round_workspace_bytes",
    "dmoe_status_string", "allocate", "allocate_meta", "DMoELayer",
    "dmoe_autograd", "fused_gather_pays",
]

DMOE_F32 = 0
DMOE_BF16 = 1
_DTYPES = {torch.float32: DMOE_F32, torch.bfloat16: DMOE_BF16}
_TORCH = {v: k for k, v in _DTYPES.items()}

_PKG = os.path.dirname(os.path.abspath(__file__))


class DMoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {dmoe_status_string(code)} (status {code})")


class DMoELibraryMissing(ImportError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("F", ctypes.c_int64), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _Meta(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "tokens_per_expert", "bins", "padded_bins", "indices", "bin_ids",
        "row_of_entry", "tile_expert", "num_padded_rows", "status",
        "row_token", "schedule")]


class _Saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x_perm", "h1", "h3", "act", "y_perm")]


class _Scratch(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dy_perm", "dh1", "dh3", "dx_perm")]


_lib = None


def library_path() -> str:
    return os.environ.get("DMOE_LIBRARY", os.path.join(_PKG, "libdmoe.so"))


def load_library() -> ctypes.CDLL:
    """Load libdmoe.so once; raise DMoELibraryMissing if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise DMoELibraryMissing(
            f"{path} is not built; run `python -m dropless_mixture_experts_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.dmoe_max_tiles.argtypes = [P(_Dims)]
    lib.dmoe_max_tiles.restype = ctypes.c_int64
    lib.dmoe_workspace_bytes.argtypes = [P(_Dims)]
    lib.dmoe_workspace_bytes.restype = ctypes.c_int64
    lib.dmoe_schedule_bytes.argtypes = [P(_Dims)]
    lib.dmoe_schedule_bytes.restype = ctypes.c_int64
    lib.dmoe_metadata.argtypes = [P(_Dims), vp, P(_Meta), vp, vp]
    lib.dmoe_metadata.restype = ctypes.c_int
    lib.dmoe_metadata_noalloc.argtypes = [P(_Dims), vp, P(_Meta), vp]
    lib.dmoe_metadata_noalloc.restype = ctypes.c_int
    lib.dmoe_forward.argtypes = [P(_Dims), vp, vp, vp, vp, vp, P(_Meta),
                                 P(_Saved), vp, vp]
    lib.dmoe_forward.restype = ctypes.c_int
    lib.dmoe_backward.argtypes = [P(_Dims), vp, vp, vp, vp, vp, P(_Meta),
                                  P(_Saved), P(_Scratch), vp, vp, vp, vp, vp, vp]
    lib.dmoe_backward.restype = ctypes.c_int
    lib.dmoe_padded_gather.argtypes = [P(_Dims), vp, P(_Meta), vp, vp]
    lib.dmoe_padded_gather.restype = ctypes.c_int
    lib.dmoe_padded_scatter.argtypes = [P(_Dims), vp, vp, P(_Meta), vp, vp]
    lib.dmoe_padded_scatter.restype = ctypes.c_int
    lib.dmoe_metadata_timed.argtypes = [P(_Dims), vp, P(_Meta), vp, vp, vp]
    lib.dmoe_metadata_timed.restype = ctypes.c_int
    lib.dmoe_forward_timed.argtypes = [P(_Dims), vp, vp, vp, vp, vp, P(_Meta),
                                       P(_Saved), vp, vp, vp]
    lib.dmoe_forward_timed.restype = ctypes.c_int
    lib.dmoe_backward_timed.argtypes = [P(_Dims), vp, vp, vp, vp, vp, P(_Meta),
                                        P(_Saved), P(_Scratch), vp, vp, vp, vp,
                                        vp, vp, vp]
    lib.dmoe_backward_timed.restype = ctypes.c_int
    lib.dmoe_backward_recompute.argtypes = lib.dmoe_backward.argtypes
    lib.dmoe_backward_recompute.restype = ctypes.c_int
    lib.dmoe_backward_recompute_timed.argtypes = lib.dmoe_backward_timed.argtypes
    lib.dmoe_backward_recompute_timed.restype = ctypes.c_int
    lib.dmoe_forward_fused_gather.argtypes = lib.dmoe_forward.argtypes
    lib.dmoe_forward_fused_gather.restype = ctypes.c_int
    lib.dmoe_forward_fused_gather_timed.argtypes = lib.dmoe_forward_timed.argtypes
    lib.dmoe_forward_fused_gather_timed.restype = ctypes.c_int
    lib.dmoe_backward_lean.argtypes = [P(_Dims), vp] + lib.dmoe_backward.argtypes[1:]
    lib.dmoe_backward_lean.restype = ctypes.c_int
    lib.dmoe_backward_lean_timed.argtypes = [P(_Dims), vp] + lib.dmoe_backward_timed.argtypes[1:]
    lib.dmoe_backward_lean_timed.restype = ctypes.c_int
    lib.dmoe_backward_fused_gather.argtypes = [P(_Dims), vp] + lib.dmoe_backward.argtypes[1:]
    lib.dmoe_backward_fused_gather.restype = ctypes.c_int
    lib.dmoe_backward_fused_gather_timed.argtypes = ([P(_Dims), vp]
                                                     + lib.dmoe_backward_timed.argtypes[1:])
    lib.dmoe_backward_fused_gather_timed.restype = ctypes.c_int
    lib.dmoe_token_round_workspace_bytes.argtypes = [P(_Dims)]
    lib.dmoe_token_round_workspace_bytes.restype = ctypes.c_int64
    lib.dmoe_token_round.argtypes = [P(_Dims), vp, ctypes.c_int32, vp, vp, vp, vp]
    lib.dmoe_token_round.restype = ctypes.c_int
    lib.dmoe_router_forward.argtypes = [P(_Dims), vp, ctypes.c_float, vp, vp, vp, vp, vp]
    lib.dmoe_router_forward.restype = ctypes.c_int
    lib.dmoe_router_backward.argtypes = [P(_Dims), vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.dmoe_router_backward.restype = ctypes.c_int
    lib.dmoe_moa_map.argtypes = [P(_Dims), vp, vp, P(_Meta), vp, vp, vp, vp]
    lib.dmoe_moa_map.restype = ctypes.c_int
    lib.dmoe_moa_reduce.argtypes = [P(_Dims), vp, vp, vp, P(_Meta), vp, vp, vp, vp]
    lib.dmoe_moa_reduce.restype = ctypes.c_int
    lib.dmoe_moa_reduce_backward.argtypes = [P(_Dims), vp, vp, vp, P(_Meta), vp, vp, vp, vp,
                                             vp, vp, vp, vp]
    lib.dmoe_moa_reduce_backward.restype = ctypes.c_int
    lib.dmoe_moa_map_backward.argtypes = [P(_Dims), vp, vp, P(_Meta), vp, vp, vp, vp, vp, vp]
    lib.dmoe_moa_map_backward.restype = ctypes.c_int
    lib.dmoe_status_string.argtypes = [ctypes.c_int]
    lib.dmoe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


@dataclasses.dataclass(frozen=True)
class Dims:
    T: int
    H: int
    F: int
    E: int
    k: int
    dtype: int = DMOE_BF16

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH[self.dtype]

    def _c(self) -> _Dims:
        return _dims_struct(self)


@functools.lru_cache(maxsize=256)
def _dims_struct(dims: "Dims") -> _Dims:
    # the library only reads the struct, so one per dims serves every call
    return _Dims(dims.T, dims.H, dims.F, dims.E, dims.k, dims.dtype)


class _Buffers:
    """Base of the buffer sets passed to the library (Meta, Saved,
    GradScratch): their ctypes struct is built and validated once and kept
    until a field is assigned.  The tensors themselves must not be resized
    or re-pointed in place (resize_, set_) while the struct is in use."""

    def __setattr__(self, name, value):
        self.__dict__.pop("_struct", None)
        self.__dict__.pop("_checked", None)
        object.__setattr__(self, name, value)

    def _cached(self, dt, build):
        c = self.__dict__.get("_struct")
        if c is None or c[0] != dt:
            c = (dt, build())
            self.__dict__["_struct"] = c
        return c[1]


@dataclasses.dataclass
class Meta(_Buffers):
    tokens_per_expert: torch.Tensor
    bins: torch.Tensor
    padded_bins: torch.Tensor
    indices: torch.Tensor
    bin_ids: torch.Tensor
    row_of_entry: torch.Tensor
    tile_expert: torch.Tensor
    num_padded_rows: torch.Tensor
    status: torch.Tensor
    row_token: torch.Tensor
    schedule: torch.Tensor      # opaque: dmoe_schedule_bytes(dims) bytes

    def _c(self) -> _Meta:
        return self._cached(None, lambda: _Meta(*[
            _ptr(getattr(self, f.name), None if f.name == "schedule" else torch.int32, f.name)
            for f in dataclasses.fields(self)]))


@dataclasses.dataclass
class Saved(_Buffers):
    x_perm: Optional[torch.Tensor]      # may be None for the fused-gather forward
    h1: torch.Tensor
    h3: torch.Tensor
    act: torch.Tensor
    y_perm: torch.Tensor

    def _c(self, dt) -> _Saved:
        return self._cached(dt, lambda: _Saved(*[
            _ptr(getattr(self, f.name), dt, f.name) for f in dataclasses.fields(self)]))


@dataclasses.dataclass
class GradScratch(_Buffers):
    dy_perm: torch.Tensor
    dh1: torch.Tensor
    dh3: torch.Tensor
    dx_perm: torch.Tensor

    def _c(self, dt) -> _Scratch:
        return self._cached(dt, lambda: _Scratch(*[
            _ptr(getattr(self, f.name), dt, f.name) for f in dataclasses.fields(self)]))


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, numel: int):
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream")
                           else int(stream))


def _check(code: int, where: str):
    if code != 0:
        raise DMoEError(code, where)


def dmoe_status_string(code: int) -> str:
    try:
        return load_library().dmoe_status_string(int(code)).decode()
    except DMoELibraryMissing:
        return f"status {code}"


@functools.lru_cache(maxsize=256)
def _sizes(dims: Dims):
    """(max_tiles, workspace bytes, schedule bytes) of dims, from the library
    (cached: these depend on the sizes only)."""
    lib = load_library()
    d = dims._c()
    out = []
    for fn, name in ((lib.dmoe_max_tiles, "dmoe_max_tiles"),
                     (lib.dmoe_workspace_bytes, "dmoe_workspace_bytes"),
                     (lib.dmoe_schedule_bytes, "dmoe_schedule_bytes")):
        v = fn(ctypes.byref(d))
        _check(v if v < 0 else 0, name)
        out.append(int(v))
    return tuple(out)


def dmoe_max_tiles(dims: Dims) -> int:
    return _sizes(dims)[0]


def dmoe_workspace_bytes(dims: Dims) -> int:
    return _sizes(dims)[1]


def dmoe_schedule_bytes(dims: Dims) -> int:
    return _sizes(dims)[2]


def _check_meta(dims: Dims, meta: Meta):
    # once per dims until a field of meta is assigned
    if meta.__dict__.get("_checked") == dims:
        return
    n = dims.T * dims.k
    nt, _, sb = _sizes(dims)
    for name, size in (("tokens_per_expert", dims.E), ("bins", dims.E),
                       ("padded_bins", dims.E), ("indices", n), ("bin_ids", n),
                       ("row_of_entry", n), ("tile_expert", nt),
                       ("num_padded_rows", 1), ("status", 1),
                       ("row_token", 128 * nt)):
        _need(getattr(meta, name), name, size)
    s = meta.schedule
    if s.numel() * s.element_size() < sb:
        raise ValueError(f"schedule: needs at least {sb} bytes, has "
                         f"{s.numel() * s.element_size()}")
    meta.__dict__["_checked"] = dims


def _ev(events, n):
    """None, or an EventArray of at least n+1 events (see hip_events)."""
    if events is None:
        return None
    if len(events) < n + 1:
        raise ValueError(f"timing needs {n + 1} events, got {len(events)}")
    return events.pointer()


def dmoe_metadata(dims: Dims, top_experts: torch.Tensor, meta: Meta,
                  ws: torch.Tensor, stream=None, events=None) -> None:
    """Routing metadata; see include/dmoe.h.  `events`: optional EventArray
    of 4 events for per-kernel timing (dmoe_metadata_timed)."""
    lib = load_library()
    _need(top_experts, "top_experts", dims.T * dims.k)
    _check_meta(dims, meta)
    _need(ws, "ws", dmoe_workspace_bytes(dims) // ws.element_size())
    args = (ctypes.byref(dims._c()), _ptr(top_experts, torch.int32, "top_experts"),
            ctypes.byref(meta._c()), _ptr(ws, None, "ws"), _stream(top_experts, stream))
    if events is None:
        _check(lib.dmoe_metadata(*args), "dmoe_metadata")
    else:
        _check(lib.dmoe_metadata_timed(*args, _ev(events, 3)), "dmoe_metadata_timed")


def dmoe_metadata_noalloc(dims: Dims, top_experts: torch.Tensor, meta: Meta,
                          stream=None) -> None:
    """dmoe_metadata with its workspace in the library's own device array
    (no ws argument, nothing allocated); see include/dmoe.h for the limit
    and for calls that overlap on one GPU."""
    lib = load_library()
    _need(top_experts, "top_experts", dims.T * dims.k)
    _check_meta(dims, meta)
    _check(lib.dmoe_metadata_noalloc(ctypes.byref(dims._c()),
                                     _ptr(top_experts, torch.int32, "top_experts"),
                                     ctypes.byref(meta._c()), _stream(top_experts, stream)),
           "dmoe_metadata_noalloc")


def _pmax(dims: Dims) -> int:
    return 128 * dmoe_max_tiles(dims)


def dmoe_forward(dims: Dims, x, weights, w1, w3, w2, meta: Meta, saved: Saved,
                 y, stream=None, events=None, fused_gather: bool = False) -> None:
    """Forward of the layer; see include/dmoe.h.  `events`: optional
    EventArray of 5 events (4 with fused_gather) for per-kernel timing.
    fused_gather: the up projection reads token rows of x directly
    (dmoe_forward_fused_gather); saved.x_perm may be None."""
    lib = load_library()
    dt = dims.torch_dtype
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    pm = _pmax(dims)
    need = [(x, "x", T * H), (weights, "weights", T * k),
            (w1, "w1", E * H * F), (w3, "w3", E * H * F),
            (w2, "w2", E * F * H), (y, "y", T * H), (saved.h1, "h1", pm * F),
            (saved.h3, "h3", pm * F), (saved.act, "act", pm * F),
            (saved.y_perm, "y_perm", pm * H)]
    if not fused_gather:
        need.append((saved.x_perm, "x_perm", pm * H))
    for t, n, s in need:
        _need(t, n, s)
    _check_meta(dims, meta)
    args = (ctypes.byref(dims._c()), _ptr(x, dt, "x"),
            _ptr(weights, torch.float32, "weights"), _ptr(w1, dt, "w1"),
            _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), ctypes.byref(meta._c()),
            ctypes.byref(saved._c(dt)), _ptr(y, dt, "y"), _stream(x, stream))
    name = "dmoe_forward_fused_gather" if fused_gather else "dmoe_forward"
    if events is None:
        _check(getattr(lib, name)(*args), name)
    else:
        _check(getattr(lib, name + "_timed")(*args, _ev(events, 3 if fused_gather else 4)),
               name + "_timed")


def dmoe_backward(dims: Dims, dy, weights, w1, w3, w2, meta: Meta, saved: Saved,
                  scratch: GradScratch, dx, dw1, dw3, dw2, d_weights,
                  stream=None, events=None, recompute: bool = False,
                  x=None, lean: bool = False) -> None:
    """Backward of the layer; see include/dmoe.h.  `events`: optional
    EventArray of 6 events (7 with recompute or x, 8 with lean) for
    per-kernel timing.  recompute: saved.act is scratch on entry and is
    rebuilt from h1 and h3 (dmoe_backward_recompute).  x: the forward's
    input; alone, after the fused-gather forward (dmoe_backward_fused_gather):
    saved.x_perm is then scratch on entry and is gathered from x first.
    lean (needs x): saved.x_perm, h1, h3 and act are all scratch on entry and
    are rebuilt from x (dmoe_backward_lean); only saved.y_perm is kept."""
    if x is not None and recompute:
        raise ValueError("the fused gather has no recompute variant")
    if lean and (x is None or recompute):
        raise ValueError("lean needs the forward's x and excludes recompute")
    lib = load_library()
    dt = dims.torch_dtype
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    pm = _pmax(dims)
    for t, n, s in ((dy, "dy", T * H), (weights, "weights", T * k),
                    (w1, "w1", E * H * F), (w3, "w3", E * H * F),
                    (w2, "w2", E * F * H), (dx, "dx", T * H),
                    (dw1, "dw1", E * H * F), (dw3, "dw3", E * H * F),
                    (dw2, "dw2", E * F * H), (d_weights, "d_weights", T * k),
                    (saved.x_perm, "x_perm", pm * H),
                    (scratch.dy_perm, "dy_perm", pm * H),
                    (scratch.dh1, "dh1", pm * F), (scratch.dh3, "dh3", pm * F),
                    (scratch.dx_perm, "dx_perm", pm * H)):
        _need(t, n, s)
    _check_meta(dims, meta)
    args = [ctypes.byref(dims._c()), _ptr(dy, dt, "dy"),
            _ptr(weights, torch.float32, "weights"), _ptr(w1, dt, "w1"),
            _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), ctypes.byref(meta._c()),
            ctypes.byref(saved._c(dt)), ctypes.byref(scratch._c(dt)),
            _ptr(dx, dt, "dx"), _ptr(dw1, dt, "dw1"), _ptr(dw3, dt, "dw3"),
            _ptr(dw2, dt, "dw2"), _ptr(d_weights, torch.float32, "d_weights"),
            _stream(dy, stream)]
    if x is not None:
        _need(x, "x", T * H)
        name = "dmoe_backward_lean" if lean else "dmoe_backward_fused_gather"
        args.insert(1, _ptr(x, dt, "x"))
    elif recompute:
        name = "dmoe_backward_recompute"
    else:
        name = "dmoe_backward"
    if events is None:
        _check(getattr(lib, name)(*args), name)
    else:
        _check(getattr(lib, name + "_timed")(
            *args, _ev(events, 7 if lean else 6 if recompute or x is not None else 5)),
            name + "_timed")


def dmoe_padded_gather(dims: Dims, x, meta: Meta, x_perm, stream=None) -> None:
    """padded_gather alone; see include/dmoe.h."""
    lib = load_library()
    dt = dims.torch_dtype
    _need(x, "x", dims.T * dims.H)
    _need(x_perm, "x_perm", _pmax(dims) * dims.H)
    _check_meta(dims, meta)
    _check(lib.dmoe_padded_gather(ctypes.byref(dims._c()), _ptr(x, dt, "x"),
                                  ctypes.byref(meta._c()), _ptr(x_perm, dt, "x_perm"),
                                  _stream(x, stream)), "dmoe_padded_gather")


def dmoe_padded_scatter(dims: Dims, src_perm, weights, meta: Meta, out,
                        stream=None) -> None:
    """padded_scatter alone (weights=None: unit weights); see include/dmoe.h."""
    lib = load_library()
    dt = dims.torch_dtype
    _need(src_perm, "src_perm", _pmax(dims) * dims.H)
    _need(out, "out", dims.T * dims.H)
    if weights is not None:
        _need(weights, "weights", dims.T * dims.k)
    _check_meta(dims, meta)
    _check(lib.dmoe_padded_scatter(
        ctypes.byref(dims._c()), _ptr(src_perm, dt, "src_perm"),
        _ptr(weights, torch.float32, "weights"), ctypes.byref(meta._c()),
        _ptr(out, dt, "out"), _stream(out, stream)), "dmoe_padded_scatter")


def dmoe_router_forward(dims: Dims, logits, top_experts, weights, zloss_coef: float = 0.0,
                        z=None, zloss=None, stream=None) -> None:
    """Top-k + softmax over the chosen logits (+ z-loss); see include/dmoe.h.

    logits [T,E] fp32; writes top_experts [T,k] int32 and weights [T,k] fp32,
    and with zloss_coef != 0 also z [T] and zloss [1] (fp32)."""
    lib = load_library()
    _need(logits, "logits", dims.T * dims.E)
    _need(top_experts, "top_experts", dims.T * dims.k)
    _need(weights, "weights", dims.T * dims.k)
    if zloss_coef != 0.0:
        if z is None or zloss is None:
            raise ValueError("zloss_coef != 0 needs z and zloss")
        _need(z, "z", dims.T)
        _need(zloss, "zloss", 1)
    _check(lib.dmoe_router_forward(
        ctypes.byref(dims._c()), _ptr(logits, torch.float32, "logits"),
        ctypes.c_float(zloss_coef), _ptr(top_experts, torch.int32, "top_experts"),
        _ptr(weights, torch.float32, "weights"), _ptr(z, torch.float32, "z"),
        _ptr(zloss, torch.float32, "zloss"), _stream(logits, stream)),
        "dmoe_router_forward")


def dmoe_token_round_workspace_bytes(dims: Dims) -> int:
    v = load_library().dmoe_token_round_workspace_bytes(ctypes.byref(dims._c()))
    _check(v if v < 0 else 0, "dmoe_token_round_workspace_bytes")
    return int(v)


def dmoe_token_round(dims: Dims, logits, top_experts, weights, ws, tile_rows: int = 128,
                     stream=None) -> None:
    """Tile-aware token rounding of the top-k routing; see include/dmoe.h.

    logits [T,E] fp32; dims.k = k routed slots (k < E); writes top_experts
    [T,k+1] int32 (-1 for an empty slot) and weights [T,k+1] fp32.  The
    layer then runs on these slots with Dims(..., k=k+1)."""
    lib = load_library()
    k1 = dims.k + 1
    _need(logits, "logits", dims.T * dims.E)
    _need(top_experts, "top_experts", dims.T * k1)
    _need(weights, "weights", dims.T * k1)
    _need(ws, "ws", dmoe_token_round_workspace_bytes(dims) // ws.element_size())
    _check(lib.dmoe_token_round(
        ctypes.byref(dims._c()), _ptr(logits, torch.float32, "logits"), ctypes.c_int32(tile_rows),
        _ptr(top_experts, torch.int32, "top_experts"), _ptr(weights, torch.float32, "weights"),
        _ptr(ws, None, "ws"), _stream(logits, stream)), "dmoe_token_round")


# --------------------------------------------------------------------------
# dMoA: the map / reduce pair of mixture of attention heads (bf16)
# --------------------------------------------------------------------------

def dmoe_moa_map(dims: Dims, x, w1, meta: Meta, x_perm, q_perm, q, stream=None) -> None:
    """q [T*k, F] = x[t] @ w1[e] per routed slot; x_perm [P_max, H] is kept
    for the backward.  See include/dmoe.h."""
    lib = load_library()
    dt, pm = dims.torch_dtype, _pmax(dims)
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    for t, n, sz in ((x, "x", T * H), (w1, "w1", E * H * F), (x_perm, "x_perm", pm * H),
                     (q_perm, "q_perm", pm * F), (q, "q", T * k * F)):
        _need(t, n, sz)
    _check_meta(dims, meta)
    _check(lib.dmoe_moa_map(ctypes.byref(dims._c()), _ptr(x, dt, "x"), _ptr(w1, dt, "w1"),
                            ctypes.byref(meta._c()), _ptr(x_perm, dt, "x_perm"),
                            _ptr(q_perm, dt, "q_perm"), _ptr(q, dt, "q"), _stream(x, stream)),
           "dmoe_moa_map")


def dmoe_moa_reduce(dims: Dims, y, weights, w2, meta: Meta, y_perm, o_perm, out,
                    stream=None) -> None:
    """out [T, H] = sum_j weights[t, j] * y[t*k+j] @ w2[e]; y_perm and o_perm
    are kept for the backward.  See include/dmoe.h."""
    lib = load_library()
    dt, pm = dims.torch_dtype, _pmax(dims)
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    for t, n, sz in ((y, "y", T * k * F), (weights, "weights", T * k), (w2, "w2", E * F * H),
                     (y_perm, "y_perm", pm * F), (o_perm, "o_perm", pm * H),
                     (out, "out", T * H)):
        _need(t, n, sz)
    _check_meta(dims, meta)
    _check(lib.dmoe_moa_reduce(ctypes.byref(dims._c()), _ptr(y, dt, "y"),
                               _ptr(weights, torch.float32, "weights"), _ptr(w2, dt, "w2"),
                               ctypes.byref(meta._c()), _ptr(y_perm, dt, "y_perm"),
                               _ptr(o_perm, dt, "o_perm"), _ptr(out, dt, "out"),
                               _stream(y, stream)), "dmoe_moa_reduce")


def dmoe_moa_reduce_backward(dims: Dims, dout, weights, w2, meta: Meta, y_perm, o_perm,
                             do_perm, dy_perm, dy, dw2, d_weights, stream=None) -> None:
    """Gradients of dmoe_moa_reduce; see include/dmoe.h."""
    lib = load_library()
    dt, pm = dims.torch_dtype, _pmax(dims)
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    for t, n, sz in ((dout, "dout", T * H), (weights, "weights", T * k),
                     (w2, "w2", E * F * H), (y_perm, "y_perm", pm * F),
                     (o_perm, "o_perm", pm * H), (do_perm, "do_perm", pm * H),
                     (dy_perm, "dy_perm", pm * F), (dy, "dy", T * k * F),
                     (dw2, "dw2", E * F * H), (d_weights, "d_weights", T * k)):
        _need(t, n, sz)
    _check_meta(dims, meta)
    _check(lib.dmoe_moa_reduce_backward(
        ctypes.byref(dims._c()), _ptr(dout, dt, "dout"), _ptr(weights, torch.float32, "weights"),
        _ptr(w2, dt, "w2"), ctypes.byref(meta._c()), _ptr(y_perm, dt, "y_perm"),
        _ptr(o_perm, dt, "o_perm"), _ptr(do_perm, dt, "do_perm"), _ptr(dy_perm, dt, "dy_perm"),
        _ptr(dy, dt, "dy"), _ptr(dw2, dt, "dw2"), _ptr(d_weights, torch.float32, "d_weights"),
        _stream(dout, stream)), "dmoe_moa_reduce_backward")


def dmoe_moa_map_backward(dims: Dims, dq, w1, meta: Meta, x_perm, dq_perm, dx_perm, dx, dw1,
                          stream=None) -> None:
    """Gradients of dmoe_moa_map; see include/dmoe.h."""
    lib = load_library()
    dt, pm = dims.torch_dtype, _pmax(dims)
    T, H, F, E, k = dims.T, dims.H, dims.F, dims.E, dims.k
    for t, n, sz in ((dq, "dq", T * k * F), (w1, "w1", E * H * F), (x_perm, "x_perm", pm * H),
                     (dq_perm, "dq_perm", pm * F), (dx_perm, "dx_perm", pm * H),
                     (dx, "dx", T * H), (dw1, "dw1", E * H * F)):
        _need(t, n, sz)
    _check_meta(dims, meta)
    _check(lib.dmoe_moa_map_backward(
        ctypes.byref(dims._c()), _ptr(dq, dt, "dq"), _ptr(w1, dt, "w1"), ctypes.byref(meta._c()),
        _ptr(x_perm, dt, "x_perm"), _ptr(dq_perm, dt, "dq_perm"), _ptr(dx_perm, dt, "dx_perm"),
        _ptr(dx, dt, "dx"), _ptr(dw1, dt, "dw1"), _stream(dq, stream)), "dmoe_moa_map_backward")


class DMoALayer:
    """map / reduce of mixture of attention heads on preallocated buffers:
    metadata(top_experts), then map(x), attention outside, reduce(y), and
    their backward in reverse (reduce_backward, then map_backward)."""

    def __init__(self, dims: Dims, device="cuda"):
        if dims.dtype != DMOE_BF16:
            raise DMoEError(-3, "DMoALayer (bf16 only)")
        self.dims = dims
        self.device = torch.device(device)
        self.meta, self.ws = allocate_meta(dims, device)
        pm = _pmax(dims)
        fl = dict(dtype=dims.torch_dtype, device=device)
        H, F = dims.H, dims.F
        self.x_perm = torch.empty(pm, H, **fl)
        self.y_perm = torch.empty(pm, F, **fl)
        self.o_perm = torch.empty(pm, H, **fl)
        self.perm_f = torch.empty(pm, F, **fl)     # q_perm, dy_perm, dq_perm (scratch)
        self.perm_h = torch.empty(pm, H, **fl)     # do_perm, dx_perm (scratch)

    def metadata(self, top_experts, stream=None):
        dmoe_metadata(self.dims, top_experts, self.meta, self.ws, stream)

    def map(self, x, w1, stream=None):
        d = self.dims
        q = torch.empty(d.T * d.k, d.F, dtype=d.torch_dtype, device=self.device)
        dmoe_moa_map(d, x, w1, self.meta, self.x_perm, self.perm_f, q, stream)
        return q

    def reduce(self, y, weights, w2, stream=None):
        d = self.dims
        out = torch.empty(d.T, d.H, dtype=d.torch_dtype, device=self.device)
        dmoe_moa_reduce(d, y, weights, w2, self.meta, self.y_perm, self.o_perm, out, stream)
        return out

    def reduce_backward(self, dout, weights, w2, stream=None):
        d = self.dims
        fl = dict(dtype=d.torch_dtype, device=self.device)
        dy = torch.empty(d.T * d.k, d.F, **fl)
        dw2 = torch.empty(d.E, d.F, d.H, **fl)
        dwt = torch.empty(d.T, d.k, dtype=torch.float32, device=self.device)
        dmoe_moa_reduce_backward(d, dout, weights, w2, self.meta, self.y_perm, self.o_perm,
                                 self.perm_h, self.perm_f, dy, dw2, dwt, stream)
        return dy, dw2, dwt

    def map_backward(self, dq, w1, stream=None):
        d = self.dims
        fl = dict(dtype=d.torch_dtype, device=self.device)
        dx = torch.empty(d.T, d.H, **fl)
        dw1 = torch.empty(d.E, d.H, d.F, **fl)
        dmoe_moa_map_backward(d, dq, w1, self.meta, self.x_perm, self.perm_f, self.perm_h,
                              dx, dw1, stream)
        return dx, dw1


def dmoe_router_backward(dims: Dims, logits, top_experts, weights, d_weights, d_logits,
                         zloss_coef: float = 0.0, stream=None) -> None:
    """d_logits [T,E] fp32 from d_weights [T,k] (+ the z-loss's); see include/dmoe.h."""
    lib = load_library()
    _need(logits, "logits", dims.T * dims.E)
    _need(d_logits, "d_logits", dims.T * dims.E)
    for t, n in ((top_experts, "top_experts"), (weights, "weights"), (d_weights, "d_weights")):
        _need(t, n, dims.T * dims.k)
    _check(lib.dmoe_router_backward(
        ctypes.byref(dims._c()), _ptr(logits, torch.float32, "logits"),
        _ptr(top_experts, torch.int32, "top_experts"), _ptr(weights, torch.float32, "weights"),
        _ptr(d_weights, torch.float32, "d_weights"), ctypes.c_float(zloss_coef),
        _ptr(d_logits, torch.float32, "d_logits"), _stream(logits, stream)),
        "dmoe_router_backward")


# --------------------------------------------------------------------------
# Buffer plumbing (torch allocates; the library never does)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Buffers:
    dims: Dims
    meta: Meta
    ws: torch.Tensor
    saved: Saved
    scratch: Optional[GradScratch]


def allocate_meta(dims: Dims, device):
    """The metadata arrays and the metadata workspace for `dims`."""
    n, E = dims.T * dims.k, dims.E
    nt, ws_bytes, sched_bytes = _sizes(dims)
    i32 = dict(dtype=torch.int32, device=device)
    meta = Meta(torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(E, **i32),
                torch.empty(n, **i32), torch.empty(n, **i32), torch.empty(n, **i32),
                torch.empty(nt, **i32), torch.empty(1, **i32), torch.empty(1, **i32),
                torch.empty(128 * nt, **i32),
                torch.empty(sched_bytes, dtype=torch.uint8, device=device))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    return meta, ws


def allocate(dims: Dims, device, with_backward: bool = True,
             lean: bool = False) -> Buffers:
    """Allocate every caller-owned buffer for `dims` on `device`.

    lean=True lets the backward scratch alias the saved activations where
    include/dmoe.h permits it (dh1 -> h1, dh3 -> h3, dx_perm -> dy_perm)."""
    pm = 128 * dmoe_max_tiles(dims)
    meta, ws = allocate_meta(dims, device)
    fl = dict(dtype=dims.torch_dtype, device=device)
    saved = Saved(torch.empty(pm, dims.H, **fl), torch.empty(pm, dims.F, **fl),
                  torch.empty(pm, dims.F, **fl), torch.empty(pm, dims.F, **fl),
                  torch.empty(pm, dims.H, **fl))
    scratch = None
    if with_backward:
        dyp = torch.empty(pm, dims.H, **fl)
        if lean:
            scratch = GradScratch(dyp, saved.h1, saved.h3, dyp)
        else:
            scratch = GradScratch(dyp, torch.empty(pm, dims.F, **fl),
                                  torch.empty(pm, dims.F, **fl),
                                  torch.empty(pm, dims.H, **fl))
    return Buffers(dims, meta, ws, saved, scratch)


# Last-level cache (MALL) of MI355X.  A padded copy of x larger than this
# is read back by the up projection from HBM, where the T token rows of x
# (each read by its k entries) would stay in the cache.
LLC_BYTES = 256 << 20


def fused_gather_pays(dims: Dims) -> bool:
    """Whether to fuse the gather into the up projection for these dims:
    bf16 (the only dtype the fused entry points take), x under 2 GB (their
    limit), and a padded copy of x that would not fit the last-level cache.
    Measured on MI355X: 1.7% off the step of the T=16384, H=1536, E=256
    layer (449 MB padded copy); level at T=4096, H=2048, E=64 (150 MB)."""
    if dims.dtype != DMOE_BF16 or dims.T * dims.H * 2 >= (1 << 31):
        return False
    return dmoe_max_tiles(dims) * 128 * dims.H * 2 > LLC_BYTES


class DMoELayer:
    """Runs metadata + forward + backward on preallocated buffers.

    fused_gather=True (bf16): the forward's up projection reads token rows
    of x directly and writes no x_perm; the backward gathers x_perm from x
    first, so the x given to forward must be unchanged until backward.
    fused_gather="auto": fused when fused_gather_pays(dims)."""

    def __init__(self, dims: Dims, device="cuda", lean: bool = False,
                 fused_gather=False):
        self.dims = dims
        if fused_gather == "auto":
            fused_gather = fused_gather_pays(dims)
        self.fused_gather = bool(fused_gather)
        self.buf = allocate(dims, device, True, lean)
        self.device = torch.device(device)
        self._x = None

    def metadata(self, top_experts, stream=None, events=None):
        dmoe_metadata(self.dims, top_experts, self.buf.meta, self.buf.ws, stream,
                      events)

    def forward(self, x, top_experts, weights, w1, w3, w2, y=None,
                stream=None, run_metadata=True, events=None):
        if run_metadata:
            self.metadata(top_experts, stream)
        if y is None:
            y = torch.empty(self.dims.T, self.dims.H, dtype=self.dims.torch_dtype,
                            device=self.device)
        dmoe_forward(self.dims, x, weights, w1, w3, w2, self.buf.meta,
                     self.buf.saved, y, stream, events, self.fused_gather)
        self._x = x
        return y

    def backward(self, dy, weights, w1, w3, w2, grads=None, stream=None,
                 events=None, recompute=False, lean=False):
        """lean: rebuild x_perm, h1, h3 and act from the forward's x
        (dmoe_backward_lean) instead of reading them."""
        d = self.dims
        if grads is None:
            fl = dict(dtype=d.torch_dtype, device=self.device)
            grads = dict(dx=torch.empty(d.T, d.H, **fl),
                         dw1=torch.empty(d.E, d.H, d.F, **fl),
                         dw3=torch.empty(d.E, d.H, d.F, **fl),
                         dw2=torch.empty(d.E, d.F, d.H, **fl),
                         d_weights=torch.empty(d.T, d.k, dtype=torch.float32,
                                               device=self.device))
        if (self.fused_gather or lean) and self._x is None:
            raise RuntimeError("backward needs the forward's x: run forward first")
        dmoe_backward(d, dy, weights, w1, w3, w2, self.buf.meta, self.buf.saved,
                      self.buf.scratch, grads["dx"], grads["dw1"], grads["dw3"],
                      grads["dw2"], grads["d_weights"], stream, events, recompute,
                      self._x if (self.fused_gather or lean) else None, lean)
        return grads


class _DMoEFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, top_experts, weights, w1, w3, w2):
        T, H = x.shape
        E, _, F = w1.shape
        dims = Dims(T, H, F, E, top_experts.shape[1], _DTYPES[x.dtype])
        layer = DMoELayer(dims, x.device)
        args = [a.contiguous() for a in (x, top_experts.to(torch.int32),
                                         weights.float(), w1, w3, w2)]
        y = layer.forward(*args)
        ctx.layer = layer
        ctx.save_for_backward(*args[2:])
        return y

    @staticmethod
    def backward(ctx, dy):
        weights, w1, w3, w2 = ctx.saved_tensors
        g = ctx.layer.backward(dy.contiguous(), weights, w1, w3, w2)
        return g["dx"], None, g["d_weights"], g["dw1"], g["dw3"], g["dw2"]


def dmoe_autograd(x, top_experts, weights, w1, w3, w2):
    """y = dMoE(x) with autograd support (gradients for x, weights, w1/w3/w2)."""
    return _DMoEFunction.apply(x, top_experts, weights, w1, w3, w2)
