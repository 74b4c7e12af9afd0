"""Python binding of the MI355X sparse MoE layer library (libstrata_moe.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  There is
no fallback: if the shared library is missing or a call fails, an error is
raised.

The C ABI is declared in include/strata_moe.h; the names here mirror it:
``workspace_bytes``, ``route``, ``forward``, ``kernel_names``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstrata_moe.so")

STRATA_OK, STRATA_EINVAL, STRATA_EUNSUPPORTED, STRATA_EWORKSPACE, STRATA_EHIP = range(5)
X_BF16, X_F32 = 0, 1
NORM_FIRST = 1


class StrataError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"strata_moe status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("bits", ctypes.c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("resident_mask", ctypes.c_void_p), ("bits", ctypes.c_int32)]


class HostLayer(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("bits", ctypes.c_int32)]


class RouteOut(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libstrata_moe.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_routed_expert_amd.build`")
    try:  # bind to the HIP runtime torch has loaded (same SONAME), so streams are shared
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.strata_moe_workspace_bytes.restype = sz
    lib.strata_moe_workspace_bytes.argtypes = [ctypes.POINTER(Shape), i32, i32]
    lib.strata_moe_route.restype = ctypes.c_int
    lib.strata_moe_route.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layer), vp, ctypes.c_int, i32,
                                     ctypes.POINTER(RouteOut), vp, sz, vp]
    lib.strata_moe_forward.restype = ctypes.c_int
    lib.strata_moe_forward.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layer), i32, vp, ctypes.c_int, i32,
                                       ctypes.c_uint32, vp, vp, ctypes.POINTER(RouteOut), vp, vp, i32, vp, vp, sz,
                                       ctypes.POINTER(ctypes.c_void_p), i32, vp]
    lib.strata_moe_forward_noalloc.restype = ctypes.c_int
    lib.strata_moe_forward_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layer), i32, vp, ctypes.c_int,
                                               i32, ctypes.c_uint32, vp, vp, ctypes.POINTER(RouteOut), vp, vp, i32,
                                               vp, ctypes.POINTER(ctypes.c_void_p), i32, vp]
    lib.strata_moe_host_workspace_bytes.restype = sz
    lib.strata_moe_host_workspace_bytes.argtypes = [ctypes.POINTER(Shape), i32, i32]
    lib.strata_moe_host_isa.restype = ctypes.c_char_p
    lib.strata_moe_host_isa.argtypes = []
    lib.strata_moe_host_misses.restype = ctypes.c_int
    lib.strata_moe_host_misses.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(HostLayer), vp, i32, vp, vp, i32, vp,
                                           vp, sz, i32]
    lib.strata_moe_forward_coprocess.restype = ctypes.c_int
    lib.strata_moe_forward_coprocess.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Layer),
                                                 ctypes.POINTER(HostLayer), i32, vp, ctypes.c_int, i32,
                                                 ctypes.c_uint32, vp, vp, ctypes.POINTER(RouteOut), vp, vp, i32, vp,
                                                 vp, sz, vp, sz, i32, vp, vp]
    lib.strata_moe_counts_accumulate.restype = ctypes.c_int
    lib.strata_moe_counts_accumulate.argtypes = [vp, vp, i32, vp]
    lib.strata_moe_resident_topn.restype = ctypes.c_int
    lib.strata_moe_resident_topn.argtypes = [vp, i32, i32, vp, vp]
    lib.strata_moe_kernel_names.restype = i32
    lib.strata_moe_kernel_names.argtypes = [ctypes.POINTER(Shape), i32, i32, ctypes.POINTER(ctypes.c_char_p), i32]
    lib.strata_status_str.restype = ctypes.c_char_p
    lib.strata_status_str.argtypes = [ctypes.c_int]
    lib.strata_probe_hbm_read.restype = ctypes.c_int
    lib.strata_probe_hbm_read.argtypes = [vp, sz, vp, i32, vp]
    lib.strata_probe_mfma_bf16.restype = ctypes.c_int
    lib.strata_probe_mfma_bf16.argtypes = [i32, vp, i32, ctypes.POINTER(ctypes.c_double), vp]
    _lib = lib
    return lib


EXPORTED_SYMBOLS = ("strata_moe_workspace_bytes", "strata_moe_route", "strata_moe_forward",
                    "strata_moe_counts_accumulate", "strata_moe_resident_topn", "strata_moe_kernel_names",
                    "strata_status_str", "strata_probe_hbm_read", "strata_probe_mfma_bf16",
                    "strata_moe_forward_noalloc", "strata_moe_host_workspace_bytes", "strata_moe_host_isa",
                    "strata_moe_host_misses", "strata_moe_forward_coprocess")

NOALLOC_SCRATCH_BYTES = 64 << 20   # STRATA_NOALLOC_SCRATCH_BYTES


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(status: int):
    if status != STRATA_OK:
        msg = load_library().strata_status_str(status).decode()
        raise StrataError(status, msg)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


@dataclass
class LayerData:
    """Device tensors of one layer (torch tensors or raw device addresses)."""
    router_w: object
    codes: object
    scales: object
    router_bias: object = None
    resident_mask: object = None
    bits: int = 0   # this layer's code width (3 or 2); 0 = the shape's

    def as_c(self) -> Layer:
        return Layer(_ptr(self.router_w), _ptr(self.router_bias), _ptr(self.codes), _ptr(self.scales),
                     _ptr(self.resident_mask), int(self.bits))


def shape(n_experts: int, top_k: int, d_model: int, d_ff: int, bits: int, n_shared: int = 1) -> Shape:
    return Shape(n_experts, top_k, n_shared, d_model, d_ff, bits)


def workspace_bytes(sh: Shape, T: int, L: int = 1) -> int:
    n = load_library().strata_moe_workspace_bytes(ctypes.byref(sh), T, L)
    if n == 0:
        raise StrataError(STRATA_EINVAL, "unsupported shape")
    return n


def kernel_names(sh: Shape, T: int, L: int = 1) -> list:
    """Kernel groups of an L-layer forward call with T tokens, in launch order."""
    lib = load_library()
    n = lib.strata_moe_kernel_names(ctypes.byref(sh), T, L, None, 0)
    arr = (ctypes.c_char_p * max(n, 1))()
    n = lib.strata_moe_kernel_names(ctypes.byref(sh), T, L, arr, n)
    return [arr[i].decode() for i in range(n)]


def _route_out(ro: Optional[dict]) -> Optional[RouteOut]:
    if ro is None:
        return None
    return RouteOut(_ptr(ro.get("topk_idx")), _ptr(ro.get("topk_w")), _ptr(ro.get("counts")),
                    _ptr(ro.get("offsets")), _ptr(ro.get("perm")), _ptr(ro.get("pos")))


def route(sh: Shape, layer: LayerData, x, xdtype: int, T: int, out: dict, ws, ws_bytes: int, stream=None):
    """Routing of one layer; `out` maps RouteOut field names to device tensors."""
    lib = load_library()
    ro = _route_out(out)
    _check(lib.strata_moe_route(ctypes.byref(sh), ctypes.byref(layer.as_c()), _ptr(x), xdtype, T,
                                ctypes.byref(ro) if ro is not None else None, _ptr(ws), ws_bytes, _stream(stream)))


def _forward_args(sh: Shape, layers: Sequence[LayerData], x, xdtype: int, T: int, y_last, ws, ws_bytes: int,
                  resid_out=None, route_outs: Optional[Sequence[dict]] = None, miss_te=None, miss_w=None,
                  miss_cap: int = 0, miss_count=None, flags: int = 0, events: Optional[Sequence[int]] = None,
                  stream=None) -> tuple:
    L = len(layers)
    c_layers = (Layer * L)(*[ly.as_c() for ly in layers])
    c_ro = None
    if route_outs is not None:
        assert len(route_outs) == L
        c_ro = (RouteOut * L)(*[_route_out(r) or RouteOut() for r in route_outs])
    ev = None
    n_ev = 0
    if events:
        ev = (ctypes.c_void_p * len(events))(*events)
        n_ev = len(events) // 2
    return (ctypes.byref(sh), c_layers, L, _ptr(x), xdtype, T, flags, _ptr(y_last), _ptr(resid_out), c_ro,
            _ptr(miss_te), _ptr(miss_w), miss_cap, _ptr(miss_count), _ptr(ws), ws_bytes, ev, n_ev, _stream(stream))


def forward(sh: Shape, layers: Sequence[LayerData], x, xdtype: int, T: int, y_last, ws, ws_bytes: int,
            resid_out=None, route_outs: Optional[Sequence[dict]] = None, miss_te=None, miss_w=None,
            miss_cap: int = 0, miss_count=None, flags: int = 0, events: Optional[Sequence[int]] = None,
            stream=None):
    """Forward of len(layers) stacked layers (see strata_moe_forward)."""
    lib = load_library()
    _check(lib.strata_moe_forward(*_forward_args(sh, layers, x, xdtype, T, y_last, ws, ws_bytes, resid_out,
                                                 route_outs, miss_te, miss_w, miss_cap, miss_count, flags, events,
                                                 stream)))


class PreparedForward:
    """A forward call whose arguments are marshalled once (same arguments as
    forward()); calling it enqueues the call again with the same pointers,
    so a loop of calls spends its host time in the library, not in argument
    marshalling."""

    def __init__(self, *args, **kwargs):
        self._fn = load_library().strata_moe_forward
        self._args = _forward_args(*args, **kwargs)

    def __call__(self):
        _check(self._fn(*self._args))


def forward_noalloc(sh: Shape, layers: Sequence[LayerData], x, xdtype: int, T: int, y_last, resid_out=None,
                    route_outs: Optional[Sequence[dict]] = None, miss_te=None, miss_w=None, miss_cap: int = 0,
                    miss_count=None, flags: int = 0, events: Optional[Sequence[int]] = None, stream=None):
    """forward() on the library's fixed per-device scratch (no workspace; see
    strata_moe_forward_noalloc)."""
    lib = load_library()
    L = len(layers)
    c_layers = (Layer * L)(*[ly.as_c() for ly in layers])
    c_ro = None
    if route_outs is not None:
        assert len(route_outs) == L
        c_ro = (RouteOut * L)(*[_route_out(r) or RouteOut() for r in route_outs])
    ev = None
    n_ev = 0
    if events:
        ev = (ctypes.c_void_p * len(events))(*events)
        n_ev = len(events) // 2
    _check(lib.strata_moe_forward_noalloc(ctypes.byref(sh), c_layers, L, _ptr(x), xdtype, T, flags, _ptr(y_last),
                                          _ptr(resid_out), c_ro, _ptr(miss_te), _ptr(miss_w), miss_cap,
                                          _ptr(miss_count), ev, n_ev, _stream(stream)))


def counts_accumulate(counts_acc, counts, n_experts: int, stream=None):
    """counts_acc[e] += counts[e] (int64 running totals, int32 per-call counts)."""
    _check(load_library().strata_moe_counts_accumulate(_ptr(counts_acc), _ptr(counts), n_experts, _stream(stream)))


def resident_topn(counts_acc, n_experts: int, n_resident: int, mask_out, stream=None):
    """mask_out = the n_resident most-picked experts (count desc, index asc)."""
    _check(load_library().strata_moe_resident_topn(_ptr(counts_acc), n_experts, n_resident, _ptr(mask_out),
                                                   _stream(stream)))


def probe_hbm_read(buf, nbytes: int, sink, blocks: int, stream=None):
    """Stream-read probe: every byte of buf loaded once (see strata_probe.h)."""
    _check(load_library().strata_probe_hbm_read(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream)))


def probe_mfma_bf16(iters: int, sink, blocks: int, stream=None) -> float:
    """bf16 matrix-core probe; returns the launch's floating-point operations."""
    fl = ctypes.c_double()
    _check(load_library().strata_probe_mfma_bf16(iters, _ptr(sink), blocks, ctypes.byref(fl), _stream(stream)))
    return fl.value


def _host_ptr(a) -> Optional[int]:
    """Address of a host buffer: a numpy array, a CPU torch tensor or an int."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "ctypes"):
        return a.ctypes.data
    return a.data_ptr()


def host_isa() -> str:
    """Instruction set of the host consumer of the miss list."""
    return load_library().strata_moe_host_isa().decode()


def host_workspace_bytes(sh: Shape, T: int, miss_cap: int) -> int:
    n = load_library().strata_moe_host_workspace_bytes(ctypes.byref(sh), T, miss_cap)
    if n == 0:
        raise StrataError(STRATA_EUNSUPPORTED, "shape not handled by the host consumer")
    return n


def host_misses(sh: Shape, codes, scales, bits: int, u, T: int, miss_te, miss_w, n_miss: int, y_add, host_ws,
                host_ws_bytes: int, n_threads: int):
    """y_add = per-token sum of gate * FFN_e(u_t) over the misses, on the host
    (see strata_moe_host_misses); every argument is host memory."""
    hl = HostLayer(_host_ptr(codes), _host_ptr(scales), int(bits))
    _check(load_library().strata_moe_host_misses(ctypes.byref(sh), ctypes.byref(hl), _host_ptr(u), T,
                                                 _host_ptr(miss_te), _host_ptr(miss_w), n_miss, _host_ptr(y_add),
                                                 _host_ptr(host_ws), host_ws_bytes, n_threads))


def forward_coprocess(sh: Shape, layers: Sequence[LayerData], host_layers: Sequence[tuple], x, xdtype: int, T: int,
                      y_last, ws, ws_bytes: int, host_ws, host_ws_bytes: int, n_threads: int, miss_te, miss_w,
                      miss_cap: int, miss_count, resid_out=None, route_outs: Optional[Sequence[dict]] = None,
                      flags: int = 0, aux_stream=None, stream=None):
    """forward() with every masked layer's misses computed on the host and
    added in (see strata_moe_forward_coprocess).  host_layers: per layer a
    (codes, scales, bits) tuple of host buffers; host_ws: page-locked host
    memory (e.g. a pinned torch tensor)."""
    lib = load_library()
    L = len(layers)
    c_layers = (Layer * L)(*[ly.as_c() for ly in layers])
    c_host = (HostLayer * L)(*[HostLayer(_host_ptr(c), _host_ptr(s_), int(b)) for c, s_, b in host_layers])
    c_ro = None
    if route_outs is not None:
        assert len(route_outs) == L
        c_ro = (RouteOut * L)(*[_route_out(r) or RouteOut() for r in route_outs])
    aux = None if aux_stream is None else (aux_stream if isinstance(aux_stream, int) else aux_stream.cuda_stream)
    _check(lib.strata_moe_forward_coprocess(ctypes.byref(sh), c_layers, c_host, L, _ptr(x), xdtype, T, flags,
                                            _ptr(y_last), _ptr(resid_out), c_ro, _ptr(miss_te), _ptr(miss_w),
                                            miss_cap, _ptr(miss_count), _ptr(ws), ws_bytes, _host_ptr(host_ws),
                                            host_ws_bytes, n_threads, aux, _stream(stream)))
