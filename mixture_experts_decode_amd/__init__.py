"""Python binding of libmoe_mi355x.so (the routed-expert MoE FFN for gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory and the current stream;
nothing else of torch is used here.  The library must be built
(``python -m mixture_experts_decode_amd.build``); without it every call raises.
"""

import contextlib
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
DT = {"f32": 0, "bf16": 1}
FMT = {"f32": 0, "mxfp8": 1, "mxfp4": 2, "fp8_blk128": 3}
PATH = {"auto": 0, "decode": 1, "grouped": 2}
PATH_NAME = {v: k for k, v in PATH.items()}
DOWN_VARIANT = {"auto": 0, "token": 1, "expert": 2}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode() if _lib else status}")


class _Weights(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("format", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
_WP = ctypes.POINTER(_Weights)

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_abi_version": (_I, []),
    "moe_decode_max_entries": (_I, []),
    "moe_gate_up": (_I, [_WP, _P, _I, _P, _I, _I, _P, _I, _P]),
    "moe_down_workspace_bytes": (_Z, [_WP, _I, _I]),
    "moe_down": (_I, [_WP, _P, _I, _P, _P, _I, _I, _P, _I, _I, _P, _Z, _P]),
    "moe_align_sort_capacity": (_Z, [_I, _I, _I, _I, _I]),
    "moe_align_sort_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "moe_align_sort": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_quant_rows": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_grouped_gate_up": (_I, [_WP, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P]),
    "moe_grouped_down": (_I, [_WP, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P, _P]),
    "moe_combine": (_I, [_P, _I, _I, _I, _P, _I, _P]),
    "moe_topk_route": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "moe_check_routing": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_choose_path": (_I, [_WP, _I, _I]),
    "moe_layer_workspace_bytes": (_Z, [_WP, _I, _I, _I, _I]),
    "moe_layer": (_I, [_WP, _P, _I, _P, _P, _I, _I, _P, _I, _I, _I, _P, _Z,
                       ctypes.POINTER(_I), _P]),
    "moe_layer_noalloc_max_bytes": (_Z, []),
    "moe_layer_noalloc": (_I, [_WP, _P, _I, _P, _P, _I, _I, _P, _I, _I, _I,
                               ctypes.POINTER(_I), _P]),
    "moe_util_copy": (_I, [_P, _P, _Z, _P]),
    "moe_util_read": (_I, [_P, _Z, _P, _P]),
    "moe_util_read_sink_len": (_I, []),
    "moe_util_fill": (_I, [_P, _Z, ctypes.c_uint32, _P]),
    "moe_util_num_cus": (_I, []),
}

EXPORTS = tuple(_SIGS)


def load(path=LIB_PATH):
    """Load the HIP library (idempotent).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run python -m mixture_experts_decode_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status, where):
    if status != OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a binding call with its `stream` argument made torch's current
    stream, so every tensor the call allocates (outputs, scratch) belongs to
    the stream its kernels are enqueued on and the caching allocator does not
    hand that memory to other work while they run."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kwargs):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return wrapped


class Weights:
    """One layer's expert weights resident on the device.

    Tensors as stored (see include/moe_mi355x.h): w13 [E+S][2][I][H*],
    w2 [E+S][H][I*] and their scales (None for "f32")."""

    def __init__(self, fmt, hidden, inter, num_experts, num_shared, w13, w13_scale, w2, w2_scale):
        self.fmt = fmt
        self.hidden, self.inter = hidden, inter
        self.num_experts, self.num_shared = num_experts, num_shared
        self.tensors = (w13, w13_scale, w2, w2_scale)
        self._s = _Weights(hidden, inter, num_experts, num_shared, FMT[fmt],
                           w13.data_ptr(), None if w13_scale is None else w13_scale.data_ptr(),
                           w2.data_ptr(), None if w2_scale is None else w2_scale.data_ptr())

    @classmethod
    def from_arrays(cls, cfg, arrays, device="cuda"):
        """Upload stacked numpy arrays (as made by the workload generators)."""
        def up(a):
            return None if a is None else torch.from_numpy(a).to(device)
        return cls(cfg.fmt, cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_shared,
                   up(arrays["w13"]), up(arrays.get("w13_scale")), up(arrays["w2"]),
                   up(arrays.get("w2_scale")))

    @property
    def ref(self):
        return ctypes.byref(self._s)

    @property
    def slots_extra(self):
        return self.num_shared

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in self.tensors if t is not None)


def _dt(t):
    if t.dtype == torch.float32:
        return DT["f32"]
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DT["bf16"]
    raise ValueError(f"unsupported activation dtype {t.dtype}")


def _alloc(shape, dtype, device):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.empty(shape, dtype=tdt, device=device)


@_on_stream
def gate_up(W, x, topk_ids, h=None, h_dtype="f32", stream=None):
    """h [T][k+S][I] for the decode path."""
    load()
    t, k = topk_ids.shape
    if h is None:
        h = _alloc((t, k + W.num_shared, W.inter), h_dtype, x.device)
    st = _lib.moe_gate_up(W.ref, _ptr(x), _dt(x), _ptr(topk_ids), t, k, _ptr(h), _dt(h),
                          _stream(stream))
    _check(st, "moe_gate_up")
    return h


@_on_stream
def down(W, h, topk_ids, topk_weights, y=None, y_dtype="f32", variant="auto", workspace=None,
         stream=None):
    """y [T][H] for the decode path.  variant: "token" (token-major), "expert"
    (expert-major with a slot buffer in `workspace`) or "auto" (as moe_layer
    does; it may pick either, so a slot buffer is passed)."""
    load()
    t, k = topk_ids.shape
    if y is None:
        y = _alloc((t, W.hidden), y_dtype, h.device)
    ws, wsb = None, 0
    if variant in ("expert", "auto"):
        wsb = _lib.moe_down_workspace_bytes(W.ref, t, k)
        if workspace is None:
            workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=h.device)
        ws, wsb = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = _lib.moe_down(W.ref, _ptr(h), _dt(h), _ptr(topk_ids), _ptr(topk_weights), t, k, _ptr(y),
                       _dt(y), DOWN_VARIANT[variant], ws, wsb, _stream(stream))
    _check(st, "moe_down")
    return y


def align_sort_capacity(t, k, num_experts, num_shared, block):
    load()
    return _lib.moe_align_sort_capacity(t, k, num_experts, num_shared, block)


@_on_stream
def align_sort(topk_ids, num_experts, num_shared, block, stream=None):
    """Returns dict of device tensors: sorted_token_ids [cap], expert_ids
    [cap/bs], expert_offsets [E+S+1], num_tokens_post_padded [1]."""
    load()
    t, k = topk_ids.shape
    dev = topk_ids.device
    cap = _lib.moe_align_sort_capacity(t, k, num_experts, num_shared, block)
    wsb = _lib.moe_align_sort_workspace_bytes(t, k, num_experts, num_shared, block)
    out = {
        "sorted_token_ids": torch.empty(cap, dtype=torch.int32, device=dev),
        "expert_ids": torch.empty(max(cap // block, 1), dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(num_experts + num_shared + 1, dtype=torch.int32, device=dev),
        "num_tokens_post_padded": torch.empty(1, dtype=torch.int32, device=dev),
    }
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    st = _lib.moe_align_sort(_ptr(topk_ids), t, k, num_experts, num_shared, block,
                             _ptr(out["sorted_token_ids"]), _ptr(out["expert_ids"]),
                             _ptr(out["expert_offsets"]), _ptr(out["num_tokens_post_padded"]),
                             _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_align_sort")
    out["capacity"] = cap
    out["_ws"] = ws
    return out


@_on_stream
def quant_rows(x, stream=None):
    """Each token row of x [T][H] quantised once to MXFP8: (xq [T][H] u8,
    xs [T][H/32] u8)."""
    load()
    t, h = x.shape
    xq = torch.empty((t, h), dtype=torch.uint8, device=x.device)
    xs = torch.empty((t, h // 32), dtype=torch.uint8, device=x.device)
    st = _lib.moe_quant_rows(_ptr(x), _dt(x), t, h, _ptr(xq), _ptr(xs), _stream(stream))
    _check(st, "moe_quant_rows")
    return xq, xs


@_on_stream
def grouped_gate_up(W, xq, xs, t, k, sorted_ids, expert_ids, npp, capacity, block, stream=None):
    """Grouped gate_up GEMM over the sorted rows; row r reads token row
    sorted_ids[r] // (k + S) of xq / xs.  Returns (hq [2][cap][I], hs [2][cap][I/32])."""
    load()
    hq = torch.empty((2, capacity, W.inter), dtype=torch.uint8, device=xq.device)
    hs = torch.empty((2, capacity, W.inter // 32), dtype=torch.uint8, device=xq.device)
    st = _lib.moe_grouped_gate_up(W.ref, _ptr(xq), _ptr(xs), t, k, _ptr(sorted_ids),
                                  _ptr(expert_ids), _ptr(npp), capacity, block, _ptr(hq), _ptr(hs),
                                  _stream(stream))
    _check(st, "moe_grouped_gate_up")
    return hq, hs


@_on_stream
def grouped_down(W, hq, hs, sorted_ids, expert_ids, npp, capacity, block, topk_weights, t, k,
                 slot_out=None, stream=None):
    load()
    if slot_out is None:
        slot_out = torch.empty((t * (k + W.num_shared), W.hidden), dtype=torch.bfloat16,
                               device=hq.device)
    if slot_out.dtype != torch.bfloat16:
        raise TypeError("slot_out holds BF16 values")
    st = _lib.moe_grouped_down(W.ref, _ptr(hq), _ptr(hs), _ptr(sorted_ids), _ptr(expert_ids),
                               _ptr(npp), capacity, block, _ptr(topk_weights), t, k,
                               _ptr(slot_out), _stream(stream))
    _check(st, "moe_grouped_down")
    return slot_out


@_on_stream
def combine(slot_out, t, slots, y=None, y_dtype="f32", stream=None):
    load()
    if slot_out.dtype != torch.bfloat16:
        raise TypeError("slot_out holds BF16 values (as grouped_down writes them)")
    h = slot_out.shape[1]
    if y is None:
        y = _alloc((t, h), y_dtype, slot_out.device)
    st = _lib.moe_combine(_ptr(slot_out), t, slots, h, _ptr(y), _dt(y), _stream(stream))
    _check(st, "moe_combine")
    return y


@_on_stream
def topk_route(scores, k, bias=None, ids=None, wts=None, stream=None):
    """Router front-end: scores [T][E] float32 (device), bias [E] or None ->
    (topk_ids int32 [T][k], topk_weights float32 [T][k]), written into ids /
    wts when given."""
    load()
    t, e = scores.shape
    if ids is None:
        ids = torch.empty((t, k), dtype=torch.int32, device=scores.device)
    if wts is None:
        wts = torch.empty((t, k), dtype=torch.float32, device=scores.device)
    st = _lib.moe_topk_route(_ptr(scores), None if bias is None else _ptr(bias), t, e, k, _ptr(ids),
                             _ptr(wts), _stream(stream))
    _check(st, "moe_topk_route")
    return ids, wts


@_on_stream
def check_routing(ids, num_experts, result=None, stream=None):
    """Device check of topk_ids [T][k] int32: returns (or fills) an int32 [2]
    device tensor (number of ids outside [0, num_experts), first such entry
    t*k + j or -1)."""
    load()
    t, k = ids.shape
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=ids.device)
    st = _lib.moe_check_routing(_ptr(ids) if ids.numel() else None, t, k, num_experts,
                                _ptr(result), _stream(stream))
    _check(st, "moe_check_routing")
    return result


def choose_path(W, t, k):
    load()
    return PATH_NAME[_lib.moe_choose_path(W.ref, t, k)]


def layer_workspace_bytes(W, t, k, path="auto", block=0):
    load()
    return _lib.moe_layer_workspace_bytes(W.ref, t, k, PATH[path], block)


@_on_stream
def layer(W, x, topk_ids, topk_weights, path="auto", block=0, y=None, y_dtype="f32",
          workspace=None, stream=None):
    """y [T][H] for the whole layer; returns (y, path that ran)."""
    load()
    t, k = topk_ids.shape
    if y is None:
        y = _alloc((t, W.hidden), y_dtype, x.device)
    need = _lib.moe_layer_workspace_bytes(W.ref, t, k, PATH[path], block)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    chosen = ctypes.c_int32(-1)
    st = _lib.moe_layer(W.ref, _ptr(x), _dt(x), _ptr(topk_ids), _ptr(topk_weights), t, k, _ptr(y),
                        _dt(y), PATH[path], block, _ptr(workspace),
                        workspace.numel() * workspace.element_size(), ctypes.byref(chosen),
                        _stream(stream))
    _check(st, "moe_layer")
    return y, PATH_NAME.get(chosen.value, "?")


def layer_noalloc_max_bytes():
    load()
    return _lib.moe_layer_noalloc_max_bytes()


def layer_noalloc(W, x, topk_ids, topk_weights, y, path="auto", block=0, stream=None):
    """moe_layer_noalloc: y [T][H] (caller-allocated, written in place) with
    the library's own device array as workspace; nothing is allocated here.
    Returns the path that ran."""
    load()
    t, k = topk_ids.shape
    chosen = ctypes.c_int32(-1)
    st = _lib.moe_layer_noalloc(W.ref, _ptr(x), _dt(x), _ptr(topk_ids), _ptr(topk_weights), t, k,
                                _ptr(y), _dt(y), PATH[path], block, ctypes.byref(chosen),
                                _stream(stream))
    _check(st, "moe_layer_noalloc")
    return PATH_NAME.get(chosen.value, "?")


# ---- measurement kernels ------------------------------------------------

def util_copy(src, dst, nbytes, stream=None):
    load()
    _check(_lib.moe_util_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "moe_util_copy")


def util_read(src, nbytes, sink, stream=None):
    load()
    _check(_lib.moe_util_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "moe_util_read")


def util_fill(dst, nbytes, value=0, stream=None):
    load()
    _check(_lib.moe_util_fill(_ptr(dst), nbytes, value, _stream(stream)), "moe_util_fill")


def num_cus():
    load()
    return _lib.moe_util_num_cus()
