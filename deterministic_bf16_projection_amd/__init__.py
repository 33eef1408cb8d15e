"""Python binding of libdpg, the MI355X projection GEMM library.

Argument marshalling only: every entry point takes torch tensors (device
memory allocated by PyTorch), passes their data pointers, row strides and the
current HIP stream to the C ABI declared in ``include/dpg.h`` and returns the
output tensor.  All arithmetic runs in the library's gfx950 kernels.  There is
no fallback: if ``libdpg.so`` is missing, importing this package raises.

Names follow the C ABI: ``dpg_forward``, ``dpg_dgrad``, ``dpg_wgrad``,
``dpg_router_forward``, ``dpg_router_dgrad``, ``dpg_router_wgrad`` and the
batched ``dpg_forward_batched``, ``dpg_dgrad_batched``, ``dpg_wgrad_batched``.
``deterministic=True`` is the default, as on the router page's description.
"""
import contextlib
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpg.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dpg.h")

if not os.path.exists(LIB_PATH):
    raise ImportError("libdpg.so is not built; run `python deterministic_bf16_projection_amd/build.py` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

BF16, F32 = 0, 1
PASS_FORWARD, PASS_DGRAD, PASS_WGRAD = 0, 1, 2
PASS_ROUTER_FORWARD, PASS_ROUTER_DGRAD, PASS_ROUTER_WGRAD = 3, 4, 5
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "alignment", 4: "workspace", 5: "HIP launch failed"}

_i64, _vp, _ci, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_GEMM_ARGS = [_vp, _i64, _vp, _i64, _vp, _i64, _ci, _i64, _i64, _i64, _ci, _ci, _vp, _sz, _vp]
_ROUTER_ARGS = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _ci, _ci, _vp, _sz, _vp]
for _name in ("dpg_forward", "dpg_dgrad", "dpg_wgrad"):
    getattr(_lib, _name).argtypes = _GEMM_ARGS
    getattr(_lib, _name).restype = _ci
for _name in ("dpg_router_forward", "dpg_router_dgrad", "dpg_router_wgrad"):
    getattr(_lib, _name).argtypes = _ROUTER_ARGS
    getattr(_lib, _name).restype = _ci
_BATCHED_ARGS = [_vp, _i64, _i64, _vp, _i64, _i64, _ci, _vp, _i64, _i64, _ci,
                 _i64, _i64, _i64, _i64, _ci, _ci, _vp, _sz, _vp]
for _name in ("dpg_forward_batched", "dpg_dgrad_batched"):
    getattr(_lib, _name).argtypes = _BATCHED_ARGS
    getattr(_lib, _name).restype = _ci
_lib.dpg_wgrad_batched.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _ci, _ci,
                                   _i64, _i64, _i64, _i64, _ci, _ci, _vp, _sz, _vp]
_lib.dpg_wgrad_batched.restype = _ci
_lib.dpg_workspace_size_batched.argtypes = [_ci, _ci, _i64, _i64, _i64, _i64, _ci, _ci, _ci]
_lib.dpg_workspace_size_batched.restype = _sz
_lib.dpg_plan_describe_batched.argtypes = [_ci, _ci, _i64, _i64, _i64, _i64, _ci, _ci, _ci, ctypes.c_char_p, _sz]
_lib.dpg_plan_describe_batched.restype = _ci
_lib.dpg_workspace_size.argtypes = [_ci, _i64, _i64, _i64, _ci, _ci, _ci]
_lib.dpg_workspace_size.restype = _sz
_lib.dpg_plan_describe.argtypes = [_ci, _i64, _i64, _i64, _ci, _ci, _ci, ctypes.c_char_p, _sz]
_lib.dpg_plan_describe.restype = _ci
_lib.dpg_clear_plan_cache.argtypes = []
_lib.dpg_clear_plan_cache.restype = None
_lib.dpg_plan_cache_stats.argtypes = [ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
_lib.dpg_plan_cache_stats.restype = None
_lib.dpg_wgrad_noalloc.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _ci, _i64, _i64, _i64, _ci, _ci, _vp]
_lib.dpg_wgrad_noalloc.restype = _ci
_lib.dpg_noalloc_scratch_bytes.argtypes = []
_lib.dpg_noalloc_scratch_bytes.restype = _sz
_lib.dpg_set_router_arithmetic.argtypes = [_ci]
_lib.dpg_set_router_arithmetic.restype = _ci
_lib.dpg_get_router_arithmetic.argtypes = []
_lib.dpg_get_router_arithmetic.restype = _ci
_lib.dpg_plan_cache_capacity.argtypes = []
_lib.dpg_plan_cache_capacity.restype = _i64
_lib.dpg_status_string.argtypes = [_ci]
_lib.dpg_status_string.restype = ctypes.c_char_p
_lib.dpg_version.argtypes = []
_lib.dpg_version.restype = ctypes.c_char_p


class DpgError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.dpg_status_string(status).decode()
        super().__init__("%s: %s (status %d)" % (where, msg, status))


def lib():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def header_symbols():
    """Names of the functions include/dpg.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(dpg_[a-z_]+)\s*\(", text)))


def version():
    return _lib.dpg_version().decode()


def _code(dtype):
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError("output dtype must be torch.bfloat16 or torch.float32")


def _ld(t, name):
    """Row stride in elements.  A matrix with at most one row never steps to a
    next row, so its stride is reported as the column count rounded up to 8."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    rows, cols = t.shape
    if rows > 0 and cols > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit column stride" % name)
    if rows <= 1:
        return max(8, (cols + 7) // 8 * 8)
    return t.stride(0)


# Raw handle of a device's current stream (the accessor torch's own compiler
# uses): about 0.3 us a call against about 3 us for a torch.cuda.Stream object.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device=None):
    """HIP stream handle of a call: `stream` as given, else the current stream
    of `device` (the device the call runs on, which is current there)."""
    if stream is None:
        if _raw_current_stream is not None and device is not None and device.index is not None:
            return _raw_current_stream(device.index)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on_stream(stream, device):
    """Context in which the binding allocates the tensors a call creates (its
    output and workspace): the stream the kernels run on.  PyTorch's caching
    allocator then reuses such a block only after that stream's work on it, so
    a workspace dropped when the call returns cannot be handed to other work
    while the kernels still read it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


_n_devices = []


def _on_device(device):
    """Context that makes the tensors' device HIP's current one, on which the
    library launches; a no-op (no device switch, no query) when it already is
    or when only one device is visible."""
    if not _n_devices:
        _n_devices.append(torch.cuda.device_count())
    if _n_devices[0] <= 1 or device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def workspace_size(pass_, T, N, K, out_dtype=torch.bfloat16, deterministic=True, split_k=0):
    n = _lib.dpg_workspace_size(pass_, T, N, K, _code(out_dtype), int(bool(deterministic)), split_k)
    if n == ctypes.c_size_t(-1).value:
        raise DpgError(1, "dpg_workspace_size")
    return n


def plan_describe(pass_, T, N, K, out_dtype=torch.bfloat16, deterministic=True, split_k=0):
    buf = ctypes.create_string_buffer(1024)
    st = _lib.dpg_plan_describe(pass_, T, N, K, _code(out_dtype), int(bool(deterministic)), split_k, buf, 1024)
    if st:
        raise DpgError(st, "dpg_plan_describe")
    return buf.value.decode()


def parse_plan(text):
    """key=value pairs of a plan description as a dict of strings."""
    return dict(kv.split("=", 1) for kv in text.split() if "=" in kv)


def clear_plan_cache():
    _lib.dpg_clear_plan_cache()


def plan_cache_stats():
    e, g = _i64(0), _i64(0)
    _lib.dpg_plan_cache_stats(ctypes.byref(e), ctypes.byref(g))
    return e.value, g.value


def plan_cache_capacity():
    return _lib.dpg_plan_cache_capacity()


ROUTER_ARITH = {"auto": 0, "bf16x3": 1, "fp32": 2}


def set_router_arithmetic(arith):
    """Process-wide router arithmetic: 'auto' (the planner's choice per shape),
    'bf16x3' or 'fp32' (FP32 fused multiply-adds).  Returns the previous one."""
    if arith not in ROUTER_ARITH:
        raise ValueError("router arithmetic must be one of %s" % sorted(ROUTER_ARITH))
    prev = get_router_arithmetic()
    st = _lib.dpg_set_router_arithmetic(ROUTER_ARITH[arith])
    if st:
        raise DpgError(st, "dpg_set_router_arithmetic")
    return prev


def get_router_arithmetic():
    code = _lib.dpg_get_router_arithmetic()
    return {v: k for k, v in ROUTER_ARITH.items()}[code]


def _workspace(pass_, T, N, K, out_code, det, split_k, workspace, device):
    need = _lib.dpg_workspace_size(pass_, T, N, K, out_code, det, split_k)
    if need == ctypes.c_size_t(-1).value:
        raise DpgError(1, "dpg_workspace_size")
    if need == 0:
        return None, 0
    _check_workspace(workspace, device)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise DpgError(4, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _call(name, pass_, a, b, out, out_code, T, N, K, deterministic, split_k, workspace, stream):
    det = int(bool(deterministic))
    with _on_device(out.device):
        with _on_stream(stream, out.device):
            ws, ws_bytes = _workspace(pass_, T, N, K, out_code, det, split_k, workspace, out.device)
        fn = getattr(_lib, name)
        args = [a.data_ptr(), _ld(a, "a"), b.data_ptr(), _ld(b, "b"), out.data_ptr(), _ld(out, "out")]
        if pass_ < 3:
            args.append(out_code)
        args += [T, N, K, det, split_k, ws.data_ptr() if ws is not None else None, ws_bytes,
                 _stream(stream, out.device)]
        st = fn(*args)
    if st:
        raise DpgError(st, name)
    return out


def _check_in(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


def _check_same_device(*named):
    """Every (name, tensor) pair on the first one's device."""
    dev = named[0][1].device
    for name, t in named[1:]:
        if t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))


def _check_out(out, shape, device, name="out"):
    """A caller-supplied output must be a device tensor of exactly the output's
    shape (the kernels write every element of it)."""
    if not out.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if out.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, out.device, device))
    if tuple(out.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(out.shape)))


def _check_workspace(workspace, device):
    if workspace is not None and (not workspace.is_cuda or workspace.device != device):
        raise ValueError("workspace must be a device tensor on %s" % device)


def dpg_forward(x, w, out=None, out_dtype=torch.bfloat16, deterministic=True, split_k=0, workspace=None,
                stream=None):
    """Y[T,N] = X[T,K] W[N,K]^T (BF16 operands, FP32 accumulation)."""
    _check_in(x, torch.bfloat16, "x")
    _check_in(w, torch.bfloat16, "w")
    T, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K]")
    _check_same_device(("x", x), ("w", w))
    if out is None:
        with _on_stream(stream, x.device):
            out = torch.empty((T, N), dtype=out_dtype, device=x.device)
    _check_out(out, (T, N), x.device)
    return _call("dpg_forward", PASS_FORWARD, x, w, out, _code(out.dtype), T, N, K, deterministic, split_k,
                 workspace, stream)


def dpg_dgrad(dy, w, out=None, out_dtype=torch.bfloat16, deterministic=True, split_k=0, workspace=None,
              stream=None):
    """dX[T,K] = dY[T,N] W[N,K]."""
    _check_in(dy, torch.bfloat16, "dy")
    _check_in(w, torch.bfloat16, "w")
    T, N = dy.shape
    K = w.shape[1]
    if w.shape[0] != N:
        raise ValueError("w must be [N, K]")
    _check_same_device(("dy", dy), ("w", w))
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty((T, K), dtype=out_dtype, device=dy.device)
    _check_out(out, (T, K), dy.device)
    return _call("dpg_dgrad", PASS_DGRAD, dy, w, out, _code(out.dtype), T, N, K, deterministic, split_k,
                 workspace, stream)


def dpg_wgrad(dy, x, out=None, out_dtype=torch.bfloat16, deterministic=True, split_k=0, workspace=None,
              stream=None):
    """dW[N,K] = dY[T,N]^T X[T,K], reducing over T."""
    _check_in(dy, torch.bfloat16, "dy")
    _check_in(x, torch.bfloat16, "x")
    T, N = dy.shape
    K = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x must be [T, K]")
    _check_same_device(("dy", dy), ("x", x))
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty((N, K), dtype=out_dtype, device=dy.device)
    _check_out(out, (N, K), dy.device)
    return _call("dpg_wgrad", PASS_WGRAD, dy, x, out, _code(out.dtype), T, N, K, deterministic, split_k,
                 workspace, stream)


def dpg_wgrad_noalloc(dy, x, out, deterministic=True, split_k=0, stream=None):
    """dW[N,K] = dY[T,N]^T X[T,K] into the caller's ``out`` without any
    allocation: split partials go to the library's static device scratch
    (``noalloc_scratch_bytes()`` per GPU).  Same plan and bits as dpg_wgrad.
    Calls that overlap on one GPU race on the scratch; do not issue them."""
    _check_in(dy, torch.bfloat16, "dy")
    _check_in(x, torch.bfloat16, "x")
    T, N = dy.shape
    K = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x must be [T, K]")
    _check_same_device(("dy", dy), ("x", x))
    _check_out(out, (N, K), dy.device)
    with _on_device(out.device):
        st = _lib.dpg_wgrad_noalloc(dy.data_ptr(), _ld(dy, "dy"), x.data_ptr(), _ld(x, "x"), out.data_ptr(),
                                    _ld(out, "out"), _code(out.dtype), T, N, K, int(bool(deterministic)), split_k,
                                    _stream(stream, out.device))
    if st:
        raise DpgError(st, "dpg_wgrad_noalloc")
    return out


def noalloc_scratch_bytes():
    return _lib.dpg_noalloc_scratch_bytes()


def dpg_router_forward(x, w, out=None, deterministic=True, split_k=0, workspace=None, stream=None):
    """y[T,E] = x[T,H] w[E,H]^T, FP32 via BF16x3."""
    _check_in(x, torch.float32, "x")
    _check_in(w, torch.float32, "w")
    T, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("w must be [E, H]")
    _check_same_device(("x", x), ("w", w))
    if out is None:
        with _on_stream(stream, x.device):
            out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check_in(out, torch.float32, "out")
    _check_out(out, (T, E), x.device)
    return _call("dpg_router_forward", PASS_ROUTER_FORWARD, x, w, out, F32, T, E, H, deterministic, split_k,
                 workspace, stream)


def dpg_router_dgrad(dy, w, out=None, deterministic=True, split_k=0, workspace=None, stream=None):
    """dx[T,H] = dy[T,E] w[E,H], FP32 via BF16x3."""
    _check_in(dy, torch.float32, "dy")
    _check_in(w, torch.float32, "w")
    T, E = dy.shape
    H = w.shape[1]
    if w.shape[0] != E:
        raise ValueError("w must be [E, H]")
    _check_same_device(("dy", dy), ("w", w))
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty((T, H), dtype=torch.float32, device=dy.device)
    _check_in(out, torch.float32, "out")
    _check_out(out, (T, H), dy.device)
    return _call("dpg_router_dgrad", PASS_ROUTER_DGRAD, dy, w, out, F32, T, E, H, deterministic, split_k,
                 workspace, stream)


def dpg_router_wgrad(dy, x, out=None, deterministic=True, split_k=0, workspace=None, stream=None):
    """dw[E,H] = dy[T,E]^T x[T,H], FP32 via BF16x3."""
    _check_in(dy, torch.float32, "dy")
    _check_in(x, torch.float32, "x")
    T, E = dy.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x must be [T, H]")
    _check_same_device(("dy", dy), ("x", x))
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty((E, H), dtype=torch.float32, device=dy.device)
    _check_in(out, torch.float32, "out")
    _check_out(out, (E, H), dy.device)
    return _call("dpg_router_wgrad", PASS_ROUTER_WGRAD, dy, x, out, F32, T, E, H, deterministic, split_k,
                 workspace, stream)


# ------------------------------------------------------------------ batched --
WEIGHT_LAYOUTS = {"nk": 0, "kn": 1}


def _wl(weight_layout):
    if weight_layout not in WEIGHT_LAYOUTS:
        raise ValueError("weight_layout must be 'nk' or 'kn'")
    return WEIGHT_LAYOUTS[weight_layout]


def _batched(t, name, batch=None):
    """(tensor, batch stride, row stride) of a [B, R, C] operand, or of a 2-D
    [R, C] one shared by every problem (batch stride 0)."""
    if t.dim() == 2:
        t3, bstride = t, 0
        rows, cols = t.shape
        rs, cs = t.stride()
    elif t.dim() == 3:
        t3 = t
        _, rows, cols = t.shape
        bstride, rs, cs = t.stride()
        if batch is not None and t.shape[0] != batch:
            raise ValueError("%s: batch %d, expected %d" % (name, t.shape[0], batch))
    else:
        raise ValueError("%s must be [B, R, C] or [R, C]" % name)
    if cols > 1 and cs != 1:
        raise ValueError("%s: the last dimension must be contiguous" % name)
    ld = rs if rows > 1 else ((cols + 7) // 8) * 8
    return t3, bstride, ld


def workspace_size_batched(pass_, batch, T, N, K, out_dtype=torch.bfloat16, deterministic=True, split_k=0,
                           weight_layout="nk"):
    return _lib.dpg_workspace_size_batched(pass_, _wl(weight_layout), batch, T, N, K, _code(out_dtype),
                                           int(bool(deterministic)), split_k)


def plan_describe_batched(pass_, batch, T, N, K, out_dtype=torch.bfloat16, deterministic=True, split_k=0,
                          weight_layout="nk"):
    buf = ctypes.create_string_buffer(1024)
    st = _lib.dpg_plan_describe_batched(pass_, _wl(weight_layout), batch, T, N, K, _code(out_dtype),
                                        int(bool(deterministic)), split_k, buf, 1024)
    if st:
        raise DpgError(st, "dpg_plan_describe_batched")
    return buf.value.decode()


def _batched_ws(pass_, wl, batch, T, N, K, out_code, det, split_k, workspace, device):
    need = _lib.dpg_workspace_size_batched(pass_, wl, batch, T, N, K, out_code, det, split_k)
    if need == ctypes.c_size_t(-1).value:
        raise DpgError(1, "dpg_workspace_size_batched")
    if need == 0:
        return None, 0
    _check_workspace(workspace, device)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise DpgError(4, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def dpg_forward_batched(x, w, out=None, out_dtype=torch.bfloat16, weight_layout="nk", deterministic=True,
                        split_k=0, workspace=None, stream=None):
    """y[b] = x[b] w[b]^T for weights [B, N, K] (weight_layout 'nk') or
    y[b] = x[b] w[b] for weights [B, K, N] ('kn'); x [B, T, K]; a 2-D weight is
    shared by every problem.  Views with any batch and row strides are taken as
    they are (unit column stride)."""
    _check_in(x, torch.bfloat16, "x")
    _check_in(w, torch.bfloat16, "w")
    wl = _wl(weight_layout)
    batch, T, K = x.shape
    N = w.shape[-2] if wl == 0 else w.shape[-1]
    if (w.shape[-1] if wl == 0 else w.shape[-2]) != K:
        raise ValueError("weight does not match K")
    _check_same_device(("x", x), ("w", w))
    if out is None:
        with _on_stream(stream, x.device):
            out = torch.empty((batch, T, N), dtype=out_dtype, device=x.device)
    _check_out(out, (batch, T, N), x.device)
    x3, sx, ldx = _batched(x, "x", batch)
    w3, sw, ldw = _batched(w, "w", batch)
    o3, so, ldo = _batched(out, "out", batch)
    det = int(bool(deterministic))
    with _on_device(x.device):
        with _on_stream(stream, x.device):
            ws, wsb = _batched_ws(PASS_FORWARD, wl, batch, T, N, K, _code(out.dtype), det, split_k, workspace,
                                  x.device)
        st = _lib.dpg_forward_batched(x3.data_ptr(), ldx, sx, w3.data_ptr(), ldw, sw, wl, o3.data_ptr(), ldo, so,
                                      _code(out.dtype), batch, T, N, K, det, split_k,
                                      ws.data_ptr() if ws is not None else None, wsb, _stream(stream, x.device))
    if st:
        raise DpgError(st, "dpg_forward_batched")
    return out


def dpg_dgrad_batched(dy, w, out=None, out_dtype=torch.bfloat16, weight_layout="nk", deterministic=True,
                      split_k=0, workspace=None, stream=None):
    """dx[b] = dy[b] w[b] for weights [B, N, K] ('nk'), or dy[b] w[b]^T for
    weights [B, K, N] ('kn'); dy [B, T, N]."""
    _check_in(dy, torch.bfloat16, "dy")
    _check_in(w, torch.bfloat16, "w")
    wl = _wl(weight_layout)
    batch, T, N = dy.shape
    K = w.shape[-1] if wl == 0 else w.shape[-2]
    if (w.shape[-2] if wl == 0 else w.shape[-1]) != N:
        raise ValueError("weight does not match N")
    _check_same_device(("dy", dy), ("w", w))
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty((batch, T, K), dtype=out_dtype, device=dy.device)
    _check_out(out, (batch, T, K), dy.device)
    d3, sd, ldd = _batched(dy, "dy", batch)
    w3, sw, ldw = _batched(w, "w", batch)
    o3, so, ldo = _batched(out, "out", batch)
    det = int(bool(deterministic))
    with _on_device(dy.device):
        with _on_stream(stream, dy.device):
            ws, wsb = _batched_ws(PASS_DGRAD, wl, batch, T, N, K, _code(out.dtype), det, split_k, workspace,
                                  dy.device)
        st = _lib.dpg_dgrad_batched(d3.data_ptr(), ldd, sd, w3.data_ptr(), ldw, sw, wl, o3.data_ptr(), ldo, so,
                                    _code(out.dtype), batch, T, N, K, det, split_k,
                                    ws.data_ptr() if ws is not None else None, wsb, _stream(stream, dy.device))
    if st:
        raise DpgError(st, "dpg_dgrad_batched")
    return out


def dpg_wgrad_batched(dy, x, out=None, out_dtype=torch.bfloat16, weight_layout="nk", deterministic=True,
                      split_k=0, workspace=None, stream=None):
    """dw[b] = dy[b]^T x[b] as [B, N, K] ('nk') or x[b]^T dy[b] as [B, K, N]
    ('kn'); dy [B, T, N], x [B, T, K]."""
    _check_in(dy, torch.bfloat16, "dy")
    _check_in(x, torch.bfloat16, "x")
    wl = _wl(weight_layout)
    batch, T, N = dy.shape
    K = x.shape[-1]
    if x.shape[-2] != T:
        raise ValueError("x must be [B, T, K]")
    _check_same_device(("dy", dy), ("x", x))
    oshape = (batch, N, K) if wl == 0 else (batch, K, N)
    if out is None:
        with _on_stream(stream, dy.device):
            out = torch.empty(oshape, dtype=out_dtype, device=dy.device)
    _check_out(out, oshape, dy.device)
    d3, sd, ldd = _batched(dy, "dy", batch)
    x3, sx, ldx = _batched(x, "x", batch)
    o3, so, ldo = _batched(out, "out", batch)
    det = int(bool(deterministic))
    with _on_device(dy.device):
        with _on_stream(stream, dy.device):
            ws, wsb = _batched_ws(PASS_WGRAD, wl, batch, T, N, K, _code(out.dtype), det, split_k, workspace,
                                  dy.device)
        st = _lib.dpg_wgrad_batched(d3.data_ptr(), ldd, sd, x3.data_ptr(), ldx, sx, o3.data_ptr(), ldo, so, wl,
                                    _code(out.dtype), batch, T, N, K, det, split_k,
                                    ws.data_ptr() if ws is not None else None, wsb, _stream(stream, dy.device))
    if st:
        raise DpgError(st, "dpg_wgrad_batched")
    return out
