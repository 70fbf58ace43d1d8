"""Thin ctypes binding of libcnhwc.so (C ABI in include/cnhwc.h).

The cnhwc_* functions mirror the C entry points one to one (argument
marshalling only: every step of the computation runs in the HIP library).
``fwd`` / ``dgrad`` / ``wgrad`` are conveniences over PyTorch device tensors: torch only
allocates the outputs and workspace and supplies the current stream.

A problem is a dict with keys n, h, w, c, k, r, s, stride, pad_h, pad_w,
groups and dtype ("f16" or "bf16").  Any non-zero status raises CnhwcError
with the library's reason text.  Loading fails loudly if the library has not
been built: there is no fallback.
"""
import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcnhwc.so")

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, MISALIGNED, HIP_ERROR = range(6)
F16, BF16 = 0, 1
OP_FWD, OP_DGRAD, OP_WGRAD = 1, 2, 4
(VAR_AUTO, VAR_DGRAD_POINTWISE, VAR_DGRAD_IGEMM, VAR_DGRAD_DW_STREAM, VAR_DGRAD_DW_ROTATED,
 VAR_FWD_DIRECT, VAR_FWD_SPLITC, VAR_FWD_GROUPED, VAR_FWD_GENERIC, VAR_DGRAD_GENERIC,
 VAR_DGRAD_DW_TILED, VAR_FWD_DW_TILED, VAR_FWD_DW_ROTATED, VAR_DGRAD_GROUPED,
 VAR_WGRAD_GENERIC, VAR_WGRAD_POINTWISE, VAR_WGRAD_SPLITK, VAR_DGRAD_SPLITK, VAR_FWD_IGEMM) = range(19)

SYMBOLS = ("cnhwc_out_dims", "cnhwc_workspace_size", "cnhwc_plan", "cnhwc_chunk_plan",
           "cnhwc_fwd", "cnhwc_dgrad", "cnhwc_wgrad", "cnhwc_last_error", "cnhwc_set_override",
           "cnhwc_fwd_static_ws")
STATIC_WS_BYTES = 32 << 20   # CNHWC_STATIC_WS_BYTES


class CnhwcError(RuntimeError):
    def __init__(self, status, reason):
        super().__init__("cnhwc status %d: %s" % (status, reason))
        self.status = status
        self.reason = reason


class Problem(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
                ("c", ctypes.c_int64), ("k", ctypes.c_int64), ("r", ctypes.c_int64),
                ("s", ctypes.c_int64), ("stride", ctypes.c_int32), ("pad_h", ctypes.c_int32),
                ("pad_w", ctypes.c_int32), ("groups", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Override(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("cpl", ctypes.c_int32), ("split_c", ctypes.c_int32),
                ("tune", ctypes.c_int32), ("chunk_limit_bytes", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # One HIP runtime per process: when PyTorch is present its bundled
        # libamdhip64.so.7 must be the one our library binds to, so load torch
        # first (the dynamic loader then reuses the already-loaded soname).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcnhwc.so is not built (%s); run "
                               "`python -m convolution_nhwc_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.cnhwc_out_dims.argtypes = [P, i64p, i64p]
        L.cnhwc_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
        L.cnhwc_plan.argtypes = [P, ctypes.c_int, ctypes.c_char_p, sz, ctypes.POINTER(ctypes.c_int32)]
        L.cnhwc_chunk_plan.argtypes = [P, ctypes.c_int, i64p, ctypes.c_int64, i64p]
        L.cnhwc_fwd.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.cnhwc_dgrad.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.cnhwc_wgrad.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.cnhwc_fwd_static_ws.argtypes = [P, vp, vp, vp, vp]
        L.cnhwc_last_error.argtypes = []
        L.cnhwc_last_error.restype = ctypes.c_char_p
        L.cnhwc_set_override.argtypes = [ctypes.POINTER(Override)]
        for fn in SYMBOLS:
            if fn != "cnhwc_last_error":
                getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _problem(p):
    if isinstance(p, Problem):
        return p
    dt = p.get("dtype", "f16")
    dt = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}.get(dt, dt)
    return Problem(int(p["n"]), int(p["h"]), int(p["w"]), int(p["c"]), int(p["k"]), int(p["r"]),
                   int(p["s"]), int(p.get("stride", 1)), int(p.get("pad_h", 0)),
                   int(p.get("pad_w", 0)), int(p.get("groups", 1)), int(dt), 0)


def last_error():
    return lib().cnhwc_last_error().decode()


def _check(status):
    if status != OK:
        raise CnhwcError(status, last_error())


def cnhwc_out_dims(p):
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().cnhwc_out_dims(ctypes.byref(_problem(p)), ctypes.byref(ho), ctypes.byref(wo)))
    return ho.value, wo.value


def cnhwc_workspace_size(p, op):
    b = ctypes.c_size_t()
    _check(lib().cnhwc_workspace_size(ctypes.byref(_problem(p)), op, ctypes.byref(b)))
    return b.value


def cnhwc_plan(p, op):
    buf = ctypes.create_string_buffer(256)
    v = ctypes.c_int32()
    _check(lib().cnhwc_plan(ctypes.byref(_problem(p)), op, buf, 256, ctypes.byref(v)))
    return buf.value.decode(), v.value


def cnhwc_chunk_plan(p, op, cap=4096):
    arr = (ctypes.c_int64 * cap)()
    n = ctypes.c_int64()
    _check(lib().cnhwc_chunk_plan(ctypes.byref(_problem(p)), op, arr, cap, ctypes.byref(n)))
    return [arr[i] for i in range(min(n.value, cap))]


def cnhwc_fwd(p, x, w, y, ws, ws_bytes, stream):
    """Raw entry point: pointers as ints (device addresses), stream as int."""
    _check(lib().cnhwc_fwd(ctypes.byref(_problem(p)), x, w, y, ws, ws_bytes, stream))


def cnhwc_fwd_static_ws(p, x, w, y, stream):
    """Forward pass with the library's static device workspace (no allocation)."""
    _check(lib().cnhwc_fwd_static_ws(ctypes.byref(_problem(p)), x, w, y, stream))


def cnhwc_dgrad(p, dy, w, dx, ws, ws_bytes, stream):
    _check(lib().cnhwc_dgrad(ctypes.byref(_problem(p)), dy, w, dx, ws, ws_bytes, stream))


def cnhwc_wgrad(p, x, dy, dw, ws, ws_bytes, stream):
    _check(lib().cnhwc_wgrad(ctypes.byref(_problem(p)), x, dy, dw, ws, ws_bytes, stream))


def cnhwc_set_override(variant=0, cpl=0, split_c=0, chunk_limit_bytes=0, tune=0):
    _check(lib().cnhwc_set_override(ctypes.byref(Override(variant, cpl, split_c, tune,
                                                          chunk_limit_bytes))))


def cnhwc_clear_override():
    _check(lib().cnhwc_set_override(None))


@contextlib.contextmanager
def override(**kw):
    """Test-only: force dispatcher choices inside a with-block."""
    cnhwc_set_override(**kw)
    try:
        yield
    finally:
        cnhwc_clear_override()


# ---- PyTorch conveniences ----------------------------------------------------

def _stream_handle(torch, device):
    return torch.cuda.current_stream(device).cuda_stream


def _storage_dtype(torch, p):
    return torch.bfloat16 if p.get("dtype", "f16") in ("bf16", BF16) else torch.float16


def fwd(x, w, p, y=None, ws=None):
    """y = forward conv of device tensors x [N,H,W,C] and w [K,R,S,C/G] (16-bit)."""
    import torch
    ho, wo = cnhwc_out_dims(p)
    if y is None:
        y = torch.empty((p["n"], ho, wo, p["k"]), dtype=_storage_dtype(torch, p), device=x.device)
    need = cnhwc_workspace_size(p, OP_FWD)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    cnhwc_fwd(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), ws.data_ptr() if ws is not None else None,
              ws.numel() * ws.element_size() if ws is not None else 0, _stream_handle(torch, x.device))
    return y


def dgrad(dy, w, p, dx=None, ws=None):
    """dx = backward-data conv of device tensors dy [N,Ho,Wo,K] and w [K,R,S,C/G]."""
    import torch
    if dx is None:
        dx = torch.empty((p["n"], p["h"], p["w"], p["c"]), dtype=_storage_dtype(torch, p),
                         device=dy.device)
    need = cnhwc_workspace_size(p, OP_DGRAD)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dy.device)
    cnhwc_dgrad(p, dy.data_ptr(), w.data_ptr(), dx.data_ptr(),
                ws.data_ptr() if ws is not None else None,
                ws.numel() * ws.element_size() if ws is not None else 0,
                _stream_handle(torch, dy.device))
    return dx


def wgrad(x, dy, p, dw=None, ws=None):
    """dw = weight gradient of device tensors x [N,H,W,C] and dy [N,Ho,Wo,K]."""
    import torch
    if dw is None:
        dw = torch.empty((p["k"], p["r"], p["s"], p["c"] // p.get("groups", 1)),
                         dtype=_storage_dtype(torch, p), device=x.device)
    need = cnhwc_workspace_size(p, OP_WGRAD)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    cnhwc_wgrad(p, x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                ws.data_ptr() if ws is not None else None,
                ws.numel() * ws.element_size() if ws is not None else 0,
                _stream_handle(torch, x.device))
    return dw
