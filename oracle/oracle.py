"""ctypes front end of the fp64 C oracle in ``oracle.c`` (test infrastructure only).

``conv_fwd``, ``conv_dgrad`` and ``conv_wgrad`` take and return float64 numpy arrays in NHWC
(activations) and KRSC (weights) layout and compute the plain definitions given
in ``oracle.c``.  ``build`` compiles the C file with gcc (OpenMP) into
``oracle/_build``; a deliberate-mistake variant can be built with ``mutation``
so the tests can show that their pins catch it.
"""
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_libs = {}
_lock = threading.Lock()


def _lib_path(mutation):
    name = "liboracle.so" if mutation == 0 else "liboracle_mut%d.so" % mutation
    return os.path.join(_BUILD, name)


def build(mutation=0, force=False):
    """Compile oracle.c (gcc -O2 -fopenmp, no fast-math) and return the .so path."""
    out = _lib_path(mutation)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    os.makedirs(_BUILD, exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-DORACLE_MUTATION=%d" % mutation, _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib(mutation=0):
    with _lock:
        if mutation not in _libs:
            lib = ctypes.CDLL(build(mutation))
            i64 = ctypes.c_int64
            dp = ctypes.POINTER(ctypes.c_double)
            for fn in ("oracle_conv_fwd_f64", "oracle_conv_dgrad_f64", "oracle_conv_wgrad_f64"):
                f = getattr(lib, fn)
                f.argtypes = [i64] * 11 + [dp, dp, dp]
                f.restype = ctypes.c_int
            lib.oracle_out_dims.argtypes = [i64] * 11 + [ctypes.POINTER(i64)] * 2
            lib.oracle_out_dims.restype = ctypes.c_int
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            _libs[mutation] = lib
        return _libs[mutation]


def _dims(p):
    return [int(p[k]) for k in ("n", "h", "w", "c", "k", "r", "s", "stride",
                                "pad_h", "pad_w", "groups")]


def out_dims(p):
    """(Ho, Wo) of problem dict ``p`` by the floor formula, or ValueError."""
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    if _lib().oracle_out_dims(*_dims(p), ctypes.byref(ho), ctypes.byref(wo)):
        raise ValueError("invalid convolution problem %r" % (p,))
    return ho.value, wo.value


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def conv_fwd(x, w, p, mutation=0):
    """y[N,Ho,Wo,K] = forward cross-correlation of x[N,H,W,C] with w[K,R,S,C/G]."""
    ho, wo = out_dims(p)
    x, w = _f64(x), _f64(w)
    assert x.shape == (p["n"], p["h"], p["w"], p["c"]), x.shape
    assert w.shape == (p["k"], p["r"], p["s"], p["c"] // p["groups"]), w.shape
    y = np.empty((p["n"], ho, wo, p["k"]), dtype=np.float64)
    if _lib(mutation).oracle_conv_fwd_f64(*_dims(p), _ptr(x), _ptr(w), _ptr(y)):
        raise ValueError("oracle refused %r" % (p,))
    return y


def conv_dgrad(dy, w, p, mutation=0):
    """dx[N,H,W,C] = adjoint of the forward map applied to dy[N,Ho,Wo,K]."""
    ho, wo = out_dims(p)
    dy, w = _f64(dy), _f64(w)
    assert dy.shape == (p["n"], ho, wo, p["k"]), dy.shape
    assert w.shape == (p["k"], p["r"], p["s"], p["c"] // p["groups"]), w.shape
    dx = np.empty((p["n"], p["h"], p["w"], p["c"]), dtype=np.float64)
    if _lib(mutation).oracle_conv_dgrad_f64(*_dims(p), _ptr(dy), _ptr(w), _ptr(dx)):
        raise ValueError("oracle refused %r" % (p,))
    return dx


def conv_wgrad(x, dy, p, mutation=0):
    """dw[K,R,S,C/G] = gradient of the forward map with respect to the weight,
    for input x[N,H,W,C] and output gradient dy[N,Ho,Wo,K]."""
    ho, wo = out_dims(p)
    x, dy = _f64(x), _f64(dy)
    assert x.shape == (p["n"], p["h"], p["w"], p["c"]), x.shape
    assert dy.shape == (p["n"], ho, wo, p["k"]), dy.shape
    dw = np.empty((p["k"], p["r"], p["s"], p["c"] // p["groups"]), dtype=np.float64)
    if _lib(mutation).oracle_conv_wgrad_f64(*_dims(p), _ptr(x), _ptr(dy), _ptr(dw)):
        raise ValueError("oracle refused %r" % (p,))
    return dw


def num_threads():
    return int(_lib().oracle_num_threads())


def set_num_threads(n):
    _lib().oracle_set_num_threads(int(n))
