"""fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  It shares no code with the GPU library
(`gated_delta_rule_30_amd`) and never imports it.

Contents
  forward()        the token-by-token fp64 recurrence (kda_oracle.c), the
                   reference every parity test compares against.
  chunked          a second, independent fp64 CPU form (chunkwise), used to
                   pin the recurrence (any chunk size must give the same
                   result) -- see chunked.py.
  bruteforce       exact rational expansion for tiny cases -- see
                   bruteforce.py.
  parity_error()   the comparison metric: per (sequence, head) slice,
                   max|x - ref| / max|ref|.

Parity status of each function is stated in its own module header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP, no GPU code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.kda_oracle_forward.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int64, P, P, ctypes.c_int]
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_backward.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.kda_oracle_backward.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(_LIB)
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile a modified copy of the oracle source (used by the test that
    plants mistakes in the oracle to show the pins catch them) and return a
    forward() bound to it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", out_path, "-lm"],
                   check=True)
    lib = _bind(out_path)

    def fwd(*args, **kw):
        return forward(*args, _lib=lib, **kw)
    fwd.backward = lambda *args, **kw: backward(*args, _lib=lib, **kw)
    return fwd


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):          # torch tensor: widen on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, beta, g, S0=None, cu_seqlens=None, out_range=None, n_threads=0,
            want_state=True, _lib=None):
    """Run the fp64 recurrence.

    q, k, g: [T_total, H, d_k]; v: [T_total, H, d_v]; beta: [T_total, H];
    S0: [N, H, d_k, d_v] or None (zeros); cu_seqlens: [N+1] or None (one
    sequence).  Any float dtype (numpy or torch); values are widened to fp64
    exactly.  Returns (o [hi-lo, H, d_v] fp64 for packed tokens in
    out_range=(lo, hi), S_T [N, H, d_k, d_v] fp64 or None).
    """
    q, k, v, beta, g, S0 = (_f64(a) for a in (q, k, v, beta, g, S0))
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
    N = len(cu) - 1
    lo, hi = (0, T) if out_range is None else (int(out_range[0]), int(out_range[1]))
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape[:2] == (T, H)
    assert beta.shape == (T, H)
    if S0 is not None:
        assert S0.shape == (N, H, dk, dv)
    o = np.zeros((hi - lo, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64) if want_state else None
    lib = _lib if _lib is not None else _load()
    rc = lib.kda_oracle_forward(T, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                    _ptr(S0), _ptr(cu), lo, hi, _ptr(o), _ptr(ST), int(n_threads))
    if rc != 0:
        raise ValueError("kda_oracle_forward failed with code %d" % rc)
    return o, ST


def backward(q, k, v, beta, g, dO, S0=None, dS_T=None, cu_seqlens=None, n_threads=0, _lib=None):
    """Gradients of the fp64 recurrence for output gradients dO [T_total, H,
    d_v] and final-state gradients dS_T [N, H, d_k, d_v] (None = zeros).
    Returns dict(dq, dk, dv, dbeta, dg, dS0) in fp64 (dg is the gradient of
    log alpha)."""
    q, k, v, beta, g, S0, dO, dS_T = (_f64(a) for a in (q, k, v, beta, g, S0, dO, dS_T))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = (np.array([0, T], dtype=np.int64) if cu_seqlens is None
          else np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64))
    N = len(cu) - 1
    assert dO.shape == (T, H, dv)
    if dS_T is not None:
        assert dS_T.shape == (N, H, dk, dv)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dbeta=np.zeros((T, H)), dg=np.zeros((T, H, dk)), dS0=np.zeros((N, H, dk, dv)))
    lib = _lib if _lib is not None else _load()
    rc = lib.kda_oracle_backward(T, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0),
                                 _ptr(cu), _ptr(dO), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]),
                                 _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dg"]), _ptr(out["dS0"]),
                                 int(n_threads))
    if rc != 0:
        raise ValueError("kda_oracle_backward failed with code %d" % rc)
    return out


def parity_error(x, ref, cu_seqlens=None, token_axis=0, head_axis=1, floor=1e-30):
    """Worst per-(sequence, head) slice of max|x - ref| / max(max|ref|, floor).

    For o-shaped arrays [T, H, d] slices are (sequence, head); pass
    cu_seqlens=None to treat all tokens as one sequence.  For state-shaped
    arrays [N, H, dk, dv] call with cu_seqlens=None, token_axis=0 meaning
    sequence axis (each [n, h] slice is one state).  `floor` keeps a slice
    whose reference has decayed below any fp32-meaningful scale (a state
    decayed by e^-750 is ~1e-326) from turning rounding to zero into a
    relative error of 1.  Any non-finite value in `x` gives inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if cu_seqlens is None:
        bounds = [(i, i + 1) for i in range(x.shape[token_axis])] if x.ndim == 4 else [(0, x.shape[0])]
    else:
        cu = np.asarray(cu_seqlens)
        bounds = [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    worst = 0.0
    for (a, b) in bounds:
        if b <= a:
            continue
        xs = np.take(x, range(a, b), axis=token_axis)
        rs = np.take(ref, range(a, b), axis=token_axis)
        for h in range(x.shape[head_axis]):
            xh = np.take(xs, h, axis=head_axis)
            rh = np.take(rs, h, axis=head_axis)
            if not np.all(np.isfinite(xh)):
                return float("inf")
            den = max(float(np.max(np.abs(rh))), floor)
            num = float(np.max(np.abs(xh - rh)))
            worst = max(worst, num / den)
    return worst
