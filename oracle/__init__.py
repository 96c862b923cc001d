"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library under ``linear_attention_token_gdn_amd``
never imports it and shares no code with it.

The arithmetic lives in ``gdn_oracle.c`` (plain token-by-token recurrence of
Eq. (1) on the explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app,
section "GDNの中身").  This module only builds that file with gcc, loads it
with ctypes and marshals numpy arrays.

Inputs are the stored values: fp32 arrays, or bf16 values widened exactly to
fp32.  Outputs are fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIB: another build of gdn_oracle.c (the sanitizer test loads an instrumented one)
_LIB = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so (gcc, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            f32p = ctypes.POINTER(ctypes.c_float)
            f64p = ctypes.POINTER(ctypes.c_double)
            i64p = ctypes.POINTER(ctypes.c_int64)
            lib.gdn_oracle_run.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, i64p, ctypes.c_int64,
                                           f64p, f64p, ctypes.c_int]
            lib.gdn_oracle_run.restype = ctypes.c_int
            lib.gdn_oracle_decode_step.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                                   f64p, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_double, ctypes.c_int]
            lib.gdn_oracle_decode_step.restype = ctypes.c_int
            lib.gdn_oracle_run_packed.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i64p,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_double, ctypes.c_uint, f64p, f64p,
                                                  ctypes.c_int]
            lib.gdn_oracle_run_packed.restype = ctypes.c_int
            lib.gdn_oracle_backward.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, f64p, f64p,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_double, f64p, f64p, f64p, f64p, f64p,
                                                f64p]
            lib.gdn_oracle_backward.restype = ctypes.c_int
            lib.gdn_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f32(a, shape):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def run(q, k, v, beta, g, s0=None, scale=1.0, chains=None, nthreads=0,
        want_state=True):
    """Recurrence of Eq. (1) over all T tokens.

    q, k: [B,T,Hk,dk]; v: [B,T,Hv,dv]; beta, g: [B,T,Hv] (g = log alpha);
    s0: [B,Hv,dk,dv] (any float dtype, widened to fp64) or None.  ``chains`` lists chain ids b*Hv+hv (None = all).
    Returns (o [n,T,dv] fp64, sT [n,dk,dv] fp64 or None), n = number of chains.
    With chains=None the results are reshaped to o [B,T,Hv,dv] and sT [B,Hv,dk,dv].
    """
    lib = _load()
    B, T, Hk, dk = np.shape(q)
    Hv, dv = np.shape(v)[2], np.shape(v)[3]
    q = _f32(q, (B, T, Hk, dk))
    k = _f32(k, (B, T, Hk, dk))
    v = _f32(v, (B, T, Hv, dv))
    beta = _f32(beta, (B, T, Hv))
    g = _f32(g, (B, T, Hv))
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (B, Hv, dk, dv):
            raise ValueError("s0 must have shape %s" % ((B, Hv, dk, dv),))
    if chains is None:
        n = B * Hv
        ch = None
    else:
        ch = np.ascontiguousarray(np.asarray(chains, dtype=np.int64).ravel())
        n = ch.size
    o = np.empty((n, T, dv), dtype=np.float64)
    sT = np.empty((n, dk, dv), dtype=np.float64) if want_state else None
    rc = lib.gdn_oracle_run(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                            _ptr(v, ctypes.c_float), _ptr(beta, ctypes.c_float),
                            _ptr(g, ctypes.c_float), _ptr(s0, ctypes.c_double),
                            B, T, Hk, Hv, dk, dv, float(scale),
                            _ptr(ch, ctypes.c_int64), n,
                            _ptr(o, ctypes.c_double), _ptr(sT, ctypes.c_double),
                            int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_run failed with code %d" % rc)
    if chains is None:
        o = o.reshape(B, Hv, T, dv).transpose(0, 2, 1, 3)
        if sT is not None:
            sT = sT.reshape(B, Hv, dk, dv)
    return o, sT


QK_L2NORM, BETA_LOGIT, G_LOGIT = 1, 2, 4  # input prologue flags


def backward(q, k, v, beta, g, dO, s0=None, dST=None, scale=1.0):
    """Gradients of the recurrence.  Shapes as ``run``; dO: [B,T,Hv,dv]; dST: [B,Hv,dk,dv]
    or None.  Returns dict dq, dk [B,T,Hk,dk], dv [B,T,Hv,dv], dbeta, dg [B,T,Hv],
    dS0 [B,Hv,dk,dv] (fp64; dg is the gradient w.r.t. g = log alpha)."""
    lib = _load()
    B, T, Hk, dk = np.shape(q)
    Hv, dv = np.shape(v)[2], np.shape(v)[3]
    q, k = _f32(q, (B, T, Hk, dk)), _f32(k, (B, T, Hk, dk))
    v = _f32(v, (B, T, Hv, dv))
    beta, g = _f32(beta, (B, T, Hv)), _f32(g, (B, T, Hv))
    f64 = lambda a, shape: None if a is None else np.ascontiguousarray(a, dtype=np.float64).reshape(shape)
    s0 = f64(s0, (B, Hv, dk, dv))
    dST = f64(dST, (B, Hv, dk, dv))
    dO = f64(dO, (B, T, Hv, dv))
    out = {"dq": np.empty((B, T, Hk, dk)), "dk": np.empty((B, T, Hk, dk)),
           "dv": np.empty((B, T, Hv, dv)), "dbeta": np.empty((B, T, Hv)),
           "dg": np.empty((B, T, Hv)), "dS0": np.empty((B, Hv, dk, dv))}
    p = lambda a: _ptr(a, ctypes.c_double)
    rc = lib.gdn_oracle_backward(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                 _ptr(v, ctypes.c_float), _ptr(beta, ctypes.c_float),
                                 _ptr(g, ctypes.c_float), p(s0), p(dO), p(dST), B, T, Hk, Hv,
                                 dk, dv, float(scale), p(out["dq"]), p(out["dk"]), p(out["dv"]),
                                 p(out["dbeta"]), p(out["dg"]), p(out["dS0"]))
    if rc != 0:
        raise RuntimeError("gdn_oracle_backward failed with code %d" % rc)
    return out


def run_packed(q, k, v, beta, g, cu_seqlens, s0=None, scale=1.0, flags=0, nthreads=0,
               want_state=True):
    """Packed sequences with the input prologue.  q, k: [T,Hk,dk]; v: [T,Hv,dv]; beta, g:
    [T,Hv]; cu_seqlens: N+1 offsets (sequence i = rows cu[i]..cu[i+1]-1); s0: [N,Hv,dk,dv] or
    None.  ``flags``: QK_L2NORM | BETA_LOGIT | G_LOGIT.  Returns (o [T,Hv,dv] fp64,
    sT [N,Hv,dk,dv] fp64 or None)."""
    lib = _load()
    T, Hk, dk = np.shape(q)
    Hv, dv = np.shape(v)[1], np.shape(v)[2]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).ravel())
    N = cu.size - 1
    q = _f32(q, (T, Hk, dk))
    k = _f32(k, (T, Hk, dk))
    v = _f32(v, (T, Hv, dv))
    beta = _f32(beta, (T, Hv))
    g = _f32(g, (T, Hv))
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (N, Hv, dk, dv):
            raise ValueError("s0 must have shape %s" % ((N, Hv, dk, dv),))
    o = np.empty((T, Hv, dv), dtype=np.float64)
    sT = np.empty((N, Hv, dk, dv), dtype=np.float64) if want_state else None
    rc = lib.gdn_oracle_run_packed(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                   _ptr(v, ctypes.c_float), _ptr(beta, ctypes.c_float),
                                   _ptr(g, ctypes.c_float), _ptr(s0, ctypes.c_double),
                                   _ptr(cu, ctypes.c_int64), N, T, Hk, Hv, dk, dv,
                                   float(scale), int(flags), _ptr(o, ctypes.c_double),
                                   _ptr(sT, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_run_packed failed with code %d" % rc)
    return o, sT


def decode_step(q, k, v, beta, g, state, scale=1.0, nthreads=0):
    """One token of Eq. (1) applied in place to ``state`` (fp64 [B,Hv,dk,dv]).

    q, k: [B,Hk,dk]; v: [B,Hv,dv]; beta, g: [B,Hv].  Returns o [B,Hv,dv] fp64.
    """
    lib = _load()
    B, Hk, dk = np.shape(q)
    Hv, dv = np.shape(v)[1], np.shape(v)[2]
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous and state.shape == (B, Hv, dk, dv)):
        raise ValueError("state must be a C-contiguous float64 array [B,Hv,dk,dv]")
    q = _f32(q, (B, Hk, dk))
    k = _f32(k, (B, Hk, dk))
    v = _f32(v, (B, Hv, dv))
    beta = _f32(beta, (B, Hv))
    g = _f32(g, (B, Hv))
    o = np.empty((B, Hv, dv), dtype=np.float64)
    rc = lib.gdn_oracle_decode_step(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                    _ptr(v, ctypes.c_float), _ptr(beta, ctypes.c_float),
                                    _ptr(g, ctypes.c_float), _ptr(state, ctypes.c_double),
                                    _ptr(o, ctypes.c_double), B, Hk, Hv, dk, dv,
                                    float(scale), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_decode_step failed with code %d" % rc)
    return o
