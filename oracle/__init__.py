"""fp64 CPU oracle for SANATAN attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The GPU library never links, loads or calls it, and it shares no
code with the GPU library; the two meet only on the seeded inputs of ``sanatan_inputs``.

The arithmetic lives in ``oracle.c`` (plain C, IEEE binary64, no fast-math); this module is
ctypes marshalling plus numpy shape handling.  See ``oracle.c`` for the definitions and the
passages of the SANATAN reading notes (page 1) and forum post (page 2) each follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GAMMA = 4.0
LAMBDA_BASE = 10000.0
EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O3, OpenMP, no fast-math, no FMA contraction).  The target is
    x86-64-v3 (AVX2), not -march=native: the library is built on one machine and run on another machine's host
    CPU.  Without fast-math and with contraction off, the vector code gives the same results as scalar code."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    i64 = ctypes.c_int64
    lib.oracle_angle.restype = ctypes.c_double
    lib.oracle_angle.argtypes = [ctypes.c_double]
    lib.oracle_root.restype = ctypes.c_double
    lib.oracle_root.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.oracle_freq.restype = ctypes.c_double
    lib.oracle_freq.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double]
    lib.oracle_features.restype = None
    lib.oracle_features.argtypes = [dp, ctypes.c_int, ctypes.c_int, i64, dp, ctypes.c_double, ctypes.c_double, dp]
    lib.oracle_kappa.restype = ctypes.c_double
    lib.oracle_kappa.argtypes = [dp, dp, ctypes.c_int, i64, i64, dp, ctypes.c_double, ctypes.c_double]
    lib.oracle_attention_direct.restype = None
    lib.oracle_attention_direct.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, dp,
                                            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                            ctypes.c_int, ip, ctypes.c_int, dp]
    lib.oracle_attention_direct4.restype = None
    lib.oracle_attention_direct4.argtypes = lib.oracle_attention_direct.argtypes
    lib.oracle_kappa4.restype = ctypes.c_double
    lib.oracle_kappa4.argtypes = lib.oracle_kappa.argtypes
    lib.oracle_recurrent.restype = None
    lib.oracle_recurrent.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, dp,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     dp, dp, dp]
    lib.oracle_recurrent_heads.restype = None
    lib.oracle_recurrent_heads.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           i64, dp, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_double, dp, dp, dp]
    lib.oracle_features_h.restype = None
    lib.oracle_features_h.argtypes = [dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, dp, ctypes.c_double,
                                      ctypes.c_double, dp]
    lib.oracle_kappa_h.restype = ctypes.c_double
    lib.oracle_kappa_h.argtypes = [dp, dp, ctypes.c_int, ctypes.c_int, i64, i64, dp, ctypes.c_double, ctypes.c_double]
    lib.oracle_attention_direct_h.restype = None
    lib.oracle_attention_direct_h.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double, ip,
                                              ctypes.c_int, dp]
    lib.oracle_recurrent_h.restype = None
    lib.oracle_recurrent_h.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, dp,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double, dp, dp, dp]
    lib.oracle_attention_direct_grad.restype = None
    lib.oracle_attention_direct_grad.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp,
                                                 ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                                 ctypes.c_double, ctypes.c_int, dp, dp, dp, dp]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def angle(u: float) -> float:
    return float(_load().oracle_angle(float(u)))


def root(u: float, omega: float, gamma: float = GAMMA) -> float:
    return float(_load().oracle_root(float(u), float(omega), float(gamma)))


def freq(a: int, d: int, base: float = LAMBDA_BASE) -> float:
    return float(_load().oracle_freq(int(a), int(d), float(base)))


def features(u, pos0: int, omega, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE) -> np.ndarray:
    """Phi of rows u[T, d] at positions pos0.. -> [T, 6d], channel-major (row c*d + a)."""
    u = _f64(u)
    T, d = u.shape
    om = _f64(omega).reshape(d)
    out = np.empty((T, 6 * d), dtype=np.float64)
    _load().oracle_features(_ptr(u), T, d, int(pos0), _ptr(om), float(gamma), float(lambda_base), _ptr(out))
    return out


def kappa(q, k, t: int, s: int, omega, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE) -> float:
    q = _f64(q).ravel()
    k = _f64(k).ravel()
    om = _f64(omega).ravel()
    return float(_load().oracle_kappa(_ptr(q), _ptr(k), q.size, int(t), int(s), _ptr(om), float(gamma),
                                      float(lambda_base)))


def kappa4(q, k, t: int, s: int, omega, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE) -> float:
    """The unclipped four-channel kernel of one (t, s) pair: sum_a 1 + r_q r_k (1 + cos dtheta)."""
    q = _f64(q).ravel()
    k = _f64(k).ravel()
    om = _f64(omega).ravel()
    return float(_load().oracle_kappa4(_ptr(q), _ptr(k), q.size, int(t), int(s), _ptr(om), float(gamma),
                                       float(lambda_base)))


def attention_direct(q, k, v, omega, pos0: int = 0, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
                     c: float | None = None, eps: float = EPS, p: int = 1, rows=None,
                     four_channel: bool = False) -> np.ndarray:
    """Direct-kappa normalised causal attention for ONE head: q,k [T,d], v [T,dv].  With four_channel, the
    unclipped four-channel kernel (kappa4) replaces the six-channel one."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, d = q.shape
    dv = v.shape[1]
    if c is None:
        c = 4.0 * d
    om = _f64(omega).reshape(d)
    if rows is None:
        out = np.empty((T, dv), dtype=np.float64)
        rp, nr = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        if r.size and (r.min() < 0 or r.max() >= T):
            raise ValueError("row index out of range")
        out = np.empty((r.size, dv), dtype=np.float64)
        rp, nr = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), int(r.size)
    fn = _load().oracle_attention_direct4 if four_channel else _load().oracle_attention_direct
    fn(_ptr(q), _ptr(k), _ptr(v), T, d, dv, int(pos0), _ptr(om), float(gamma), float(lambda_base), float(c),
       float(eps), int(p), rp, nr, _ptr(out))
    return out


def recurrent(q, k, v, omega, pos0: int = 0, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
              c: float | None = None, eps: float = EPS, S=None, z=None, want_out: bool = True):
    """p=1 recurrence for ONE head. Returns (out [T,dv] or None, S [6d,dv], z [6d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, d = k.shape
    dv = v.shape[1]
    if c is None:
        c = 4.0 * d
    S = np.zeros((6 * d, dv)) if S is None else _f64(S).copy()
    z = np.zeros((6 * d,)) if z is None else _f64(z).copy()
    out = np.empty((T, dv), dtype=np.float64) if want_out else None
    _load().oracle_recurrent(_ptr(q), _ptr(k), _ptr(v), T, d, dv, int(pos0), _ptr(_f64(omega).reshape(d)),
                             float(gamma), float(lambda_base), float(c), float(eps), _ptr(S), _ptr(z),
                             _ptr(out) if want_out else None)
    return out, S, z


def recurrent_heads(q, k, v, omega, pos0: int = 0, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
                    c: float | None = None, eps: float = EPS, S=None, z=None, want_out: bool = True):
    """p=1 recurrence over NH independent heads (OpenMP over heads).

    q,k [NH,T,d], v [NH,T,dv], omega [n_param_heads, d] (head j uses row j % n_param_heads).
    Returns (out [NH,T,dv] or None, S [NH,6d,dv], z [NH,6d]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    NH, T, d = k.shape
    dv = v.shape[2]
    if c is None:
        c = 4.0 * d
    om = _f64(omega).reshape(-1, d)
    S = np.zeros((NH, 6 * d, dv)) if S is None else _f64(S).copy()
    z = np.zeros((NH, 6 * d)) if z is None else _f64(z).copy()
    out = np.empty((NH, T, dv), dtype=np.float64) if want_out else None
    _load().oracle_recurrent_heads(_ptr(q), _ptr(k), _ptr(v), NH, T, d, dv, int(pos0), _ptr(om), om.shape[0],
                                   float(gamma), float(lambda_base), float(c), float(eps), _ptr(S), _ptr(z),
                                   _ptr(out) if want_out else None)
    return out, S, z


def attention_direct_grad(q, k, v, dout, omega, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
                          c: float | None = None, eps: float = EPS, p: int = 1):
    """Gradient of sum_t <dout_t, o_t> of the direct form for ONE head: q,k [T,d], v,dout [T,dv], omega [d].
    Returns (dq [T,d], dk [T,d], dv [T,dv], domega [d])."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, d = q.shape
    dv = v.shape[1]
    if c is None:
        c = 4.0 * d
    om = _f64(omega).reshape(d)
    dq, dk = np.empty((T, d)), np.empty((T, d))
    dvv, dom = np.empty((T, dv)), np.empty((d,))
    _load().oracle_attention_direct_grad(_ptr(q), _ptr(k), _ptr(v), _ptr(g), T, d, dv, _ptr(om), float(gamma),
                                         float(lambda_base), float(c), float(eps), int(p), _ptr(dq), _ptr(dk),
                                         _ptr(dvv), _ptr(dom))
    return dq, dk, dvv, dom


def features_h(u, pos0: int, omega, nh: int, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE) -> np.ndarray:
    """Phi_h (spectral harmonics n = 1..nh) of rows u[T, d] at positions pos0.. -> [T, (2 + 4 nh) d]."""
    u = _f64(u)
    T, d = u.shape
    out = np.empty((T, (2 + 4 * nh) * d), dtype=np.float64)
    _load().oracle_features_h(_ptr(u), T, d, int(nh), int(pos0), _ptr(_f64(omega).reshape(d)), float(gamma),
                              float(lambda_base), _ptr(out))
    return out


def kappa_h(q, k, t: int, s: int, omega, nh: int, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE) -> float:
    q, k, om = _f64(q).ravel(), _f64(k).ravel(), _f64(omega).ravel()
    return float(_load().oracle_kappa_h(_ptr(q), _ptr(k), q.size, int(nh), int(t), int(s), _ptr(om), float(gamma),
                                        float(lambda_base)))


def attention_direct_h(q, k, v, omega, nh: int, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
                       c: float | None = None, eps: float = EPS, rows=None) -> np.ndarray:
    """Direct-kappa_h normalised causal p = 1 attention for ONE head (spectral harmonics n = 1..nh)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, d = q.shape
    dv = v.shape[1]
    if c is None:
        c = 4.0 * d
    if rows is None:
        out = np.empty((T, dv))
        rp, nr = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        out = np.empty((r.size, dv))
        rp, nr = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), int(r.size)
    _load().oracle_attention_direct_h(_ptr(q), _ptr(k), _ptr(v), T, d, dv, int(nh), _ptr(_f64(omega).reshape(d)),
                                      float(gamma), float(lambda_base), float(c), float(eps), rp, nr, _ptr(out))
    return out


def recurrent_h(q, k, v, omega, nh: int, pos0: int = 0, gamma: float = GAMMA, lambda_base: float = LAMBDA_BASE,
                c: float | None = None, eps: float = EPS, S=None, z=None, want_out: bool = True):
    """p = 1 recurrence on Phi_h for ONE head.  Returns (out [T,dv] or None, S [(2+4nh)d, dv], z [(2+4nh)d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, d = k.shape
    dv = v.shape[1]
    if c is None:
        c = 4.0 * d
    D = (2 + 4 * nh) * d
    S = np.zeros((D, dv)) if S is None else _f64(S).copy()
    z = np.zeros((D,)) if z is None else _f64(z).copy()
    out = np.empty((T, dv)) if want_out else None
    _load().oracle_recurrent_h(_ptr(q), _ptr(k), _ptr(v), T, d, dv, int(nh), int(pos0), _ptr(_f64(omega).reshape(d)),
                               float(gamma), float(lambda_base), float(c), float(eps), _ptr(S), _ptr(z),
                               _ptr(out) if want_out else None)
    return out, S, z
