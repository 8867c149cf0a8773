"""fp64 CPU oracle for HYPIC's linear-attention state algebra.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  The GPU
library never calls it, and it shares no code with the GPU library.

Two independent implementations live here:

* ``liboracle.so`` (``hypic_oracle.c``): the plain token-by-token recurrence,
  fp64, OpenMP over independent (segment, head) / (chain, head) units;
* :mod:`oracle.brute`: numpy brute force that forms every token transition
  matrix explicitly and multiplies the ordered products out (tiny inputs only);
* :func:`compose_gemm`: the composition with numpy's fp64 matrix product per
  step (for request batches too large for the C loop), pinned to the C routine.

Sources are cited by short key, as in ``hypic_oracle.c``: [ZH] is the Chinese
page "首 token 延迟降 3.25 倍！…HYPIC…" (sections 2.1 linear layers, 2.2 seam
windows); [ES] is the Spanish page "…presentan HYPIC…".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hypic_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GATE_HEAD, GATE_TOKEN, GATE_DIAG = 0, 1, 2


class _Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("delta", ctypes.c_int32)]


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_build.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, P, P, P, P, P, P, P, P]
        lib.oracle_run.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.c_int64,
                                   P, P, P, P, P, ctypes.c_double, P, P]
        lib.oracle_compose.argtypes = [ctypes.c_int32] * 6 + [P, P, P, P]
        lib.oracle_seam_advance.argtypes = ([ctypes.POINTER(_Dims), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, P, P, P, P, P, P, ctypes.c_double, P,
                                             ctypes.c_int32, P, P, P, P])
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(H, dk, dv, gate, delta):
    return _Dims(int(H), int(dk), int(dv), int(gate), int(delta))


def _check_tokens(k, v, H, dk, dv):
    assert k.ndim == 3 and k.shape[1:] == (H, dk), k.shape
    assert v.ndim == 3 and v.shape[1:] == (H, dv) and v.shape[0] == k.shape[0], v.shape


def segment_build(k, v, g, beta, seg_begin, seg_end, *, gate: int, delta: int, want_T: bool = True):
    """(T_C, S(C|0)) per (segment, head) by the token recurrence ([ZH] 2.1).

    Returns ``T`` [n_seg, H, d_k, d_k] (or None) and ``S`` [n_seg, H, d_k, d_v].
    """
    k, v = _f64(k), _f64(v)
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    _check_tokens(k, v, H, dk, dv)
    g = _f64(g)
    beta = _f64(beta) if beta is not None else np.zeros((n_tok, H))
    sb = np.ascontiguousarray(np.asarray(seg_begin, dtype=np.int64))
    se = np.ascontiguousarray(np.asarray(seg_end, dtype=np.int64))
    assert sb.shape == se.shape and np.all(sb >= 0) and np.all(se <= n_tok) and np.all(se >= sb)
    n_seg = sb.shape[0]
    T = np.empty((n_seg, H, dk, dk)) if want_T else None
    S = np.empty((n_seg, H, dk, dv))
    d = _dims(H, dk, dv, gate, delta)
    _load().oracle_build(ctypes.byref(d), n_seg, _ptr(sb), _ptr(se), _ptr(k), _ptr(v), _ptr(g),
                         _ptr(beta), _ptr(T), _ptr(S))
    return T, S


def run(k, v, g, beta, *, gate: int, delta: int, t0: int = 0, t1: int | None = None,
        S0=None, q=None, scale: float = 1.0):
    """Plain recurrence over tokens [t0, t1) from state S0 (default 0).

    Returns (S_final [H, d_k, d_v], outputs [t1 - t0, H, d_v] or None).
    """
    k, v = _f64(k), _f64(v)
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    _check_tokens(k, v, H, dk, dv)
    t1 = n_tok if t1 is None else t1
    assert 0 <= t0 <= t1 <= n_tok
    g = _f64(g)
    beta = _f64(beta) if beta is not None else np.zeros((n_tok, H))
    S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True, order="C")
    q = _f64(q)
    out = np.empty((t1 - t0, H, dv)) if q is not None else None
    d = _dims(H, dk, dv, gate, delta)
    _load().oracle_run(ctypes.byref(d), t0, t1, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                       float(scale), _ptr(S), _ptr(out))
    return S, out


def compose(T_cache, S_cache, pair_id, S_run=None, *, t_scalar: bool = False):
    """Ordered composition S_run <- T[id] S_run + S[id] along each chain ([ZH] 2.1).

    ``pair_id`` is [n_chain, n_step] (id < 0 skips); S_run is [n_chain, H, d_k, d_v]
    (default zeros).  Returns the new S_run (a copy).
    """
    S_cache = _f64(S_cache)
    T_cache = _f64(T_cache)
    n_pair, H, dk, dv = S_cache.shape
    ids = np.ascontiguousarray(np.asarray(pair_id, dtype=np.int32))
    n_chain, n_step = ids.shape
    assert np.all(ids < n_pair)
    if t_scalar:
        assert T_cache.shape == (n_pair, H)
    else:
        assert T_cache.shape == (n_pair, H, dk, dk)
    R = (np.zeros((n_chain, H, dk, dv)) if S_run is None
         else np.array(S_run, dtype=np.float64, copy=True, order="C"))
    _load().oracle_compose(H, dk, dv, int(bool(t_scalar)), n_chain, n_step, _ptr(ids), _ptr(T_cache),
                           _ptr(S_cache), _ptr(R))
    return R


def compose_gemm(T_cache, S_cache, pair_id, S_run=None, *, workers: int | None = None):
    """The composition of :func:`compose` -- S_run <- T[id] S_run + S[id] for every step of
    every chain, in order ([ZH] 2.1: left-multiply by the cached T_C, then add S(C|0)) --
    with each step's product taken by numpy's fp64 matrix product over all heads at once.
    Chains are independent and run on a thread pool (one BLAS thread each).  For chain sets
    that the token-loop C routine would take minutes over (a batch of requests composing
    hundreds of cached segments); the tests pin it to :func:`compose`.

    ``pair_id`` [n_chain, n_step] (id < 0 skips); T_cache [n_pair, H, d_k, d_k] (dense),
    S_cache [n_pair, H, d_k, d_v]; S_run [n_chain, H, d_k, d_v] (default zeros).  Returns the
    new S_run (a copy)."""
    import concurrent.futures

    from threadpoolctl import threadpool_limits

    S_cache = _f64(S_cache)
    T_cache = _f64(T_cache)
    n_pair, H, dk, dv = S_cache.shape
    assert T_cache.shape == (n_pair, H, dk, dk)
    ids = np.ascontiguousarray(np.asarray(pair_id, dtype=np.int64))
    n_chain, n_step = ids.shape
    assert np.all(ids < n_pair)
    R = (np.zeros((n_chain, H, dk, dv)) if S_run is None
         else np.array(S_run, dtype=np.float64, copy=True, order="C"))

    def chain(c):
        r, nxt = R[c].copy(), np.empty_like(R[c])
        for j in range(n_step):
            i = ids[c, j]
            if i >= 0:
                np.matmul(T_cache[i], r, out=nxt)
                nxt += S_cache[i]
                r, nxt = nxt, r
        R[c] = r

    n_workers = workers or min(16, os.cpu_count() or 1)
    with threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(n_workers) as ex:
            list(ex.map(chain, range(n_chain)))
    return R


def seam_advance(q, k, v, g, beta, seam_start, *, gate: int, delta: int, w: int, scale: float,
                 pair_id=None, T_cache=None, S_cache=None, S_run=None, t_scalar: bool = False):
    """Seam windows then composition, step by step along each chain ([ZH] 2.2).

    Returns (S_run [n_chain, H, d_k, d_v], out [n_chain, n_step, w, H, d_v]);
    out rows of steps without a seam are NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    _check_tokens(k, v, H, dk, dv)
    g = _f64(g)
    beta = _f64(beta) if beta is not None else np.zeros((n_tok, H))
    ss = np.ascontiguousarray(np.asarray(seam_start, dtype=np.int64))
    n_chain, n_step = ss.shape
    assert np.all((ss < 0) | (ss + w <= n_tok))
    ids = None
    if pair_id is not None:
        ids = np.ascontiguousarray(np.asarray(pair_id, dtype=np.int32))
        assert ids.shape == ss.shape
        T_cache, S_cache = _f64(T_cache), _f64(S_cache)
    R = (np.zeros((n_chain, H, dk, dv)) if S_run is None
         else np.array(S_run, dtype=np.float64, copy=True, order="C"))
    out = np.full((n_chain, n_step, w, H, dv), np.nan)
    d = _dims(H, dk, dv, gate, delta)
    _load().oracle_seam_advance(ctypes.byref(d), n_chain, n_step, w, _ptr(ss), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(ids),
                                int(bool(t_scalar)), _ptr(T_cache), _ptr(S_cache), _ptr(R),
                                _ptr(out))
    return R, out


def naive_sum(S_cache, pair_id):
    """The strawman the pages reject ([ZH] 2.1): add the zero-initial final
    states, dropping T.  Exact only for plain linear attention."""
    S_cache = _f64(S_cache)
    ids = np.asarray(pair_id)
    n_chain = ids.shape[0]
    out = np.zeros((n_chain,) + S_cache.shape[1:])
    for c in range(n_chain):
        for i in ids[c]:
            if i >= 0:
                out[c] += S_cache[i]
    return out


def rel_f(x, ref):
    """Relative Frobenius error ||x - ref||_F / ||ref||_F over the last two axes."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    return num / np.where(den == 0, 1.0, den)
