"""fp64 CPU oracle for Error-Free Linear Attention (EFLA) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
The product path (the HIP library and its Python binding) never imports, links or calls it.

The arithmetic lives in ``efla_oracle.c`` (plain C, double precision, token by token), built
into ``liboracle_efla.so`` with gcc; this module only marshals numpy arrays into it.

What it computes follows "Exact Flow Linear Attention: Exact Solution from Continuous-Time
Dynamics" (gist.science), Metodologia items 2-3, and "Error-Free Linear Attention is a Free
Lunch" (howistudyai.com), Steps 1-3 and the pipeline summary:
    alpha_t = (1 - exp(-beta_t ||k_t||^2)) / ||k_t||^2
    S_t     = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
    o_t     = S_t^T q_t
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "efla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_efla.so")

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile an oracle C source with gcc (-O2, OpenMP, no fast-math) into a shared library.  ``extra_flags``
    are added to the command (the sanitizer test builds an instrumented copy elsewhere with them)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", *extra_flags, src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one built oracle library (the default one is ``liboracle_efla.so``)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        lib.efla_oracle_alpha.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        lib.efla_oracle_alpha.restype = None
        lib.efla_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.efla_oracle_fwd.restype = ctypes.c_int
        lib.efla_oracle_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.efla_oracle_step.restype = ctypes.c_int
        lib.efla_oracle_ut.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.efla_oracle_ut.restype = ctypes.c_int
        lib.efla_oracle_bwd.argtypes = [_dp] * 12 + [ctypes.c_int] * 7
        lib.efla_oracle_bwd.restype = ctypes.c_int
        self.lib = lib

    def alpha(self, k, beta, gate=0):
        """alpha for keys k [..., d_k] and steps beta [...]; returns float64 [...].

        gate 0: the exact coefficient; gate p >= 1: the p-th order Runge-Kutta coefficient."""
        k = _f64(k)
        beta = _f64(beta)
        d_k = k.shape[-1]
        assert beta.shape == k.shape[:-1]
        out = np.empty(beta.shape, dtype=np.float64)
        self.lib.efla_oracle_alpha(_ptr(k), _ptr(beta), _ptr(out), int(beta.size), int(d_k), int(gate))
        return out

    def fwd(self, q, k, v, beta, initial_state=None, n_threads=0, want_o=True, want_state=True, gate=0):
        """Token-by-token recurrence over [B,H,L,*] inputs.

        Returns (o [B,H,L,d_v] float64 or None, final_state [B,H,d_k,d_v] float64 or None, threads).
        """
        q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
        B, H, L, d_k = k.shape
        d_v = v.shape[-1]
        assert q.shape == k.shape and v.shape[:3] == (B, H, L) and beta.shape == (B, H, L)
        s0 = None
        if initial_state is not None:
            s0 = _f64(initial_state)
            assert s0.shape == (B, H, d_k, d_v)
        o = np.empty((B, H, L, d_v), dtype=np.float64) if want_o else None
        sf = np.empty((B, H, d_k, d_v), dtype=np.float64) if want_state else None
        used = self.lib.efla_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(o), _ptr(sf),
                                        B, H, L, d_k, d_v, int(gate), int(n_threads))
        return o, sf, used

    def bwd(self, q, k, v, beta, initial_state, d_o, d_final=None, n_threads=0, gate=0):
        """Gradients of sum(o * d_o) + sum(S_L * d_final) with respect to q, k, v, beta and the initial state
        (the adjoint of the token recurrence, see efla_oracle_bwd).

        Returns (dq, dk, dv, dbeta, d_initial) as float64 arrays of the inputs' shapes ([B,H,d_k,d_v] for
        d_initial, also when initial_state is None)."""
        q, k, v, beta, d_o = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(d_o)
        B, H, L, d_k = k.shape
        d_v = v.shape[-1]
        assert q.shape == k.shape and v.shape[:3] == (B, H, L) and beta.shape == (B, H, L)
        assert d_o.shape == v.shape
        s0 = None if initial_state is None else _f64(initial_state)
        dsf = None if d_final is None else _f64(d_final)
        for x in (s0, dsf):
            assert x is None or x.shape == (B, H, d_k, d_v)
        dq, dk = np.empty_like(q), np.empty_like(k)
        dv, db = np.empty_like(v), np.empty_like(beta)
        ds0 = np.empty((B, H, d_k, d_v), dtype=np.float64)
        self.lib.efla_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s0), _ptr(d_o), _ptr(dsf),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(ds0), B, H, L, d_k, d_v, int(gate),
                                 int(n_threads))
        return dq, dk, dv, db, ds0

    def ut(self, k, beta, chunk, n_threads=0, gate=0):
        """Intra-chunk transform T diag(alpha), T = (I + strict_lower(diag(alpha) K K^T))^{-1}, per chunk.

        Returns float64 [B,H,ceil(L/chunk),chunk,chunk] (rows/columns past a short last chunk are zero).
        """
        k, beta = _f64(k), _f64(beta)
        B, H, L, d_k = k.shape
        assert beta.shape == (B, H, L)
        nc = (L + chunk - 1) // chunk
        out = np.empty((B, H, nc, chunk, chunk), dtype=np.float64)
        self.lib.efla_oracle_ut(_ptr(k), _ptr(beta), _ptr(out), B, H, L, d_k, int(chunk), int(gate), int(n_threads))
        return out

    def step(self, q, k, v, beta, state, n_threads=0, gate=0):
        """One decode step for [NH,*] inputs; ``state`` [NH,d_k,d_v] is copied, updated and returned.

        Returns (o [NH,d_v] float64, new_state float64, threads).
        """
        q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
        NH, d_k = k.shape
        d_v = v.shape[-1]
        s = np.array(state, dtype=np.float64, copy=True, order="C")
        assert s.shape == (NH, d_k, d_v) and beta.shape == (NH,)
        o = np.empty((NH, d_v), dtype=np.float64)
        used = self.lib.efla_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(s), _ptr(o),
                                         int(NH), int(d_k), int(d_v), int(gate), int(n_threads))
        return o, s, used


_default = None


def default() -> Oracle:
    """The oracle built from ``efla_oracle.c`` (built on first use if no library is there)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _default = Oracle(_LIB_PATH)
    return _default


def alpha(k, beta, gate=0):
    return default().alpha(k, beta, gate)


def fwd(q, k, v, beta, initial_state=None, n_threads=0, want_o=True, want_state=True, gate=0):
    return default().fwd(q, k, v, beta, initial_state, n_threads, want_o, want_state, gate)


def step(q, k, v, beta, state, n_threads=0, gate=0):
    return default().step(q, k, v, beta, state, n_threads, gate)


def bwd(q, k, v, beta, initial_state, d_o, d_final=None, n_threads=0, gate=0):
    return default().bwd(q, k, v, beta, initial_state, d_o, d_final, n_threads, gate)


def ut(k, beta, chunk, n_threads=0, gate=0):
    return default().ut(k, beta, chunk, n_threads, gate)


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)
