"""fp64 CPU oracle for Exact Flow Linear Attention (EFLA).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  The product
library (``delta_rule_sequence_efla_amd``) never imports it and shares no code
with it.

The oracle is ``efla_oracle.c``: the token-by-token EFLA recurrence of the
"Exact Flow Linear Attention" summary pages (Method, steps 2-3), run in double
precision, plus the readout ``o_t = S_t^T q_t`` on the post-update state.  This
module compiles it with gcc and exposes it through ctypes on numpy float64
arrays.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against quantities computed by other routes (matrix exponential of the ODE,
RK4 integration, closed forms, high-precision evaluation of the coefficient).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "efla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libefla_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (no GPU, no HIP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC",
               "-shared", "-pthread", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_alpha.restype = ctypes.c_double
        lib.oracle_alpha.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.oracle_coeff.restype = ctypes.c_int
        lib.oracle_coeff.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [_D, _D, _D, _D, _D, _D, _D, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_step.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_coeff_rule.restype = ctypes.c_int
        lib.oracle_coeff_rule.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        lib.oracle_forward_rule.restype = ctypes.c_int
        lib.oracle_forward_rule.argtypes = [_D, _D, _D, _D, _D, _D, _D, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_step_rule.restype = ctypes.c_int
        lib.oracle_step_rule.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_alpha_grad.restype = ctypes.c_int
        lib.oracle_alpha_grad.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int, _D]
        lib.oracle_backward_rule.restype = ctypes.c_int
        lib.oracle_backward_rule.argtypes = [_D] * 12 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_int]
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def alpha(beta: float, lam: float) -> float:
    """alpha = (1 - exp(-beta*lam)) / lam, with its limit beta at lam == 0."""
    return float(_load().oracle_alpha(float(beta), float(lam)))


# update rules: the exact flow (Method step 3) or one explicit Euler step of
# length beta, the delta rule of DeltaNet (alpha = beta)
RULES = {"exact": 0, "euler": 1}


def _rule(rule) -> int:
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule!r}")
    return RULES[rule]


def coeff(k, beta, rule: str = "exact"):
    """lambda = ||k||^2 and alpha per token.  k [..., dk], beta [...]."""
    k = _f64(k)
    beta = _f64(beta)
    dk = k.shape[-1]
    n = int(np.prod(k.shape[:-1], dtype=np.int64))
    if beta.size != n:
        raise ValueError("beta must have one value per key row")
    lam = np.empty(n, np.float64)
    alp = np.empty(n, np.float64)
    rc = _load().oracle_coeff_rule(_p(k), _p(beta), _p(lam), _p(alp), n, dk, _rule(rule))
    if rc != 0:
        raise RuntimeError(f"oracle_coeff failed ({rc})")
    return lam.reshape(k.shape[:-1]), alp.reshape(k.shape[:-1])


def forward(q, k, v, beta, s0=None, nthreads: int | None = None, rule: str = "exact"):
    """Token-by-token EFLA over q,k [B,L,H,dk], v [B,L,H,dv], beta [B,L,H].

    s0 [B,H,dk,dv] or None (zeros).  Returns (o [B,L,H,dv], S_L [B,H,dk,dv]).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, L, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:3] != (B, L, H) or beta.shape != (B, L, H):
        raise ValueError("shape mismatch")
    if s0 is not None:
        s0 = _f64(s0)
        if s0.shape != (B, H, dk, dv):
            raise ValueError("s0 shape mismatch")
    o = np.empty((B, L, H, dv), np.float64)
    sf = np.empty((B, H, dk, dv), np.float64)
    nt = default_threads() if nthreads is None else int(nthreads)
    rc = _load().oracle_forward_rule(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(o),
                                     _p(sf), B, H, L, dk, dv, nt, _rule(rule))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed ({rc})")
    return o, sf


def alpha_grad(beta: float, lam: float, rule: str = "exact"):
    """(d alpha / d beta, d alpha / d lambda) of the coefficient under a rule."""
    out = np.empty(2, np.float64)
    if _load().oracle_alpha_grad(float(beta), float(lam), _rule(rule), _p(out)) != 0:
        raise RuntimeError("oracle_alpha_grad failed")
    return float(out[0]), float(out[1])


def backward(q, k, v, beta, s0, do, dsf=None, nthreads: int | None = None, rule: str = "exact"):
    """Gradients of a scalar loss through forward(): given do = dLoss/do
    [B,L,H,dv] and dsf = dLoss/dS_L [B,H,dk,dv] (None: zero), returns
    (dq, dk, dv, dbeta, ds0) with the shapes of q, k, v, beta and
    [B,H,dk,dv] (reverse-mode differentiation of the token recurrence)."""
    q, k, v, beta, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(do)
    B, L, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape[:3] != (B, L, H) or beta.shape != (B, L, H) or do.shape != v.shape:
        raise ValueError("shape mismatch")
    s0 = None if s0 is None else _f64(s0)
    dsf = None if dsf is None else _f64(dsf)
    for s in (s0, dsf):
        if s is not None and s.shape != (B, H, dk, dv):
            raise ValueError("state shape mismatch")
    gq, gk, gv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    gb = np.empty_like(beta)
    gs0 = np.empty((B, H, dk, dv), np.float64)
    nt = default_threads() if nthreads is None else int(nthreads)
    rc = _load().oracle_backward_rule(_p(q), _p(k), _p(v), _p(beta), _p(s0), _p(do), _p(dsf), _p(gq), _p(gk),
                                      _p(gv), _p(gb), _p(gs0), B, H, L, dk, dv, nt, _rule(rule))
    if rc != 0:
        raise RuntimeError(f"oracle_backward failed ({rc})")
    return gq, gk, gv, gb, gs0


def step(q, k, v, beta, state, rule: str = "exact"):
    """One decode step.  q,k [N,H,dk], v [N,H,dv], beta [N,H], state [N,H,dk,dv].

    Returns (o [N,H,dv], new_state); the input state is not modified.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    N, H, dk = k.shape
    dv = v.shape[-1]
    if st.shape != (N, H, dk, dv) or beta.shape != (N, H) or q.shape != k.shape:
        raise ValueError("shape mismatch")
    o = np.empty((N, H, dv), np.float64)
    rc = _load().oracle_step_rule(_p(q), _p(k), _p(v), _p(beta), _p(st), _p(o), N, H, dk, dv, _rule(rule))
    if rc != 0:
        raise RuntimeError(f"oracle_step failed ({rc})")
    return o, st


def forward_varlen(q, k, v, beta, cu_seqlens, s0=None, nthreads: int | None = None, rule: str = "exact"):
    """A packed variable-length batch: q, k [T,H,dk], v [T,H,dv], beta [T,H],
    offsets cu_seqlens [N+1].  Every sequence is an independent run of
    forward() from its own initial state s0[i] (or zeros).  Returns o [T,H,dv]
    (zeros for tokens outside every sequence) and the final states [N,H,dk,dv]."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    cu = np.asarray(cu_seqlens, dtype=np.int64).ravel()
    T, H, dk = k.shape
    dv = v.shape[-1]
    N = cu.size - 1
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    for i in range(N):
        a, e = int(cu[i]), int(cu[i + 1])
        si = None if s0 is None else _f64(s0)[i:i + 1]
        oi, sfi = forward(q[None, a:e], k[None, a:e], v[None, a:e], beta[None, a:e], si,
                          nthreads=nthreads, rule=rule)
        o[a:e] = oi[0]
        sf[i] = sfi[0]
    return o, sf
