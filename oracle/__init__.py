"""fp64 CPU oracle of the Kimi Delta Attention recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU path (``gated_delta_rule_18_amd``)
and imports nothing from it.

The arithmetic lives in ``kda_oracle.c`` (plain sequential loops in double
precision; see its header for the cited passages).  This module only converts
numpy arrays to contiguous float64 and calls the C entry points through ctypes.

Functions
---------
prefill(q, k, v, g, beta, S0=None, nthreads=None) -> (o, S_T)
    q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; S0 [B,H,dk,dv] or None.
prefill_snapshots(q, k, v, g, beta, S0, snap_every, n_snaps, nthreads=None) -> (o, S_T, snaps)
    as prefill, plus snaps [n_snaps,B,H,dk,dv]: snapshot s is the state after the
    first (s + 1) * snap_every tokens.
prefill_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit,
             eps=1e-6, nthreads=None) -> (q, k, v, g, beta, conv_final)
    q_pre, k_pre, z [B,T,H,dk]; v_pre [B,T,H,dv]; beta_logit [B,T,H];
    conv_w [H,2dk+dv,width]; A [H]; conv_init [B,H,width-1,2dk+dv] (oldest
    first) or None for a zero history.  conv_final holds the last width-1
    pre-activations, oldest first.
decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S,
            eps=1e-6, nthreads=None) -> o
    conv_cache and S are updated in place (they must be float64 C-contiguous
    arrays owned by the caller).
output_gate(o, gate, w=None, eps=1e-6) -> y
    o, gate [..., H, dv]; w [dv] or None (ones).  y = Sigmoid(gate) * RMSNorm(o) * w,
    the RMSNorm taken over the dv channels of each (row, head).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
L2NORM_EPS = 1e-6
RMSNORM_EPS = 1e-6


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_prefill.argtypes = [_dp] * 8 + [ctypes.c_long] * 5 + [ctypes.c_int]
        lib.kda_oracle_prefill_snapshots.restype = ctypes.c_int
        lib.kda_oracle_prefill_snapshots.argtypes = [_dp] * 9 + [ctypes.c_long] * 7 + [ctypes.c_int]
        lib.kda_oracle_prefill_prep.restype = ctypes.c_int
        lib.kda_oracle_prefill_prep.argtypes = (
            [_dp] * 14 + [ctypes.c_long] * 6 + [ctypes.c_double, ctypes.c_int])
        lib.kda_oracle_output_gate.restype = ctypes.c_int
        lib.kda_oracle_output_gate.argtypes = [_dp] * 4 + [ctypes.c_long] * 3 + [ctypes.c_double]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = (
            [_dp] * 5 + [ctypes.c_long] + [_dp] * 4 + [ctypes.c_long] * 5 + [ctypes.c_double, ctypes.c_int])
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads():
    return max(1, min(os.cpu_count() or 1, 16))


def prefill(q, k, v, g, beta, S0=None, nthreads=None):
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("oracle.prefill: inconsistent shapes")
    S0a = None if S0 is None else _f64(S0)
    if S0a is not None and S0a.shape != (B, H, dk, dv):
        raise ValueError("oracle.prefill: S0 shape")
    o = np.empty((B, T, H, dv))
    S_T = np.empty((B, H, dk, dv))
    rc = _load().kda_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0a),
                                    _ptr(o), _ptr(S_T), B, T, H, dk, dv,
                                    nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill failed ({rc})")
    return o, S_T


def prefill_snapshots(q, k, v, g, beta, S0, snap_every, n_snaps, nthreads=None):
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("oracle.prefill_snapshots: inconsistent shapes")
    S0a = None if S0 is None else _f64(S0)
    if S0a is not None and S0a.shape != (B, H, dk, dv):
        raise ValueError("oracle.prefill_snapshots: S0 shape")
    o = np.empty((B, T, H, dv))
    S_T = np.empty((B, H, dk, dv))
    snaps = np.empty((n_snaps, B, H, dk, dv))
    rc = _load().kda_oracle_prefill_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0a),
                                              _ptr(o), _ptr(S_T), _ptr(snaps), int(snap_every), int(n_snaps),
                                              B, T, H, dk, dv, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill_snapshots failed ({rc})")
    return o, S_T, snaps


def prefill_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit,
                 eps=L2NORM_EPS, nthreads=None):
    q_pre, k_pre, v_pre, conv_w, z, A, beta_logit = (
        _f64(x) for x in (q_pre, k_pre, v_pre, conv_w, z, A, beta_logit))
    B, T, H, dk = q_pre.shape
    dv = v_pre.shape[-1]
    width = conv_w.shape[-1]
    nch = 2 * dk + dv
    init = None if conv_init is None else _f64(conv_init)
    if (k_pre.shape != q_pre.shape or z.shape != q_pre.shape or v_pre.shape != (B, T, H, dv)
            or beta_logit.shape != (B, T, H) or conv_w.shape != (H, nch, width) or A.shape != (H,)
            or (init is not None and init.shape != (B, H, width - 1, nch))):
        raise ValueError("oracle.prefill_prep: inconsistent shapes")
    q, k, g = (np.empty((B, T, H, dk)) for _ in range(3))
    v = np.empty((B, T, H, dv))
    beta = np.empty((B, T, H))
    conv_final = np.empty((B, H, width - 1, nch))
    rc = _load().kda_oracle_prefill_prep(
        _ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w), _ptr(init), _ptr(z), _ptr(A),
        _ptr(beta_logit), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_final),
        B, T, H, dk, dv, width, float(eps), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill_prep failed ({rc})")
    return q, k, v, g, beta, conv_final


def decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S,
                eps=L2NORM_EPS, nthreads=None):
    q_pre, k_pre, v_pre, conv_w, g, beta = (_f64(x) for x in (q_pre, k_pre, v_pre, conv_w, g, beta))
    for name, a in (("conv_cache", conv_cache), ("S", S)):
        if not (isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags.c_contiguous):
            raise TypeError(f"oracle.decode_step: {name} must be a C-contiguous float64 array (updated in place)")
    N, H, dk = q_pre.shape
    dv = v_pre.shape[-1]
    width = conv_w.shape[-1]
    nch = 2 * dk + dv
    if (k_pre.shape != (N, H, dk) or v_pre.shape != (N, H, dv) or conv_w.shape != (H, nch, width)
            or conv_cache.shape != (N, H, width - 1, nch) or g.shape != (N, H, dk)
            or beta.shape != (N, H) or S.shape != (N, H, dk, dv)):
        raise ValueError("oracle.decode_step: inconsistent shapes")
    o = np.empty((N, H, dv))
    rc = _load().kda_oracle_decode_step(_ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w),
                                        _ptr(conv_cache), int(conv_pos), _ptr(g), _ptr(beta),
                                        _ptr(S), _ptr(o), N, H, dk, dv, width, float(eps),
                                        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_step failed ({rc})")
    return o


def output_gate(o, gate, w=None, eps=RMSNORM_EPS):
    o, gate = _f64(o), _f64(gate)
    if o.shape != gate.shape or o.ndim < 2:
        raise ValueError("oracle.output_gate: o and gate must share a shape [..., H, dv]")
    H, dv = o.shape[-2], o.shape[-1]
    rows = int(np.prod(o.shape[:-2], dtype=np.int64))
    wa = None if w is None else _f64(w)
    if wa is not None and wa.shape != (dv,):
        raise ValueError("oracle.output_gate: w shape")
    y = np.empty(o.shape)
    rc = _load().kda_oracle_output_gate(_ptr(o), _ptr(gate), _ptr(wa), _ptr(y), rows, H, dv, float(eps))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_output_gate failed ({rc})")
    return y
