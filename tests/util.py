"""Shared helpers of the parity tests: tolerances and oracle calls on subsets."""
import numpy as np
import torch

import oracle
from gated_delta_rule_18_amd.inputs import to_f64

# Parity bars: max|do| <= TOL_O * |o|_inf and max|dS| <= TOL_S * |S|_inf, with the
# infinity norms taken from the oracle's result.
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
# Gradient bars (kda_chunk_bwd), max|diff| <= TOL_GRAD * |ref|_inf per gradient tensor.
# A gradient element is a sum over up to 16 dk dv signed products, some of whose
# factors reach e^{+-75} at the decay bound before they cancel; fp32 accumulation
# of such sums carries ~1e-5 of the largest term, so fp32 mode is held to 1e-4
# (measured worst: 3.2e-5).  bf16 mode keeps the forward's bar.
TOL_GRAD = {"bf16": 2e-2, "fp32": 1e-4}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    return err / scale if scale > 0 else err


def assert_parity(got, ref, tol, what):
    got64 = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got64).all(), f"{what}: non-finite values"
    e = rel_err(got64, ref)
    assert e <= tol, f"{what}: max|diff|/|ref|_inf = {e:.3e} > {tol:.1e}"
    return e


def oracle_prefill_heads(inp, heads, cols=None, S0=None):
    """Oracle over the full sequence for a subset of (b, h) pairs and, optionally, a
    subset of value columns (value columns of the state never interact).
    heads: list of (b, h).  Returns (o [n, T, dv'], S [n, dk, dv'])."""
    outs, states = [], []
    for b, h in heads:
        sl = lambda t: to_f64(t[b:b + 1, :, h:h + 1])
        q, k, g = sl(inp["q"]), sl(inp["k"]), sl(inp["g"])
        v = sl(inp["v"])
        beta = to_f64(inp["beta"][b:b + 1, :, h:h + 1])
        s0 = S0 if S0 is not None else inp.get("S0")
        s0 = None if s0 is None else to_f64(s0[b:b + 1, h:h + 1])
        if cols is not None:
            v = np.ascontiguousarray(v[..., cols])
            s0 = None if s0 is None else np.ascontiguousarray(s0[..., cols])
        o, S = oracle.prefill(q, k, v, g, beta, s0)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return np.stack(outs), np.stack(states)
