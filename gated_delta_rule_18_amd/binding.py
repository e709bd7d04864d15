"""Python binding of libkda.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; torch is used
for device memory and for the current HIP stream.  If the library is missing
the calls raise (there is no fallback).

    o, S_T        = chunk_fwd(q, k, v, g, beta, S0=None, chunk=64)
    o, S_T, snaps = chunk_fwd_snapshots(q, k, v, g, beta, S0, snap_every, n_snaps, chunk=64)
    o             = decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S)
    q, k, v, g, beta, conv_final = prefill_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A,
                                                beta_logit)
    y             = output_gate(o, gate, norm_w=None, eps=1e-6)
    dq, dk, dv, dg, dbeta, dS0 = chunk_bwd(q, k, v, g, beta, S0, dO, dS_T=None)
    y             = decode_step_gated(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta,
                                      S, gate, norm_w=None, eps=1e-6)

Shapes and dtypes follow include/kda.h: bf16 activations with an fp32 state,
or fp32 everywhere (test mode).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

KDA_BF16, KDA_FP32 = 0, 1
KDA_OK, KDA_ERR_INVALID, KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH, KDA_ERR_TOO_LARGE = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 64 << 20      # KDA_NOALLOC_SCRATCH_BYTES
EXPORTS = ("kda_chunk_bwd", "kda_chunk_bwd_ex", "kda_chunk_bwd_noalloc", "kda_chunk_bwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_ex",
           "kda_chunk_fwd_from_proj", "kda_chunk_fwd_from_proj_workspace_size", "kda_chunk_fwd_gated",
           "kda_chunk_fwd_gated_workspace_size", "kda_chunk_fwd_snapshots",
           "kda_decode_step", "kda_decode_step_gated", "kda_output_gate", "kda_prefill_prep", "kda_strerror",
           "kda_validate_inputs", "kda_version", "kda_workgroup_xcds")

_lib = None


class FwdOptions(ctypes.Structure):
    """struct kda_fwd_options of kda.h."""
    _fields_ = [("spin_limit", ctypes.c_int)]


class BwdOptions(ctypes.Structure):
    """struct kda_bwd_options of kda.h."""
    _fields_ = [("fail_xcd_check", ctypes.c_int)]


class KdaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (kda status {code})")
        self.code = code


def lib():
    """Load libkda.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with "
                              "`python -m gated_delta_rule_18_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, i = ctypes.c_void_p, ctypes.c_int
        L.kda_chunk_fwd.restype = i
        L.kda_chunk_fwd.argtypes = [vp] * 8 + [i] * 7 + [vp]
        L.kda_chunk_fwd_snapshots.restype = i
        L.kda_chunk_fwd_snapshots.argtypes = [vp] * 9 + [i] * 9 + [vp]
        L.kda_chunk_fwd_ex.restype = i
        L.kda_chunk_fwd_ex.argtypes = [vp] * 9 + [i] * 9 + [ctypes.POINTER(FwdOptions), vp]
        L.kda_chunk_fwd_gated.restype = i
        L.kda_chunk_fwd_gated.argtypes = ([vp] * 8 + [ctypes.c_float] + [vp] * 3 + [ctypes.c_size_t] + [i] * 6
                                          + [ctypes.POINTER(FwdOptions), vp])
        L.kda_chunk_fwd_gated_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_fwd_gated_workspace_size.argtypes = [i] * 3
        L.kda_chunk_fwd_from_proj.restype = i
        L.kda_chunk_fwd_from_proj.argtypes = ([vp] * 17 + [vp, ctypes.c_size_t] + [i] * 7
                                              + [ctypes.POINTER(FwdOptions), vp])
        L.kda_chunk_fwd_from_proj_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_fwd_from_proj_workspace_size.argtypes = [i] * 3
        L.kda_decode_step.restype = i
        L.kda_decode_step.argtypes = [vp] * 5 + [i] + [vp] * 4 + [i] * 6 + [vp]
        L.kda_decode_step_gated.restype = i
        L.kda_decode_step_gated.argtypes = ([vp] * 5 + [i] + [vp] * 5 + [ctypes.c_float, vp]
                                            + [i] * 6 + [vp])
        L.kda_chunk_bwd.restype = i
        L.kda_chunk_bwd.argtypes = [vp] * 15 + [ctypes.c_size_t] + [i] * 6 + [vp]
        L.kda_chunk_bwd_ex.restype = i
        L.kda_chunk_bwd_ex.argtypes = [vp] * 15 + [ctypes.c_size_t] + [i] * 6 + [ctypes.POINTER(BwdOptions), vp]
        L.kda_chunk_bwd_noalloc.restype = i
        L.kda_chunk_bwd_noalloc.argtypes = [vp] * 14 + [i] * 6 + [vp]
        L.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        L.kda_chunk_bwd_workspace_size.argtypes = [i] * 5
        L.kda_output_gate.restype = i
        L.kda_output_gate.argtypes = [vp] * 4 + [i] * 3 + [ctypes.c_float, i, vp]
        L.kda_prefill_prep.restype = i
        L.kda_prefill_prep.argtypes = [vp] * 14 + [i] * 7 + [vp]
        L.kda_validate_inputs.restype = i
        L.kda_validate_inputs.argtypes = [vp] * 3 + [i] * 5 + [vp]
        L.kda_workgroup_xcds.restype = i
        L.kda_workgroup_xcds.argtypes = [vp, i, i, vp]
        L.kda_strerror.restype = ctypes.c_char_p
        L.kda_strerror.argtypes = [i]
        L.kda_version.restype = i
        L.kda_version.argtypes = []
        _lib = L
    return _lib


def version():
    return lib().kda_version()


def _check(rc):
    if rc != KDA_OK:
        raise KdaError(rc, lib().kda_strerror(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32")


def _want(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device or device.type != "cuda":
        raise ValueError(f"{name}: device {t.device}, expected the GPU tensor device {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd(q, k, v, g, beta, S0=None, chunk=64, o=None, S_T=None, return_state=True, spin_limit=None):
    """Chunkwise prefill.  q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H];
    S0 [B,H,dk,dv] fp32 or None.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv] fp32 or None).
    S_T may be passed as S0 itself for in-place streaming over segments.  Every chunk
    size (16, 32, 64) gives the same bits.  spin_limit (testing): see kda_chunk_fwd_ex."""
    o, S_T, _ = _chunk_fwd(q, k, v, g, beta, S0, chunk, o, S_T, return_state, None, 0, 0, spin_limit)
    return o, S_T


def chunk_fwd_snapshots(q, k, v, g, beta, S0, snap_every, n_snaps, chunk=64, o=None, S_T=None,
                        snaps=None, return_state=True, spin_limit=None):
    """chunk_fwd that also returns snaps [n_snaps,B,H,dk,dv] fp32: snapshot s is the
    state after the first (s+1)*snap_every tokens (snap_every a multiple of chunk)."""
    return _chunk_fwd(q, k, v, g, beta, S0, chunk, o, S_T, return_state, snaps, snap_every, n_snaps,
                      spin_limit)


def _chunk_fwd(q, k, v, g, beta, S0, chunk, o, S_T, return_state, snaps, snap_every, n_snaps,
               spin_limit=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _want(t, name, shp, dt, dev)
    if S0 is not None:
        _want(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _want(o, "o", (B, T, H, dv), dt, dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _want(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    if n_snaps and snaps is None:
        snaps = torch.empty((n_snaps, B, H, dk, dv), dtype=torch.float32, device=dev)
    elif snaps is not None:
        _want(snaps, "snaps", (n_snaps, B, H, dk, dv), torch.float32, dev)
    if spin_limit is not None:
        opts = FwdOptions(spin_limit=int(spin_limit))
        rc = lib().kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                    _ptr(S_T), _ptr(snaps), int(snap_every), int(n_snaps), B, T, H, dk, dv,
                                    code, int(chunk), ctypes.byref(opts), _stream(dev))
    elif n_snaps or snaps is not None:
        rc = lib().kda_chunk_fwd_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                           _ptr(o), _ptr(S_T), _ptr(snaps), int(snap_every), int(n_snaps),
                                           B, T, H, dk, dv, code, int(chunk), _stream(dev))
    else:
        rc = lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                 _ptr(S_T), B, T, H, dk, dv, code, int(chunk), _stream(dev))
    _check(rc)
    return o, S_T, snaps


def chunk_fwd_gated(q, k, v, g, beta, S0, gate, norm_w=None, eps=1e-6, y=None, S_T=None, return_state=True,
                    workspace=None, spin_limit=None):
    """Prefill with the output exposure gate fused: returns (y [B,T,H,dv], S_T or None),
    y = Sigmoid(gate) * RMSNorm(o) * norm_w with o the prefill's readout -- the same
    bits as output_gate(chunk_fwd(...)[0], gate, norm_w, eps).  gate [B,T,H,dv] like v;
    norm_w fp32 [dv] or None (ones).  workspace: a uint8 device tensor of at least
    gated_workspace_size(B, H, dv) bytes, or None (allocated here).  spin_limit
    (testing): see kda_chunk_fwd_ex."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)), ("gate", gate, (B, T, H, dv))):
        _want(t, name, shp, dt, dev)
    if S0 is not None:
        _want(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if norm_w is not None:
        _want(norm_w, "norm_w", (dv,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _want(y, "y", (B, T, H, dv), dt, dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _want(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    need = gated_workspace_size(B, H, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    opts = FwdOptions(spin_limit=int(spin_limit)) if spin_limit is not None else None
    rc = lib().kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(gate),
                                   _ptr(norm_w), float(eps), _ptr(y), _ptr(S_T), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), B, T, H, dk, dv, code,
                                   ctypes.byref(opts) if opts is not None else None, _stream(dev))
    _check(rc)
    return y, S_T


def chunk_fwd_from_proj(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, S0=None, out=None, o=None,
                        S_T=None, return_state=True, workspace=None, spin_limit=None):
    """prefill_prep and chunk_fwd in one launch.  Arguments as prefill_prep (whose
    outputs q, k, v, g, beta, conv_final are returned too, in `out` if given), then
    S0, o, S_T as chunk_fwd.  Returns (o, S_T or None, dict(q, k, v, g, beta,
    conv_final)): the same bits as prefill_prep followed by chunk_fwd.  workspace: a
    uint8 device tensor of at least from_proj_workspace_size(B, T, H) bytes, or None
    (allocated here).  spin_limit (testing): see kda_chunk_fwd_ex."""
    B, T, H, dk = q_pre.shape
    dv = v_pre.shape[-1]
    dev, dt = q_pre.device, q_pre.dtype
    code = _dtype_code(q_pre)
    W = conv_w.shape[-1]
    nch = 2 * dk + dv
    for name, t, shp in (("q_pre", q_pre, (B, T, H, dk)), ("k_pre", k_pre, (B, T, H, dk)),
                         ("v_pre", v_pre, (B, T, H, dv)), ("z", z, (B, T, H, dk)),
                         ("beta_logit", beta_logit, (B, T, H))):
        _want(t, name, shp, dt, dev)
    _want(conv_w, "conv_w", (H, nch, W), torch.float32, dev)
    _want(A, "A", (H,), torch.float32, dev)
    if conv_init is not None:
        _want(conv_init, "conv_init", (B, H, W - 1, nch), dt, dev)
    if out is None:
        out = dict(q=torch.empty((B, T, H, dk), dtype=dt, device=dev), k=torch.empty((B, T, H, dk), dtype=dt, device=dev),
                   v=torch.empty((B, T, H, dv), dtype=dt, device=dev), g=torch.empty((B, T, H, dk), dtype=dt, device=dev),
                   beta=torch.empty((B, T, H), dtype=dt, device=dev),
                   conv_final=torch.empty((B, H, W - 1, nch), dtype=dt, device=dev))
    if S0 is not None:
        _want(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _want(o, "o", (B, T, H, dv), dt, dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _want(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    if workspace is None:
        workspace = torch.empty(max(from_proj_workspace_size(B, T, H), 16), dtype=torch.uint8, device=dev)
    opts = FwdOptions(spin_limit=int(spin_limit)) if spin_limit is not None else None
    rc = lib().kda_chunk_fwd_from_proj(
        _ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w), _ptr(conv_init), _ptr(z), _ptr(A), _ptr(beta_logit),
        _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["g"]), _ptr(out["beta"]), _ptr(out.get("conv_final")),
        _ptr(S0), _ptr(o), _ptr(S_T), _ptr(workspace), workspace.numel() * workspace.element_size(),
        B, T, H, dk, dv, W, code, ctypes.byref(opts) if opts is not None else None, _stream(dev))
    _check(rc)
    return o, S_T, out


def from_proj_workspace_size(B, T, H):
    """Bytes of workspace chunk_fwd_from_proj needs (kda_chunk_fwd_from_proj_workspace_size)."""
    return int(lib().kda_chunk_fwd_from_proj_workspace_size(int(B), int(T), int(H)))


def gated_workspace_size(B, H, dv):
    """Bytes of workspace chunk_fwd_gated needs (kda_chunk_fwd_gated_workspace_size)."""
    return int(lib().kda_chunk_fwd_gated_workspace_size(int(B), int(H), int(dv)))


def _bwd_outputs(q, k, v, g, beta, S0, dO, dS_T, return_dS0, out):
    """Checks the backward's inputs; returns the sizes, the dtype code and the fp32
    outputs (dq, dk, dv, dg, dbeta, dS0): `out` when given (checked), else new tensors."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H)), ("dO", dO, (B, T, H, dv))):
        _want(t, name, shp, dt, dev)
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _want(t, name, (B, H, dk, dv), torch.float32, dev)
    shapes = ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H, dk), (B, T, H), (B, H, dk, dv))
    if out is None:
        out = tuple(torch.empty(s, dtype=torch.float32, device=dev) for s in shapes)
        if not return_dS0:
            out = out[:5] + (None,)
    else:
        for name, t, s in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), out, shapes):
            if t is not None:
                _want(t, name, s, torch.float32, dev)
    return (B, T, H, dk, dv), code, tuple(out)


def chunk_bwd(q, k, v, g, beta, S0, dO, dS_T=None, return_dS0=True, workspace=None, fail_xcd_check=False):
    """Gradients of <dO, o> + <dS_T, S_T> through chunk_fwd.  Inputs as chunk_fwd plus
    dO [B,T,H,dv] (input dtype) and dS_T [B,H,dk,dv] fp32 or None (zero).  Returns fp32
    (dq, dk, dv, dg, dbeta, dS0); dS0 is None when return_dS0 is False.  `workspace`
    may supply a uint8 device tensor of at least workspace_size(...) bytes.
    fail_xcd_check (testing): see kda_chunk_bwd_ex."""
    (B, T, H, dk, dv), code, (dq, dk_, dv_, dg, db, dS0) = _bwd_outputs(q, k, v, g, beta, S0, dO, dS_T,
                                                                          return_dS0, None)
    dev = q.device
    need = workspace_size(B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < need or workspace.device != dev:
        raise ValueError(f"workspace: need {need} bytes on {dev}")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
            _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dS0), _ptr(workspace),
            int(workspace.numel()), B, T, H, dk, dv, code)
    if fail_xcd_check:
        rc = lib().kda_chunk_bwd_ex(*args, ctypes.byref(BwdOptions(fail_xcd_check=1)), _stream(dev))
    else:
        rc = lib().kda_chunk_bwd(*args, _stream(dev))
    _check(rc)
    return dq, dk_, dv_, dg, db, dS0


def chunk_bwd_noalloc(q, k, v, g, beta, S0, dO, dS_T=None, out=None, return_dS0=True):
    """chunk_bwd through kda_chunk_bwd_noalloc: the library's per-GPU scratch array in
    place of a workspace (sizes needing more than NOALLOC_SCRATCH_BYTES raise
    KdaError with code KDA_ERR_TOO_LARGE).  `out` = (dq, dk, dv, dg, dbeta, dS0)
    supplies preallocated fp32 outputs (dS0 may be None); without it they are
    allocated here, as in chunk_bwd."""
    (B, T, H, dk, dv), code, (dq, dk_, dv_, dg, db, dS0) = _bwd_outputs(q, k, v, g, beta, S0, dO, dS_T,
                                                                          return_dS0, out)
    rc = lib().kda_chunk_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO),
                                     _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db),
                                     _ptr(dS0), B, T, H, dk, dv, code, _stream(q.device))
    _check(rc)
    return dq, dk_, dv_, dg, db, dS0


def workspace_size(B, T, H, dk, dv):
    """Bytes of workspace chunk_bwd needs."""
    return int(lib().kda_chunk_bwd_workspace_size(B, T, H, dk, dv))


def decode_step(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, o=None):
    """One decode step.  q_pre, k_pre [N,H,dk]; v_pre [N,H,dv]; conv_w fp32 [H,2dk+dv,W];
    conv_cache [N,H,W-1,2dk+dv] (updated); g [N,H,dk]; beta [N,H]; S fp32 [N,H,dk,dv]
    (updated in place).  Returns o [N,H,dv]."""
    return _decode(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, o, None, None, 0.0)


def decode_step_gated(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, gate,
                      norm_w=None, eps=1e-6, y=None):
    """decode_step with the output exposure gate fused: returns y [N,H,dv] =
    Sigmoid(gate) * RMSNorm(o) * norm_w (norm_w fp32 [dv] or None for ones)."""
    return _decode(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, y, gate, norm_w, eps)


def _decode(q_pre, k_pre, v_pre, conv_w, conv_cache, conv_pos, g, beta, S, o, gate, norm_w, eps):
    N, H, dk = q_pre.shape
    dv = v_pre.shape[-1]
    W = conv_w.shape[-1]
    nch = 2 * dk + dv
    dev, dt = q_pre.device, q_pre.dtype
    code = _dtype_code(q_pre)
    for name, t, shp in (("q_pre", q_pre, (N, H, dk)), ("k_pre", k_pre, (N, H, dk)),
                         ("v_pre", v_pre, (N, H, dv)), ("g", g, (N, H, dk)), ("beta", beta, (N, H)),
                         ("conv_cache", conv_cache, (N, H, W - 1, nch))):
        _want(t, name, shp, dt, dev)
    _want(conv_w, "conv_w", (H, nch, W), torch.float32, dev)
    _want(S, "S", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _want(o, "o", (N, H, dv), dt, dev)
    if gate is None:
        rc = lib().kda_decode_step(_ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w), _ptr(conv_cache),
                                   int(conv_pos), _ptr(g), _ptr(beta), _ptr(S), _ptr(o), N, H, dk, dv,
                                   W, code, _stream(dev))
    else:
        _want(gate, "gate", (N, H, dv), dt, dev)
        if norm_w is not None:
            _want(norm_w, "norm_w", (dv,), torch.float32, dev)
        rc = lib().kda_decode_step_gated(_ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w),
                                         _ptr(conv_cache), int(conv_pos), _ptr(g), _ptr(beta), _ptr(S),
                                         _ptr(gate), _ptr(norm_w), float(eps), _ptr(o), N, H, dk, dv, W,
                                         code, _stream(dev))
    _check(rc)
    return o


def output_gate(o, gate, norm_w=None, eps=1e-6, y=None):
    """Output exposure gate: y = Sigmoid(gate) * RMSNorm(o) * norm_w, RMSNorm over the
    last (dv) axis of each head.  o, gate [..., H, dv] (bf16 or fp32); norm_w fp32 [dv]
    or None (ones).  y may be passed as o or gate itself (in place)."""
    if o.dim() < 2:
        raise ValueError("o must be [..., H, dv]")
    H, dv = o.shape[-2], o.shape[-1]
    rows = 1
    for n in o.shape[:-2]:
        rows *= n
    dev, dt = o.device, o.dtype
    code = _dtype_code(o)
    _want(o, "o", o.shape, dt, dev)
    _want(gate, "gate", o.shape, dt, dev)
    if norm_w is not None:
        _want(norm_w, "norm_w", (dv,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(o)
    else:
        _want(y, "y", o.shape, dt, dev)
    rc = lib().kda_output_gate(_ptr(o), _ptr(gate), _ptr(norm_w), _ptr(y), rows, H, dv, float(eps), code,
                               _stream(dev))
    _check(rc)
    return y


def validate_inputs(g, beta):
    """Debug check of the value domains: g [B,T,H,dk] in [-5, 0], beta [B,T,H] in [0, 1]
    (NaN outside both).  Waits for the GPU and returns dict(bad_g, first_bad_g, bad_beta,
    first_bad_beta) with flat indices, -1 where nothing is outside."""
    B, T, H, dk = g.shape
    dev, dt = g.device, g.dtype
    code = _dtype_code(g)
    _want(g, "g", (B, T, H, dk), dt, dev)
    _want(beta, "beta", (B, T, H), dt, dev)
    report = torch.empty(4, dtype=torch.int64, device=dev)
    rc = lib().kda_validate_inputs(_ptr(g), _ptr(beta), _ptr(report), B, T, H, dk, code, _stream(dev))
    _check(rc)
    r = [int(x) for x in report.cpu()]
    return dict(bad_g=r[0], first_bad_g=r[1], bad_beta=r[2], first_bad_beta=r[3])


def workgroup_xcds(n, lds_bytes=0, device=None):
    """Debug check of the workgroup placement the fused launches assume: an int32
    tensor [n] whose element i is the XCD workgroup i of one n-workgroup launch (each
    workgroup requesting lds_bytes of LDS) ran on; the fused launches expect xcd[i] == xcd[i % 8]
    with xcd[0..7] all different (round-robin placement from any first XCD)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    xcd = torch.full((max(int(n), 0),), -1, dtype=torch.int32, device=dev)
    _check(lib().kda_workgroup_xcds(_ptr(xcd) if n > 0 else None, int(n), int(lds_bytes), _stream(dev)))
    return xcd


def prefill_prep(q_pre, k_pre, v_pre, conv_w, conv_init, z, A, beta_logit, out=None,
                 conv_final=None, return_final=True):
    """Prefill preprocessing.  q_pre, k_pre, z [B,T,H,dk]; v_pre [B,T,H,dv]; beta_logit [B,T,H];
    conv_w fp32 [H,2dk+dv,W]; conv_init [B,H,W-1,2dk+dv] or None (zero history); A fp32 [H].
    Returns (q, k, v, g, beta, conv_final); conv_final may be passed as conv_init itself.
    `out` may supply preallocated (q, k, v, g, beta)."""
    B, T, H, dk = q_pre.shape
    dv = v_pre.shape[-1]
    W = conv_w.shape[-1]
    nch = 2 * dk + dv
    dev, dt = q_pre.device, q_pre.dtype
    code = _dtype_code(q_pre)
    for name, t, shp in (("q_pre", q_pre, (B, T, H, dk)), ("k_pre", k_pre, (B, T, H, dk)),
                         ("z", z, (B, T, H, dk)), ("v_pre", v_pre, (B, T, H, dv)),
                         ("beta_logit", beta_logit, (B, T, H))):
        _want(t, name, shp, dt, dev)
    _want(conv_w, "conv_w", (H, nch, W), torch.float32, dev)
    _want(A, "A", (H,), torch.float32, dev)
    if conv_init is not None:
        _want(conv_init, "conv_init", (B, H, W - 1, nch), dt, dev)
    shapes = ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H, dk), (B, T, H))
    if out is None:
        out = tuple(torch.empty(s, dtype=dt, device=dev) for s in shapes)
    else:
        for name, t, s in zip(("q", "k", "v", "g", "beta"), out, shapes):
            _want(t, name, s, dt, dev)
    if conv_final is None and return_final:
        conv_final = torch.empty((B, H, W - 1, nch), dtype=dt, device=dev)
    elif conv_final is not None:
        _want(conv_final, "conv_final", (B, H, W - 1, nch), dt, dev)
    q, k, v, g, beta = out
    rc = lib().kda_prefill_prep(_ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_w), _ptr(conv_init),
                                _ptr(z), _ptr(A), _ptr(beta_logit), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(conv_final), B, T, H, dk, dv, W, code, _stream(dev))
    _check(rc)
    return q, k, v, g, beta, conv_final
