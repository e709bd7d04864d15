"""Seeded synthetic inputs for the KDA prefill and decode paths.

This module only draws random numbers and casts them; it holds none of the
recurrence's arithmetic.  Both the GPU path's tests/benchmark and the CPU
oracle's tests take their inputs from here, so the two sides see the same
values.  (q, k are L2-normalised here because the prefill workloads hand the
kernel already-normalised q, k; that normalisation is part of the input recipe,
not of the kernel under test.)

Workloads (shapes as named; every value is synthetic):
  tiny_fp32      B=1  H=2  T=256    d=64   fp32  chunk 16  S0 = 0          seed 0 (CPU)
  prefill_b4h32  B=4  H=32 T=4096   d=128  bf16  S0 ~ 0.02 N(0,1)         seed 1 (CPU)
  k3_prefill     B=1  H=96 T=65536  d=128  bf16  + 10% of tokens g=-4.99   seed 2
  stream_1m      16 segments of k3_prefill's shape, state carried          seed 3000+s
  decode         N=256 H=96 d=128, 64 steps, bf16                          seed 4000+step
  k3_prep        B=1  H=96 T=65536  d=128  bf16  prefill preprocessing     seed 5
  k3_gate        rows=65536 H=96 dv=128 bf16  output exposure gate         seed 6
Long-memory variants (make the state matter across chunks):
  L1  tiny_fp32 shape, g = -5 sigmoid(N(0,1) - 7), upper half of the key channels g = 0
  L2  prefill_b4h32 shape with the L1 gate distribution
  L3  prefill_b4h32 shape, beta = 0, g = -1e-3, S0 ~ N(0,1)

Draw order per call: q, k, v, beta logits, g logits, S0, then the bound mask
(k3_prefill only).  Decode state: conv weights, conv cache, S.  Decode step:
q_pre, k_pre, v_pre, beta logits, g logits.  Prefill preprocessing: conv weights,
A, conv history, then q_pre, k_pre, v_pre, z, beta logits.  Output gate: o,
gate pre-activations, RMSNorm weight.  Decode gate pre-activations: one draw per
step from seed seed_base + 10000 + step.  Backward upstream gradients: dO, then
dS_T, from seed spec.seed + 7000.
"""
from dataclasses import dataclass, field

import torch

G_MIN = -5.0


@dataclass(frozen=True)
class PrefillSpec:
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str = "bf16"          # "bf16" or "fp32"
    seed: int = 0
    s0_std: float = 0.02         # 0 -> S0 is None (zero state)
    gate: str = "standard"       # "standard" | "long" | "const"
    g_const: float = 0.0
    beta_zero: bool = False
    bound_frac: float = 0.0      # fraction of tokens whose g is set to bound_value
    bound_value: float = -4.99
    chunk: int = 32


@dataclass(frozen=True)
class DecodeSpec:
    N: int
    H: int
    dk: int
    dv: int
    width: int = 4
    steps: int = 64
    dtype: str = "bf16"
    seed_base: int = 4000
    state_seed: int = 4999
    gate: str = "standard"


@dataclass(frozen=True)
class PrepSpec:
    B: int
    T: int
    H: int
    dk: int
    dv: int
    width: int = 4
    dtype: str = "bf16"
    seed: int = 5
    history: bool = True         # False -> conv_init is None (zero history)


WORKLOADS = {
    "tiny_fp32": PrefillSpec(B=1, H=2, T=256, dk=64, dv=64, dtype="fp32", seed=0, s0_std=0.0, chunk=16),
    "prefill_b4h32": PrefillSpec(B=4, H=32, T=4096, dk=128, dv=128, seed=1),
    "k3_prefill": PrefillSpec(B=1, H=96, T=65536, dk=128, dv=128, seed=2, bound_frac=0.1),
    "L1": PrefillSpec(B=1, H=2, T=256, dk=64, dv=64, dtype="fp32", seed=10, s0_std=0.0, gate="long", chunk=16),
    "L1_bf16": PrefillSpec(B=1, H=2, T=256, dk=64, dv=64, dtype="bf16", seed=11, s0_std=0.0, gate="long"),
    "L2": PrefillSpec(B=4, H=32, T=4096, dk=128, dv=128, seed=12, gate="long"),
    "L3": PrefillSpec(B=4, H=32, T=4096, dk=128, dv=128, seed=13, s0_std=1.0, gate="const",
                      g_const=-1e-3, beta_zero=True),
}
PREP_K3 = PrepSpec(B=1, T=65536, H=96, dk=128, dv=128, seed=5)
GATE_K3 = dict(rows=65536, H=96, dv=128, dtype="bf16", seed=6)
STREAM_1M = dict(base=WORKLOADS["k3_prefill"], segments=16, seed_base=3000)
DECODE = DecodeSpec(N=256, H=96, dk=128, dv=128)


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


def prefill_inputs(spec: PrefillSpec, device="cpu", seed=None, T=None):
    """Return dict(q, k, v, g, beta, S0) for one prefill call.

    q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H] in spec.dtype;
    S0: [B,H,dk,dv] fp32, or None when spec.s0_std == 0.
    """
    seed = spec.seed if seed is None else seed
    T = spec.T if T is None else T
    B, H, dk, dv = spec.B, spec.H, spec.dk, spec.dv
    dt = torch_dtype(spec.dtype)
    gen = _gen(device, seed)
    q = _unit(_randn((B, T, H, dk), gen, device))
    k = _unit(_randn((B, T, H, dk), gen, device))
    v = _randn((B, T, H, dv), gen, device)
    beta_logit = _randn((B, T, H), gen, device)
    g_logit = _randn((B, T, H, dk), gen, device)
    if spec.beta_zero:
        beta = torch.zeros_like(beta_logit)
    else:
        beta = torch.sigmoid(beta_logit)
    if spec.gate == "standard":
        g = G_MIN * torch.sigmoid(g_logit)
    elif spec.gate == "long":
        g = G_MIN * torch.sigmoid(g_logit - 7.0)
        g[..., dk // 2:] = 0.0
    elif spec.gate == "const":
        g = torch.full_like(g_logit, spec.g_const)
    else:
        raise ValueError(spec.gate)
    S0 = None
    if spec.s0_std > 0:
        S0 = spec.s0_std * _randn((B, H, dk, dv), gen, device)
    if spec.bound_frac > 0:
        mask = torch.rand((B, T, H), generator=gen, device=device) < spec.bound_frac
        g = torch.where(mask[..., None], torch.full_like(g, spec.bound_value), g)
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                g=g.to(dt).contiguous(), beta=beta.to(dt).contiguous(),
                S0=None if S0 is None else S0.contiguous())


def identical_key_inputs(B, T, H, dk, dv, dtype="bf16", seed=77, device="cpu"):
    """Edge of the input domain: every token of a head shares one unit key, beta = 1
    and g = 0 (no decay); q unit, v ~ N(0,1), S0 ~ 0.02 N(0,1).  Within a chunk A is
    then the strict lower part of all ones.  Same dict layout as prefill_inputs."""
    dt = torch_dtype(dtype)
    gen = _gen(device, seed)
    key = _unit(_randn((1, 1, H, dk), gen, device))
    k = key.expand(B, T, H, dk)
    q = _unit(_randn((B, T, H, dk), gen, device))
    v = _randn((B, T, H, dv), gen, device)
    S0 = (0.02 * _randn((B, H, dk, dv), gen, device)).contiguous()
    g = torch.zeros((B, T, H, dk), device=device)
    beta = torch.ones((B, T, H), device=device)
    out = {n: x.to(dt).contiguous() for n, x in dict(q=q, k=k, v=v, g=g, beta=beta).items()}
    out["S0"] = S0
    return out


def decode_state(spec: DecodeSpec, device="cpu", N=None):
    """Initial decode state: conv_w fp32 [H, 2dk+dv, width] ~ 0.5 N(0,1);
    conv_cache [N, H, width-1, 2dk+dv] ~ N(0,1) in spec.dtype; S fp32 [N,H,dk,dv] ~ 0.02 N(0,1)."""
    N = spec.N if N is None else N
    H, dk, dv, W = spec.H, spec.dk, spec.dv, spec.width
    nch = 2 * dk + dv
    gen = _gen(device, spec.state_seed)
    conv_w = 0.5 * _randn((H, nch, W), gen, device)
    cache = _randn((N, H, W - 1, nch), gen, device).to(torch_dtype(spec.dtype))
    S = 0.02 * _randn((N, H, dk, dv), gen, device)
    return dict(conv_w=conv_w.contiguous(), conv_cache=cache.contiguous(), S=S.contiguous())


def decode_step_inputs(spec: DecodeSpec, step: int, device="cpu", N=None):
    """Per-step decode inputs: q_pre, k_pre [N,H,dk]; v_pre [N,H,dv] ~ N(0,1);
    beta = sigmoid(N(0,1)) [N,H]; g = -5 sigmoid(N(0,1)) [N,H,dk] (or near 0 for gate="long")."""
    N = spec.N if N is None else N
    H, dk, dv = spec.H, spec.dk, spec.dv
    dt = torch_dtype(spec.dtype)
    gen = _gen(device, spec.seed_base + step)
    q = _randn((N, H, dk), gen, device)
    k = _randn((N, H, dk), gen, device)
    v = _randn((N, H, dv), gen, device)
    beta = torch.sigmoid(_randn((N, H), gen, device))
    g_logit = _randn((N, H, dk), gen, device)
    if spec.gate == "standard":
        g = G_MIN * torch.sigmoid(g_logit)
    elif spec.gate == "long":
        g = G_MIN * torch.sigmoid(g_logit - 7.0)
    else:
        raise ValueError(spec.gate)
    return dict(q_pre=q.to(dt).contiguous(), k_pre=k.to(dt).contiguous(), v_pre=v.to(dt).contiguous(),
                g=g.to(dt).contiguous(), beta=beta.to(dt).contiguous())


def prep_inputs(spec: PrepSpec, device="cpu", seed=None, T=None):
    """Prefill-preprocessing inputs: conv_w fp32 [H, 2dk+dv, width] ~ 0.5 N(0,1);
    A fp32 [H] ~ N(0,1); conv_init [B, H, width-1, 2dk+dv] ~ N(0,1) (or None);
    q_pre, k_pre, z [B,T,H,dk], v_pre [B,T,H,dv], beta_logit [B,T,H] ~ N(0,1)."""
    seed = spec.seed if seed is None else seed
    T = spec.T if T is None else T
    B, H, dk, dv, W = spec.B, spec.H, spec.dk, spec.dv, spec.width
    nch = 2 * dk + dv
    dt = torch_dtype(spec.dtype)
    gen = _gen(device, seed)
    conv_w = 0.5 * _randn((H, nch, W), gen, device)
    A = _randn((H,), gen, device)
    init = _randn((B, H, W - 1, nch), gen, device).to(dt).contiguous() if spec.history else None
    x = {n: _randn(shp, gen, device).to(dt).contiguous()
         for n, shp in (("q_pre", (B, T, H, dk)), ("k_pre", (B, T, H, dk)), ("v_pre", (B, T, H, dv)),
                        ("z", (B, T, H, dk)), ("beta_logit", (B, T, H)))}
    x.update(conv_w=conv_w.contiguous(), A=A.contiguous(), conv_init=init)
    return x


def backward_inputs(spec: PrefillSpec, device="cpu", seed=None, T=None, ds_std=1.0):
    """Upstream gradients for a backward call: dO ~ N(0,1) [B,T,H,dv] in spec.dtype and
    dS_T ~ ds_std N(0,1) [B,H,dk,dv] fp32 (None when ds_std == 0); seed spec.seed + 7000."""
    seed = spec.seed + 7000 if seed is None else seed
    T = spec.T if T is None else T
    gen = _gen(device, seed)
    dO = _randn((spec.B, T, spec.H, spec.dv), gen, device).to(torch_dtype(spec.dtype)).contiguous()
    dS = (ds_std * _randn((spec.B, spec.H, spec.dk, spec.dv), gen, device)).contiguous() if ds_std else None
    return dict(dO=dO, dS_T=dS)


def gate_inputs(rows, H, dv, dtype="bf16", seed=6, device="cpu", weight=True):
    """Output-gate inputs: o ~ N(0,1) and gate ~ 2 N(0,1), both [rows, H, dv] in dtype;
    norm_w fp32 [dv] ~ 1 + 0.1 N(0,1) (None when weight is False)."""
    dt = torch_dtype(dtype)
    gen = _gen(device, seed)
    o = _randn((rows, H, dv), gen, device).to(dt).contiguous()
    gate = (2.0 * _randn((rows, H, dv), gen, device)).to(dt).contiguous()
    w = (1.0 + 0.1 * _randn((dv,), gen, device)).contiguous() if weight else None
    return dict(o=o, gate=gate, norm_w=w)


def decode_gate_inputs(spec: DecodeSpec, step: int, device="cpu", N=None):
    """Gate pre-activations of one decode step: [N, H, dv] ~ 2 N(0,1) in spec.dtype."""
    N = spec.N if N is None else N
    gen = _gen(device, spec.seed_base + 10000 + step)
    return (2.0 * _randn((N, spec.H, spec.dv), gen, device)).to(torch_dtype(spec.dtype)).contiguous()


def to_f64(t):
    """Exact upcast of a (possibly bf16) torch tensor to a float64 numpy array."""
    import numpy as np
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy().astype(np.float64, copy=False)
