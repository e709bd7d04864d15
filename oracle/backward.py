"""fp64 CPU oracle of the KDA recurrence's gradients -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the GPU path and imports nothing from it.

The pages say training runs the chunked form of the recurrence (page "Kimi K3：
架构、训练与百万 Token Agentic RL 技术解读", section 3.3, the chunk interface used
for training and long prefill) but derive no backward pass.  The plainest
reading is the exact gradient of the forward map
    (q, k, v, g, beta, S0) -> (o, S_T)
defined by the recurrence of section 3.1 in the one-step order of section 3.2:
    Sbar = Diag(exp(g_t)) S_{t-1};  vhat = Sbar^T k_t;
    S_t  = Sbar + beta_t k_t (v_t - vhat)^T;  o_t = S_t^T q_t.
Given upstream gradients dO = dL/do and dS_T = dL/dS_T, this module returns
(dq, dk, dv, dg, dbeta, dS0).  The loop below is that forward, token by token
in float64 torch CPU tensors, differentiated by torch.autograd (a library
primitive used as one step; nothing else is added).

Layouts: q, k, g [B, T, H, dk]; v, dO [B, T, H, dv]; beta [B, T, H];
S0, dS_T [B, H, dk, dv] (row = key channel).  S0 None means zero.
"""
import numpy as np
import torch


def _t(a):
    return torch.as_tensor(np.ascontiguousarray(np.asarray(a, dtype=np.float64)))


def forward_torch(q, k, v, g, beta, S0):
    """The recurrence on float64 torch tensors (differentiable).  Returns (o, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = S0 if S0 is not None else torch.zeros((B, H, dk, dv), dtype=torch.float64)
    outs = []
    for t in range(T):
        alpha = torch.exp(g[:, t])                                   # [B, H, dk]
        Sbar = alpha[..., None] * S                                  # rows scaled
        vhat = torch.einsum("bhij,bhi->bhj", Sbar, k[:, t])          # Sbar^T k
        S = Sbar + beta[:, t][..., None, None] * k[:, t][..., None] * (v[:, t] - vhat)[..., None, :]
        outs.append(torch.einsum("bhij,bhi->bhj", S, q[:, t]))       # S^T q, after the write
    o = torch.stack(outs, dim=1) if T else torch.zeros((B, 0, H, dv), dtype=torch.float64)
    return o, S


def backward(q, k, v, g, beta, S0, dO, dS_T):
    """Exact gradients of <dO, o> + <dS_T, S_T>.  Returns float64 numpy arrays
    (dq, dk, dv, dg, dbeta, dS0); dS0 is returned even when S0 is None (the
    gradient with respect to a zero initial state)."""
    q, k, v, g, beta = (_t(x).requires_grad_(True) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0t = _t(np.zeros((B, H, dk, dv)) if S0 is None else S0).requires_grad_(True)
    o, S_T = forward_torch(q, k, v, g, beta, S0t)
    loss = (o * _t(dO)).sum() + (S_T * _t(dS_T)).sum()
    grads = torch.autograd.grad(loss, (q, k, v, g, beta, S0t), allow_unused=True)
    out = []
    for x, gr in zip((q, k, v, g, beta, S0t), grads):
        out.append(np.zeros(tuple(x.shape)) if gr is None else gr.detach().numpy())
    return tuple(out)
