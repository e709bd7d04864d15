"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Every check here is independent of the oracle's own loop: hand-derived exact
values, closed forms of special cases, explicit matrix products, invariants,
a second (chunkwise) derivation, and library routines for the preprocessing.
Page cited throughout: "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读"
(sections 3.1-3.3) and "Kimi K3 架构篇：一文详解 2.8 万亿参数的巨型怪兽".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.chunk_model import chunk_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-12


def _rand_inputs(rng, B, T, H, dk, dv, unit=True, gscale=1.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * gscale / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, S0


def _close(a, b, tol=RTOL):
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


def test_scalar_worked_example():
    """d_k = d_v = 1 worked by hand with exact fractions (section 3.2 edit order)."""
    with open(os.path.join(GOLDEN, "scalar_recurrence.json")) as f:
        gd = json.load(f)
    T = len(gd["q"])
    shp = (1, T, 1, 1)
    o, S = oracle.prefill(np.array(gd["q"]).reshape(shp), np.array(gd["k"]).reshape(shp),
                          np.array(gd["v"]).reshape(shp), np.log(np.array(gd["alpha"])).reshape(shp),
                          np.array(gd["beta"]).reshape(1, T, 1), np.full((1, 1, 1, 1), gd["S0"]))
    np.testing.assert_allclose(o.ravel(), gd["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S.ravel(), [gd["S_T"]], rtol=0, atol=1e-15)


def test_bound_facts():
    """g_min = -5: alpha > e^-5 ~ 0.0067; a 16-position tile sums to >= -80; e^80 fits bf16."""
    with open(os.path.join(GOLDEN, "bound_facts.json")) as f:
        gd = json.load(f)
    assert round(math.exp(gd["g_min"]), gd["alpha_min_decimals"]) == gd["alpha_min_approx"]
    assert gd["tile_positions"] * gd["g_min"] == gd["tile_cumulative_log_decay_min"]
    assert math.exp(-gd["tile_cumulative_log_decay_min"]) < torch.finfo(torch.bfloat16).max
    # the workload's bound-stress value rounds onto the bound itself in bf16
    assert torch.tensor(-4.99).to(torch.bfloat16).item() == gd["g_min"]


def test_decay_only_closed_form():
    """beta = 0: S_t = Diag(exp(sum_{s<=t} g_s)) S0 and o_t = S_t^T q_t -- decay scales rows only."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 40, 3, 8, 5)
    beta[:] = 0.0
    o, S = oracle.prefill(q, k, v, g, beta, S0)
    G = np.cumsum(g, axis=1)                                   # [B,T,H,dk]
    St = np.exp(G)[..., None] * S0[:, None]                    # [B,T,H,dk,dv]
    _close(o, np.einsum("bthij,bthi->bthj", St, q))
    _close(S, St[:, -1])


def test_linear_attention_reduction():
    """alpha = 1, S0 = 0, orthonormal keys: S_t = sum_{i<=t} beta_i k_i v_i^T;
    with beta = 1 this is the plain linear-attention prefix sum of section 3.1 eq. 1."""
    rng = np.random.default_rng(2)
    T, dk, dv = 12, 16, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T].reshape(1, T, 1, dk)
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    g = np.zeros((1, T, 1, dk))
    for beta in (rng.random((1, T, 1)), np.ones((1, T, 1))):
        o, S = oracle.prefill(q, k, v, g, beta, None)
        outer = beta[0, :, 0, None, None] * k[0, :, 0, :, None] * v[0, :, 0, None, :]
        St = np.cumsum(outer, axis=0)
        _close(o[0, :, 0], np.einsum("tij,ti->tj", St, q[0, :, 0]))
        _close(S[0, 0], St[-1])


def test_delta_recall():
    """beta = 1 and unit k: S_t^T k_t = v_t exactly, for any alpha (read with q = k).
    General beta and non-unit k: S_t^T k_t = vhat_t + beta_t |k_t|^2 (v_t - vhat_t)."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 30, 2, 8, 6)
    beta1 = np.ones_like(beta)
    o, _ = oracle.prefill(k, k, v, g, beta1, S0)
    _close(o, v, 1e-12)
    k2 = 1.7 * k
    o2, _ = oracle.prefill(k2, k2, v, g, beta, S0)
    for t in (0, 5, 29):
        if t == 0:
            Sprev = S0
        else:
            _, Sprev = oracle.prefill(q[:, :t], k2[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0)
        for h in range(2):
            vhat = (np.exp(g[0, t, h])[:, None] * Sprev[0, h]).T @ k2[0, t, h]
            nk2 = k2[0, t, h] @ k2[0, t, h]
            expect = vhat + beta[0, t, h] * nk2 * (v[0, t, h] - vhat)
            _close(o2[0, t, h], expect)


def test_unrolled_product_bruteforce():
    """T <= 8: S_T = (prod A_t) S0 + sum_i (prod_{t>i} A_t) beta_i k_i v_i^T with
    A_t = (I - beta_t k_t k_t^T) Diag(alpha_t) formed explicitly (section 3.1 eq. 3)."""
    rng = np.random.default_rng(4)
    for T in (1, 2, 5, 8):
        q, k, v, g, beta, S0 = _rand_inputs(rng, 1, T, 1, 6, 4, unit=False)
        o, S = oracle.prefill(q, k, v, g, beta, S0)
        dk = 6
        Ss = S0[0, 0].copy()
        for t in range(T):
            kt = k[0, t, 0]
            At = (np.eye(dk) - beta[0, t, 0] * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, 0]))
            Ss = At @ Ss + beta[0, t, 0] * np.outer(kt, v[0, t, 0])
            _close(o[0, t, 0], Ss.T @ q[0, t, 0])
        # closed product form of the final state
        P = np.eye(dk)
        acc = np.zeros_like(S0[0, 0])
        for t in reversed(range(T)):
            kt = k[0, t, 0]
            acc += P @ (beta[0, t, 0] * np.outer(kt, v[0, t, 0]))
            P = P @ ((np.eye(dk) - beta[0, t, 0] * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, 0])))
        _close(S[0, 0], P @ S0[0, 0] + acc)
        _close(Ss, S[0, 0])


def test_linearity_and_value_permutation():
    """(V, S0) -> (O, S_T) is linear; permuting value channels permutes o and S columns."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 25, 2, 8, 6)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    o1, s1 = oracle.prefill(q, k, v, g, beta, S0)
    o2, s2 = oracle.prefill(q, k, v2, g, beta, S02)
    o3, s3 = oracle.prefill(q, k, v - 2.5 * v2, g, beta, S0 - 2.5 * S02)
    _close(o3, o1 - 2.5 * o2, 1e-11)
    _close(s3, s1 - 2.5 * s2, 1e-11)
    perm = rng.permutation(6)
    o4, s4 = oracle.prefill(q, k, v[..., perm], g, beta, S0[..., perm])
    _close(o4, o1[..., perm])
    _close(s4, s1[..., perm])


def test_state_passing():
    """One call over T equals two calls over T1 and T-T1 with S0 = S_T of the first (section 3.3)."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 37, 3, 8, 5)
    o, S = oracle.prefill(q, k, v, g, beta, S0)
    for T1 in (1, 16, 36):
        oa, Sa = oracle.prefill(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
        ob, Sb = oracle.prefill(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa)
        _close(np.concatenate([oa, ob], axis=1), o)
        _close(Sb, S)


def test_zero_length_and_threads():
    """T = 0 returns S_T = S0; thread count does not change the result."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 0, 3, 4, 4)
    o, S = oracle.prefill(q, k, v, g, beta, S0)
    assert o.shape == (2, 0, 3, 4)
    np.testing.assert_array_equal(S, S0)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 9, 3, 4, 4)
    a = oracle.prefill(q, k, v, g, beta, S0, nthreads=1)
    b = oracle.prefill(q, k, v, g, beta, S0, nthreads=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("C", [5, 8, 16, 32, 64])
@pytest.mark.parametrize("ref", ["direct", "center"])
def test_chunk_form_matches_oracle(C, ref):
    """The chunkwise WY/UT form (a separate derivation) reproduces the sequential oracle."""
    if ref == "center" and C > 32:
        pytest.skip("centre split of a 64-chunk spans 32 positions: e^160 overflows")
    rng = np.random.default_rng(8 + C)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 150, 2, 16, 8)
    o, S = oracle.prefill(q, k, v, g, beta, S0)
    for h in range(2):
        oc, Sc = chunk_forward(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h], S0[0, h], C, ref)
        _close(oc, o[0, :, h], 1e-10)
        _close(Sc, S[0, h], 1e-10)


def test_chunk_form_at_the_bound():
    """g = -5 everywhere (the bound): the centre-split 32-chunk stays finite and exact in fp64."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 96, 1, 16, 8)
    g[:] = -5.0
    o, S = oracle.prefill(q, k, v, g, beta, S0)
    oc, Sc = chunk_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0], 32, "center")
    assert np.isfinite(oc).all()
    _close(oc, o[0, :, 0], 1e-10)
    _close(Sc, S[0, 0], 1e-10)


# ------------------------------------------------------------------- decode --

def _decode_expected(qp, kp, vp, w, cache0, g, beta, S0, eps):
    """Preprocessing from library routines: np.convolve for the causal conv,
    torch's silu for Swish, np.linalg.norm for L2Norm; then the (pinned) prefill oracle."""
    Tn, N, H, dk = qp.shape
    dv = vp.shape[-1]
    W = w.shape[-1]
    x = np.concatenate([qp, kp, vp], axis=-1)                 # [T, N, H, nch]
    hist = np.concatenate([np.transpose(cache0, (2, 0, 1, 3)), x], axis=0)  # [W-1+T, N, H, nch]
    u = np.zeros_like(x)
    for n in range(N):
        for h in range(H):
            for c in range(x.shape[-1]):
                full = np.convolve(hist[:, n, h, c], w[h, c, ::-1], mode="valid")
                u[:, n, h, c] = full[:Tn]
    s = torch.nn.functional.silu(torch.from_numpy(u)).numpy()
    q = s[..., :dk] / np.sqrt(np.linalg.norm(s[..., :dk], axis=-1, keepdims=True) ** 2 + eps)
    k = s[..., dk:2 * dk] / np.sqrt(np.linalg.norm(s[..., dk:2 * dk], axis=-1, keepdims=True) ** 2 + eps)
    vv = s[..., 2 * dk:]
    # prefill oracle over T steps with (B, T, H) = (N, Tn, H)
    tr = lambda a: np.ascontiguousarray(np.transpose(a, (1, 0, 2, 3)))
    o, S = oracle.prefill(tr(q), tr(k), tr(vv), np.ascontiguousarray(np.transpose(g, (1, 0, 2, 3))),
                          np.ascontiguousarray(np.transpose(beta, (1, 0, 2))), S0)
    return np.transpose(o, (1, 0, 2, 3)), S


@pytest.mark.parametrize("W", [4, 2])
def test_decode_matches_preprocessing_and_prefill(W):
    rng = np.random.default_rng(11)
    Tn, N, H, dk, dv = 7, 2, 3, 8, 6
    nch = 2 * dk + dv
    qp = rng.standard_normal((Tn, N, H, dk))
    kp = rng.standard_normal((Tn, N, H, dk))
    vp = rng.standard_normal((Tn, N, H, dv))
    w = 0.5 * rng.standard_normal((H, nch, W))
    cache0 = rng.standard_normal((N, H, W - 1, nch))
    g = -5 / (1 + np.exp(-rng.standard_normal((Tn, N, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((Tn, N, H))))
    S0 = 0.1 * rng.standard_normal((N, H, dk, dv))
    eo, eS = _decode_expected(qp, kp, vp, w, cache0, g, beta, S0, oracle.L2NORM_EPS)
    cache = cache0.copy()
    S = S0.copy()
    pos = 5   # any start offset of the ring: rotate the initial cache to match
    cache = np.roll(cache0, shift=pos % (W - 1), axis=2).copy()
    for t in range(Tn):
        o = oracle.decode_step(qp[t], kp[t], vp[t], w, cache, pos + t, g[t], beta[t], S)
        _close(o, eo[t], 1e-11)
    _close(S, eS, 1e-11)


def test_decode_identity_conv_and_unit_norm():
    """Conv taps (0,...,0,1) pass x_t through; with beta = 1, g = 0, S = 0 the new state is
    k v^T with |k| = 1 (L2Norm) and v = silu(v_pre)."""
    rng = np.random.default_rng(12)
    N, H, dk, dv, W = 3, 2, 8, 5, 4
    nch = 2 * dk + dv
    w = np.zeros((H, nch, W))
    w[..., -1] = 1.0
    cache = rng.standard_normal((N, H, W - 1, nch))
    qp, kp = rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk))
    vp = rng.standard_normal((N, H, dv))
    S = np.zeros((N, H, dk, dv))
    o = oracle.decode_step(qp, kp, vp, w, cache, 0, np.zeros((N, H, dk)), np.ones((N, H)), S)
    vs = torch.nn.functional.silu(torch.from_numpy(vp)).numpy()
    ks = torch.nn.functional.silu(torch.from_numpy(kp)).numpy()
    kn = ks / np.sqrt((ks ** 2).sum(-1, keepdims=True) + oracle.L2NORM_EPS)
    _close(S, kn[..., :, None] * vs[..., None, :], 1e-13)
    # the oldest slot now holds x_t
    np.testing.assert_array_equal(cache[:, :, 0, :dk], qp)
    np.testing.assert_array_equal(cache[:, :, 0, 2 * dk:], vp)
    assert np.allclose(np.linalg.norm(kn, axis=-1), 1.0, atol=1e-6)
    assert o.shape == (N, H, dv)


# ---------------------------------------------------------------- snapshots --

def test_snapshots_are_prefix_final_states():
    """Snapshot s (the state after (s+1)*every tokens) is, independently, the final
    state of a prefill over that prefix -- the state a cached prefix resumes from
    (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section 9, the
    KDA-checkpoint / hash-block prefix cache figure)."""
    rng = np.random.default_rng(31)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 100, 3, 8, 4)
    o, S_T, snaps = oracle.prefill_snapshots(q, k, v, g, beta, S0, 16, 6)
    for s in range(6):
        t = (s + 1) * 16
        _, S_pre = oracle.prefill(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0)
        assert np.array_equal(S_pre, snaps[s])
    o2, S2 = oracle.prefill(q, k, v, g, beta, S0)
    assert np.array_equal(o, o2) and np.array_equal(S_T, S2)


def test_snapshot_at_the_end_is_the_final_state_and_resumes():
    """With T a multiple of the interval the last snapshot is S_T, and a prefill of
    the suffix started from a snapshot reproduces the tail of o and S_T."""
    rng = np.random.default_rng(32)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 96, 2, 8, 4)
    o, S_T, snaps = oracle.prefill_snapshots(q, k, v, g, beta, S0, 32, 3)
    assert np.array_equal(snaps[2], S_T)
    o_tail, S_tail = oracle.prefill(q[:, 32:], k[:, 32:], v[:, 32:], g[:, 32:], beta[:, 32:], snaps[0])
    _close(o_tail, o[:, 32:], 1e-12)
    _close(S_tail, S_T, 1e-12)


def test_snapshot_arguments_rejected():
    rng = np.random.default_rng(33)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 20, 1, 4, 4)
    with pytest.raises(RuntimeError):
        oracle.prefill_snapshots(q, k, v, g, beta, S0, 8, 3)   # 3 * 8 > 20
    with pytest.raises(RuntimeError):
        oracle.prefill_snapshots(q, k, v, g, beta, S0, 0, 1)


# -------------------------------------------------------- prefill preprocessing --

def _prep_inputs(rng, B, T, H, dk, dv, W=4, history=True):
    nch = 2 * dk + dv
    qp = rng.standard_normal((B, T, H, dk))
    kp = rng.standard_normal((B, T, H, dk))
    vp = rng.standard_normal((B, T, H, dv))
    w = 0.5 * rng.standard_normal((H, nch, W))
    init = rng.standard_normal((B, H, W - 1, nch)) if history else None
    z = 2.0 * rng.standard_normal((B, T, H, dk))
    A = rng.standard_normal(H)
    bl = 2.0 * rng.standard_normal((B, T, H))
    return qp, kp, vp, w, init, z, A, bl


def test_gate_and_beta_worked_values():
    """Hand-derived values where Sigmoid lands on an exact ratio (note, sections 3.2 and 3.3)."""
    with open(os.path.join(GOLDEN, "gate_beta_worked.json")) as f:
        gd = json.load(f)
    n = len(gd["gate"])
    H, dk, dv = n, 4, 2
    rng = np.random.default_rng(31)
    qp, kp, vp, w, init, _, _, _ = _prep_inputs(rng, 1, 1, H, dk, dv)
    A = np.array([math.log(e["eA"]) for e in gd["gate"]])
    z = np.empty((1, 1, H, dk))
    for h, e in enumerate(gd["gate"]):
        z[0, 0, h, :] = e["z_factor"] * math.log(e["z_ln_arg"])
    bl = np.array([[[e["logit_factor"] * math.log(e["logit_ln_arg"])
                     for e in (gd["beta"] * H)[:H]]]])
    _, _, _, g, beta, _ = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    for h, e in enumerate(gd["gate"]):
        np.testing.assert_allclose(g[0, 0, h], e["g"], rtol=0, atol=1e-14)
    for h in range(H):
        np.testing.assert_allclose(beta[0, 0, h], (gd["beta"] * H)[h]["beta"], rtol=0, atol=1e-15)


def test_gate_range_and_monotonicity():
    """g lies in (-5, 0), falls as z grows (for any A), and z = 0 gives -5/2 for every A."""
    rng = np.random.default_rng(32)
    H, dk, dv = 3, 64, 2
    qp, kp, vp, w, init, _, _, bl = _prep_inputs(rng, 1, 1, H, dk, dv)
    A = np.array([-2.0, 0.0, 1.5])
    zs = np.linspace(-8, 8, dk)
    z = np.broadcast_to(zs, (1, 1, H, dk)).copy()
    z[0, 0, :, dk // 2] = 0.0
    _, _, _, g, _, _ = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    g = g[0, 0]
    assert np.all(g > -5.0) and np.all(g < 0.0)
    np.testing.assert_allclose(g[:, dk // 2], -2.5, rtol=0, atol=1e-15)
    order = np.argsort(z[0, 0, 0], kind="stable")
    assert np.all(np.diff(g[:, order], axis=1) <= 0)
    # a larger A sharpens the map: further from -5/2 at the same z != 0
    far = np.abs(g + 2.5)
    nz = z[0, 0, 0] != 0
    assert np.all(far[2, nz] > far[1, nz]) and np.all(far[1, nz] > far[0, nz])


@pytest.mark.parametrize("history", [True, False])
def test_prep_matches_library_routines(history):
    """Conv by np.convolve, Swish by torch's silu, L2Norm by np.linalg.norm, sigmoids by
    scipy's expit (note, section 3.2 input branches; section 3.3 gate)."""
    from scipy.special import expit
    rng = np.random.default_rng(33)
    B, T, H, dk, dv, W = 2, 9, 3, 8, 6, 4
    qp, kp, vp, w, init, z, A, bl = _prep_inputs(rng, B, T, H, dk, dv, W, history)
    q, k, v, g, beta, fin = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    nch = 2 * dk + dv
    x = np.concatenate([qp, kp, vp], axis=-1)                       # [B, T, H, nch]
    hist = np.zeros((B, H, W - 1, nch)) if init is None else init
    seq = np.concatenate([np.transpose(hist, (0, 2, 1, 3)), x], axis=1)  # [B, W-1+T, H, nch]
    u = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            for c in range(nch):
                u[b, :, h, c] = np.convolve(seq[b, :, h, c], w[h, c, ::-1], mode="valid")
    s = torch.nn.functional.silu(torch.from_numpy(u)).numpy()
    eq = s[..., :dk] / np.sqrt(np.linalg.norm(s[..., :dk], axis=-1, keepdims=True) ** 2 + oracle.L2NORM_EPS)
    ek = s[..., dk:2 * dk] / np.sqrt(np.linalg.norm(s[..., dk:2 * dk], axis=-1, keepdims=True) ** 2
                                     + oracle.L2NORM_EPS)
    _close(q, eq, 1e-13)
    _close(k, ek, 1e-13)
    _close(v, s[..., 2 * dk:], 1e-13)
    _close(beta, expit(bl), 1e-15)
    _close(g, -5.0 * expit(np.exp(A)[None, None, :, None] * z), 1e-14)
    np.testing.assert_array_equal(fin, np.transpose(seq[:, -(W - 1):], (0, 2, 1, 3)))


def test_prep_split_resumes_through_conv_final():
    """Preprocessing T tokens at once equals two calls joined by conv_final -> conv_init,
    also when the second call is shorter than the conv history."""
    rng = np.random.default_rng(34)
    B, T, H, dk, dv = 2, 11, 2, 8, 4
    qp, kp, vp, w, init, z, A, bl = _prep_inputs(rng, B, T, H, dk, dv)
    full = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    for t1 in (0, 1, 5, 9, 10):
        cut = lambda a, sl: np.ascontiguousarray(a[:, sl])
        first = oracle.prefill_prep(cut(qp, slice(0, t1)), cut(kp, slice(0, t1)), cut(vp, slice(0, t1)),
                                    w, init, cut(z, slice(0, t1)), A, cut(bl, slice(0, t1)))
        second = oracle.prefill_prep(cut(qp, slice(t1, T)), cut(kp, slice(t1, T)), cut(vp, slice(t1, T)),
                                     w, first[5], cut(z, slice(t1, T)), A, cut(bl, slice(t1, T)))
        for i in range(5):
            np.testing.assert_array_equal(np.concatenate([first[i], second[i]], axis=1), full[i])
        np.testing.assert_array_equal(second[5], full[5])


def test_prep_then_prefill_equals_decode_steps():
    """The decode oracle (pinned separately against library routines) stepped token by token
    from the same conv history reproduces prep + prefill: outputs, state and conv history."""
    rng = np.random.default_rng(35)
    B, T, H, dk, dv, W = 2, 7, 3, 8, 6, 4
    qp, kp, vp, w, init, z, A, bl = _prep_inputs(rng, B, T, H, dk, dv, W)
    q, k, v, g, beta, fin = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, g, beta, S0)
    cache = init.copy()          # ring at position 0: slot 0 holds the oldest token
    S = S0.copy()
    for t in range(T):
        ot = oracle.decode_step(qp[:, t], kp[:, t], vp[:, t], w, cache, t, g[:, t], beta[:, t], S)
        _close(ot, o[:, t], 1e-12)
    _close(S, S_T, 1e-12)
    # after T steps the ring's oldest slot is T mod (W-1)
    np.testing.assert_array_equal(np.roll(cache, -(T % (W - 1)), axis=2), fin)


def test_prep_empty_and_rejects():
    rng = np.random.default_rng(36)
    qp, kp, vp, w, init, z, A, bl = _prep_inputs(rng, 2, 0, 2, 4, 4)
    q, k, v, g, beta, fin = oracle.prefill_prep(qp, kp, vp, w, init, z, A, bl)
    assert q.shape == (2, 0, 2, 4) and beta.shape == (2, 0, 2)
    np.testing.assert_array_equal(fin, init)
    with pytest.raises(ValueError):
        oracle.prefill_prep(qp, kp, vp, w, init, z, A[:1], bl)
    with pytest.raises(ValueError):
        oracle.prefill_prep(qp, kp, vp, w, init[:, :, :2], z, A, bl)


# ---------------------------------------------------------------------------
# Output exposure gate: y = Sigmoid(gate) * RMSNorm(o) * w (note, section 3.2,
# output equation, before W_o), RMSNorm over the dv channels of one head.

def test_output_gate_worked_values():
    with open(os.path.join(GOLDEN, "output_gate_worked.json")) as fh:
        ref = json.load(fh)
    for case in ref["cases"]:
        o = np.array(case["o"])[None, None]
        gate = np.log(np.array(case["gate_ln_arg"]))[None, None]   # Sigmoid(ln a) = a / (1 + a)
        w = None if case["w"] is None else np.array(case["w"])
        y = oracle.output_gate(o, gate, w, eps=case["eps"])
        want = np.array(case["y_sqrt2_factor"]) * math.sqrt(2.0)
        np.testing.assert_allclose(y[0, 0], want, rtol=1e-14, atol=1e-15)


def test_output_gate_matches_library_routines():
    rng = np.random.default_rng(41)
    o = rng.standard_normal((5, 3, 3, 64)) * 2.5
    gate = rng.standard_normal(o.shape) * 3
    w = rng.standard_normal(64)
    eps = 1e-3
    y = oracle.output_gate(o, gate, w, eps=eps)
    to = torch.from_numpy(o)
    ref = torch.sigmoid(torch.from_numpy(gate)) * torch.nn.functional.rms_norm(
        to, (64,), weight=torch.from_numpy(w), eps=eps)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_output_gate_invariants():
    rng = np.random.default_rng(42)
    o = rng.standard_normal((7, 4, 128))
    gate = rng.standard_normal(o.shape)
    # an open gate and unit weight leave exactly unit root-mean-square (eps = 0)
    y = oracle.output_gate(o, np.full(o.shape, 800.0), None, eps=0.0)
    np.testing.assert_allclose(np.mean(y ** 2, axis=-1), 1.0, rtol=1e-13)
    # scale invariance of RMSNorm (eps = 0) and oddness in o
    base = oracle.output_gate(o, gate, None, eps=0.0)
    np.testing.assert_allclose(oracle.output_gate(37.5 * o, gate, None, eps=0.0), base, rtol=1e-12)
    np.testing.assert_allclose(oracle.output_gate(-o, gate, None, eps=0.0), -base, rtol=0, atol=0)
    # a closed-at-half gate (0) halves the normalised readout, channel by channel
    half = oracle.output_gate(o, np.zeros(o.shape), None, eps=0.0)
    np.testing.assert_allclose(half * 2, oracle.output_gate(o, np.full(o.shape, 800.0), None, eps=0.0),
                               rtol=1e-13)
    # heads are normalised separately: scaling one head leaves the others alone
    o2 = o.copy()
    o2[:, 1] *= 1e3
    y2 = oracle.output_gate(o2, gate, None, eps=1e-6)
    y1 = oracle.output_gate(o, gate, None, eps=1e-6)
    np.testing.assert_array_equal(y2[:, 0], y1[:, 0])
    np.testing.assert_array_equal(y2[:, 2:], y1[:, 2:])


def test_output_gate_rejects():
    o = np.zeros((2, 3, 4))
    with pytest.raises(ValueError):
        oracle.output_gate(o, np.zeros((2, 3, 5)))
    with pytest.raises(ValueError):
        oracle.output_gate(o, o, np.ones(3))


# ---------------------------------------------------------------------------
# Backward: exact gradients of <dO, o> + <dS_T, S_T> (oracle/backward.py).

from oracle import backward as obwd
from tests.chunk_model import chunk_backward


def _bwd_case(rng, B, T, H, dk, dv, **kw):
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, **kw)
    dO = rng.standard_normal((B, T, H, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, S0, dO, dS


def _objective(q, k, v, g, beta, S0, dO, dS):
    o, S_T = oracle.prefill(q, k, v, g, beta, S0)
    return float(np.sum(o * dO) + np.sum(S_T * dS))


def test_backward_matches_central_differences_of_the_forward_oracle():
    """Directional derivatives of the (pinned) C forward oracle, by central
    differences, against <gradient, direction> for every input."""
    rng = np.random.default_rng(51)
    x = list(_bwd_case(rng, 1, 7, 2, 5, 4))
    grads = obwd.backward(*x)
    names = ("q", "k", "v", "g", "beta", "S0")
    h = 1e-6
    for idx, name in enumerate(names):
        d = rng.standard_normal(np.shape(x[idx]))
        xp = list(x)
        xm = list(x)
        xp[idx] = x[idx] + h * d
        xm[idx] = x[idx] - h * d
        fd = (_objective(*xp) - _objective(*xm)) / (2 * h)
        an = float(np.sum(grads[idx] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_backward_decay_only_closed_form():
    """beta = 0: S_t = Diag(e^{G_t}) S0, o_t = S_t^T q_t, so dv = 0, dq_t = S_t dO_t and
    dS0 = Diag(e^{G_T}) dS_T + sum_t Diag(e^{G_t}) q_t dO_t^T."""
    rng = np.random.default_rng(52)
    q, k, v, g, beta, S0, dO, dS = _bwd_case(rng, 1, 9, 1, 6, 5)
    beta = np.zeros_like(beta)
    dq, dk_, dv_, dg, db, dS0 = obwd.backward(q, k, v, g, beta, S0, dO, dS)
    G = np.cumsum(g[0, :, 0], axis=0)                       # [T, dk]
    np.testing.assert_allclose(dv_, 0.0, atol=1e-15)
    want_dq = np.stack([(np.exp(G[t])[:, None] * S0[0, 0]) @ dO[0, t, 0] for t in range(9)])
    np.testing.assert_allclose(dq[0, :, 0], want_dq, rtol=1e-12, atol=1e-13)
    want_dS0 = np.exp(G[-1])[:, None] * dS[0, 0] + sum(
        np.exp(G[t])[:, None] * np.outer(q[0, t, 0], dO[0, t, 0]) for t in range(9))
    np.testing.assert_allclose(dS0[0, 0], want_dS0, rtol=1e-12, atol=1e-13)
    # d/dg_s of sum_t <dO_t, S_t^T q_t> + <dS, S_T>: channel c of g_s scales rows c of S_t for t >= s
    terms = np.stack([np.exp(G[t]) * (S0[0, 0] @ dO[0, t, 0]) * q[0, t, 0] for t in range(9)])
    last = np.exp(G[-1]) * np.sum(S0[0, 0] * dS[0, 0], axis=1)
    want_dg = np.cumsum(terms[::-1], axis=0)[::-1] + last[None, :]
    np.testing.assert_allclose(dg[0, :, 0], want_dg, rtol=1e-12, atol=1e-13)


def test_backward_is_linear_in_the_upstream_gradients():
    rng = np.random.default_rng(53)
    q, k, v, g, beta, S0, dO, dS = _bwd_case(rng, 1, 6, 2, 4, 4)
    a = obwd.backward(q, k, v, g, beta, S0, dO, dS)
    b = obwd.backward(q, k, v, g, beta, S0, 2.5 * dO, 2.5 * dS)
    c = obwd.backward(q, k, v, g, beta, S0, dO, np.zeros_like(dS))
    d = obwd.backward(q, k, v, g, beta, S0, np.zeros_like(dO), dS)
    for x, y, u, w in zip(a, b, c, d):
        np.testing.assert_allclose(y, 2.5 * x, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(u + w, x, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C,inverse", [(16, "solve"), (16, "product"), (5, "solve"), (32, "solve")])
def test_chunk_backward_matches_oracle(C, inverse):
    """The chunk-form reverse mode (a second derivation) equals the autograd oracle."""
    rng = np.random.default_rng(54)
    q, k, v, g, beta, S0, dO, dS = _bwd_case(rng, 1, 40, 1, 8, 6)
    ref = obwd.backward(q, k, v, g, beta, S0, dO, dS)
    got = chunk_backward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0],
                         dO[0, :, 0], dS[0, 0], C, inverse=inverse)
    for name, r, x in zip(("dq", "dk", "dv", "dg", "dbeta"), ref[:5], got[:5]):
        np.testing.assert_allclose(x, r[0, :, 0], rtol=1e-9, atol=1e-10, err_msg=name)
    np.testing.assert_allclose(got[5], ref[5][0, 0], rtol=1e-9, atol=1e-10, err_msg="dS0")


def test_chunk_backward_at_the_bound():
    """g = -5 everywhere (the pages' lower bound): the reciprocal decay reaches e^{75}
    inside a 16-token chunk; the chunk form still matches the oracle."""
    rng = np.random.default_rng(55)
    q, k, v, g, beta, S0, dO, dS = _bwd_case(rng, 1, 32, 1, 8, 6)
    g = np.full_like(g, -5.0)
    ref = obwd.backward(q, k, v, g, beta, S0, dO, dS)
    got = chunk_backward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0],
                         dO[0, :, 0], dS[0, 0], 16)
    for name, r, x in zip(("dq", "dk", "dv", "dg", "dbeta"), ref[:5], got[:5]):
        scale = max(1.0, float(np.abs(r).max()))
        assert np.abs(x - r[0, :, 0]).max() <= 1e-9 * scale, name
