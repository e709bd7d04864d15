"""CPU pins of the algebra the chunk-16 prefill kernel evaluates (no GPU).

The kernel forms, per 16-token chunk, the decayed operands with the chunk start as
the single reference point, inverts I + A (A strictly lower triangular) as the
exact finite product (I - A)(I + A^2)(I + A^4)(I + A^8), and evaluates that
product on 16x16x4 fp32 matrix instructions with every matrix held in the
accumulator layout, building T^T (T's register image as an A operand).  These
tests check each step against the fp64 oracle or a dense inverse:
  * the chunk-start form with the product inverse reproduces the oracle;
  * the product equals the dense inverse for any strictly lower A, including A
    with entries of the size beta <k_r, k_i> reaches (|A| <= 1, up to 15 rows);
  * a lane-exact model of the matrix instruction and of the composition the
    kernel uses reproduces T^T in the consumers' operand layout.
The kernel's chunk relation is the pages' chunk interface (X_[c], S_in) ->
(Y_[c], S_out) (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读",
section 3.3); the inversion is exact algebra, not an approximation.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_18_amd.inputs import PrefillSpec, backward_inputs, prefill_inputs
from tests.chunk_model import chunk_backward, chunk_forward, nilpotent_inverse


def _inputs(rng, T, dk, dv, gscale=1.0):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = -5.0 * gscale / (1.0 + np.exp(-rng.standard_normal((T, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.02 * rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("gscale", [1.0, 0.0])
def test_chunk_start_form_with_product_inverse_matches_oracle(gscale):
    rng = np.random.default_rng(21)
    q, k, v, g, beta, S0 = _inputs(rng, 100, 16, 8, gscale)
    args = [x[None, :, None] for x in (q, k, v, g)] + [beta[None, :, None], S0[None, None]]
    o, S = oracle.prefill(*args)
    oc, Sc = chunk_forward(q, k, v, g, beta, S0, 16, ref="start", inverse="product")
    assert np.abs(oc - o[0, :, 0]).max() <= 1e-10 * np.abs(o).max()
    assert np.abs(Sc - S[0, 0]).max() <= 1e-10 * np.abs(S).max()


def test_chunk_start_form_at_the_bound():
    """g = -5 on every token: the column factor reaches e^75 and stays finite."""
    rng = np.random.default_rng(22)
    q, k, v, g, beta, S0 = _inputs(rng, 64, 16, 8)
    g[:] = -5.0
    args = [x[None, :, None] for x in (q, k, v, g)] + [beta[None, :, None], S0[None, None]]
    o, S = oracle.prefill(*args)
    oc, Sc = chunk_forward(q, k, v, g, beta, S0, 16, ref="start", inverse="product")
    assert np.isfinite(oc).all()
    assert np.abs(oc - o[0, :, 0]).max() <= 1e-10 * np.abs(o).max()


@pytest.mark.parametrize("n", [1, 2, 7, 16])
@pytest.mark.parametrize("scale", [0.3, 1.0])
def test_product_inverse_equals_dense_inverse(n, scale):
    rng = np.random.default_rng(23 + n)
    A = np.tril(rng.uniform(-scale, scale, (n, n)), -1)
    inv = np.linalg.inv(np.eye(n) + A)
    got = nilpotent_inverse(A)
    assert np.abs(got - inv).max() <= 1e-12 * max(1.0, np.abs(inv).max())


def test_product_inverse_worst_case_growth():
    """A = strict lower part of all ones (beta = 1, identical unit keys, no decay):
    (I + A)^{-1} has entries of size 1 and the product is still exact."""
    A = np.tril(np.ones((16, 16)), -1)
    inv = np.linalg.inv(np.eye(16) + A)
    assert np.abs(nilpotent_inverse(A) - inv).max() <= 1e-12 * np.abs(inv).max()


# ---- lane-exact model of the 16x16x4 fp32 matrix instruction -------------------

def _acc_layout(X):
    """Accumulator layout: lane n + 16 g holds rows 4g .. 4g+3 of column n."""
    out = np.zeros((64, 4))
    for lane in range(64):
        n, g = lane % 16, lane // 16
        out[lane] = X[4 * g:4 * g + 4, n]
    return out


def _from_acc(R):
    X = np.zeros((16, 16))
    for lane in range(64):
        n, g = lane % 16, lane // 16
        X[4 * g:4 * g + 4, n] = R[lane]
    return X


def _mfma_16x16x4(a, b, c):
    """D = A B + C with A[i][kk] from lane i + 16 kk, B[kk][n] from lane n + 16 kk."""
    A = np.array([[a[i + 16 * kk] for kk in range(4)] for i in range(16)])
    B = np.array([[b[n + 16 * kk] for n in range(16)] for kk in range(4)])
    return c + _acc_layout(A @ B)


def _mul(xt, y):
    """The kernel's product: X Y from X^T and Y in accumulator layout, step s taking
    element s of every lane (contraction index 4 g + s in lane group g)."""
    acc = np.zeros((64, 4))
    for s in range(4):
        acc = _mfma_16x16x4(xt[:, s], y[:, s], acc)
    return acc


def test_mul_is_the_matrix_product():
    rng = np.random.default_rng(24)
    X, Y = rng.standard_normal((16, 16)), rng.standard_normal((16, 16))
    assert np.allclose(_from_acc(_mul(_acc_layout(X.T), _acc_layout(Y))), X @ Y, rtol=0, atol=1e-12)
    # the transposed product from the same registers
    assert np.allclose(_from_acc(_mul(_acc_layout(Y), _acc_layout(X.T))), (X @ Y).T, rtol=0, atol=1e-12)


def test_transposed_inverse_in_operand_layout():
    """T^T = Diag(beta)(I - A^T)(I + A2^T)(I + A4^T)(I + A8^T) built from A and A^T in
    accumulator layout equals (inv(I + A) Diag(beta))^T, i.e. lane r + 16 g holds
    T[r][4g .. 4g+3] -- the A-operand image the consumers read."""
    rng = np.random.default_rng(25)
    Kt, Kc = rng.standard_normal((16, 32)) * 0.2, rng.standard_normal((16, 32)) * 0.2
    beta = rng.uniform(0, 1, 16)
    raw = Kt @ Kc.T
    A_full = np.tril(beta[:, None] * raw, -1)
    A, AT = _acc_layout(A_full), _acc_layout(A_full.T)
    A2, A2T = _mul(AT, A), _mul(A, AT)
    A4, A4T = _mul(A2T, A2), _mul(A2, A2T)
    A8T = _mul(A4, A4T)
    I4 = _acc_layout(np.eye(16))
    WT = I4 + A4T + A8T + _mul(A4, A8T)
    W2T = WT + _mul(A2, WT)
    LiT = W2T - _mul(A, W2T)
    br = _acc_layout(np.repeat(beta[:, None], 16, axis=1))     # beta of each lane's rows
    TT = br * LiT
    T = np.linalg.inv(np.eye(16) + A_full) @ np.diag(beta)
    image = np.array([T[lane % 16, 4 * (lane // 16):4 * (lane // 16) + 4] for lane in range(64)])
    assert np.abs(TT - image).max() <= 1e-12 * np.abs(T).max()


def test_fp32_backward_at_the_bound_needs_subnormal_operands():
    """g = -5 on every token and channel: the operand k e^G of the last tokens of a chunk
    falls below fp32's smallest normal number for small |k|, and dg sums products such as
    dKt Kt and dKc Kc whose factors reach e^{+-80} before they cancel.  The float32
    chunk-form reverse mode (float32 inverse, as the kernel's fp32 mode) keeps every
    other gradient within 1e-6 of the fp64 gradients but dg only within 2e-5 (5.5e-6 to
    1.2e-5 over seeds) when the sub-normal values are kept, and dg drifts to between 1e-5
    and 1e-4 when they are flushed to zero, as fp32 matrix units flush them.  This is the
    measured basis of the fp32-mode dg bar of the GPU backward test at the bound."""
    from oracle import backward as obwd
    spec = PrefillSpec(B=1, H=2, T=48, dk=128, dv=128, dtype="fp32", seed=99, gate="const", g_const=-5.0)
    x = prefill_inputs(spec)
    gr = backward_inputs(spec)
    f = lambda t: t.double().numpy()
    worst = {False: np.zeros(6), True: np.zeros(6)}
    for h in range(spec.H):
        q, k, v, g = (f(x[n][0, :, h]) for n in "qkvg")
        beta, S0 = f(x["beta"][0, :, h]), f(x["S0"][0, h])
        dO, dS = f(gr["dO"][0, :, h]), f(gr["dS_T"][0, h])
        ref = obwd.backward(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                            beta[None, :, None], S0[None, None], dO[None, :, None], dS[None, None])
        ref = [r[0, :, 0] for r in ref[:5]] + [ref[5][0, 0]]
        for flush in (False, True):
            got = chunk_backward(q, k, v, g, beta, S0, dO, dS, 16, dtype=np.float32, flush_subnormal=flush)
            for i, (a, r) in enumerate(zip(got, ref)):
                worst[flush][i] = max(worst[flush][i], np.abs(a - r).max() / np.abs(r).max())
    dg = 3
    assert np.delete(worst[False], dg).max() < 1e-6 and worst[False][dg] < 2e-5, worst[False]
    assert np.delete(worst[True], dg).max() < 2e-6, worst[True]
    assert 1e-5 < worst[True][dg] < 1e-4, worst[True]
