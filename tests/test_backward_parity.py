"""GPU backward (kda_chunk_bwd through the C ABI) against the fp64 autograd oracle:
gradients of <dO, o> + <dS_T, S_T> with respect to q, k, v, g, beta and S0."""
import numpy as np
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import PrefillSpec, backward_inputs, identical_key_inputs, prefill_inputs, to_f64
from oracle import backward as obwd
from tests.util import TOL_GRAD, assert_parity

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _check(spec, gpu, T=None, ds_std=1.0, heads=None, tol=None, what="", x=None, tol_by_name=None):
    x = prefill_inputs(spec, device=gpu, T=T) if x is None else x
    gr = backward_inputs(spec, device=gpu, T=T, ds_std=ds_std)
    got = binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    torch.cuda.synchronize()
    tol = TOL_GRAD[spec.dtype] if tol is None else tol
    heads = heads or [(b, h) for b in range(spec.B) for h in range(spec.H)]
    Tn = x["q"].shape[1]
    worst = dict.fromkeys(NAMES, 0.0)
    for b, h in heads:
        sl = lambda t: None if t is None else to_f64(t[b:b + 1, :, h:h + 1])
        S0 = None if x["S0"] is None else to_f64(x["S0"][b:b + 1, h:h + 1])
        dS = np.zeros((1, 1, spec.dk, spec.dv)) if gr["dS_T"] is None else to_f64(gr["dS_T"][b:b + 1, h:h + 1])
        ref = obwd.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                            to_f64(x["beta"][b:b + 1, :, h:h + 1]), S0, sl(gr["dO"]), dS)
        mine = [to_f64(t[b:b + 1, :, h:h + 1]) for t in got[:4]]
        mine.append(to_f64(got[4][b:b + 1, :, h:h + 1]))
        mine.append(to_f64(got[5][b:b + 1, h:h + 1]))
        for name, m, r in zip(NAMES, mine, ref):
            if Tn == 0 and name != "dS0":
                continue
            t = (tol_by_name or {}).get(name, tol)
            worst[name] = max(worst[name], assert_parity(m, r, t, f"{what} b{b} h{h} {name}"))
    print(f"backward {what}: " + " ".join(f"{k} {v:.1e}" for k, v in worst.items()), flush=True)
    return got


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 16, 32, 40])
def test_backward_small(gpu, dtype, dk, dv, T):
    spec = PrefillSpec(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype, seed=90 + T, s0_std=0.3)
    _check(spec, gpu, what=f"{dtype} dk{dk} dv{dv} T{T}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_identical_keys(gpu, dtype):
    """Identical unit keys, beta = 1, g = 0: in every chunk A is all ones below the
    diagonal, the hardest case for the chunk inverse (T = 40: a ragged last chunk)."""
    spec = PrefillSpec(B=1, H=2, T=40, dk=128, dv=128, dtype=dtype, seed=99)
    x = identical_key_inputs(1, 40, 2, 128, 128, dtype=dtype, device=gpu)
    _check(spec, gpu, x=x, what=f"identical keys {dtype}")


def test_backward_zero_initial_state_and_no_final_gradient(gpu):
    spec = PrefillSpec(B=1, H=3, T=50, dk=128, dv=128, dtype="fp32", seed=97, s0_std=0.0)
    _check(spec, gpu, ds_std=0.0, what="S0=None dS_T=None")


def test_backward_empty_sequence(gpu):
    spec = PrefillSpec(B=1, H=2, T=0, dk=64, dv=64, dtype="fp32", seed=98, s0_std=0.3)
    x = prefill_inputs(spec, device=gpu)
    gr = backward_inputs(spec, device=gpu)
    got = binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    torch.cuda.synchronize()
    assert torch.equal(got[5], gr["dS_T"])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_at_the_bound(gpu, dtype):
    """g = -5 for every token and channel: the reciprocal decay reaches e^{75} in a chunk,
    and the chunk-start-referenced operands k e^G fall to e^-80 |k|, below fp32's smallest
    normal number (1.2e-38) for |k| < 6.6e-3.  dg sums products whose factors reach
    e^{+-80} before they cancel: the float32 evaluation of this chunk algebra holds dg to
    5.5e-6 - 1.2e-5 of its norm with sub-normal operands kept and 2.3e-5 - 4.1e-5 with them
    flushed to zero, as the fp32 matrix cores flush them
    (tests/test_chunk_algebra.py::test_fp32_backward_at_the_bound_needs_subnormal_operands).
    dg alone is held to 1e-4 here; every other gradient to the 1e-5 bar."""
    spec = PrefillSpec(B=1, H=2, T=48, dk=128, dv=128, dtype=dtype, seed=99, gate="const", g_const=-5.0)
    _check(spec, gpu, what=f"g=-5 {dtype}", tol_by_name={"dg": 1e-4} if dtype == "fp32" else None)


@pytest.mark.parametrize("name", ["L1", "L1_bf16"])
def test_backward_long_memory(gpu, name):
    from gated_delta_rule_18_amd.inputs import WORKLOADS
    spec = WORKLOADS[name]
    _check(spec, gpu, what=name)


def test_backward_b4h32_sampled_heads(gpu):
    """B4 H32 T4096 d128 bf16 (the training-sized prefill config): 3 heads checked."""
    spec = PrefillSpec(B=4, H=32, T=4096, dk=128, dv=128, seed=1)
    _check(spec, gpu, heads=[(0, 0), (1, 17), (3, 31)], what="B4 H32 T4096 (3 heads)")


def test_backward_deterministic(gpu):
    spec = PrefillSpec(B=1, H=4, T=200, dk=128, dv=128, seed=100)
    x = prefill_inputs(spec, device=gpu)
    gr = backward_inputs(spec, device=gpu)
    a = binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    b = binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


@pytest.mark.parametrize("B,H,T", [(8, 40, 100), (3, 97, 33)])
def test_backward_grid_larger_than_the_chip(gpu, B, H, T):
    """640 workgroups (320 heads) and 592 (291 heads, not a multiple of 8: 582 busy) for 256 CUs: the
    two value-slice workgroups of a head hand partial gradients to each other through the
    L2 of their XCD, and heads run in several waves.  Heads from the first, middle and last
    waves against the oracle."""
    spec = PrefillSpec(B=B, H=H, T=T, dk=128, dv=128, seed=700 + H)
    heads = [(0, 0), (0, 7), (B // 2, H // 2), (B - 1, H - 9), (B - 1, H - 1)]
    _check(spec, gpu, heads=heads, what=f"B{B} H{H} T{T} ({B * H * 2} workgroups)")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_failed_handoff_marks_the_head_nan(gpu, dtype):
    """The failure path of the value slices' hand-off, forced from the host through
    kda_chunk_bwd_ex (the second slice takes the first for one on another XCD): every
    dq, dk, dg, dbeta of a two-slice head is NaN, while dv and dS0, which each slice
    writes itself, equal the normal call's bit for bit; every kernel exits normally."""
    spec = PrefillSpec(B=2, H=3, T=100, dk=128, dv=128, dtype=dtype, seed=140)
    x = prefill_inputs(spec, device=gpu)
    gr = backward_inputs(spec, device=gpu)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    good = binding.chunk_bwd(*args)
    bad = binding.chunk_bwd(*args, fail_xcd_check=True)
    torch.cuda.synchronize()
    for name, t in zip(("dq", "dk", "dg", "dbeta"), (bad[0], bad[1], bad[3], bad[4])):
        assert torch.isnan(t).all(), f"{name}: {int((~torch.isnan(t)).sum())} values not NaN"
    assert torch.equal(bad[2], good[2]), "dv changed"
    assert torch.equal(bad[5], good[5]), "dS0 changed"
    assert not any(torch.isnan(t).any() for t in good), "the normal call marked NaN"
    print(f"failed hand-off ({dtype}): dq, dk, dg, dbeta all NaN; dv, dS0 exact", flush=True)
