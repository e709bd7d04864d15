"""GPU prefill with the output exposure gate fused (kda_chunk_fwd_gated through the C
ABI): bit for bit kda_chunk_fwd followed by kda_output_gate (whose own parity with the
oracle is checked in test_gate_parity.py), and in fp32 mode the fp64 oracle's gate of the
oracle's prefill.  The cases span a grid that leaves CUs idle for the gate workers
(H * dv / 64 workgroups well below 256) and grids that fill the chip, where the workers
start only as prefill workgroups finish."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import WORKLOADS, PrefillSpec, gate_inputs, prefill_inputs, to_f64
from tests.util import TOL, assert_parity

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _gate_for(spec, gpu, seed, weight=True):
    gi = gate_inputs(spec.B * spec.T, spec.H, spec.dv, dtype=spec.dtype, seed=seed, device=gpu, weight=weight)
    return gi["gate"].view(spec.B, spec.T, spec.H, spec.dv), gi["norm_w"]


def _both(spec, gpu, seed, weight=True):
    x = prefill_inputs(spec, device=gpu)
    gate, w = _gate_for(spec, gpu, seed, weight)
    o, S = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
    y_ref = binding.output_gate(o, gate, w, eps=EPS)
    y, S2 = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w, eps=EPS)
    torch.cuda.synchronize()
    return x, gate, w, y, S2, y_ref, S


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (2, 3, 77), (1, 5, 300), (3, 2, 16)])
def test_gated_equals_prefill_then_gate(gpu, dtype, dk, dv, B, H, T):
    spec = PrefillSpec(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, seed=100 + T + H)
    _, _, _, y, S2, y_ref, S = _both(spec, gpu, seed=200 + T, weight=(T % 2 == 1))
    assert torch.equal(y, y_ref), f"y differs from prefill + gate: {(y.float() - y_ref.float()).abs().max()}"
    assert torch.equal(S2, S)
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_gated_fp32_matches_oracle(gpu, dk, dv):
    spec = PrefillSpec(B=2, H=3, T=77, dk=dk, dv=dv, dtype="fp32", seed=31)
    x, gate, w, y, S2, _, _ = _both(spec, gpu, seed=32)
    o_ref, S_ref = oracle.prefill(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]), to_f64(x["g"]),
                                  to_f64(x["beta"]), to_f64(x["S0"]))
    y_ref = oracle.output_gate(o_ref, to_f64(gate), to_f64(w), eps=EPS)
    # The prefill's bar, |do| <= 1e-5 |o|_inf, reaches y through the row's RMS
    # normalisation: |dy| <= |Sigmoid(gate) w| (|do| + |o| |d rms| / rms) / rms, at most
    # 2 |Sigmoid(gate) w| 1e-5 |o|_inf / rms per element, plus fp32 rounding of the gate.
    rms = np.sqrt((o_ref ** 2).mean(axis=-1, keepdims=True) + EPS)
    sw = np.abs(1.0 / (1.0 + np.exp(-to_f64(gate))) * to_f64(w))
    bar = 2 * TOL["fp32"][0] * np.abs(o_ref).max() * sw / rms + 1e-5 * np.abs(y_ref) + 1e-6 * np.abs(y_ref).max()
    got = to_f64(y)
    assert np.isfinite(got).all()
    excess = float((np.abs(got - y_ref) - bar).max())
    assert excess <= 0.0, f"gated prefill y exceeds its bar by {excess:.3e}"
    assert_parity(to_f64(S2), S_ref, TOL["fp32"][1], "gated prefill S_T")
    print(f"gated prefill fp32 dk{dk} dv{dv}: y max|diff| {np.abs(got - y_ref).max():.2e}", flush=True)


@pytest.mark.parametrize("B,H,T", [(4, 32, 1024), (8, 32, 333)])
def test_gated_when_the_prefill_fills_the_chip(gpu, B, H, T):
    """B*H*2 = 256 and 512 prefill workgroups: the gate workers start as they finish."""
    spec = PrefillSpec(B=B, H=H, T=T, dk=128, dv=128, seed=41)
    _, _, _, y, S2, y_ref, S = _both(spec, gpu, seed=42)
    assert torch.equal(y, y_ref) and torch.equal(S2, S)


def test_gated_workspace_reuse_and_in_place_state(gpu):
    """Two calls through one workspace (its stale counters are cleared by the call), the
    second streaming the state in place (S_T = S0)."""
    spec = PrefillSpec(B=2, H=5, T=250, dk=128, dv=128, seed=51)
    x = prefill_inputs(spec, device=gpu)
    gate, w = _gate_for(spec, gpu, 52)
    ws = torch.empty(binding.gated_workspace_size(2, 5, 128), dtype=torch.uint8, device=gpu)
    y1, S1 = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w, eps=EPS,
                                     workspace=ws)
    S_run = S1.clone()
    y2, _ = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], S_run, gate, w, eps=EPS,
                                    S_T=S_run, workspace=ws)
    o_a, S_a = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
    o_b, S_b = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], S_a, chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(y1, binding.output_gate(o_a, gate, w, eps=EPS)) and torch.equal(S1, S_a)
    assert torch.equal(y2, binding.output_gate(o_b, gate, w, eps=EPS)) and torch.equal(S_run, S_b)


def test_gated_empty_sequence_copies_the_state(gpu):
    spec = PrefillSpec(B=1, H=2, T=0, dk=64, dv=64, seed=61)
    x = prefill_inputs(spec, device=gpu)
    gate = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device=gpu)
    y, S = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, None, eps=EPS)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(S, x["S0"])


def test_gated_marks_nan_when_waits_give_up(gpu):
    """spin_limit 0 (forced from the host): every wait gives up at its first unsatisfied
    poll; the kernel still finishes and every y row is NaN, never stale or partial."""
    spec = PrefillSpec(B=1, H=4, T=200, dk=128, dv=128, seed=71)
    x = prefill_inputs(spec, device=gpu)
    gate, w = _gate_for(spec, gpu, 72)
    y, S = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w, eps=EPS,
                                   spin_limit=0)
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all(), "y not marked"
    assert torch.isnan(S).all(), "S_T not marked"
    y2, _ = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w, eps=EPS)
    o, _ = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(y2, binding.output_gate(o, gate, w, eps=EPS))


def test_gated_k3_shape_equals_prefill_then_gate(gpu):
    """The K3 prefill shape (B1 H96 T65536 d128 bf16), in the launch the benchmark times:
    the whole y equals prefill + gate bit for bit, and S_T too."""
    spec = WORKLOADS["k3_prefill"]
    x = prefill_inputs(spec, device=gpu)
    gate, w = _gate_for(spec, gpu, 6)
    o, S = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
    y_ref = binding.output_gate(o, gate, w, eps=EPS)
    del o
    y, S2 = binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w, eps=EPS)
    torch.cuda.synchronize()
    same = torch.eq(y, y_ref)
    if not bool(same.all()):
        bad = (~same).nonzero()
        raise AssertionError(f"{bad.shape[0]} y elements differ, first at {bad[0].tolist()}")
    assert torch.equal(S2, S)
    print("gated K3: y and S_T equal prefill + gate", flush=True)
