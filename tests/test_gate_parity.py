"""GPU output exposure gate (kda_output_gate, kda_decode_step_gated through the C ABI)
against the fp64 CPU oracle: y = Sigmoid(gate) * RMSNorm(o) * w per (row, head)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import (DecodeSpec, PrefillSpec, decode_gate_inputs, decode_state,
                                            decode_step_inputs, gate_inputs, prefill_inputs, to_f64)
from tests.util import TOL, assert_close_elementwise, assert_parity

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dv", [128, 64])
@pytest.mark.parametrize("rows,H,weight", [(1, 1, True), (37, 3, True), (300, 5, False), (4096, 7, True)])
def test_output_gate_small(gpu, dtype, dv, rows, H, weight):
    x = gate_inputs(rows, H, dv, dtype=dtype, seed=rows + H, device=gpu, weight=weight)
    y = binding.output_gate(x["o"], x["gate"], x["norm_w"], eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.output_gate(to_f64(x["o"]), to_f64(x["gate"]), to_f64(x["norm_w"]), eps=EPS)
    e = assert_close_elementwise(to_f64(y), ref, dtype, f"gate {dtype} dv{dv} rows{rows} H{H}")
    print(f"output gate {dtype} dv{dv} {rows}x{H}: err {e:.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_output_gate_in_place_and_tiny_rows(gpu, dtype):
    x = gate_inputs(129, 2, 128, dtype=dtype, seed=5, device=gpu)
    ref = oracle.output_gate(to_f64(x["o"]), to_f64(x["gate"]), to_f64(x["norm_w"]), eps=EPS)
    o = x["o"].clone()
    y = binding.output_gate(o, x["gate"], x["norm_w"], eps=EPS, y=o)     # in place over o
    torch.cuda.synchronize()
    assert y.data_ptr() == o.data_ptr()
    assert_close_elementwise(to_f64(o), ref, dtype, "in place over o")
    g = x["gate"].clone()
    binding.output_gate(x["o"], g, x["norm_w"], eps=EPS, y=g)           # in place over gate
    torch.cuda.synchronize()
    assert_close_elementwise(to_f64(g), ref, dtype, "in place over gate")
    # all-zero readout rows stay zero; a large eps damps a small readout
    z = torch.zeros_like(x["o"])
    assert torch.count_nonzero(binding.output_gate(z, x["gate"], x["norm_w"], eps=EPS)) == 0
    big = binding.output_gate(x["o"], x["gate"], None, eps=1e4)
    ref_big = oracle.output_gate(to_f64(x["o"]), to_f64(x["gate"]), None, eps=1e4)
    assert_close_elementwise(to_f64(big), ref_big, dtype, "large eps")


def test_output_gate_k3_shape_sampled(gpu):
    """The K3 prefill output shape: 65536 tokens x 96 heads x 128, bf16; 512 sampled rows."""
    x = gate_inputs(65536, 96, 128, dtype="bf16", seed=6, device=gpu)
    y = binding.output_gate(x["o"], x["gate"], x["norm_w"], eps=EPS)
    torch.cuda.synchronize()
    rows = torch.as_tensor(np.r_[0:8, 65528:65536, np.random.default_rng(7).integers(0, 65536, 496)],
                           device=gpu)
    ref = oracle.output_gate(to_f64(x["o"][rows]), to_f64(x["gate"][rows]), to_f64(x["norm_w"]), eps=EPS)
    e = assert_close_elementwise(to_f64(y[rows]), ref, "bf16", "k3 gate")
    print(f"output gate 65536x96x128 bf16 (512 rows): err {e:.2e}", flush=True)


def test_prefill_then_gate_matches_oracle(gpu):
    """kda_output_gate on kda_chunk_fwd's output in its [B, T, H, dv] layout equals the
    oracle gate of that same output.  (The gate divides each row by its own RMS, so
    prefill's rounding, bounded relative to the largest |o|, is not a fixed fraction
    of a small row's y: the recurrence's parity is checked by the prefill tests.)"""
    spec = PrefillSpec(B=2, H=3, T=100, dk=128, dv=128, seed=8)
    x = prefill_inputs(spec, device=gpu)
    o, _ = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
    gi = gate_inputs(2 * 100, 3, 128, seed=9, device=gpu)
    gate = gi["gate"].view(2, 100, 3, 128)
    y = binding.output_gate(o, gate, gi["norm_w"], eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.output_gate(to_f64(o), to_f64(gate), to_f64(gi["norm_w"]), eps=EPS)
    e = assert_parity(to_f64(y), ref, TOL["bf16"][0], "prefill + gate")
    print(f"prefill + gate: err {e:.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv,weight", [(128, 128, True), (64, 64, False), (128, 64, True), (64, 128, True)])
def test_decode_gated_matches_oracle_and_plain_decode(gpu, dtype, dk, dv, weight):
    spec = DecodeSpec(N=5, H=3, dk=dk, dv=dv, dtype=dtype, seed_base=80, state_seed=81)
    st = decode_state(spec, device=gpu)
    S_g, cache_g = st["S"].clone(), st["conv_cache"].clone()
    S_p, cache_p = st["S"].clone(), st["conv_cache"].clone()
    S_o, cache_o = to_f64(st["S"]).copy(), to_f64(st["conv_cache"]).copy()
    w_o = to_f64(st["conv_w"])
    nw = (1.0 + 0.1 * torch.randn(dv, generator=torch.Generator().manual_seed(3))).to(gpu) if weight else None
    to, ts = TOL[dtype]
    for step in range(5):
        x = decode_step_inputs(spec, step, device=gpu)
        gate = decode_gate_inputs(spec, step, device=gpu)
        y = binding.decode_step_gated(x["q_pre"], x["k_pre"], x["v_pre"], st["conv_w"], cache_g, 3 + step,
                                      x["g"], x["beta"], S_g, gate, nw, eps=EPS)
        binding.decode_step(x["q_pre"], x["k_pre"], x["v_pre"], st["conv_w"], cache_p, 3 + step,
                            x["g"], x["beta"], S_p)
        torch.cuda.synchronize()
        oo = oracle.decode_step(to_f64(x["q_pre"]), to_f64(x["k_pre"]), to_f64(x["v_pre"]), w_o, cache_o,
                                3 + step, to_f64(x["g"]), to_f64(x["beta"]), S_o)
        ref = oracle.output_gate(oo, to_f64(gate), None if nw is None else to_f64(nw), eps=EPS)
        assert_parity(to_f64(y), ref, to, f"step {step} y")
        assert_parity(to_f64(S_g), S_o, ts, f"step {step} S")
        # the fused epilogue leaves the state and the cache exactly as the plain step does
        assert torch.equal(S_g, S_p) and torch.equal(cache_g, cache_p)
