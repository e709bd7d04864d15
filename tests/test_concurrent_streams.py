"""Calls on two streams at once.  The library keeps no state between calls, so two calls on
different buffers may run concurrently; the kernels whose workgroups hand data to each other
through an XCD's L2 (the backward's value slices, the gated and fused prefill launches) must
then still find their partners where they expect them, while another grid shares the chip.
Each case runs two different problems on two streams, several times, and compares every
output bit for bit with the same problems run one after the other."""
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import (PrefillSpec, PrepSpec, backward_inputs, gate_inputs,
                                            prefill_inputs, prep_inputs)

pytestmark = pytest.mark.gpu
REPEATS = 3


def _both(run_a, run_b):
    """Serial reference, then REPEATS concurrent runs on two streams; outputs compared bitwise."""
    ref_a, ref_b = run_a(), run_b()
    torch.cuda.synchronize()
    ref_a, ref_b = [t.clone() for t in ref_a], [t.clone() for t in ref_b]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(REPEATS):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            out_a = run_a()
        with torch.cuda.stream(s2):
            out_b = run_b()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(out_a, ref_a)):
            assert torch.equal(x, y), f"repeat {rep}: first problem, output {i} differs under concurrency"
        for i, (x, y) in enumerate(zip(out_b, ref_b)):
            assert torch.equal(x, y), f"repeat {rep}: second problem, output {i} differs under concurrency"


def test_backward_on_two_streams(gpu):
    specs = [PrefillSpec(B=2, H=32, T=1024, dk=128, dv=128, seed=801),
             PrefillSpec(B=2, H=30, T=700, dk=128, dv=128, seed=802)]
    data = [(prefill_inputs(s, device=gpu), backward_inputs(s, device=gpu)) for s in specs]

    def run(i):
        x, gr = data[i]
        return lambda: [t for t in binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"],
                                                     gr["dO"], gr["dS_T"]) if t is not None]
    _both(run(0), run(1))
    print("backward on two streams: bit-identical to serial", flush=True)


def test_prefill_gated_on_two_streams(gpu):
    specs = [PrefillSpec(B=1, H=24, T=3000, dk=128, dv=128, seed=811),
             PrefillSpec(B=2, H=16, T=2048, dk=128, dv=128, seed=812)]
    data = []
    for s in specs:
        x = prefill_inputs(s, device=gpu)
        gi = gate_inputs(s.B * s.T, s.H, s.dv, seed=s.seed + 1, device=gpu)
        data.append((x, gi["gate"].view(s.B, s.T, s.H, s.dv), gi["norm_w"]))

    def run(i):
        x, gate, w = data[i]
        return lambda: list(binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate, w))
    _both(run(0), run(1))
    print("gated prefill on two streams: bit-identical to serial", flush=True)


def test_plain_prefill_on_two_streams(gpu):
    specs = [PrefillSpec(B=1, H=40, T=2000, dk=128, dv=128, seed=821),
             PrefillSpec(B=3, H=8, T=1500, dk=128, dv=128, seed=822)]
    data = [prefill_inputs(s, device=gpu) for s in specs]

    def run(i):
        x = data[i]
        return lambda: list(binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16))
    _both(run(0), run(1))
    print("prefill on two streams: bit-identical to serial", flush=True)


def test_prefill_from_proj_on_two_streams(gpu):
    specs = [PrepSpec(B=1, T=2000, H=12, dk=128, dv=128, seed=831),
             PrepSpec(B=1, T=1600, H=10, dk=128, dv=128, seed=832)]
    data = [prep_inputs(s, device=gpu) for s in specs]

    def run(i):
        p = data[i]
        def call():
            o, S_T, out = binding.chunk_fwd_from_proj(p["q_pre"], p["k_pre"], p["v_pre"], p["conv_w"],
                                                      p["conv_init"], p["z"], p["A"], p["beta_logit"])
            return [o, S_T] + [out[n] for n in sorted(out) if out[n] is not None]
        return call
    _both(run(0), run(1))
    print("fused preprocessing + prefill on two streams: bit-identical to serial", flush=True)
