"""The allocation-free backward, kda_chunk_bwd_noalloc called through the C ABI, against
the workspace entry point kda_chunk_bwd on the same inputs.  Two calls in a row, the
second with smaller inputs, so that the second runs on a scratch array still holding
the first call's chunk states and partials: both must give exactly the gradients of
kda_chunk_bwd (the two share every kernel and the backward adds its slice partials in
a fixed order, so equality is bitwise), and one (sequence, head) of each call is also
checked against the fp64 oracle at the gradient bar."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import PrefillSpec, backward_inputs, prefill_inputs, to_f64
from oracle import backward as obwd
from tests.util import TOL_GRAD, assert_parity

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _noalloc(x, gr, out):
    """kda_chunk_bwd_noalloc through ctypes, into preallocated outputs."""
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    code = binding.KDA_FP32 if x["q"].dtype == torch.float32 else binding.KDA_BF16
    stream = ctypes.c_void_p(torch.cuda.current_stream(x["q"].device).cuda_stream)
    args = [p(x[n]) for n in ("q", "k", "v", "g", "beta", "S0")] + [p(gr["dO"]), p(gr["dS_T"])]
    args += [p(t) for t in out]
    return binding.lib().kda_chunk_bwd_noalloc(*args, B, T, H, dk, dv, code, stream)


def _oracle_check(x, gr, got, b, h, dtype, what):
    sl = lambda t: to_f64(t[b:b + 1, :, h:h + 1])
    S0 = None if x["S0"] is None else to_f64(x["S0"][b:b + 1, h:h + 1])
    ref = obwd.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), to_f64(x["beta"][b:b + 1, :, h:h + 1]),
                        S0, sl(gr["dO"]), to_f64(gr["dS_T"][b:b + 1, h:h + 1]))
    mine = [sl(t) for t in got[:4]] + [to_f64(got[4][b:b + 1, :, h:h + 1]), to_f64(got[5][b:b + 1, h:h + 1])]
    for name, m, r in zip(NAMES, mine, ref):
        assert_parity(m, r, TOL_GRAD[dtype], f"{what} b{b} h{h} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_backward_matches_workspace_entry_twice(gpu, dtype):
    # first call: 11500 token-heads at dk = dv = 128 (64.8 MB of the 64 MiB array: chunk
    # states, slice 0's partials, flags); second call smaller, with a ragged chunk
    first = PrefillSpec(B=2, H=5, T=1150, dk=128, dv=128, dtype=dtype, seed=301, s0_std=0.3)
    second = PrefillSpec(B=1, H=3, T=77, dk=128, dv=128, dtype=dtype, seed=302, s0_std=0.3)
    for n, spec in enumerate((first, second)):
        what = f"noalloc call {n + 1} {dtype} B{spec.B} H{spec.H} T{spec.T}"
        print(what, flush=True)
        need = binding.workspace_size(spec.B, spec.T, spec.H, spec.dk, spec.dv)
        assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
        x = prefill_inputs(spec, device=gpu)
        gr = backward_inputs(spec, device=gpu)
        ref = binding.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
        out = [torch.full_like(t, float("nan")) for t in ref]
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(gpu)
        rc = _noalloc(x, gr, out)
        assert rc == binding.KDA_OK, binding.lib().kda_strerror(rc)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(gpu) == before
        for name, a, r in zip(NAMES, out, ref):
            assert torch.equal(a, r), f"{what}: {name} differs from kda_chunk_bwd"
        _oracle_check(x, gr, out, spec.B - 1, spec.H - 1, dtype, what)


def test_noalloc_backward_binding_and_limit(gpu):
    """The binding's chunk_bwd_noalloc (outputs allocated by the binding) equals
    chunk_bwd; sizes beyond the scratch array are refused with KDA_ERR_TOO_LARGE
    before anything is launched."""
    spec = PrefillSpec(B=1, H=2, T=50, dk=64, dv=128, dtype="bf16", seed=303)
    x = prefill_inputs(spec, device=gpu)
    gr = backward_inputs(spec, device=gpu)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gr["dO"], gr["dS_T"])
    ref = binding.chunk_bwd(*args)
    got = binding.chunk_bwd_noalloc(*args)
    torch.cuda.synchronize()
    for name, a, r in zip(NAMES, got, ref):
        assert torch.equal(a, r), name
    big = PrefillSpec(B=1, H=4, T=4096, dk=128, dv=128, dtype="bf16", seed=304)
    assert binding.workspace_size(big.B, big.T, big.H, big.dk, big.dv) > binding.NOALLOC_SCRATCH_BYTES
    xb = prefill_inputs(big, device=gpu)
    gb = backward_inputs(big, device=gpu)
    with pytest.raises(binding.KdaError) as err:
        binding.chunk_bwd_noalloc(xb["q"], xb["k"], xb["v"], xb["g"], xb["beta"], xb["S0"], gb["dO"], gb["dS_T"])
    assert err.value.code == binding.KDA_ERR_TOO_LARGE
    assert np.isfinite(to_f64(got[3])).all()
