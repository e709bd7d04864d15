"""GPU kda_validate_inputs (through the C ABI) against the plain definition of the value
domains, g in [-5, 0] and beta in [0, 1] with NaN outside both, evaluated with numpy on a
host copy of the same tensors."""
import numpy as np
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import WORKLOADS, PrefillSpec, prefill_inputs, to_f64

pytestmark = pytest.mark.gpu


def _expected(g, beta):
    out = {}
    for name, t, lo, hi in (("g", g, -5.0, 0.0), ("beta", beta, 0.0, 1.0)):
        x = to_f64(t).reshape(-1)
        bad = ~((x >= lo) & (x <= hi))
        idx = np.flatnonzero(bad)
        out[f"bad_{name}"] = int(bad.sum())
        out[f"first_bad_{name}"] = int(idx[0]) if idx.size else -1
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_validate_clean_inputs(gpu, dtype):
    spec = PrefillSpec(B=2, H=3, T=100, dk=128, dv=128, dtype=dtype, seed=13, bound_frac=0.1)
    x = prefill_inputs(spec, device=gpu)
    assert binding.validate_inputs(x["g"], x["beta"]) == dict(bad_g=0, first_bad_g=-1, bad_beta=0,
                                                              first_bad_beta=-1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_validate_finds_planted_values(gpu, dtype):
    x = prefill_inputs(PrefillSpec(B=2, H=3, T=100, dk=64, dv=64, dtype=dtype, seed=14), device=gpu)
    g, beta = x["g"].clone(), x["beta"].clone()
    gf, bf = g.view(-1), beta.view(-1)
    # the closed ends of both domains are inside
    gf[0], gf[1], bf[0], bf[1] = -5.0, 0.0, 0.0, 1.0
    for i, val in ((777, 0.25), (5, float("nan")), (30000, -5.5), (gf.numel() - 1, 3.0)):
        gf[i] = val
    for i, val in ((100, 1.5), (3, -0.01), (bf.numel() - 1, float("nan"))):
        bf[i] = val
    torch.cuda.synchronize()
    got = binding.validate_inputs(g, beta)
    assert got == _expected(g, beta)
    assert got["bad_g"] == 4 and got["first_bad_g"] == 5 and got["bad_beta"] == 3 and got["first_bad_beta"] == 3


def test_validate_empty_sequence(gpu):
    x = prefill_inputs(PrefillSpec(B=1, H=2, T=0, dk=64, dv=64, seed=15), device=gpu)
    assert binding.validate_inputs(x["g"], x["beta"]) == dict(bad_g=0, first_bad_g=-1, bad_beta=0,
                                                              first_bad_beta=-1)


def test_validate_k3_full_size(gpu):
    """The benchmark workload's g and beta (B1 H96 T65536 d128 bf16, 805 M g elements) are
    inside the domains; one value planted at the end is found at its index."""
    x = prefill_inputs(WORKLOADS["k3_prefill"], device=gpu)
    assert binding.validate_inputs(x["g"], x["beta"]) == dict(bad_g=0, first_bad_g=-1, bad_beta=0,
                                                              first_bad_beta=-1)
    n = x["g"].numel()
    x["g"].view(-1)[n - 2] = 0.5
    got = binding.validate_inputs(x["g"], x["beta"])
    assert got == dict(bad_g=1, first_bad_g=n - 2, bad_beta=0, first_bad_beta=-1)
