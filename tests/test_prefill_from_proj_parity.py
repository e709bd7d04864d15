"""GPU prefill with the preprocessing fused (kda_chunk_fwd_from_proj through the C ABI):
every output -- o, S_T, and the preprocessing's q, k, v, g, beta and conv_final -- is bit
for bit what kda_prefill_prep followed by kda_chunk_fwd writes (each of which is checked
against the oracle in test_prep_parity.py and test_prefill_parity.py).  The cases span
grids that leave CUs to the prep workers (the fused launch) and grids that fill the chip
(the call then runs the two passes)."""
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import PREP_K3, PrepSpec, prep_inputs

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "beta", "conv_final")


def _s0(spec, gpu, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return (0.02 * torch.randn((spec.B, spec.H, spec.dk, spec.dv), generator=gen)).to(gpu)


def _two_pass(x, S0):
    q, k, v, g, beta, cf = binding.prefill_prep(x["q_pre"], x["k_pre"], x["v_pre"], x["conv_w"], x["conv_init"],
                                                x["z"], x["A"], x["beta_logit"])
    o, S = binding.chunk_fwd(q, k, v, g, beta, S0, chunk=16)
    return o, S, dict(q=q, k=k, v=v, g=g, beta=beta, conv_final=cf)


def _fused(x, S0, **kw):
    return binding.chunk_fwd_from_proj(x["q_pre"], x["k_pre"], x["v_pre"], x["conv_w"], x["conv_init"], x["z"],
                                       x["A"], x["beta_logit"], S0, **kw)


def _assert_same(a, b, what):
    same = torch.eq(a, b)
    if not bool(same.all()):
        bad = (~same).nonzero()
        raise AssertionError(f"{what}: {bad.shape[0]} elements differ, first at {bad[0].tolist()}")


def _check(x, S0):
    o2, S2, p2 = _two_pass(x, S0)
    o, S, p = _fused(x, S0)
    torch.cuda.synchronize()
    _assert_same(o, o2, "o")
    _assert_same(S, S2, "S_T")
    for n in NAMES:
        _assert_same(p[n], p2[n], n)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("B,H,T,history", [(1, 1, 1, True), (2, 3, 77, False), (1, 5, 300, True),
                                           (3, 2, 1000, True)])
def test_from_proj_equals_prep_then_prefill(gpu, dtype, dk, dv, B, H, T, history):
    spec = PrepSpec(B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, seed=300 + T + H, history=history)
    x = prep_inputs(spec, device=gpu)
    _check(x, _s0(spec, gpu, 301) if T % 2 == 0 else None)


@pytest.mark.parametrize("B,H,T", [(1, 16, 2048), (1, 80, 300), (1, 96, 200), (4, 32, 1024)])
def test_from_proj_wide_grids(gpu, B, H, T):
    """32 prefill workgroups (224 CUs of prep workers), 160 (96, the fewest the fused
    launch runs with), 192 and 256 (too few idle CUs: the call runs the preprocessing
    pass and then the prefill)."""
    spec = PrepSpec(B=B, T=T, H=H, dk=128, dv=128, seed=311)
    x = prep_inputs(spec, device=gpu)
    _check(x, _s0(spec, gpu, 312))


def test_from_proj_empty_sequence(gpu):
    spec = PrepSpec(B=2, T=0, H=3, dk=128, dv=128, seed=321)
    x = prep_inputs(spec, device=gpu)
    S0 = _s0(spec, gpu, 322)
    o, S, p = _fused(x, S0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, S0)
    assert torch.equal(p["conv_final"], x["conv_init"])


def test_from_proj_workspace_reuse_and_in_place_state(gpu):
    """Two calls through one workspace (its stale flags are cleared by the call), the
    second streaming the state in place (S_T = S0) and the conv history (conv_init =
    the first call's conv_final)."""
    spec = PrepSpec(B=2, T=500, H=4, dk=128, dv=128, seed=331)
    x = prep_inputs(spec, device=gpu)
    ws = torch.empty(binding.from_proj_workspace_size(2, 500, 4), dtype=torch.uint8, device=gpu)
    S0 = _s0(spec, gpu, 332)
    o1, S1, p1 = _fused(x, S0, workspace=ws)
    S_run = S1.clone()
    x2 = dict(x, conv_init=p1["conv_final"].clone())
    o2, _, p2 = _fused(x2, S_run, S_T=S_run, workspace=ws)
    torch.cuda.synchronize()
    r1o, r1S, r1p = _two_pass(x, S0)
    r2o, r2S, r2p = _two_pass(x2, r1S)
    torch.cuda.synchronize()
    _assert_same(o1, r1o, "o, first call")
    _assert_same(o2, r2o, "o, second call")
    _assert_same(S_run, r2S, "S_T, second call")
    for n in NAMES:
        _assert_same(p2[n], r2p[n], n)


def test_from_proj_marks_nan_when_waits_give_up(gpu):
    """spin_limit 0 (forced from the host): the prefill's waits give up at their first
    unsatisfied poll; the kernel still finishes, o and S_T are NaN (the mark), and the
    preprocessing's outputs, which wait for nothing, are exact."""
    spec = PrepSpec(B=1, T=400, H=4, dk=128, dv=128, seed=341)
    x = prep_inputs(spec, device=gpu)
    S0 = _s0(spec, gpu, 342)
    o, S, p = _fused(x, S0, spin_limit=0)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all(), "o not marked"
    assert torch.isnan(S).all(), "S_T not marked"
    _, _, r = _two_pass(x, S0)
    torch.cuda.synchronize()
    for n in NAMES:
        _assert_same(p[n], r[n], n)


@pytest.mark.parametrize("H", [96, 48])
def test_from_proj_full_length_equals_prep_then_prefill(gpu, H):
    """The K3 layer shape (B1 H96 T65536 d128 bf16; the call runs the two passes) and
    half of its heads (H48, what one GPU holds at two-way head parallelism; the fused
    launch), in the calls the benchmark times."""
    spec = PrepSpec(B=1, T=65536, H=H, dk=128, dv=128, seed=PREP_K3.seed)
    x = prep_inputs(spec, device=gpu)
    S0 = _s0(spec, gpu, 351)
    _check(x, S0)
    print(f"from_proj H{H} T65536: o, S_T and the preprocessing outputs equal the two passes", flush=True)
