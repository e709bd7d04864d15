"""The workgroup placement the fused launches rely on (kda_chunk_fwd_gated, kda_chunk_fwd_from_proj
and the two-slice backward hand data between workgroups through the L2 of one XCD):
workgroup i of a launch runs on XCD i mod 8, checked through the C ABI's diagnostic
kda_workgroup_xcds at the LDS sizes those kernels request (none, one workgroup per CU,
the whole LDS) and for grids several times the chip."""
import pytest
import torch

from gated_delta_rule_18_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lds", [0, 81 * 1024, 160 * 1024])
@pytest.mark.parametrize("n", [8, 1000, 4096])
def test_workgroup_i_runs_on_xcd_i_mod_8(gpu, n, lds):
    xcd = binding.workgroup_xcds(n, lds, device=gpu)
    torch.cuda.synchronize()
    want = torch.arange(n, dtype=torch.int32, device=gpu) % 8
    bad = (xcd != want).nonzero()
    assert bad.numel() == 0, f"{bad.numel()} workgroups off their XCD, first {bad[0].item()}: {xcd[bad[0]].item()}"
