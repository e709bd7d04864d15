"""The workgroup placement the fused launches rely on (kda_chunk_fwd_gated, kda_chunk_fwd_from_proj
and the two-slice backward hand data between workgroups through the L2 of one XCD): a launch's
workgroups go round-robin over the 8 XCDs, so workgroups i and i + 8 share one; which XCD takes
workgroup 0 varies between launches (it was seen to change after work on other streams).
Checked through the C ABI's diagnostic kda_workgroup_xcds at the LDS sizes those kernels
request (none, one workgroup per CU, the whole LDS) and for grids several times the chip."""
import pytest
import torch

from gated_delta_rule_18_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lds", [0, 81 * 1024, 160 * 1024])
@pytest.mark.parametrize("n", [8, 1000, 4096])
def test_workgroups_eight_apart_share_an_xcd(gpu, n, lds):
    xcd = binding.workgroup_xcds(n, lds, device=gpu)
    torch.cuda.synchronize()
    first = xcd[:8]
    assert sorted(first.tolist()) == list(range(8)), f"workgroups 0..7 ran on XCDs {first.tolist()}"
    want = first[torch.arange(n, device=gpu) % 8]
    bad = (xcd != want).nonzero()
    assert bad.numel() == 0, (f"{bad.numel()} workgroups off the XCD of workgroup i mod 8, first {bad[0].item()}: "
                              f"{xcd[bad[0]].item()} (workgroups 0..7: {first.tolist()})")
    print(f"n={n} lds={lds}: workgroups 0..7 on XCDs {first.tolist()}", flush=True)
