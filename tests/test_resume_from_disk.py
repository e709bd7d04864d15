"""Resume across processes: one process runs the prefill over the first segment of a
sequence, writes the state it ends with (S_T) to disk and exits; this process reads it
back as S0 for the rest of the sequence.  The chunk interface (page "Kimi K3：架构、训练与
百万 Token Agentic RL 技术解读", section 3.3: the state leaving a segment is the state
entering the next) makes the split run equal the uninterrupted one; with the split on a
16-token boundary the kernel computes the same fp32 state either way, so the outputs
match bit for bit.  The preprocessing's ShortConv history (conv_final -> conv_init)
resumes the same way."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import PrefillSpec, PrepSpec, prefill_inputs, prep_inputs

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SPEC = PrefillSpec(B=2, H=3, T=1000, dk=128, dv=128, seed=901)
SPLIT = 16 * 37
PSPEC = PrepSpec(B=2, T=700, H=3, dk=128, dv=128, seed=911, history=True)
PSPLIT = 333          # any token: the conv history carries the last 3 inputs

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r})
from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import PrefillSpec, PrepSpec, prefill_inputs, prep_inputs
gpu = torch.device("cuda:0")
x = prefill_inputs(PrefillSpec(B=2, H=3, T=1000, dk=128, dv=128, seed=901))
x = {{n: (None if t is None else (t if n == "S0" else t[:, :{split}]).contiguous().to(gpu)) for n, t in x.items()}}
o, S = binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=16)
p = prep_inputs(PrepSpec(B=2, T=700, H=3, dk=128, dv=128, seed=911, history=True))
cut = lambda t: t[:, :{psplit}].contiguous().to(gpu)
outs = binding.prefill_prep(cut(p["q_pre"]), cut(p["k_pre"]), cut(p["v_pre"]), p["conv_w"].to(gpu),
                            p["conv_init"].to(gpu), cut(p["z"]), p["A"].to(gpu), cut(p["beta_logit"]))
torch.cuda.synchronize()
np.save({d!r} + "/state.npy", S.cpu().numpy())
np.save({d!r} + "/o_first.npy", o.float().cpu().numpy())
np.save({d!r} + "/conv_final.npy", outs[5].float().cpu().numpy())
print("child wrote the checkpoint", flush=True)
"""


def test_prefill_and_prep_resume_from_a_checkpoint_written_by_another_process(gpu, tmp_path):
    d = str(tmp_path)
    script = CHILD.format(root=ROOT, split=SPLIT, psplit=PSPLIT, d=d)
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]

    # the uninterrupted runs
    full = {n: None if t is None else t.to(gpu) for n, t in prefill_inputs(SPEC).items()}
    o_ref, S_ref = binding.chunk_fwd(full["q"], full["k"], full["v"], full["g"], full["beta"], full["S0"],
                                     chunk=16)
    p = {n: None if t is None else t.to(gpu) for n, t in prep_inputs(PSPEC).items()}
    ref = binding.prefill_prep(p["q_pre"], p["k_pre"], p["v_pre"], p["conv_w"], p["conv_init"], p["z"], p["A"],
                               p["beta_logit"])

    # the rest, resumed from what the other process left on disk
    S_mid = torch.from_numpy(np.load(os.path.join(d, "state.npy"))).to(gpu)
    rest = lambda t: t[:, SPLIT:].contiguous()
    o2, S2 = binding.chunk_fwd(rest(full["q"]), rest(full["k"]), rest(full["v"]), rest(full["g"]),
                               rest(full["beta"]), S_mid, chunk=16)
    conv_mid = torch.from_numpy(np.load(os.path.join(d, "conv_final.npy"))).to(gpu).to(p["conv_init"].dtype)
    prest = lambda t: t[:, PSPLIT:].contiguous()
    outs2 = binding.prefill_prep(prest(p["q_pre"]), prest(p["k_pre"]), prest(p["v_pre"]), p["conv_w"], conv_mid,
                                 prest(p["z"]), p["A"], prest(p["beta_logit"]))
    torch.cuda.synchronize()

    o_first = torch.from_numpy(np.load(os.path.join(d, "o_first.npy"))).to(gpu)
    assert torch.equal(o_first, o_ref[:, :SPLIT].float()), "first segment differs"
    assert torch.equal(o2, o_ref[:, SPLIT:]), "resumed segment differs"
    assert torch.equal(S2, S_ref), "final state differs"
    for a, b, n in zip(outs2, ref, ("q", "k", "v", "g", "beta", "conv_final")):
        want = b[:, PSPLIT:] if n != "conv_final" else b
        assert torch.equal(a, want), f"resumed preprocessing output {n} differs"
    print(f"resume from disk: prefill split at {SPLIT} of {SPEC.T}, prep split at {PSPLIT} of {PSPEC.T}: "
          "bit-identical", flush=True)
