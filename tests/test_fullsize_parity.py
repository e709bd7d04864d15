"""Full-size prefill parity at the K3 shape, in the launch configuration the benchmark
times (chunk 16, bf16, B1 H96 T65536 d128), on sampled heads and value columns the
oracle can afford.  Value columns of the state never interact (Diag(alpha) scales
rows), so the oracle may run on a subset of them exactly."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_18_amd import binding
from gated_delta_rule_18_amd.inputs import STREAM_1M, WORKLOADS, prefill_inputs, to_f64
from tests.util import TOL, assert_parity

pytestmark = pytest.mark.gpu

HEADS = (0, 47, 95)
# 16 of the 128 value columns: column 16 w + j sits at lane position j of consumer
# wavefront w % 4 of value slice w // 4; one column per lane position j, spread over
# all eight (slice, wavefront) pairs
COLS = np.array([16 * (j % 8) + j for j in range(16)])


def _oracle_segment(inp, S0_cols, heads=HEADS, cols=COLS, snap_every=0, n_snaps=0):
    """Oracle on (head, column-subset) for one segment, the sampled heads run as a batch
    (one thread each); S0_cols [n, dk, len(cols)] or None.  Returns o [n, T, c], S [n, dk, c]
    (and snapshots [n_snaps, n, dk, c] when asked)."""
    hs = list(heads)
    sl = lambda t: np.ascontiguousarray(np.transpose(to_f64(t[0, :, hs]), (1, 0, 2))[:, :, None, :])
    q, k, g = sl(inp["q"]), sl(inp["k"]), sl(inp["g"])
    v = np.ascontiguousarray(sl(inp["v"])[..., cols])
    beta = np.ascontiguousarray(to_f64(inp["beta"][0, :, hs]).T[:, :, None])
    s0 = None if S0_cols is None else np.ascontiguousarray(S0_cols[:, None])
    if n_snaps:
        o, S, sn = oracle.prefill_snapshots(q, k, v, g, beta, s0, snap_every, n_snaps)
        return o[:, :, 0], S[:, 0], sn[:, :, 0]
    o, S = oracle.prefill(q, k, v, g, beta, s0)
    return o[:, :, 0], S[:, 0]


def test_k3_prefill_full_size_sampled():
    """B1 H96 T65536 bf16 with 10% of tokens at g = -4.99: full GPU run, oracle on 3 heads."""
    dev = torch.device("cuda:0")
    spec = WORKLOADS["k3_prefill"]
    inp = prefill_inputs(spec, device=dev)
    o, S_T = binding.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], chunk=16)
    torch.cuda.synchronize()
    S0c = np.stack([to_f64(inp["S0"][0, h])[:, COLS] for h in HEADS])
    oo, so = _oracle_segment(inp, S0c)
    og = np.stack([to_f64(o[0, :, h])[:, COLS] for h in HEADS])
    sg = np.stack([to_f64(S_T[0, h])[:, COLS] for h in HEADS])
    to, ts = TOL["bf16"]
    eo = assert_parity(og, oo, to, "k3 o")
    es = assert_parity(sg, so, ts, "k3 S_T")
    # every head, every column: finite
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    print(f"k3_prefill: err_o {eo:.2e} err_S {es:.2e}", flush=True)


def test_k3_prefill_snapshots_sampled():
    """The K3 shape with a state snapshot every 4096 tokens (16 snapshots): sampled heads
    and columns of every snapshot against the oracle's states at those token counts."""
    dev = torch.device("cuda:0")
    spec = WORKLOADS["k3_prefill"]
    inp = prefill_inputs(spec, device=dev)
    every, n = 4096, spec.T // 4096
    o, S_T, snaps = binding.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                inp["S0"], every, n, chunk=16)
    torch.cuda.synchronize()
    S0c = np.stack([to_f64(inp["S0"][0, h])[:, COLS] for h in HEADS])
    oo, so, sn = _oracle_segment(inp, S0c, snap_every=every, n_snaps=n)
    ts = TOL["bf16"][1]
    worst = 0.0
    for s in range(n):
        got = np.stack([to_f64(snaps[s, 0, h])[:, COLS] for h in HEADS])
        worst = max(worst, assert_parity(got, sn[s], ts, f"k3 snapshot {s}"))
    assert torch.isfinite(snaps).all()
    print(f"k3 snapshots: {n} x every {every}, worst err_S {worst:.2e}", flush=True)


@pytest.mark.slow
def test_stream_1m_sampled():
    """1,048,576 tokens as 16 sequential 65536-token segments, the state carried in place
    (S_T is S0); heads {0, 47, 95} and 16 value columns checked after every segment."""
    dev = torch.device("cuda:0")
    base = STREAM_1M["base"]
    S = None
    S_or = None
    worst = [0.0, 0.0]
    to, ts = TOL["bf16"]
    for seg in range(STREAM_1M["segments"]):
        inp = prefill_inputs(base, device=dev, seed=STREAM_1M["seed_base"] + seg)
        if S is None:
            S = inp["S0"].clone()
            S_or = np.stack([to_f64(S[0, h])[:, COLS] for h in HEADS])
        o, st = binding.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S, chunk=16, S_T=S)
        torch.cuda.synchronize()
        assert st is S
        oo, S_or = _oracle_segment(inp, S_or)
        og = np.stack([to_f64(o[0, :, h])[:, COLS] for h in HEADS])
        sg = np.stack([to_f64(S[0, h])[:, COLS] for h in HEADS])
        worst[0] = max(worst[0], assert_parity(og, oo, to, f"segment {seg} o"))
        worst[1] = max(worst[1], assert_parity(sg, S_or, ts, f"segment {seg} S"))
        print(f"segment {seg}: err_o {worst[0]:.2e} err_S {worst[1]:.2e}", flush=True)
        del inp, o
