"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
    python bench.py --sweep-heads 1,32,96,128,144   (prefill time against the head count)

Timed phases, each W untimed steps then K timed steps bracketed by
torch.cuda.synchronize():
  prefill  one kda_chunk_fwd over the K3-shaped layer: B=1, H=96, T=65536,
           dk=dv=128, bf16 inputs, fp32 state, 10 % of tokens at g = -4.99
           (the headline: `value` is its tokens/s);
  configs  the other prefill configurations: B=4, H=32, T=4096 (under
           "configs.prefill_b4h32") and the 1,048,576-token stream of 16 K3-shaped
           segments with the state carried in place ("configs.stream_1m": the
           sum of the 16 launch times, each segment's inputs drawn untimed);
  decode   one kda_decode_step over N=256 sequences x H=96 heads, dk=dv=128,
           bf16, ShortConv width 4 (reported under "decode");
  snapshots  kda_chunk_fwd_snapshots on the prefill workload with a state
           snapshot every 512 tokens (128 snapshots);
  prep     kda_prefill_prep on the same B=1, H=96, T=65536 shape: projected
           pre-activations to q, k, v, g, beta;
  gate     kda_output_gate on the prefill output shape (65536 tokens x 96 heads
           x 128, bf16), and kda_decode_step_gated on the decode batch (under
           "decode.gated");
  from_proj  kda_chunk_fwd_from_proj (preprocessing and prefill in one call) on the
           prep shape and on half of its heads (H48), next to kda_prefill_prep +
           kda_chunk_fwd on the same inputs;
  gated    kda_chunk_fwd_gated, the prefill with the output gate fused, on the
           prefill workload, next to kda_chunk_fwd + kda_output_gate on the same
           inputs (each timed on its own);
  bwd      kda_chunk_bwd, the backward pass, on the B=4, H=32, T=4096,
           dk=dv=128 bf16 prefill shape (gradients fp32).
Inputs are synthetic, seeded, and resident in HBM before the timed region.
Kernel durations come from HIP events recorded on the stream the kernels are
launched on, at the two ends of the K timed steps (their interval divided by K).  The CPU baselines time the fp64 oracle (as it stands) on the host
cores: the whole K3-shaped prefill (cpu_baseline), the whole B4 H32 T4096
prefill, and a sample of the decode batch; each records the host it ran on.

Prints one JSON line.
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 (matrix and vector), TFLOP/s


def prefill_bytes(B, T, H, dk, dv):
    """Algorithmic HBM bytes of one kda_chunk_fwd call (bf16 activations, fp32 state):
    per token-head 2(2dk+dv) [q,k,v] + 2dk [g] + 2 [beta] + 2dv [o]; per head 8 dk dv [S0 in, S_T out]."""
    per_token_head = 2 * (2 * dk + dv) + 2 * dk + 2 + 2 * dv
    return B * T * H * per_token_head + B * H * 8 * dk * dv


def prefill_flops(B, T, H, dk, dv, C):
    """Chunk-form flops at chunk C: per token-head C(6dk + 4dv) + 6 dk dv + C^2/3."""
    return B * T * H * (C * (6 * dk + 4 * dv) + 6 * dk * dv + C * C / 3.0)


def decode_bytes(N, H, dk, dv, W=4):
    """Algorithmic HBM bytes of one kda_decode_step: per (sequence, head) the fp32 state
    read + write 8 dk dv, x_t 2(2dk+dv), cache read 2(W-1)(2dk+dv), cache append 2(2dk+dv),
    g 2dk, beta 2, o 2dv."""
    nch = 2 * dk + dv
    return N * H * (8 * dk * dv + 2 * nch + 2 * (W - 1) * nch + 2 * nch + 2 * dk + 2 + 2 * dv)


def prep_bytes(B, T, H, dk, dv, W=4):
    """Algorithmic HBM bytes of one kda_prefill_prep call (bf16): per token-head the
    pre-activations 2(2dk+dv), z 2dk and the beta logit 2 in, q, k, v, g and beta out
    (the same sizes); per head the fp32 taps 4(2dk+dv)W and the conv history in and out
    2 * 2(W-1)(2dk+dv)."""
    nch = 2 * dk + dv
    per_token_head = 2 * (2 * nch + 2 * dk + 2)
    return B * T * H * per_token_head + H * 4 * nch * W + B * H * 4 * (W - 1) * nch


def bwd_flops(B, T, H, dk, dv, C=16):
    """Arithmetic of one kda_chunk_bwd call: per token-head the chunk reverse mode,
    2(7 dk dv + 2C(dk + 2dv) + 4C dk) + 2 dk dv / C (the products X, Ke D, dO S^T,
    U D^T, dX S^T, the two state-gradient products; B, M, U, dX, dM, dTm; the small
    Kc / Qt / Kt products; rowsum(D S)), plus the forward recompute F(C)."""
    per = 2 * (7 * dk * dv + 2 * C * (dk + 2 * dv) + 4 * C * dk) + 2 * dk * dv / C
    return B * T * H * (per + prefill_flops(1, 1, 1, dk, dv, C))


def bwd_bytes(B, T, H, dk, dv, es=2, C=16):
    """Algorithmic HBM bytes of one kda_chunk_bwd call: inputs q, k, v, g, beta, dO in the
    activation dtype; the incoming state of every chunk, kept in the activation dtype, written
    once by the recompute and read once by the reverse walk (2 es dk dv per chunk-head); fp32
    gradients dq, dk, dg, dv, dbeta out; S0, dS_T in and dS0 out."""
    nch = (T + C - 1) // C
    per_token = es * (3 * dk + 2 * dv + 1) + 4 * (3 * dk + dv + 1)
    return B * T * H * per_token + B * H * (nch * 2 * es * dk * dv + 12 * dk * dv)


def gate_bytes(rows, H, dv):
    """Algorithmic HBM bytes of one kda_output_gate call (bf16): read o and gate, write y,
    2 bytes each per element; the fp32 weight (4 dv bytes) once."""
    return rows * H * dv * 2 * 3 + 4 * dv


def measured_traffic(profile, sources, key="traffic_bytes"):
    """HBM bytes per launch from a committed rocprofv3 counter summary (its `key:` line),
    or None when the kernel sources have changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "gated_delta_rule_18_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    try:
        with open(os.path.join(ROOT, "profiles", profile)) as fh:
            text = fh.read()
    except OSError:
        return None
    if h.hexdigest()[:16] not in text:
        return None
    for line in text.splitlines():
        if line.startswith(key + ":"):
            return int(line.split(":")[1])
    return None


def _timed(fn, steps, warmup, torch):
    """W warmups, then K steps between synchronisations.  Returns (wall ms/step,
    mean kernel ms per step: the interval between two events recorded on the current
    stream at the two ends of the K steps, divided by K -- the launches run back to
    back, so an event between every two launches does not add its own dispatch gap)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kern = start.elapsed_time(end) / steps
    return wall, kern


def host_description():
    """The host the CPU baseline runs on: logical CPU count, the CPUs this process may
    use, and the CPU model."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "affinity": avail, "model": model}


def oracle_threads():
    """Threads for the oracle: every CPU this process may use, at most 16 (the host CPU
    share that goes with one GPU on the benchmark machines)."""
    return max(1, min(16, host_description()["affinity"]))


def cpu_baseline(x, H_total, heads=96, tokens=65536, label="K3-shaped"):
    """Time the fp64 oracle (as it stands) on a bounded sample of a prefill workload:
    the first `heads` heads of the generated inputs over `tokens` tokens."""
    import oracle
    from gated_delta_rule_18_amd.inputs import to_f64
    tokens = min(tokens, x["q"].shape[1])
    heads = min(heads, x["q"].shape[2])
    B = x["q"].shape[0]
    sl = lambda t: to_f64(t[:, :tokens, :heads].contiguous())
    S0 = None if x["S0"] is None else to_f64(x["S0"][:, :heads].contiguous())
    args = [sl(x[n]) for n in ("q", "k", "v", "g", "beta")] + [S0]
    nthreads = oracle_threads()
    dk, dv = x["q"].shape[-1], x["v"].shape[-1]
    t0 = time.perf_counter()
    oracle.prefill(*args, nthreads=nthreads)
    dt = time.perf_counter() - t0
    token_heads = B * heads * tokens
    host = host_description()
    return {
        "value": token_heads / dt / H_total,
        "unit": "tokens/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"fp64 oracle on {nthreads} threads: prefill of B{B} x {heads} of {H_total} heads x "
                   f"{tokens} tokens (dk={dk}, dv={dv}) of the same {label} inputs, {dt:.2f} s; "
                   f"value = token-heads/s / {H_total}, i.e. layer tokens/s"),
        "seconds": dt,
        "gflops_fp64": token_heads * 7 * dk * dv / dt / 1e9,
        "host": host,
    }


def cpu_baseline_decode(ds, st, steps_in, seqs=32):
    """Time the fp64 oracle's decode step on a bounded sample of the decode batch: the
    first `seqs` sequences (all heads) over every prepared step."""
    import numpy as np

    import oracle
    from gated_delta_rule_18_amd.inputs import to_f64
    seqs = min(seqs, ds.N)
    S = np.ascontiguousarray(to_f64(st["S"][:seqs]))
    cache = np.ascontiguousarray(to_f64(st["conv_cache"][:seqs]))
    w = to_f64(st["conv_w"])
    ins = [{n: to_f64(d[n][:seqs]) for n in ("q_pre", "k_pre", "v_pre", "g", "beta")} for d in steps_in]
    nthreads = oracle_threads()
    t0 = time.perf_counter()
    for i, d in enumerate(ins):
        oracle.decode_step(d["q_pre"], d["k_pre"], d["v_pre"], w, cache, i, d["g"], d["beta"], S,
                           nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {
        "value": seqs * len(ins) / dt,
        "unit": "tokens/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"fp64 oracle on {nthreads} threads: {len(ins)} decode steps of {seqs} of {ds.N} sequences "
                   f"x {ds.H} heads, {dt:.2f} s; value = sequence-steps/s (one token per sequence)"),
        "seconds": dt,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-snapshots", action="store_true")
    ap.add_argument("--skip-prep", action="store_true")
    ap.add_argument("--skip-gate", action="store_true")
    ap.add_argument("--skip-bwd", action="store_true")
    ap.add_argument("--skip-configs", action="store_true",
                    help="skip the B4 H32 T4096 prefill and the 1M-token streaming legs")
    ap.add_argument("--sweep-heads", type=str, default="", metavar="H1,H2,...",
                    help="only time the prefill on B1 T65536 d128 bf16 for each head count "
                         "(two workgroups per head: how the time grows as the grid fills the chip); "
                         "one JSON line per head count")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run torch's device-to-device copy of MIB MiB, --steps times "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_18_amd import binding
    from gated_delta_rule_18_amd.inputs import (DECODE, GATE_K3, PREP_K3, STREAM_1M, WORKLOADS, PrepSpec,
                                                backward_inputs,
                                                decode_gate_inputs,
                                                decode_state, decode_step_inputs, gate_inputs,
                                                prefill_inputs, prep_inputs)

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "launches": args.steps}), flush=True)
        return
    binding.lib()

    if args.sweep_heads:
        base = WORKLOADS["k3_prefill"]
        for Hs in [int(h) for h in args.sweep_heads.split(",")]:
            sp = dataclasses.replace(base, H=Hs)
            xs = prefill_inputs(sp, device=dev)
            os_ = torch.empty((sp.B, sp.T, Hs, sp.dv), dtype=torch.bfloat16, device=dev)
            ss = torch.empty((sp.B, Hs, sp.dk, sp.dv), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            _, kern = _timed(lambda i=0: binding.chunk_fwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["S0"],
                                                           chunk=16, o=os_, S_T=ss), args.steps, args.warmup, torch)
            by = prefill_bytes(sp.B, sp.T, Hs, sp.dk, sp.dv)
            print(json.dumps({"sweep_heads": Hs, "workgroups": 2 * sp.B * Hs, "kernel_ms": kern,
                              "gbps": by / (kern * 1e-3) / 1e9, "hbm_frac": by / (kern * 1e-3) / 1e9 / HBM_PEAK_GBPS}),
                  flush=True)
            del xs, os_, ss
            torch.cuda.empty_cache()
        return

    # ---------------- prefill --------------------------------------------------
    spec = WORKLOADS["k3_prefill"]
    B, T, H, dk, dv, C = spec.B, spec.T, spec.H, spec.dk, spec.dv, args.chunk
    x = prefill_inputs(spec, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def prefill_step(i=0):
        binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], chunk=C, o=o, S_T=S_T)

    p_wall, p_kern = _timed(prefill_step, args.steps, args.warmup, torch)
    p_bytes = prefill_bytes(B, T, H, dk, dv)
    p_flops = prefill_flops(B, T, H, dk, dv, C)
    p_gbps = p_bytes / (p_kern * 1e-3) / 1e9
    p_tflops = p_flops / (p_kern * 1e-3) / 1e12
    snapshots = None
    if not args.skip_snapshots:
        every = 512
        n_snaps = T // every
        snaps = torch.empty((n_snaps, B, H, dk, dv), dtype=torch.float32, device=dev)

        def snap_step(i=0):
            binding.chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], every, n_snaps,
                                        chunk=C, o=o, S_T=S_T, snaps=snaps)

        s_wall, s_kern = _timed(snap_step, args.steps, args.warmup, torch)
        s_bytes = p_bytes + n_snaps * B * H * dk * dv * 4
        s_gbps = s_bytes / (s_kern * 1e-3) / 1e9
        snapshots = {
            "workload": f"k3_prefill with a state snapshot every {every} tokens ({n_snaps} snapshots, "
                        f"{n_snaps * B * H * dk * dv * 4 / 1e9:.3f} GB written)",
            "ms_per_step": s_wall,
            "kernel_ms": s_kern,
            "tokens_per_s": B * T / (s_wall * 1e-3),
            "extra_ms_vs_prefill": s_kern - p_kern,
            "roofline": {"bound": "hbm", "achieved": s_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": s_gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("prefill_k3_hbm_counters.txt",
                                                     ["kda_prefill_ws.hip", "kda_device.h"],
                                                     key="snapshots_traffic_bytes"),
                         "bytes_per_launch": s_bytes},
        }
        del snaps
    gated = None
    if not args.skip_gate:
        gk = GATE_K3
        gi = gate_inputs(gk["rows"], gk["H"], gk["dv"], dtype=gk["dtype"], seed=gk["seed"], device=dev)
        gate_t = gi["gate"].view(B, T, H, dv)
        y = torch.empty_like(o)
        gws = torch.empty(max(binding.gated_workspace_size(B, H, dv), 16), dtype=torch.uint8, device=dev)
        del gi["o"]
        torch.cuda.synchronize()

        def gated_step(i=0):
            binding.chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate_t, gi["norm_w"],
                                    y=y, S_T=S_T, workspace=gws)

        def gate_only(i=0):
            binding.output_gate(o, gate_t, gi["norm_w"], y=y)

        f_wall, f_kern = _timed(gated_step, args.steps, args.warmup, torch)
        _, g_only = _timed(gate_only, args.steps, args.warmup, torch)
        _, p_again = _timed(prefill_step, args.steps, args.warmup, torch)
        f_bytes = p_bytes + gate_bytes(B * T, H, dv) - 2 * (B * T * H * dv * 2)   # o stays on chip
        f_gbps = f_bytes / (f_kern * 1e-3) / 1e9
        gated = {
            "workload": f"k3_prefill with the output gate fused (kda_chunk_fwd_gated), gate ~ 2 N(0,1), "
                        f"RMSNorm weight ~ 1 + 0.1 N(0,1), eps 1e-6",
            "ms_per_step": f_wall,
            "kernel_ms": f_kern,
            "tokens_per_s": B * T / (f_wall * 1e-3),
            "two_pass_kernel_ms": p_again + g_only,
            "two_pass_parts_ms": {"prefill": p_again, "gate": g_only},
            "speedup_vs_two_pass": (p_again + g_only) / f_kern,
            "roofline": {"bound": "hbm", "achieved": f_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": f_gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("prefill_gated_k3_hbm_counters.txt",
                                                     ["kda_prefill_ws.hip", "kda_device.h"]),
                         "bytes_per_launch": f_bytes},
        }
        del gi, gate_t, y, gws
    cpu = None if args.no_cpu else cpu_baseline(x, H)
    del x, o

    # ---------------- the other prefill configurations ------------------------------
    configs = None
    if not args.skip_configs:
        configs = {}
        # B4 H32 T4096: 256 workgroups, every CU busy
        c2 = WORKLOADS["prefill_b4h32"]
        x2 = prefill_inputs(c2, device=dev)
        o2 = torch.empty((c2.B, c2.T, c2.H, c2.dv), dtype=torch.bfloat16, device=dev)
        s2 = torch.empty((c2.B, c2.H, c2.dk, c2.dv), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        # a 0.2 ms launch: the C entry point is called directly with its arguments
        # marshalled once, so the host keeps ahead of the device and the launches run
        # back to back (through the checking Python wrapper the host needs ~0.27 ms per
        # call and the device would idle between launches)
        import ctypes
        lib = binding.lib()
        c2_args = [ctypes.c_void_p(t.data_ptr()) for t in (x2["q"], x2["k"], x2["v"], x2["g"], x2["beta"],
                                                          x2["S0"], o2, s2)]
        c2_args += [c2.B, c2.T, c2.H, c2.dk, c2.dv, binding.KDA_BF16, C,
                    ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]

        def c2_step(i=0):
            rc = lib.kda_chunk_fwd(*c2_args)
            if rc != binding.KDA_OK:
                raise binding.KdaError(rc, lib.kda_strerror(rc).decode())

        w2, k2 = _timed(c2_step, args.steps, args.warmup, torch)
        b2 = prefill_bytes(c2.B, c2.T, c2.H, c2.dk, c2.dv)
        configs["prefill_b4h32"] = {
            "workload": f"prefill B{c2.B} H{c2.H} T{c2.T} dk=dv={c2.dk} bf16 chunk{C}",
            "ms_per_step": w2, "kernel_ms": k2, "tokens_per_s": c2.B * c2.T / (w2 * 1e-3),
            "tflops": prefill_flops(c2.B, c2.T, c2.H, c2.dk, c2.dv, C) / (k2 * 1e-3) / 1e12,
            "roofline": {"bound": "hbm", "achieved": b2 / (k2 * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": b2 / (k2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                         "bytes_per_launch": b2},
        }
        if not args.no_cpu:
            configs["prefill_b4h32"]["cpu_baseline"] = cpu_baseline(x2, c2.H, heads=c2.H, tokens=c2.T,
                                                                    label="B4 H32 T4096")
        del x2, o2, s2
        # 1,048,576 tokens as 16 segments of the K3 shape, the state carried in place;
        # each segment's inputs are drawn (untimed) before its launch, the kernel time
        # is the sum of the 16 launches
        base, nseg = STREAM_1M["base"], STREAM_1M["segments"]
        S = None
        o4 = torch.empty((base.B, base.T, base.H, base.dv), dtype=torch.bfloat16, device=dev)
        seg_ms = []
        for seg in range(-1, nseg):          # segment -1: an untimed warm-up
            xs = prefill_inputs(base, device=dev, seed=STREAM_1M["seed_base"] + max(seg, 0))
            if S is None or seg == 0:
                S = xs["S0"].clone()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            binding.chunk_fwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], S, chunk=C, o=o4, S_T=S)
            e1.record()
            torch.cuda.synchronize()
            if seg >= 0:
                seg_ms.append(e0.elapsed_time(e1))
            del xs
        tot = sum(seg_ms)
        b4 = nseg * prefill_bytes(base.B, base.T, base.H, base.dk, base.dv)
        configs["stream_1m"] = {
            "workload": f"1M-token streaming prefill: {nseg} x (B{base.B} H{base.H} T{base.T}) segments, "
                        f"state carried in place, bf16 chunk{C}",
            "kernel_ms": tot, "segment_ms": [round(t, 4) for t in seg_ms],
            "tokens_per_s": nseg * base.B * base.T / (tot * 1e-3),
            "roofline": {"bound": "hbm", "achieved": b4 / (tot * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": b4 / (tot * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                         "bytes_per_launch": b4 // nseg},
        }
        if cpu is not None:
            configs["stream_1m"]["cpu_baseline"] = {
                "value": cpu["value"], "unit": "tokens/s", "cores": cpu["cores"], "kind": "oracle",
                "sample": "one K3-shaped segment (the headline cpu_baseline); the 16 segments of the "
                          "stream are the same work 16 times, so the rate is the same",
                "extrapolated_seconds": nseg * cpu["seconds"]}
        del o4, S

    # ---------------- decode ---------------------------------------------------
    decode = None
    if not args.skip_decode:
        ds = DECODE
        st = decode_state(ds, device=dev)
        nin = args.steps + args.warmup
        steps_in = [decode_step_inputs(ds, s % ds.steps, device=dev) for s in range(min(nin, ds.steps))]
        od = torch.empty((ds.N, ds.H, ds.dv), dtype=torch.bfloat16, device=dev)
        pos = [0]
        torch.cuda.synchronize()

        def decode_step(i=0):
            d = steps_in[pos[0] % len(steps_in)]
            binding.decode_step(d["q_pre"], d["k_pre"], d["v_pre"], st["conv_w"], st["conv_cache"], pos[0],
                                d["g"], d["beta"], st["S"], o=od)
            pos[0] += 1

        d_wall, d_kern = _timed(decode_step, args.steps, args.warmup, torch)
        d_cpu = None if args.no_cpu else cpu_baseline_decode(ds, st, steps_in[:8])
        d_bytes = decode_bytes(ds.N, ds.H, ds.dk, ds.dv, ds.width)
        d_gbps = d_bytes / (d_kern * 1e-3) / 1e9
        decode = {
            "workload": f"decode N{ds.N} H{ds.H} dk=dv={ds.dk} bf16 ShortConv{ds.width}",
            "ms_per_step": d_wall,
            "kernel_ms": d_kern,
            "tokens_per_s": ds.N / (d_wall * 1e-3),
            "gbps": d_gbps,
            "roofline": {"bound": "hbm", "achieved": d_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": d_gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("decode_n256_hbm_counters.txt",
                                                     ["kda_decode.hip", "kda_device.h"]),
                         "bytes_per_launch": d_bytes},
        }
        if d_cpu is not None:
            decode["cpu_baseline"] = d_cpu
        # the same step with the output exposure gate fused (y written in place of o)
        if not args.skip_gate:
            gates = [decode_gate_inputs(ds, s % ds.steps, device=dev) for s in range(len(steps_in))]
            nw = torch.ones(ds.dv, dtype=torch.float32, device=dev)
            torch.cuda.synchronize()

            def decode_gated_step(i=0):
                d = steps_in[pos[0] % len(steps_in)]
                binding.decode_step_gated(d["q_pre"], d["k_pre"], d["v_pre"], st["conv_w"], st["conv_cache"],
                                          pos[0], d["g"], d["beta"], st["S"], gates[pos[0] % len(gates)], nw,
                                          y=od)
                pos[0] += 1

            g_wall, g_kern = _timed(decode_gated_step, args.steps, args.warmup, torch)
            g_bytes = d_bytes + ds.N * ds.H * ds.dv * 2 + ds.dv * 4
            decode["gated"] = {
                "ms_per_step": g_wall, "kernel_ms": g_kern, "extra_ms_vs_decode": g_kern - d_kern,
                "roofline": {"bound": "hbm", "achieved": g_bytes / (g_kern * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": g_bytes / (g_kern * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                             "traffic": measured_traffic("decode_n256_hbm_counters.txt",
                                                         ["kda_decode.hip", "kda_device.h"],
                                                         key="gated_traffic_bytes"),
                             "bytes_per_launch": g_bytes},
            }
            del gates
        del st, steps_in

    # ---------------- prefill preprocessing --------------------------------------
    prep = None
    if not args.skip_prep:
        ps = PREP_K3
        xp = prep_inputs(ps, device=dev)
        outs = tuple(torch.empty(sh, dtype=torch.bfloat16, device=dev)
                     for sh in ((ps.B, ps.T, ps.H, ps.dk), (ps.B, ps.T, ps.H, ps.dk), (ps.B, ps.T, ps.H, ps.dv),
                                (ps.B, ps.T, ps.H, ps.dk), (ps.B, ps.T, ps.H)))
        fin = torch.empty_like(xp["conv_init"])
        torch.cuda.synchronize()

        def prep_step(i=0):
            binding.prefill_prep(xp["q_pre"], xp["k_pre"], xp["v_pre"], xp["conv_w"], xp["conv_init"], xp["z"],
                                 xp["A"], xp["beta_logit"], out=outs, conv_final=fin)

        r_wall, r_kern = _timed(prep_step, args.steps, args.warmup, torch)
        r_bytes = prep_bytes(ps.B, ps.T, ps.H, ps.dk, ps.dv, ps.width)
        r_gbps = r_bytes / (r_kern * 1e-3) / 1e9
        prep = {
            "workload": f"prefill preprocessing B{ps.B} H{ps.H} T{ps.T} dk=dv={ps.dk} bf16 ShortConv{ps.width}",
            "ms_per_step": r_wall,
            "kernel_ms": r_kern,
            "tokens_per_s": ps.B * ps.T / (r_wall * 1e-3),
            "roofline": {"bound": "hbm", "achieved": r_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": r_gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("prep_k3_hbm_counters.txt",
                                                     ["kda_prep.hip", "kda_prep_unit.h", "kda_device.h"]),
                         "bytes_per_launch": r_bytes},
        }
        del xp, outs, fin

    # ---------------- preprocessing and prefill in one call ------------------------
    from_proj = None
    if not args.skip_prep:
        from_proj = {}
        for hh in (PREP_K3.H, PREP_K3.H // 2):
            sp = PrepSpec(B=PREP_K3.B, T=PREP_K3.T, H=hh, dk=PREP_K3.dk, dv=PREP_K3.dv, seed=PREP_K3.seed)
            xp = prep_inputs(sp, device=dev)
            bf = dict(dtype=torch.bfloat16, device=dev)
            outs = dict(q=torch.empty((sp.B, sp.T, hh, sp.dk), **bf), k=torch.empty((sp.B, sp.T, hh, sp.dk), **bf),
                        v=torch.empty((sp.B, sp.T, hh, sp.dv), **bf), g=torch.empty((sp.B, sp.T, hh, sp.dk), **bf),
                        beta=torch.empty((sp.B, sp.T, hh), **bf), conv_final=torch.empty_like(xp["conv_init"]))
            of = torch.empty((sp.B, sp.T, hh, sp.dv), **bf)
            sf = torch.empty((sp.B, hh, sp.dk, sp.dv), dtype=torch.float32, device=dev)
            pws = torch.empty(max(binding.from_proj_workspace_size(sp.B, sp.T, hh), 16), dtype=torch.uint8,
                              device=dev)
            torch.cuda.synchronize()

            def fused_step(i=0):
                binding.chunk_fwd_from_proj(xp["q_pre"], xp["k_pre"], xp["v_pre"], xp["conv_w"], xp["conv_init"],
                                            xp["z"], xp["A"], xp["beta_logit"], None, out=outs, o=of, S_T=sf,
                                            workspace=pws)

            def prep_only(i=0):
                binding.prefill_prep(xp["q_pre"], xp["k_pre"], xp["v_pre"], xp["conv_w"], xp["conv_init"], xp["z"],
                                     xp["A"], xp["beta_logit"],
                                     out=(outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"]),
                                     conv_final=outs["conv_final"])

            def prefill_only(i=0):
                binding.chunk_fwd(outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"], None, chunk=16, o=of,
                                  S_T=sf)

            u_wall, u_kern = _timed(fused_step, args.steps, args.warmup, torch)
            _, u_prep = _timed(prep_only, args.steps, args.warmup, torch)
            _, u_pre = _timed(prefill_only, args.steps, args.warmup, torch)
            grid = -(-sp.B * hh // 8) * 8 * (sp.dv // 64)
            from_proj[f"H{hh}"] = {
                "workload": f"kda_chunk_fwd_from_proj B{sp.B} H{hh} T{sp.T} dk=dv={sp.dk} bf16 "
                            f"(pre-activations as prep, S0 = 0)",
                "launch": "fused" if grid <= 160 else "prep pass, then prefill",
                "ms_per_step": u_wall,
                "kernel_ms": u_kern,
                "tokens_per_s": sp.B * sp.T / (u_wall * 1e-3),
                "two_pass_kernel_ms": u_prep + u_pre,
                "two_pass_parts_ms": {"prep": u_prep, "prefill": u_pre},
                "speedup_vs_two_pass": (u_prep + u_pre) / u_kern,
            }
            del xp, outs, of, sf, pws

    # ---------------- output exposure gate --------------------------------------
    gate = None
    if not args.skip_gate:
        gk = GATE_K3
        xg = gate_inputs(gk["rows"], gk["H"], gk["dv"], dtype=gk["dtype"], seed=gk["seed"], device=dev)
        yg = torch.empty_like(xg["o"])
        torch.cuda.synchronize()

        def gate_step(i=0):
            binding.output_gate(xg["o"], xg["gate"], xg["norm_w"], y=yg)

        q_wall, q_kern = _timed(gate_step, args.steps, args.warmup, torch)
        q_bytes = gate_bytes(gk["rows"], gk["H"], gk["dv"])
        q_gbps = q_bytes / (q_kern * 1e-3) / 1e9
        gate = {
            "workload": f"output exposure gate rows={gk['rows']} H{gk['H']} dv={gk['dv']} {gk['dtype']}",
            "ms_per_step": q_wall,
            "kernel_ms": q_kern,
            "tokens_per_s": gk["rows"] / (q_wall * 1e-3),
            "roofline": {"bound": "hbm", "achieved": q_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": q_gbps / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("gate_k3_hbm_counters.txt", ["kda_gate.hip", "kda_device.h"]),
                         "bytes_per_launch": q_bytes},
        }
        del xg, yg

    # ---------------- backward (training) -----------------------------------------
    bwd = None
    if not args.skip_bwd:
        bs = WORKLOADS["prefill_b4h32"]
        xb = prefill_inputs(bs, device=dev)
        gb = backward_inputs(bs, device=dev)
        ws = torch.empty(max(binding.workspace_size(bs.B, bs.T, bs.H, bs.dk, bs.dv), 1), dtype=torch.uint8,
                         device=dev)
        torch.cuda.synchronize()

        def bwd_step(i=0):
            binding.chunk_bwd(xb["q"], xb["k"], xb["v"], xb["g"], xb["beta"], xb["S0"], gb["dO"], gb["dS_T"],
                              workspace=ws)

        b_wall, b_kern = _timed(bwd_step, args.steps, args.warmup, torch)
        b_fl = bwd_flops(bs.B, bs.T, bs.H, bs.dk, bs.dv)
        b_by = bwd_bytes(bs.B, bs.T, bs.H, bs.dk, bs.dv)
        b_tf = b_fl / (b_kern * 1e-3) / 1e12
        bwd = {
            "workload": f"backward B{bs.B} H{bs.H} T{bs.T} dk=dv={bs.dk} bf16 inputs, fp32 gradients",
            "ms_per_step": b_wall,
            "kernel_ms": b_kern,
            "tokens_per_s": bs.B * bs.T / (b_wall * 1e-3),
            "gbps": b_by / (b_kern * 1e-3) / 1e9,
            "hbm_frac": b_by / (b_kern * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "roofline": {"bound": "mfma", "achieved": b_tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": b_tf / FP32_PEAK_TFLOPS,
                         "traffic": measured_traffic("bwd_b4h32_hbm_counters.txt",
                                                     ["kda_bwd.hip", "kda_prefill_ws.hip", "kda_device.h"])
                         if (bs.B, bs.H, bs.T) == (4, 32, 4096) else None,
                         "flops_per_launch": b_fl,
                         "bytes_per_launch": b_by},
        }
        del xb, gb, ws

    line = {
        "metric": "KDA prefill tokens/s & TFLOP/s (% MFMA peak); decode-step HBM GB/s (% peak)",
        "value": B * T / (p_wall * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p_wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"k3_prefill B{B} H{H} T{T} dk=dv={dk} bf16 chunk{C} "
                               "(10% tokens g=-4.99)", "global_batch": B, "seq_len": T, "heads": H,
                   "chunk": C},
        "kernel_ms": p_kern,
        "tflops": p_tflops,
        "mfma_frac": p_tflops / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "hbm", "achieved": p_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": p_gbps / HBM_PEAK_GBPS,
                     "traffic": (measured_traffic("prefill_k3_hbm_counters.txt",
                                                  ["kda_prefill_ws.hip", "kda_device.h"])
                                 if C == 16 else None),
                     "bytes_per_launch": p_bytes},
        "decode": decode,
        "snapshots": snapshots,
        "prep": prep,
        "gate": gate,
        "gated": gated,
        "from_proj": from_proj,
        "bwd": bwd,
        "configs": configs,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
