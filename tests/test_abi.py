"""The C-ABI library loads, exports every symbol include/kda.h declares, and rejects
bad arguments before touching the GPU (no compute calls here: runs on the CPU)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_18_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "kda.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(kda_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exports():
    assert _declared() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_version_and_strerror():
    assert binding.version() == 150
    L = binding.lib()
    for code in (0, -1, -2, -3, -4, 17):
        assert isinstance(L.kda_strerror(code), bytes) and L.kda_strerror(code)


# fake, 16-byte aligned device addresses: validation rejects before any use
A = 0x10000
MIS = 0x10002


def _prefill(**kw):
    args = dict(q=A, k=A, v=A, g=A, beta=A, S0=A, o=A, S_T=A, B=1, T=8, H=2, dk=64, dv=64,
                dtype=0, chunk=32, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_chunk_fwd(vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]),
                                       vp(args["beta"]), vp(args["S0"]), vp(args["o"]), vp(args["S_T"]),
                                       args["B"], args["T"], args["H"], args["dk"], args["dv"],
                                       args["dtype"], args["chunk"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(chunk=48), -1), (dict(chunk=128), -1), (dict(chunk=7), -1), (dict(dtype=2), -1), (dict(B=-1), -1),
    (dict(T=-3), -1), (dict(dk=0), -1), (dict(dk=96), -2), (dict(dv=256), -2),
    (dict(q=None), -1), (dict(o=None), -1), (dict(k=MIS), -1), (dict(S_T=A + 64), -1),
    # index ranges: B and H at most 65535 each, B*H at most 2^24
    (dict(B=65536, T=1), -1), (dict(H=65536, T=1), -1), (dict(B=4096, H=4097, T=1), -1),
])
def test_prefill_rejects(kw, code):
    assert _prefill(**kw) == code


def test_prefill_index_range_limits_are_inclusive():
    # the largest accepted sizes pass validation (B*H = 2^24 exactly); nothing is
    # launched because T = 0 and S_T is S0
    assert _prefill(B=4096, H=4096, T=0, S_T=A, S0=A) == 0
    assert _prefill(B=65535, H=1, T=0, S_T=A, S0=A) == 0


def _prefill_ex(spin_limit=-1, **kw):
    args = dict(q=A, k=A, v=A, g=A, beta=A, S0=A, o=A, S_T=A, snaps=None, every=0, n=0,
                B=1, T=8, H=2, dk=64, dv=64, dtype=0, chunk=16, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    opts = binding.FwdOptions(spin_limit=spin_limit)
    return binding.lib().kda_chunk_fwd_ex(
        vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]), vp(args["beta"]), vp(args["S0"]),
        vp(args["o"]), vp(args["S_T"]), vp(args["snaps"]), args["every"], args["n"], args["B"], args["T"],
        args["H"], args["dk"], args["dv"], args["dtype"], args["chunk"], ctypes.byref(opts), args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(spin_limit=-2), -1), (dict(chunk=48), -1), (dict(dk=96), -2), (dict(B=65536), -1),
    (dict(n=1, every=16, snaps=None), -1),
])
def test_prefill_ex_rejects(kw, code):
    assert _prefill_ex(**kw) == code


def test_prefill_ex_empty_is_a_no_op():
    assert _prefill_ex(B=0, q=None, k=None, v=None, g=None, beta=None, o=None, spin_limit=0) == 0


def test_prefill_empty_batch_is_a_no_op():
    assert _prefill(B=0, q=None, k=None, v=None, g=None, beta=None, o=None) == 0
    assert _prefill(H=0) == 0


def _prefill_snap(**kw):
    args = dict(q=A, k=A, v=A, g=A, beta=A, S0=A, o=A, S_T=A, snaps=A + (1 << 20), every=32, n=2,
                B=1, T=64, H=2, dk=64, dv=64, dtype=0, chunk=16, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_chunk_fwd_snapshots(
        vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]), vp(args["beta"]), vp(args["S0"]),
        vp(args["o"]), vp(args["S_T"]), vp(args["snaps"]), args["every"], args["n"], args["B"], args["T"],
        args["H"], args["dk"], args["dv"], args["dtype"], args["chunk"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), -1), (dict(snaps=None), -1), (dict(every=24), -1), (dict(every=0), -1),
    (dict(n=3), -1), (dict(snaps=MIS), -1), (dict(snaps=A + 64), -1),
    (dict(chunk=64), -1),                       # every = 32 is not a multiple of the chunk
    (dict(chunk=48), -1),
    (dict(every=64, chunk=32, n=2), -1), (dict(dk=96), -2),
])
def test_prefill_snapshots_rejects(kw, code):
    assert _prefill_snap(**kw) == code


def test_prefill_snapshots_empty_batch_is_a_no_op():
    assert _prefill_snap(B=0, T=0, n=0, snaps=None, q=None, k=None, v=None, g=None, beta=None, o=None) == 0
    assert _prefill_snap(H=0) == 0


def _decode(**kw):
    args = dict(qp=A, kp=A, vp=A, w=A, cache=A, pos=0, g=A, beta=A, S=A, o=A, N=2, H=3, dk=64,
                dv=64, width=4, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_decode_step(vp(args["qp"]), vp(args["kp"]), vp(args["vp"]), vp(args["w"]),
                                         vp(args["cache"]), args["pos"], vp(args["g"]), vp(args["beta"]),
                                         vp(args["S"]), vp(args["o"]), args["N"], args["H"], args["dk"],
                                         args["dv"], args["width"], args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(width=3), -1), (dict(width=5), -1), (dict(pos=-1), -1), (dict(dtype=7), -1),
    (dict(dk=32), -2), (dict(S=None), -1), (dict(cache=MIS), -1), (dict(N=-2), -1),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_is_a_no_op():
    assert _decode(N=0, S=None) == 0


def _prep(**kw):
    big = 1 << 24      # separate fake regions for every output: no overlap unless asked for
    args = dict(qp=A, kp=A, vp=A, w=A, init=A, z=A, Ah=A, bl=A, q=A + big, k=A + 2 * big,
                v=A + 3 * big, g=A + 4 * big, beta=A + 5 * big, fin=A + 6 * big, B=1, T=8, H=2,
                dk=64, dv=64, width=4, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    n = ("qp", "kp", "vp", "w", "init", "z", "Ah", "bl", "q", "k", "v", "g", "beta", "fin")
    return binding.lib().kda_prefill_prep(*(vp(args[a]) for a in n), args["B"], args["T"], args["H"],
                                          args["dk"], args["dv"], args["width"], args["dtype"],
                                          args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(width=3), -1), (dict(dtype=5), -1), (dict(T=-1), -1), (dict(dk=96), -2), (dict(dv=32), -2),
    (dict(qp=None), -1), (dict(bl=None), -1), (dict(w=None), -1), (dict(Ah=None), -1),
    (dict(g=None), -1), (dict(q=MIS), -1), (dict(init=MIS), -1),
    (dict(k=A + (1 << 24) + 64), -1),        # k overlaps q
    (dict(v=A + 64), -1),                    # an output overlapping an input
    (dict(fin=A + 64), -1),                  # conv_final partly overlapping conv_init
])
def test_prep_rejects(kw, code):
    assert _prep(**kw) == code


def test_prep_accepts_in_place_history_and_empty_batch():
    # conv_final == conv_init exactly is allowed; nothing is launched for B*H == 0
    assert _prep(B=0, fin=A) == 0
    assert _prep(H=0, qp=None, w=None) == 0


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        binding.chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1))


def _gate(**kw):
    big = 1 << 24
    args = dict(o=A, gate=A + big, w=A + 2 * big, y=A + 3 * big, rows=8, H=2, dv=64, eps=1e-6, dtype=0,
                stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_output_gate(vp(args["o"]), vp(args["gate"]), vp(args["w"]), vp(args["y"]),
                                         args["rows"], args["H"], args["dv"], args["eps"], args["dtype"],
                                         args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(eps=0.0), -1), (dict(eps=-1.0), -1), (dict(eps=float("nan")), -1), (dict(dtype=3), -1),
    (dict(rows=-1), -1), (dict(dv=96), -2), (dict(o=None), -1), (dict(gate=None), -1), (dict(y=None), -1),
    (dict(w=MIS), -1), (dict(y=MIS), -1),
    (dict(y=A + 64), -1),                    # y partly overlapping o
    (dict(y=A + (1 << 24) + 64), -1),        # y partly overlapping gate
    (dict(w=A + 3 * (1 << 24) + 32), -1),    # the weight inside y
])
def test_output_gate_rejects(kw, code):
    assert _gate(**kw) == code


def test_output_gate_in_place_and_empty_are_accepted():
    assert _gate(rows=0, o=None, gate=None, y=None) == 0
    assert _gate(H=0) == 0


def _fwd_gated(**kw):
    big = 1 << 24
    args = dict(q=A, k=A + big, v=A + 2 * big, g=A + 3 * big, beta=A + 4 * big, S0=A + 5 * big,
                gate=A + 6 * big, w=A + 7 * big, eps=1e-6, y=A + 8 * big, S_T=A + 9 * big, ws=A + 10 * big,
                wsb=1 << 12, B=1, T=8, H=2, dk=64, dv=64, dtype=0, spin=None, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    opts = ctypes.byref(binding.FwdOptions(spin_limit=args["spin"])) if args["spin"] is not None else None
    return binding.lib().kda_chunk_fwd_gated(
        vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]), vp(args["beta"]), vp(args["S0"]),
        vp(args["gate"]), vp(args["w"]), args["eps"], vp(args["y"]), vp(args["S_T"]), vp(args["ws"]),
        args["wsb"], args["B"], args["T"], args["H"], args["dk"], args["dv"], args["dtype"], opts,
        args["stream"])


def test_fwd_gated_workspace_size():
    # one progress counter per (sequence, head, 64-column value slice, consumer wavefront)
    assert binding.gated_workspace_size(2, 3, 128) == 2 * 3 * 2 * 4 * 4
    assert binding.gated_workspace_size(2, 3, 64) == 2 * 3 * 1 * 4 * 4
    L = binding.lib()
    assert L.kda_chunk_fwd_gated_workspace_size(2, 3, 96) == 0
    assert L.kda_chunk_fwd_gated_workspace_size(-1, 3, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(gate=None), -1), (dict(gate=MIS), -1), (dict(w=MIS), -1), (dict(eps=0.0), -1),
    (dict(eps=float("inf")), -1), (dict(y=None), -1), (dict(y=MIS), -1), (dict(ws=None), -1),
    (dict(ws=MIS), -1), (dict(wsb=2 * 4 * 4 - 1), -1), (dict(spin=-2), -1), (dict(dtype=2), -1),
    (dict(dk=96), -2), (dict(dv=32), -2), (dict(B=65536), -1), (dict(H=70000), -1),
    (dict(y=A + 64), -1),                        # y overlapping q
    (dict(y=A + 6 * (1 << 24) + 16), -1),        # y overlapping gate
    (dict(ws=A + 8 * (1 << 24) + 16), -1),       # the workspace inside y
    (dict(ws=A + 5 * (1 << 24)), -1),            # the workspace over S0
    (dict(S_T=A + 5 * (1 << 24) + 64), -1),      # S_T partly overlapping S0
])
def test_fwd_gated_rejects(kw, code):
    assert _fwd_gated(**kw) == code


def test_fwd_gated_smallest_workspace_and_empty_calls():
    # exactly the workspace size passes validation; nothing is launched for an empty batch
    # or (S_T = S0, T = 0) an empty sequence
    assert _fwd_gated(B=0, wsb=0, ws=None, gate=None) == 0
    assert _fwd_gated(T=0, S_T=A + 5 * (1 << 24), ws=None, gate=None) == 0


def _from_proj(**kw):
    big = 1 << 24
    names = ("qp", "kp", "vp", "w", "ci", "z", "A", "bl", "q", "k", "v", "g", "beta", "cf", "S0", "o", "S_T", "ws")
    args = {n: A + i * big for i, n in enumerate(names)}
    args["ci"] = None
    args.update(dict(wsb=1 << 12, B=1, T=200, H=2, dk=64, dv=64, width=4, dtype=0, spin=None, stream=None))
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    opts = ctypes.byref(binding.FwdOptions(spin_limit=args["spin"])) if args["spin"] is not None else None
    return binding.lib().kda_chunk_fwd_from_proj(*(vp(args[n]) for n in names), args["wsb"], args["B"], args["T"],
                                                 args["H"], args["dk"], args["dv"], args["width"], args["dtype"],
                                                 opts, args["stream"])


def test_from_proj_workspace_size():
    # one flag per (sequence, head, 128-token tile)
    assert binding.from_proj_workspace_size(2, 300, 3) == 2 * 3 * 3 * 4
    assert binding.from_proj_workspace_size(2, 0, 3) == 0
    assert binding.lib().kda_chunk_fwd_from_proj_workspace_size(-1, 5, 3) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(width=3), -1), (dict(dtype=2), -1), (dict(dk=96), -2), (dict(B=65536), -1), (dict(spin=-2), -1),
    (dict(ws=None), -1), (dict(ws=MIS), -1), (dict(wsb=2 * 2 * 4 - 1), -1), (dict(w=None), -1),
    (dict(qp=None), -1), (dict(q=None), -1), (dict(o=None), -1), (dict(o=MIS), -1),
    (dict(o=A + 64), -1),                          # o over q_pre
    (dict(o=A + 9 * (1 << 24) + 64), -1),          # o over k (a preprocessing output)
    (dict(S_T=A + 14 * (1 << 24) + 64), -1),       # S_T partly over S0
    (dict(ws=A + 15 * (1 << 24) + 16), -1),        # the workspace over o
    (dict(S0=A + 8 * (1 << 24) + 32), -1),         # S0 over q (written by the preprocessing)
])
def test_from_proj_rejects(kw, code):
    assert _from_proj(**kw) == code


def test_from_proj_empty_batch_is_a_no_op():
    assert _from_proj(B=0, ws=None, wsb=0) == 0


def _decode_gated(**kw):
    big = 1 << 24
    args = dict(qp=A, kp=A, vp=A, w=A, cache=A, pos=0, g=A, beta=A, S=A, gate=A + big, nw=None,
                eps=1e-6, y=A + 2 * big, N=2, H=3, dk=64, dv=64, width=4, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_decode_step_gated(
        vp(args["qp"]), vp(args["kp"]), vp(args["vp"]), vp(args["w"]), vp(args["cache"]), args["pos"],
        vp(args["g"]), vp(args["beta"]), vp(args["S"]), vp(args["gate"]), vp(args["nw"]), args["eps"],
        vp(args["y"]), args["N"], args["H"], args["dk"], args["dv"], args["width"], args["dtype"],
        args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(gate=None), -1), (dict(gate=MIS), -1), (dict(nw=MIS), -1), (dict(eps=0.0), -1),
    (dict(y=None), -1), (dict(width=3), -1), (dict(dk=32), -2),
])
def test_decode_gated_rejects(kw, code):
    assert _decode_gated(**kw) == code


def test_decode_gated_empty_is_a_no_op():
    assert _decode_gated(N=0, S=None, gate=None) == 0


def _bwd(**kw):
    big = 1 << 26
    args = dict(q=A, k=A, v=A, g=A, beta=A, S0=None, dO=A, dST=None, dq=A + big, dk=A + 2 * big,
                dv=A + 3 * big, dg=A + 4 * big, db=A + 5 * big, dS0=A + 6 * big, ws=A + 7 * big,
                wsb=1 << 26, B=1, T=40, H=2, dk_=64, dv_=128, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    n = ("q", "k", "v", "g", "beta", "S0", "dO", "dST", "dq", "dk", "dv", "dg", "db", "dS0", "ws")
    return binding.lib().kda_chunk_bwd(*(vp(args[a]) for a in n), args["wsb"], args["B"], args["T"], args["H"],
                                       args["dk_"], args["dv_"], args["dtype"], args["stream"])


def test_bwd_workspace_size():
    # two slices of 64 value columns: the incoming state of chunks 0, 1, 2 (sized
    # as fp32 for either dtype), slice 0's partials and one flag per head
    want_states = 3 * 2 * 64 * 128 * 4
    want_parts = 1 * 40 * 2 * (3 * 64 + 1) * 4
    rnd = lambda b: (b + 255) // 256 * 256
    assert binding.workspace_size(1, 40, 2, 64, 128) == rnd(want_states) + rnd(want_parts) + rnd(2 * 4)
    assert binding.workspace_size(1, 0, 2, 64, 128) == 0                            # no tokens, no flags
    assert binding.workspace_size(1, 40, 2, 64, 64) == rnd(3 * 2 * 64 * 64 * 4)    # one slice: no partials
    assert binding.workspace_size(1, 16, 2, 64, 64) == 2 * 64 * 64 * 4              # one chunk: its S0
    assert binding.workspace_size(1, 0, 2, 64, 64) == 0                             # no tokens: nothing
    assert binding.workspace_size(1, 40, 2, 96, 64) == 0                            # unsupported size


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -1), (dict(T=-1), -1), (dict(dk_=96), -2), (dict(dv_=32), -2),
    (dict(q=None), -1), (dict(dO=None), -1), (dict(dq=None), -1), (dict(db=None), -1),
    (dict(wsb=64), -1),                         # workspace too small
    (dict(ws=A + (7 << 26) + 16), -1),          # workspace not 256-byte aligned
    (dict(ws=None), -1),
    (dict(dq=MIS), -1), (dict(S0=MIS), -1),
    (dict(dk=A + (1 << 26) + 64), -1),          # dk overlaps dq
    (dict(dv=A + 64), -1),                      # an output overlapping an input
])
def test_bwd_rejects(kw, code):
    assert _bwd(**kw) == code


def test_bwd_empty_batch_is_a_no_op():
    assert _bwd(B=0, q=None, ws=None, wsb=0) == 0


def _bwd_noalloc(**kw):
    args = dict(q=A, k=A, v=A, g=A, beta=A, S0=A, dO=A, dST=A, dq=A + (1 << 26), dk=A + (2 << 26),
                dv=A + (3 << 26), dg=A + (4 << 26), db=A + (5 << 26), dS0=A + (6 << 26),
                B=1, T=40, H=2, dk_=64, dv_=128, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    n = ("q", "k", "v", "g", "beta", "S0", "dO", "dST", "dq", "dk", "dv", "dg", "db", "dS0")
    return binding.lib().kda_chunk_bwd_noalloc(*(vp(args[a]) for a in n), args["B"], args["T"], args["H"],
                                               args["dk_"], args["dv_"], args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -1), (dict(T=-1), -1), (dict(dk_=96), -2), (dict(dv_=32), -2),
    (dict(q=None), -1), (dict(dO=None), -1), (dict(dq=None), -1), (dict(dq=MIS), -1),
    (dict(B=65536, T=1), -1),
    # more workspace than the library's scratch array holds
    (dict(B=1, T=65536, H=8, dk_=128, dv_=128), -4),
    (dict(B=4, T=4096, H=32, dk_=128, dv_=128), -4),
])
def test_bwd_noalloc_rejects(kw, code):
    assert _bwd_noalloc(**kw) == code


def test_bwd_noalloc_scratch_limit():
    """Sizes at the scratch array's limit: at dk = dv = 128 a token-head takes 4 KiB of
    chunk states (64 KiB per 16 tokens) and 1540 bytes of slice 0's partials, plus a flag
    per head, so 8192 token-heads (44 MiB) fit and 16384 do not."""
    lim = binding.NOALLOC_SCRATCH_BYTES
    assert lim == 64 << 20
    assert binding.workspace_size(1, 4096, 2, 128, 128) == 4096 * 2 * (4096 + 1540) + 256
    assert binding.workspace_size(1, 4096, 2, 128, 128) <= lim
    assert binding.workspace_size(1, 8192, 2, 128, 128) > lim
    assert binding.workspace_size(1, 8192, 4, 64, 64) <= lim


def test_bwd_noalloc_empty_batch_is_a_no_op():
    assert _bwd_noalloc(B=0, q=None) == 0


def _validate(**kw):
    args = dict(g=A, beta=A + (1 << 24), report=A + (2 << 24), B=1, T=4, H=2, dk=64, dtype=0, stream=None)
    args.update(kw)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return binding.lib().kda_validate_inputs(vp(args["g"]), vp(args["beta"]), vp(args["report"]), args["B"],
                                             args["T"], args["H"], args["dk"], args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(report=None), -1), (dict(report=A + (2 << 24) + 4), -1),   # report missing or not 8-byte aligned
    (dict(dtype=2), -1), (dict(T=-1), -1), (dict(dk=0), -1), (dict(g=None), -1), (dict(beta=None), -1),
])
def test_validate_rejects(kw, code):
    assert _validate(**kw) == code


@pytest.mark.parametrize("n,lds,ptr,code", [
    (-1, 0, A, -1), ((1 << 20) + 1, 0, A, -1), (8, -1, A, -1), (8, 160 * 1024 + 1, A, -1),
    (8, 0, None, -1), (8, 0, A + 2, -1), (0, 0, None, 0), (0, 160 * 1024, None, 0),
])
def test_workgroup_xcds_rejects(n, lds, ptr, code):
    vp = ctypes.c_void_p(ptr) if ptr is not None else None
    assert binding.lib().kda_workgroup_xcds(vp, n, lds, None) == code
