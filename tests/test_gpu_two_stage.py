"""GPU checks of the two-stage prefill (chunk records for every chunk at once,
then the chain), which kda_chunk_fwd runs for bf16 q/k/v with d_k in {64, 128}.

Against the oracle and against the single-kernel pipeline on the same inputs:
ragged tails, both head sizes, S0 on and off, and decay steep enough that the
pipeline regroups chunks (the two-stage records never need to).  The blocked
path -- a sequence longer than the workspace cap runs block by block, the state
carried through S_T or a pool buffer -- is forced at small sizes by a test
build's workspace cap, with snapshots and in-place state across block edges; a
packed batch over the cap falls back to the pipeline.
"""
import math

import pytest
import torch

import ctypes

import numpy as np

import chunk_records as cr
import kda_inputs as ki
import oracle
from kda_check import assert_close, forced_prefill, gpu_o_heads, gpu_s_heads, log, oracle_prefill, to_host

pytestmark = pytest.mark.gpu

REC128 = cr.offsets(128)["BYTES"]  # bytes of one d_k = 128 chunk record
REC64 = cr.offsets(64)["BYTES"]


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _inp(gpu, B, T, H, dk, dv, seed, mu=3.0):
    return ki.make_prefill(B, T, H, dk, dv, torch.bfloat16, mu, 0.1, seed=seed, device=gpu)


def _run(inp, S0=True, **kw):
    kda = _kda()
    o, st = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"] if S0 else None,
                              **kw)
    torch.cuda.synchronize()
    return o, st


def _check(inp, o, st, what, S0=True):
    ref = dict(inp)
    if not S0:
        ref["S0"] = None
    ro, rs = oracle_prefill(ref)
    eo = assert_close(gpu_o_heads(o), ro, True, f"{what} o")
    es = assert_close(gpu_s_heads(st), rs, True, f"{what} S_T")
    return eo, es


def _hooks():
    import gated_delta_rule_07_amd as kda
    lib = kda.bind(kda.library_path().with_name("libkda_testhooks.so"))
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.kda_test_prep.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp]
    lib.kda_test_prep.restype = i
    lib.kda_test_chain.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.kda_test_chain.restype = i
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("dk", [128, 64])
def test_stage1_records_match_reference(gpu, dk):
    """Stage 1 alone: every field of every record (ragged last chunk included)
    against the fp64 reference, within the fp16 rounding of the operands."""
    B, T, H = 2, 100, 3
    inp = _inp(gpu, B, T, H, dk, dk, seed=11 + dk)
    inp["alpha"][0, 40:72, 1, ::4] = math.exp(-5.0)  # a steep chunk in some channels
    nc = (T + 31) // 32
    rb = cr.offsets(dk)["BYTES"]
    rec = torch.zeros(B * nc * H * rb, dtype=torch.uint8, device=gpu)
    lib = _hooks()
    st = lib.kda_test_prep(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["alpha"].data_ptr(), inp["beta"].data_ptr(),
                           B, T, H, dk, rec.data_ptr(), _stream())
    assert st == 0
    torch.cuda.synchronize()
    got = rec.cpu().numpy().reshape(-1, rb)
    h = {n: to_host(inp[n]).double().numpy() for n in ("q", "k", "alpha", "beta")}
    ref = cr.records(h["q"], h["k"], h["alpha"], h["beta"]).reshape(-1, rb)
    names = ("KG", "QG", "KH", "T", "PT", "gamma")
    tol = {"KG": 2e-3, "QG": 2e-3, "KH": 2e-3, "T": 1e-2, "PT": 1e-2, "gamma": 1e-5}
    worst = {n: 0.0 for n in names}
    for r in range(got.shape[0]):
        g = cr.unpack(dk, got[r])
        e = cr.unpack(dk, ref[r])
        for n, x, y in zip(names, g, e):
            if n in ("T", "PT"):
                x, y = np.tril(x), np.tril(y)
            d = float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-30))
            worst[n] = max(worst[n], d)
            assert d <= tol[n], f"record {r} ({divmod(r, H)}): {n} differs by {d:.2e} of its max"
    log("  worst relative difference per field: " + ", ".join(f"{n} {worst[n]:.1e}" for n in names))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_stage2_chain_from_reference_records(gpu, dk, dv):
    """Stage 2 alone, fed records built by the fp64 reference: o and S_T against
    the oracle (the records carry only the fp16 rounding of the operands)."""
    B, T, H = 1, 150, 2
    inp = _inp(gpu, B, T, H, dk, dv, seed=21 + dk)
    h = {n: to_host(inp[n]).double().numpy() for n in ("q", "k", "alpha", "beta")}
    rec = torch.from_numpy(cr.records(h["q"], h["k"], h["alpha"], h["beta"])).to(gpu)
    o = torch.zeros(B, T, H, dv, device=gpu)
    st = torch.zeros(B, H, dk, dv, device=gpu)
    lib = _hooks()
    s = lib.kda_test_chain(inp["v"].data_ptr(), rec.data_ptr(), inp["S0"].data_ptr(), o.data_ptr(), st.data_ptr(),
                           B, T, H, dk, dv, _stream())
    assert s == 0
    torch.cuda.synchronize()
    _check(inp, o, st, f"chain d={dk}x{dv}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 32)])
@pytest.mark.parametrize("S0", [True, False])
def test_two_stage_matches_oracle_and_pipeline(gpu, dk, dv, S0):
    log(f"two-stage d={dk}x{dv} S0={S0}")
    inp = _inp(gpu, 2, 357, 3, dk, dv, seed=dk + dv + S0)
    with forced_prefill(2):
        o2, s2 = _run(inp, S0)
    with forced_prefill(1):
        o1, s1 = _run(inp, S0)
    _check(inp, o2, s2, "two-stage", S0)
    _check(inp, o1, s1, "pipeline", S0)
    # same method and fp16 operands, different factorisations of L and P
    d = (o2.float() - o1.float()).abs().max().item() / o1.float().pow(2).mean().sqrt().item()
    log(f"  two-stage vs pipeline: {d:.2e} of the RMS")
    assert d < 1e-2


def test_default_path_is_two_stage(gpu):
    """The library's choice for these shapes equals the forced two-stage run bit for bit."""
    inp = _inp(gpu, 1, 200, 2, 128, 128, seed=3)
    o0, s0 = _run(inp)
    with forced_prefill(2):
        o2, s2 = _run(inp)
    assert torch.equal(o0, o2) and torch.equal(s0, s2)


@pytest.mark.parametrize("dk", [128, 64])
def test_two_stage_any_decay(gpu, dk):
    """Decays at and far below the e^-5 bound, and exact zeros: the bounded factors
    need no regrouping whatever the decay (the pipeline is limited to alpha >= e^-5)."""
    inp = _inp(gpu, 1, 300, 2, dk, dk, seed=50 + dk)
    a = inp["alpha"]
    a[:, 0:64] = math.exp(-5.0)
    a[:, 64:100, :, ::3] = math.exp(-20.0)
    a[:, 130:131] = 0.0
    a[:, 200:260, 1, 5] = 1e-30
    log(f"two-stage extreme decay d={dk}")
    with forced_prefill(2):
        o, st = _run(inp)
    _check(inp, o, st, "extreme decay")


@pytest.mark.parametrize("nblk_chunks", [1, 3, 5])
@pytest.mark.parametrize("with_st", [True, False])
@pytest.mark.parametrize("overlap", [0, 1])
def test_blocked_sequence(gpu, nblk_chunks, with_st, overlap):
    """A workspace cap of a few chunks per sequence: the sequence runs in blocks,
    the state carried through S_T (or a pool buffer when S_T is not wanted);
    one block's stage 1 then its chain, or (overlap) each block's chain in one
    launch with stage 1 of the next, in two alternating record buffers."""
    kda = _kda()
    B, T, H = 2, 300, 2
    inp = _inp(gpu, B, T, H, 128, 128, seed=60 + nblk_chunks)
    cap = nblk_chunks * B * H * REC128
    log(f"blocked: {nblk_chunks} chunks per block, S_T {'wanted' if with_st else 'not wanted'}, overlap {overlap}")
    with forced_prefill(2, rec_cap=cap, overlap=overlap):
        o, st = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                                  want_state=with_st)
        torch.cuda.synchronize()
    with forced_prefill(2):
        o_one, st_one = _run(inp)
    # blocks only cut the chain between chunks: the same arithmetic, bit for bit
    assert torch.equal(o, o_one)
    if with_st:
        assert torch.equal(st, st_one)
    ro, _ = oracle_prefill(inp)
    assert_close(gpu_o_heads(o), ro, True, "blocked o")


@pytest.mark.parametrize("overlap", [0, 1])
def test_blocked_in_place_state_and_snapshots(gpu, overlap):
    """S0 and S_T one buffer, snapshots on and between block edges."""
    kda = _kda()
    B, T, H = 1, 333, 2
    inp = _inp(gpu, B, T, H, 64, 64, seed=70)
    pos = [32, 64, 96, 160, 320, 333]
    cap = 2 * B * H * REC64  # 64-token blocks
    S = inp["S0"].clone()
    with forced_prefill(2, rec_cap=cap, overlap=overlap):
        o, st, sn = kda.kda_chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S,
                                                snap_tokens=pos, chunk=32, S_T=S)
        torch.cuda.synchronize()
    with forced_prefill(2):
        o1, st1, sn1 = kda.kda_chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                                   inp["S0"], snap_tokens=pos, chunk=32)
        torch.cuda.synchronize()
    assert st.data_ptr() == S.data_ptr()
    assert torch.equal(o, o1) and torch.equal(S, st1) and torch.equal(sn, sn1)
    for j, t in enumerate(pos):
        h = {n: to_host(inp[n][:, :t].contiguous()) for n in ("q", "k", "v", "alpha", "beta")}
        _, rs = oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], to_host(inp["S0"]), want_o=False)
        assert_close(gpu_s_heads(sn[:, :, j]), rs, True, f"snapshot at {t}")


def test_varlen_two_stage_and_over_cap(gpu):
    """A packed batch: the two-stage records (slots cu[b] / 32 + b + c) and, with
    the cap below the batch's records, the pipeline fallback; both per sequence
    against the oracle and bit-equal to separate calls on their own path."""
    kda = _kda()
    lens, H, dk, dv = [0, 1, 63, 64, 100, 257, 31], 2, 128, 128
    seqs = [ki.make_prefill(1, max(n, 1), H, dk, dv, torch.bfloat16, 3.0, 0.1, seed=80 + i, device=gpu)
            for i, n in enumerate(lens)]
    x = {nm: torch.cat([s[nm][0, :n] for s, n in zip(seqs, lens)], 0).contiguous()
         for nm in ("q", "k", "v", "alpha", "beta")}
    S0 = torch.cat([s["S0"] for s in seqs], 0).contiguous()
    cu = torch.tensor([0] + torch.cumsum(torch.tensor(lens), 0).tolist(), dtype=torch.int32, device=gpu)
    outs = {}
    for name, cap in (("two-stage", 0), ("fallback", REC128)):
        with forced_prefill(2, rec_cap=cap):
            o, st = kda.kda_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["alpha"], x["beta"], cu, S0)
            torch.cuda.synchronize()
        outs[name] = (o, st)
        offs = cu.tolist()
        for b, n in enumerate(lens):
            if n == 0:
                assert torch.equal(st[b], S0[b])
                continue
            s = offs[b]
            h = {nm: to_host(x[nm][s:s + n][None]) for nm in ("q", "k", "v", "alpha", "beta")}
            ro, rs = oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], to_host(S0[b:b + 1]))
            assert_close(o[s:s + n].float().permute(1, 0, 2).cpu().double().numpy(), ro, True, f"{name} seq{b} o")
            assert_close(st[b].cpu().double().numpy(), rs, True, f"{name} seq{b} S_T")
    with forced_prefill(1):
        o1, st1 = kda.kda_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["alpha"], x["beta"], cu, S0)
        torch.cuda.synchronize()
    assert torch.equal(outs["fallback"][0], o1) and torch.equal(outs["fallback"][1], st1)


@pytest.mark.parametrize("dk", [128, 64])
def test_gated_two_stage(gpu, dk):
    """The fused gate formed in stage 1, fast-forgetting heads included."""
    kda = _kda()
    B, T, H = 1, 300, 4
    inp = ki.make_prefill(B, T, H, dk, dk, torch.bfloat16, 3.0, 0.1, seed=90 + dk, device=gpu)
    z, A = ki.make_gate((B, T, H, dk), H, torch.bfloat16, seed=91 + dk, device=gpu, z_mu=-3.0, z_std=1.0, a_std=0.3)
    with forced_prefill(2):
        o, st = kda.kda_chunk_fwd_gated(inp["q"], inp["k"], inp["v"], z, A, inp["beta"], inp["S0"], chunk=32)
        torch.cuda.synchronize()
    h = {n: x.cpu() for n, x in inp.items()}
    ro, rs = oracle.forward(h["q"], h["k"], h["v"], oracle.gate_alpha(z.cpu(), A.cpu()), h["beta"], h["S0"])
    eo = assert_close(gpu_o_heads(o), ro, True, f"gated two-stage d={dk} o")
    assert_close(gpu_s_heads(st), rs, True, f"gated two-stage d={dk} S_T")
    log(f"  fast-forgetting worst head: {eo:.2e}")


@pytest.mark.parametrize("dk", [128, 64])
def test_blocked_gated_overlap(gpu, dk):
    """The gated call in blocks with each block's chain beside the next block's
    stage 1 (the gate formed there): bit-equal to one block and to the serial
    blocks."""
    kda = _kda()
    B, T, H = 1, 420, 3
    inp = ki.make_prefill(B, T, H, dk, dk, torch.bfloat16, 3.0, 0.1, seed=95 + dk, device=gpu)
    z, A = ki.make_gate((B, T, H, dk), H, torch.bfloat16, seed=96 + dk, device=gpu)
    cap = 4 * B * H * cr.offsets(dk)["BYTES"]  # 128-token blocks, the last one ragged
    outs = []
    for rec_cap, overlap in ((0, -1), (cap, 0), (cap, 1)):
        with forced_prefill(2, rec_cap=rec_cap, overlap=overlap):
            outs.append(kda.kda_chunk_fwd_gated(inp["q"], inp["k"], inp["v"], z, A, inp["beta"], inp["S0"], chunk=32))
            torch.cuda.synchronize()
    for o, st in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(st, outs[0][1])
