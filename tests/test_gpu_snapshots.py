"""GPU checks of kda_chunk_fwd_snapshots (state recorded at listed token counts).

Each snapshot must equal (a) the oracle's state after that many tokens, to the
operator's tolerance, and (b) bit for bit, the final state of kda_chunk_fwd run
on the truncated sequence -- the chunks before the position are computed
identically.  Requesting snapshots must not change o or S_T.  Both prefill
kernels are covered (the pipelined bf16 d_k in {64,128} kernel and the generic
tile kernel), including ragged tails, regrouped (steep-decay) chunks and the
64K workload shape.
"""
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_check import assert_close, gpu_s_heads, log, to_host

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _slice(inp, t):
    out = {}
    for name in ("q", "k", "v", "alpha", "beta"):
        out[name] = inp[name][:, :t].contiguous()
    out["S0"] = inp.get("S0")
    return out


def _oracle_state(inp, t, heads=None):
    h = {n: to_host(x) for n, x in _slice(inp, t).items()}
    _, st = oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], h["S0"], heads=heads, want_o=False)
    return st


def _run(inp, pos, chunk):
    kda = _kda()
    o, st, sn = kda.kda_chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                                            snap_tokens=pos, chunk=chunk)
    torch.cuda.synchronize()
    return o, st, sn


CASES = [
    # (name, B, T, H, dk, dv, dtype, chunk, positions)
    ("pipe d128 ragged", 2, 300, 2, 128, 128, torch.bfloat16, 64, [64, 128, 256, 300]),
    ("pipe d64 chunk32", 1, 200, 3, 64, 64, torch.bfloat16, 32, [32, 96, 160, 192]),
    ("generic bf16 d32", 2, 150, 2, 32, 32, torch.bfloat16, 64, [64, 128, 150]),
    ("generic f32 chunk16", 1, 100, 2, 32, 16, torch.float32, 16, [16, 48, 64, 96, 100]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_snapshots_match_oracle_and_truncated_calls(gpu, case):
    name, B, T, H, dk, dv, dtype, chunk, pos = case
    log(f"snapshots {name}: B={B} T={T} H={H} d={dk}x{dv} {dtype} chunk={chunk} at {pos}")
    inp = ki.make_prefill(B, T, H, dk, dv, dtype, 3.0, 0.1, seed=T + dk, device=gpu)
    o, st, sn = _run(inp, pos, chunk)
    bf = dtype == torch.bfloat16
    kda = _kda()
    for j, t in enumerate(pos):
        got = gpu_s_heads(sn[:, :, j].contiguous())
        assert_close(got, _oracle_state(inp, t), bf, f"{name} snapshot@{t}")
        s = _slice(inp, t)
        _, st_t = kda.kda_chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["S0"], chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(sn[:, :, j], st_t), f"{name}: snapshot@{t} differs from S_T of the truncated call"


def test_snapshots_leave_outputs_unchanged(gpu):
    """o and S_T are bit-identical with and without snapshots; a snapshot at T is S_T."""
    kda = _kda()
    for dk, dtype in ((128, torch.bfloat16), (32, torch.float32)):
        inp = ki.make_prefill(2, 257, 2, dk, dk, dtype, 3.0, 0.1, seed=7, device=gpu)
        o0, st0 = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
        o1, st1, sn = _run(inp, [64, 192, 257], 64)
        assert torch.equal(o0, o1) and torch.equal(st0, st1)
        assert torch.equal(sn[:, :, 2], st1)
        o2, st2, sn0 = _run(inp, [], 64)
        assert sn0.shape[2] == 0 and torch.equal(o0, o2) and torch.equal(st0, st2)


def test_snapshots_through_regrouped_chunks(gpu):
    """Decay at the lower bound forces short segments; snapshots around them stay exact."""
    inp = ki.make_prefill(1, 256, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=5, device=gpu)
    a = inp["alpha"].clone()
    a[:, 40:140] = 0.0067379470  # e^-5
    inp["alpha"] = a
    pos = [64, 128, 192]
    o, st, sn = _run(inp, pos, 64)
    kda = _kda()
    for j, t in enumerate(pos):
        assert_close(gpu_s_heads(sn[:, :, j].contiguous()), _oracle_state(inp, t), True, f"steep snapshot@{t}")
        s = _slice(inp, t)
        _, st_t = kda.kda_chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["S0"])
        torch.cuda.synchronize()
        assert torch.equal(sn[:, :, j], st_t)


def test_snapshots_64k_workload(gpu):
    """The 64K prefill shape (B=2, H=32, d=128) with a snapshot every 4096 tokens:
    every snapshot equals the truncated call's S_T bit for bit for all heads, and
    two of them match the oracle on sampled heads."""
    kda = _kda()
    inp = ki.make_workload_prefill(2, seed=0, device=gpu)
    T = inp["q"].shape[1]
    pos = list(range(4096, T + 1, 4096))
    log(f"64K snapshots at {len(pos)} positions")
    o, st, sn = _run(inp, pos, 64)
    for j in (0, len(pos) // 2 - 1):
        t = pos[j]
        s = _slice(inp, t)
        _, st_t = kda.kda_chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["S0"])
        torch.cuda.synchronize()
        assert torch.equal(sn[:, :, j], st_t), f"snapshot@{t} differs from the truncated call"
        del s, st_t
    assert torch.equal(sn[:, :, -1], st)
    heads = [0, 37]
    for j in (0, 3):
        t = pos[j]
        ref = _oracle_state(inp, t, heads=heads)
        assert_close(gpu_s_heads(sn[:, :, j].contiguous(), heads), ref, True, f"64K snapshot@{t}")
