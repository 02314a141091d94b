"""GPU checks that the calls run on the stream they are given: on a side
stream, and captured into a HIP graph (capture fails for work enqueued on any
other stream).  Every graph is replayed several times, with the program's own
eager work and a synchronisation between replays, and every replay must equal
the eager calls bit for bit (the kernels are deterministic).  Nothing is
allocated or cleared inside a capture: buffers and workspaces are made first.
"""
import pytest
import torch

import kda_inputs as ki
from kda_check import log

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _capture(fn):
    """Capture fn() into a graph after one warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_prefill_on_a_side_stream(gpu):
    kda = _kda()
    x = ki.make_prefill(2, 300, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=61, device=gpu)
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    o_ref, s_ref = kda.kda_chunk_fwd(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, st = kda.kda_chunk_fwd(*args)
    side.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


def test_decode_steps_in_a_graph(gpu):
    """Five in-place decode steps captured once and replayed, as a serving loop would."""
    kda = _kda()
    B, H, d, steps = 16, 4, 128, 5
    S0 = ki.make_state(B, H, d, d, 0.1, 62, gpu)
    toks = [ki.make_decode_token(B, H, d, d, torch.bfloat16, 3.0, seed=62, step=t, device=gpu) for t in range(steps)]
    S_e = S0.clone()
    o_e = torch.stack([kda.kda_decode_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S_e) for t in toks])
    S_g = S0.clone()
    o_g = torch.empty(steps, B, H, d, device=gpu, dtype=torch.float32)

    def run():
        for i, t in enumerate(toks):
            kda.kda_decode_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S_g, o=o_g[i])

    g = _capture(run)
    for rep in range(3):
        S_g.copy_(S0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  decode graph replay {rep}")
        assert torch.equal(S_g, S_e) and torch.equal(o_g, o_e), f"replay {rep} differs from the eager steps"


@pytest.mark.parametrize("parts", [1, 4, 12])
def test_prefill_in_a_graph(gpu, parts):
    """The prefill (one kernel) and the split prefill (three kernels and a workspace; with 12
    parts, a tree of combine launches) in a graph."""
    kda = _kda()
    B, T, H, d = 1, 640, 2, 128
    x = ki.make_prefill(B, T, H, d, d, torch.bfloat16, 3.0, 0.1, seed=63, device=gpu)
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    n, ws_bytes = kda.kda_chunk_fwd_split_plan(torch.bfloat16, B, T, H, d, d, parts=parts)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=gpu)
    o_e, s_e = kda.kda_chunk_fwd_split(*args, parts=n, workspace=ws)
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    s_g = torch.empty_like(s_e)

    def run():
        kda.kda_chunk_fwd_split(*args, parts=n, workspace=ws, o=o_g, S_T=s_g)

    g = _capture(run)
    for rep in range(3):
        o_g.fill_(float("nan"))  # eager work between replays; a replay must overwrite all of it
        s_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  prefill graph ({n} parts) replay {rep}")
        assert torch.equal(o_g, o_e) and torch.equal(s_g, s_e), f"replay {rep} differs from the eager call"
