"""GPU checks of kda_chunk_fwd_split (the prefill with each sequence cut into
parts that run side by side: transitions of the parts, a combine, then every
part from its incoming state).

o and S_T must match the oracle's single pass to the operator's tolerance for
forced and automatic part counts, ragged last parts, parts of one chunk, d_k 64
and 128, with and without S0, in place (S0 == S_T), through steep decay, and on
the 4K-token workload shape with the library's own choice.  One part must be
kda_chunk_fwd bit for bit.
"""
import math

import pytest
import torch

import kda_inputs as ki
from kda_check import assert_close, gpu_o_heads, gpu_s_heads, log, oracle_prefill

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _check(inp, parts, what, S0=True, heads=None, o_dtype=torch.float32):
    kda = _kda()
    n, ws = kda.kda_chunk_fwd_split_plan(inp["q"].dtype, *inp["q"].shape, inp["v"].shape[-1], parts=parts)
    log(f"split {what}: {n} parts, workspace {ws} bytes")
    s0 = inp["S0"] if S0 else None
    o, st = kda.kda_chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], s0, parts=parts,
                                    o_dtype=o_dtype)
    torch.cuda.synchronize()
    ref = dict(inp)
    if not S0:
        ref["S0"] = None
    ro, rs = oracle_prefill(ref, heads=heads)
    assert_close(gpu_o_heads(o.float(), heads), ro, True, f"{what} o")
    assert_close(gpu_s_heads(st, heads), rs, True, f"{what} S_T")
    return n


CASES = [
    # (name, B, T, H, dk, parts)
    ("d128 2 parts", 1, 1000, 2, 128, 2),
    ("d128 3 parts ragged", 2, 333, 2, 128, 3),
    ("d128 5 parts", 1, 1000, 3, 128, 5),
    ("d64 4 parts", 2, 700, 3, 64, 4),
    ("d128 one chunk per part", 1, 200, 2, 128, 7),
    ("d64 more parts than chunks", 1, 100, 2, 64, 50),
]


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (128, 32)])
def test_split_unequal_head_sizes(gpu, dk, dv):
    """d_k != d_v: pass 1 runs d_v value columns and d_k transition columns."""
    inp = ki.make_prefill(2, 450, 2, dk, dv, torch.bfloat16, 3.0, 0.1, seed=dk + 3 * dv, device=gpu)
    _check(inp, 3, f"d_k={dk} d_v={dv}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle(gpu, case):
    name, B, T, H, dk, parts = case
    inp = ki.make_prefill(B, T, H, dk, dk, torch.bfloat16, 3.0, 0.1, seed=T + parts, device=gpu)
    n = _check(inp, parts, name)
    assert 1 < n <= min(parts, -(-T // 32))


TREE_CASES = [
    # (name, B, T, H, dk, dv, parts, S0): part counts >= 9 run the combine as a tree
    ("d128 10 parts", 1, 1200, 2, 128, 128, 12, True),
    ("d128 16 parts ragged", 2, 1500, 2, 128, 128, 16, True),
    ("d64 33 parts", 1, 2100, 3, 64, 64, 33, True),
    ("d128 10 parts no S0", 1, 1200, 2, 128, 128, 12, False),
    ("d128x64 10 parts", 1, 1200, 2, 128, 64, 12, True),
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[c[0] for c in TREE_CASES])
def test_split_tree_combine(gpu, case):
    """Enough parts that the states entering them are formed by a tree over the
    part maps (log2 levels of pairwise compositions, then one product with S0).
    Slow decay (alpha = sigmoid(N(8, 1)), about 0.9997) keeps S0 and the early
    parts visible at the end, so the composed transitions are what is tested."""
    name, B, T, H, dk, dv, parts, s0 = case
    inp = ki.make_prefill(B, T, H, dk, dv, torch.bfloat16, 8.0, 0.1, seed=T + parts + dv, device=gpu)
    n = _check(inp, parts, name, S0=s0)
    assert n >= 9, f"{name}: {n} parts do not reach the tree"


def test_split_without_initial_state_and_bf16_output(gpu):
    """No S0 against the oracle; a bf16 o is the fp32 o rounded to nearest even,
    bit for bit (the rounding of a bf16 o alone can spend the whole tolerance)."""
    kda = _kda()
    inp = ki.make_prefill(1, 640, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=12, device=gpu)
    _check(inp, 4, "no S0", S0=False)
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    o32, s32 = kda.kda_chunk_fwd_split(*args, parts=4)
    o16, s16 = kda.kda_chunk_fwd_split(*args, parts=4, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)


def test_split_edge_lengths(gpu):
    """A last part of one token (T = 33, 2 parts) and an empty sequence (T = 0:
    S_T = S0, the single pass)."""
    kda = _kda()
    inp = ki.make_prefill(1, 33, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=16, device=gpu)
    assert _check(inp, 2, "T=33, 2 parts") == 2
    x0 = ki.make_prefill(1, 1, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=17, device=gpu)
    empty = {n: t[:, :0].contiguous() if n != "S0" else t for n, t in x0.items()}
    o, st = kda.kda_chunk_fwd_split(empty["q"], empty["k"], empty["v"], empty["alpha"], empty["beta"],
                                    empty["S0"], parts=4)
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(st, x0["S0"])


def test_split_in_place_state(gpu):
    """S0 == S_T: the last part writes the state while earlier parts still run;
    only the combine reads S0, so the result is the single pass's."""
    kda = _kda()
    inp = ki.make_prefill(2, 500, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=13, device=gpu)
    o_ref, s_ref = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    S = inp["S0"].clone()
    o, st = kda.kda_chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S, S_T=S, parts=4)
    torch.cuda.synchronize()
    assert st.data_ptr() == S.data_ptr()
    e = (st - s_ref).abs().max().item() / s_ref.pow(2).mean().sqrt().item()
    eo = (o - o_ref).abs().max().item() / o_ref.pow(2).mean().sqrt().item()
    log(f"  in place vs single pass: S_T {e:.2e}, o {eo:.2e}")
    assert e < 1e-2 and eo < 1e-2


def test_split_one_part_is_the_single_pass(gpu):
    kda = _kda()
    inp = ki.make_prefill(1, 300, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=14, device=gpu)
    o1, s1 = kda.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])
    o2, s2 = kda.kda_chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"], parts=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_split_through_steep_decay(gpu):
    """Decay at the lower bound in some channels: parts and transitions run the
    segment path; a part boundary falls inside the steep run."""
    inp = ki.make_prefill(1, 600, 2, 128, 128, torch.bfloat16, 3.0, 0.1, seed=15, device=gpu)
    a = inp["alpha"]
    a[:, 100:400, :, ::3] = math.exp(-5.0)
    _check(inp, 3, "steep")


def test_split_4k_workload_auto(gpu):
    """B=1, H=8, T=4096: the library's part count (one: the two-stage single pass
    models faster than any split) and an explicit split; every head against the
    oracle."""
    inp = ki.make_workload_prefill(1, seed=2, device=gpu)
    n = _check(inp, 0, "4K workload auto")
    assert n == 1, "the 4K workload's single pass beats a split on this GPU"
    _check(inp, 5, "4K workload, 5 parts")
