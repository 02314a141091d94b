"""GPU checks of kda_chunk_fwd_varlen (a packed batch of sequences of different
lengths).  Every sequence must match the oracle run on that sequence alone (o
and its final state), sequences of length 0 and 1 and ragged tails included;
on the pipelined path the packed call must equal separate kda_chunk_fwd calls
bit for bit.  Offsets are clamped in the kernels: rows no sequence covers are
left untouched and a decreasing offset pair is an empty sequence.
"""
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_check import assert_close, log, to_host

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _packed(gpu, lens, H, dk, dv, dtype, seed):
    """Packed inputs [total,H,d] built from independent per-sequence draws, plus S0 [N,H,dk,dv]."""
    seqs = [ki.make_prefill(1, max(n, 1), H, dk, dv, dtype, 3.0, 0.1, seed=seed + i, device=gpu)
            for i, n in enumerate(lens)]
    cat = {}
    for name in ("q", "k", "v", "alpha", "beta"):
        cat[name] = torch.cat([s[name][0, :n] for s, n in zip(seqs, lens)], 0).contiguous()
    S0 = torch.cat([s["S0"] for s in seqs], 0).contiguous()
    cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens), 0).tolist()), dtype=torch.int32, device=gpu)
    return cat, S0, cu


CASES = [
    ("pipe bf16 d128", [0, 1, 63, 64, 100, 257], 2, 128, 128, torch.bfloat16, 64),
    ("pipe bf16 d64 chunk32", [40, 0, 97, 32], 3, 64, 64, torch.bfloat16, 32),
    ("generic f32 d32 chunk16", [5, 16, 0, 70, 33], 2, 32, 32, torch.float32, 16),
    ("generic bf16 d32", [130, 1, 64], 2, 32, 64, torch.bfloat16, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_matches_oracle_per_sequence(gpu, case):
    name, lens, H, dk, dv, dtype, chunk = case
    kda = _kda()
    log(f"varlen {name}: lengths {lens}")
    x, S0, cu = _packed(gpu, lens, H, dk, dv, dtype, seed=len(lens) * 7 + dk)
    o, st = kda.kda_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["alpha"], x["beta"], cu, S0, chunk=chunk)
    torch.cuda.synchronize()
    bf = dtype == torch.bfloat16
    offs = cu.tolist()
    for b, n in enumerate(lens):
        s0 = offs[b]
        if n == 0:
            assert torch.equal(st[b], S0[b]), f"empty sequence {b}: S_T must equal S0"
            continue
        h = {nm: to_host(x[nm][s0:s0 + n][None]) for nm in ("q", "k", "v", "alpha", "beta")}
        ro, rs = oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], to_host(S0[b:b + 1]))
        got_o = o[s0:s0 + n].float().permute(1, 0, 2).cpu().double().numpy()
        assert_close(got_o, ro, bf, f"{name} seq{b} (T={n}) o")
        assert_close(st[b].cpu().double().numpy(), rs, bf, f"{name} seq{b} S_T")


def test_varlen_equals_separate_calls(gpu):
    """Pipelined path: the packed call is bit-identical to one kda_chunk_fwd per sequence."""
    kda = _kda()
    lens = [77, 256, 1, 130]
    H, dk, dv = 2, 128, 128
    x, S0, cu = _packed(gpu, lens, H, dk, dv, torch.bfloat16, seed=3)
    o, st = kda.kda_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["alpha"], x["beta"], cu, S0)
    offs = cu.tolist()
    for b, n in enumerate(lens):
        s0 = offs[b]
        one = {nm: x[nm][s0:s0 + n][None].clone() for nm in ("q", "k", "v", "alpha", "beta")}  # aligned copies
        o1, st1 = kda.kda_chunk_fwd(one["q"], one["k"], one["v"], one["alpha"], one["beta"], S0[b:b + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[s0:s0 + n], o1[0]), f"seq {b}: o differs from the separate call"
        assert torch.equal(st[b], st1[0]), f"seq {b}: S_T differs from the separate call"


@pytest.mark.parametrize("offs,ranges", [
    ([3, 90, 150, 120], [(3, 90), (90, 150), (150, 150)]),   # starts past 0; last pair goes backwards
    ([0, 90, 500], [(0, 90), (90, 200)]),                     # the end lies past the packed length
])
def test_varlen_clamped_offsets(gpu, offs, ranges):
    """Offsets are clamped to [0, total] and lengths to >= 0: uncovered rows stay untouched,
    a backwards pair is an empty sequence (S_T = S0), a past-the-end offset stops at the end."""
    kda = _kda()
    H, dk, dv, total = 2, 64, 64, 200
    x = ki.make_prefill(1, total, H, dk, dv, torch.bfloat16, 3.0, 0.1, seed=9, device=gpu)
    flat = {nm: x[nm][0].contiguous() for nm in ("q", "k", "v", "alpha", "beta")}
    N = len(offs) - 1
    S0 = torch.cat([x["S0"]] * N, 0).contiguous()
    cu = torch.tensor(offs, dtype=torch.int32, device=gpu)
    o = torch.full((total, H, dv), 7.0, device=gpu, dtype=torch.float32)
    o, st = kda.kda_chunk_fwd_varlen(flat["q"], flat["k"], flat["v"], flat["alpha"], flat["beta"], cu, S0, o=o)
    torch.cuda.synchronize()
    covered = torch.zeros(total, dtype=torch.bool)
    for b, (s0, e) in enumerate(ranges):
        covered[s0:e] = True
        if e == s0:
            assert torch.equal(st[b], S0[b]), f"sequence {b} is empty: S_T must equal S0"
            continue
        h = {nm: to_host(flat[nm][s0:e][None]) for nm in flat}
        ro, rs = oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], to_host(S0[b:b + 1]))
        assert_close(st[b].cpu().double().numpy(), rs, True, f"clamped seq{b} [{s0},{e}) S_T")
        assert_close(o[s0:e].float().permute(1, 0, 2).cpu().double().numpy(), ro, True, f"clamped seq{b} o")
    assert torch.all(o[~covered.to(o.device)] == 7.0), "rows no sequence covers were written"
