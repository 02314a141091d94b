"""GPU parity over a seeded sweep of shapes, against the fp64 oracle.

Each case draws B, T (ragged, sometimes a single token), H, d_k, d_v, the
q/k/v dtype, the chunk size, whether S0 is given, and the decay strength
(alpha = sigmoid(N(mu, 1)) with mu = 1 making many chunks decay below e^-10, so
the segment path runs).  Every case runs kda_chunk_fwd; where the shape is one
the pipelined kernel serves, the same inputs also run kda_chunk_fwd_split with a
drawn part count, and kda_chunk_fwd_gated with a drawn gate.  Tolerances are the
operator's (1e-4 absolute for fp32 inputs, 2e-2 of the RMS per head for bf16).
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_check import assert_close, gpu_o_heads, gpu_s_heads, log, oracle_prefill

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        bf = rng.random() < 0.7
        dk = int(rng.choice([16, 32, 64, 128] if bf else [16, 32]))
        dv = int(rng.choice([16, 32, 64, 128]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        T = 1 if rng.random() < 0.1 else int(rng.integers(2, 330))
        chunk = int(rng.choice([16, 32, 64]))
        s0 = bool(rng.random() < 0.7)
        mu = float(rng.choice([1.0, 3.0, 5.0]))
        parts = int(rng.integers(2, 6))
        out.append((i, B, T, H, dk, dv, torch.bfloat16 if bf else torch.float32, chunk, s0, mu, parts))
    return out


CASES = _cases()


def _pipe_shape(dk, dv, dtype, chunk):
    return dtype == torch.bfloat16 and dk in (64, 128) and dv % 32 == 0 and chunk in (32, 64)


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}-B{c[1]}T{c[2]}H{c[3]}d{c[4]}x{c[5]}"
                                             f"{'bf16' if c[6] == torch.bfloat16 else 'f32'}C{c[7]}" for c in CASES])
def test_random_shape(gpu, case):
    import gated_delta_rule_07_amd as kda
    i, B, T, H, dk, dv, dtype, chunk, s0, mu, parts = case
    bf = dtype == torch.bfloat16
    log(f"case {i}: B={B} T={T} H={H} d={dk}x{dv} {dtype} chunk={chunk} S0={s0} mu={mu}")
    x = ki.make_prefill(B, T, H, dk, dv, dtype, mu, 0.1 if s0 else 0.0, seed=1000 + i, device=gpu)
    S0 = x["S0"] if s0 else None
    ref = dict(x)
    ref["S0"] = S0
    ro, rs = oracle_prefill(ref)
    o, st = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0, chunk=chunk)
    torch.cuda.synchronize()
    assert_close(gpu_o_heads(o), ro, bf, f"case {i} o")
    assert_close(gpu_s_heads(st), rs, bf, f"case {i} S_T")
    if not _pipe_shape(dk, dv, dtype, chunk):
        return
    o2, st2 = kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0, parts=parts, chunk=chunk)
    torch.cuda.synchronize()
    assert_close(gpu_o_heads(o2), ro, bf, f"case {i} split({parts}) o")
    assert_close(gpu_s_heads(st2), rs, bf, f"case {i} split({parts}) S_T")
    z, A = ki.make_gate((B, T, H, dk), H, dtype, seed=2000 + i, device=gpu, z_mu=-4.5 + (3.0 - mu), z_std=0.6)
    og, sg = kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], z, A, x["beta"], S0, chunk=chunk)
    torch.cuda.synchronize()
    h = {n: t.cpu() for n, t in x.items()}
    rgo, rgs = oracle.forward(h["q"], h["k"], h["v"], oracle.gate_alpha(z.cpu(), A.cpu()), h["beta"],
                              h["S0"] if s0 else None)
    assert_close(gpu_o_heads(og), rgo, bf, f"case {i} gated o")
    assert_close(gpu_s_heads(sg), rgs, bf, f"case {i} gated S_T")
