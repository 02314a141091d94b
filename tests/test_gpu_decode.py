"""GPU parity of kda_decode_step (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_check import TOL_BF16_REL, TOL_F32_ABS, PerHeadSeqErr, abs_err, log, rel_err_per_head

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _run_steps(gpu, B, H, dk, dv, dtype, steps, seed=0, check_every=1):
    kda = _kda()
    S = ki.make_state(B, H, dk, dv, 0.1, seed + 1, gpu)
    S_ref = S.detach().cpu().double().numpy().copy()
    worst_o = 0.0
    per_head = PerHeadSeqErr()  # bf16: each head's error over its own outputs' RMS
    for step in range(steps):
        tok = ki.make_decode_token(B, H, dk, dv, dtype, 3.0, seed=seed, step=step, device=gpu)
        o = kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S)
        h = {k: v.cpu() for k, v in tok.items()}
        o_ref = oracle.decode_step(h["q"], h["k"], h["v"], h["alpha"], h["beta"], S_ref)
        if step % check_every == 0 or step == steps - 1:
            got = o.float().cpu().double().numpy().reshape(B * H, dv)
            ref = o_ref.reshape(B * H, dv)
            if dtype == torch.bfloat16:
                per_head.add(got, ref)
            else:
                worst_o = max(worst_o, abs_err(got, ref))
    if dtype == torch.bfloat16:
        worst_o = per_head.value()
    torch.cuda.synchronize()
    gs = S.cpu().double().numpy().reshape(B * H, dk, dv)
    rs = S_ref.reshape(B * H, dk, dv)
    if dtype == torch.bfloat16:
        es = rel_err_per_head(gs, rs)
        log(f"  o err {worst_o:.2e}  S err {es:.2e}")
        assert worst_o <= TOL_BF16_REL and es <= TOL_BF16_REL
    else:
        es = abs_err(gs, rs)
        log(f"  o err {worst_o:.2e}  S err {es:.2e}")
        assert worst_o <= TOL_F32_ABS and es <= TOL_F32_ABS


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
def test_decode_shapes(gpu, dtype, dk, dv):
    log(f"decode dk={dk} dv={dv} {dtype}")
    _run_steps(gpu, 3, 5, dk, dv, dtype, steps=6, seed=dk + dv)


def test_decode_many_steps(gpu):
    _run_steps(gpu, 4, 8, 128, 128, torch.bfloat16, steps=40, seed=3)


def test_decode_identity_step(gpu):
    """alpha = 1, beta = 0 leaves every state bit-exact."""
    kda = _kda()
    B, H, d = 8, 4, 128
    S = ki.make_state(B, H, d, d, 0.1, 0, gpu)
    S0 = S.clone()
    tok = ki.make_decode_token(B, H, d, d, torch.bfloat16, seed=1, device=gpu)
    tok["alpha"].fill_(1.0)
    tok["beta"].zero_()
    kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


def test_decode_deterministic(gpu):
    kda = _kda()
    B, H, d = 16, 8, 128
    S1 = ki.make_state(B, H, d, d, 0.1, 0, gpu)
    S2 = S1.clone()
    tok = ki.make_decode_token(B, H, d, d, torch.bfloat16, seed=2, device=gpu)
    o1 = kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S1)
    o2 = kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_decode_bf16_output_is_rounded_fp32_output(gpu):
    kda = _kda()
    B, H, d = 16, 8, 128
    S1 = ki.make_state(B, H, d, d, 0.1, 0, gpu)
    S2 = S1.clone()
    tok = ki.make_decode_token(B, H, d, d, torch.bfloat16, seed=4, device=gpu)
    o32 = kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S1)
    o16 = kda.kda_decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S2, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(S1, S2)
