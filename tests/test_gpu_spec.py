"""GPU checks of speculative decoding: kda_decode_verify then kda_decode_commit.

verify applies K draft tokens to the state without writing it: its outputs
must equal the oracle run over the K tokens from the same state (o), the state
in memory must be untouched (bit for bit), and each write vector u_t must equal
beta_t (v_t - (Diag(alpha_t) S_{t-1})^T k_t) with S_{t-1} the oracle's state
after t-1 drafts.  commit with j accepted drafts must leave the oracle's state
after j tokens (j = 0: untouched; out-of-range counts are clamped).  Tolerances
are the decode ones (fp32 arithmetic throughout): 1e-4 absolute for fp32
inputs, 2e-2 of the RMS for bf16.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_check import TOL_BF16_REL, TOL_F32_ABS, abs_err, log, rel_err_per_head, to_host

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


def _drafts(gpu, B, K, H, dk, dv, dtype, seed):
    d = ki.make_prefill(B, K, H, dk, dv, dtype, 3.0, 0.1, seed=seed, device=gpu)
    S = d.pop("S0")
    return d, S


def _oracle_after(d, S, t):
    """Oracle (o over the first t drafts, state after them), fp64, heads in (b, h) order."""
    h = {n: to_host(x[:, :t].contiguous()) for n, x in d.items()}
    return oracle.forward(h["q"], h["k"], h["v"], h["alpha"], h["beta"], to_host(S))


def _close(got, ref, bf, what):
    if bf:
        e = rel_err_per_head(got, ref)
        tol = TOL_BF16_REL
    else:
        e = abs_err(got, ref)
        tol = TOL_F32_ABS
    log(f"  {what}: {e:.3e} (tol {tol})")
    assert e <= tol, f"{what}: {e:.3e} > {tol}"


SHAPES = [(128, 128, torch.bfloat16), (64, 32, torch.bfloat16), (32, 32, torch.float32), (16, 128, torch.float32),
          (128, 16, torch.bfloat16)]


def _check_verify(d, S, B, H, K, dk, dv, dtype):
    kda = _kda()
    S_before = S.clone()
    o, u = kda.kda_decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S)
    torch.cuda.synchronize()
    assert torch.equal(S, S_before), "verify wrote the state"
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(u).all()), "verify produced a non-finite value"
    bf = dtype == torch.bfloat16
    ro, _ = _oracle_after(d, S, K)
    got_o = o.float().permute(0, 2, 1, 3).reshape(B * H, K, dv).cpu().double().numpy()
    _close(got_o, ro, bf, "o")
    # u_t from the oracle's state before token t
    hs = {n: to_host(x).double().numpy() for n, x in d.items()}
    prev = S.cpu().double().numpy().reshape(B * H, dk, dv)
    got_u = u.cpu().double().numpy().reshape(B * H, K, dv)
    ref_u = np.zeros_like(got_u)
    for t in range(K):
        if t > 0:
            _, st = _oracle_after(d, S, t)
            prev = st
        for bh in range(B * H):
            b, h = divmod(bh, H)
            a = hs["alpha"][b, t, h]
            x = (a[:, None] * prev[bh]).T @ hs["k"][b, t, h]
            ref_u[bh, t] = hs["beta"][b, t, h] * (hs["v"][b, t, h] - x)
    _close(got_u, ref_u, bf, "u")


@pytest.mark.parametrize("dk,dv,dtype", SHAPES)
@pytest.mark.parametrize("K", [1, 4, 16])
def test_verify_matches_oracle_and_leaves_state(gpu, dk, dv, dtype, K):
    B, H = 2, 3
    log(f"verify d={dk}x{dv} {dtype} K={K}")
    d, S = _drafts(gpu, B, K, H, dk, dv, dtype, seed=dk + dv + K)
    _check_verify(d, S, B, H, K, dk, dv, dtype)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (16, 128, torch.float32), (64, 32, torch.bfloat16)])
@pytest.mark.parametrize("B,H,K", [(1, 5, 3), (3, 1, 2)])
def test_verify_odd_state_count(gpu, dk, dv, dtype, B, H, K):
    """Up to four drafts a workgroup takes two states: an odd count of
    (sequence, head) states leaves the last workgroup one."""
    log(f"verify odd count B={B} H={H} d={dk}x{dv} {dtype} K={K}")
    d, S = _drafts(gpu, B, K, H, dk, dv, dtype, seed=dk + dv + 7 * K + B)
    _check_verify(d, S, B, H, K, dk, dv, dtype)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (32, 32, torch.float32)])
@pytest.mark.parametrize("K", [4, 8])
def test_verify_steep_decay(gpu, dk, dv, dtype, K):
    """Channels whose decay over the drafts leaves fp32's comfortable range:
    alpha = 0 (the channel is wiped), alpha = 1e-30, and alpha = 2^-20 on every
    draft (the running product passes 2^-64 at the fourth), beside ordinary
    channels; the kernel multiplies the state by keys and queries decayed to
    each draft's position, whose decay products reach zero or the subnormal
    range on these channels."""
    B, H = 2, 3
    log(f"verify steep decay d={dk}x{dv} {dtype} K={K}")
    d, S = _drafts(gpu, B, K, H, dk, dv, dtype, seed=dk + 5)
    a = d["alpha"].clone()
    a[:, 2, :, 0::7] = 0.0
    a[:, min(5, K - 1), :, 1::5] = 1e-30
    a[:, :, :, 3::4] = 2.0 ** -20
    a[1, :, 2, :] = 2.0 ** -20  # every channel of one head
    d["alpha"] = a.contiguous()
    _check_verify(d, S, B, H, K, dk, dv, dtype)


@pytest.mark.parametrize("dk,dv,dtype", SHAPES[:3])
def test_commit_accepted_prefix(gpu, dk, dv, dtype):
    """Sequences accept 0, 1, 2, K, more than K (clamped) and a negative count (clamped to 0)."""
    kda = _kda()
    K, H = 5, 2
    accept = [0, 1, 2, K, K + 3, -1]
    B = len(accept)
    log(f"commit d={dk}x{dv} {dtype} accept={accept}")
    d, S = _drafts(gpu, B, K, H, dk, dv, dtype, seed=11 + dk)
    S0 = S.clone()
    o, u = kda.kda_decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S)
    n = torch.tensor(accept, dtype=torch.int32, device=gpu)
    kda.kda_decode_commit(d["k"], d["alpha"], u, n, S)
    torch.cuda.synchronize()
    bf = dtype == torch.bfloat16
    for b, j in enumerate(accept):
        jj = min(max(j, 0), K)
        if jj == 0:
            assert torch.equal(S[b], S0[b]), f"sequence {b}: nothing accepted but the state changed"
            continue
        db = {n_: x[b:b + 1] for n_, x in d.items()}
        _, ref = _oracle_after(db, S0[b:b + 1], jj)
        _close(S[b:b + 1].cpu().double().numpy().reshape(H, dk, dv), ref, bf, f"S after {jj} accepted")


def test_verify_commit_equal_sequential_decode(gpu):
    """All K drafts accepted: o and the state agree with K kda_decode_step calls."""
    kda = _kda()
    B, K, H, dk, dv = 3, 6, 4, 128, 128
    d, S = _drafts(gpu, B, K, H, dk, dv, torch.bfloat16, seed=21)
    S_seq = S.clone()
    o, u = kda.kda_decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S)
    kda.kda_decode_commit(d["k"], d["alpha"], u, torch.full((B,), K, dtype=torch.int32, device=gpu), S)
    o_seq = []
    for t in range(K):
        o_seq.append(kda.kda_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                         d["v"][:, t].contiguous(), d["alpha"][:, t].contiguous(),
                                         d["beta"][:, t].contiguous(), S_seq))
    torch.cuda.synchronize()
    o_seq = torch.stack(o_seq, dim=1)
    eo = (o - o_seq).abs().max().item() / o_seq.pow(2).mean().sqrt().item()
    es = (S - S_seq).abs().max().item() / S_seq.pow(2).mean().sqrt().item()
    log(f"  vs sequential decode: o {eo:.2e}, S {es:.2e} (relative to RMS)")
    assert eo < 1e-5 and es < 1e-5


def test_spec_workload_shape(gpu):
    """B=256, H=32, d=128 with 4 drafts, acceptances 0..4: sampled states against the oracle."""
    kda = _kda()
    B, K, H, dk, dv = 256, 4, 32, 128, 128
    d, S = _drafts(gpu, B, K, H, dk, dv, torch.bfloat16, seed=31)
    S0 = S.clone()
    o, u = kda.kda_decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S)
    accept = torch.arange(B, dtype=torch.int32, device=gpu) % (K + 1)
    kda.kda_decode_commit(d["k"], d["alpha"], u, accept, S)
    torch.cuda.synchronize()
    for b in (1, 4, 130, 255):
        j = int(accept[b])
        db = {n_: x[b:b + 1] for n_, x in d.items()}
        ro, ref = _oracle_after(db, S0[b:b + 1], max(j, 1) if j else 1)
        if j == 0:
            assert torch.equal(S[b], S0[b])
        else:
            _close(S[b:b + 1].cpu().double().numpy().reshape(H, dk, dv), ref, True, f"seq {b} S after {j}")
        got_o = o[b:b + 1, :1].float().permute(0, 2, 1, 3).reshape(H, 1, dv).cpu().double().numpy()
        _close(got_o, ro[:, :1], True, f"seq {b} o_1")
