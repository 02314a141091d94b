"""CPU checks (oracle only) of the algebra behind the split prefill.

One token of the recurrence (section 3.3 of the "Kimi K3 Technical Report
review") maps the state S to (I - beta k k^T) Diag(alpha) S + beta k v^T, the
same d_k x d_k matrix on every state column, so a run of tokens maps its
incoming state to M S + N.  Running the oracle from a zero state over the value
columns and, with v = 0, over d_k extra columns that start as the identity
gives N and M; chaining S_in(j+1) = M_j S_in(j) + N_j and rerunning each part
from S_in(j) must reproduce the single run (o and S_T) to fp64 rounding.  This
is the decomposition the GPU path computes; here it is checked against the
oracle's own single pass, for arbitrary cut points.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = 1.0 / (1.0 + np.exp(-(3.0 + rng.standard_normal((B, T, H, dk)))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, alpha, beta, S0


def _split_run(q, k, v, alpha, beta, S0, cuts):
    """The two-level scan over parts [cuts[j], cuts[j+1]) in fp64 with the oracle."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bounds = [0] + list(cuts) + [T]
    parts = list(zip(bounds[:-1], bounds[1:]))
    trans = []
    for lo, hi in parts[:-1]:
        vaug = np.concatenate([v[:, lo:hi], np.zeros((B, hi - lo, H, dk))], axis=-1)
        s_aug = np.zeros((B, H, dk, dv + dk))
        s_aug[..., dv:] = np.eye(dk)
        _, st = oracle.forward(q[:, lo:hi], k[:, lo:hi], vaug, alpha[:, lo:hi], beta[:, lo:hi], s_aug,
                               want_o=False)
        st = st.reshape(B, H, dk, dv + dk)
        trans.append((st[..., dv:], st[..., :dv]))  # (M, N)
    s_in = [S0]
    for M, N in trans:
        s_in.append(np.einsum("bhij,bhjc->bhic", M, s_in[-1]) + N)
    outs = []
    st = None
    for (lo, hi), s in zip(parts, s_in):
        o, st = oracle.forward(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], alpha[:, lo:hi], beta[:, lo:hi], s)
        outs.append(o)
    return np.concatenate(outs, axis=1), st


@pytest.mark.parametrize("cuts", [[40], [32, 64], [7, 50, 51, 90], [1, 2, 3]])
def test_two_level_scan_reproduces_the_single_pass(cuts):
    rng = np.random.default_rng(len(cuts) * 11 + cuts[0])
    B, T, H, dk, dv = 2, 96, 2, 8, 4
    x = _inputs(rng, B, T, H, dk, dv)
    ro, rs = oracle.forward(*x)
    so, ss = _split_run(*x, cuts)
    assert np.abs(so - ro).max() < 1e-12 * max(1.0, np.abs(ro).max())
    assert np.abs(ss - rs).max() < 1e-12 * max(1.0, np.abs(rs).max())


def _part_maps(q, k, v, alpha, beta, cuts):
    """(M_j, N_j) of every part but the last, from the oracle."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bounds = [0] + list(cuts) + [T]
    maps = []
    for lo, hi in list(zip(bounds[:-1], bounds[1:]))[:-1]:
        vaug = np.concatenate([v[:, lo:hi], np.zeros((B, hi - lo, H, dk))], axis=-1)
        s_aug = np.zeros((B, H, dk, dv + dk))
        s_aug[..., dv:] = np.eye(dk)
        _, st = oracle.forward(q[:, lo:hi], k[:, lo:hi], vaug, alpha[:, lo:hi], beta[:, lo:hi], s_aug,
                               want_o=False)
        st = st.reshape(B, H, dk, dv + dk)
        maps.append((st[..., dv:], st[..., :dv]))
    return maps


@pytest.mark.parametrize("nparts", [2, 3, 9, 10, 17, 33])
def test_tree_of_part_maps_equals_the_chain(nparts):
    """The tree the GPU path takes from 9 parts on: an inclusive scan over the
    part maps with (M_a, N_a) o (M_b, N_b) = (M_a M_b, M_a N_b + N_a), in levels
    d = 1, 2, 4, ... where part j >= d is composed with part j - d of the
    previous level, then S_in(j + 1) = M*_j S0 + N*_j.  It must give the chain's
    incoming states to fp64 rounding (associativity), for part counts around
    the powers of two."""
    rng = np.random.default_rng(nparts)
    B, H, dk, dv = 1, 2, 6, 3
    T = 3 * nparts
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    maps = _part_maps(q, k, v, alpha, beta, [3 * j for j in range(1, nparts)])
    chain = [S0]
    for M, N in maps:
        chain.append(np.einsum("bhij,bhjc->bhic", M, chain[-1]) + N)
    cur = list(maps)
    d = 1
    while d < len(cur):
        nxt = list(cur)
        for j in range(d, len(cur)):
            (Ma, Na), (Mb, Nb) = cur[j], cur[j - d]
            nxt[j] = (np.einsum("bhij,bhjk->bhik", Ma, Mb), np.einsum("bhij,bhjc->bhic", Ma, Nb) + Na)
        cur = nxt
        d *= 2
    tree = [S0] + [np.einsum("bhij,bhjc->bhic", M, S0) + N for M, N in cur]
    for j, (a, b) in enumerate(zip(tree, chain)):
        assert np.abs(a - b).max() < 1e-12 * max(1.0, np.abs(b).max()), f"S_in({j})"


def test_transition_is_the_product_of_token_maps():
    """M over a few tokens equals the product of the dense per-token matrices
    (I - beta k k^T) Diag(alpha), built independently here."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 5, 1, 6, 3
    q, k, v, alpha, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    s_aug = np.zeros((B, H, dk, dv + dk))
    s_aug[..., dv:] = np.eye(dk)
    vaug = np.concatenate([v, np.zeros((B, T, H, dk))], axis=-1)
    _, st = oracle.forward(q, k, vaug, alpha, beta, s_aug, want_o=False)
    M = st.reshape(dk, dv + dk)[:, dv:]
    ref = np.eye(dk)
    for t in range(T):
        kt = k[0, t, 0]
        ref = (np.eye(dk) - beta[0, t, 0] * np.outer(kt, kt)) @ np.diag(alpha[0, t, 0]) @ ref
    assert np.abs(M - ref).max() < 1e-13
