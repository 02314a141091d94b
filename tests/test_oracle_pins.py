"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

None of these re-types the oracle's own step order; each pins it against an
independent fact (a printed worked example, a closed form, an invariant, or a
separate matrix-product expansion of the update equation).  Every pin is also run
against the oracle with a deliberately planted mistake, and each mistake must be
caught by at least one pin.

Citations name the page and section:
  P1 = "Kimi K3 Technical Report review" (jw9603.github.io)
  P2 = "Kimi 모델 분석" (rlaope.github.io), KDA and chunkwise sections
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _unit(x):
    return x / np.linalg.norm(x)


def _run(mutation):
    """Oracle forward with an optional planted mistake; returns (o, S_T) with o
    as [B,T,H,dv] and S_T as [B,H,dk,dv] for convenience."""
    def run(q, k, v, a, b, S0=None, order="page1"):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        o, st = oracle.forward(q, k, v, a, b, S0, mutation=mutation, order=order, threads=2)
        o = o.reshape(B, H, T, dv).transpose(0, 2, 1, 3)
        st = st.reshape(B, H, dk, dv)
        return o, st
    return run


def _single(dk, dv, T, rng, unit_k=True, alpha=None, beta=None):
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    if unit_k:
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, dv))
    a = rng.uniform(0.3, 1.0, (1, T, 1, dk)) if alpha is None else alpha
    b = rng.uniform(0.1, 0.9, (1, T, 1)) if beta is None else beta
    S0 = rng.standard_normal((1, 1, dk, dv))
    return q, k, v, a, b, S0


# ---------------------------------------------------------------- pins


def pin_worked_example(run):
    """P1 section 3.4: prediction 0.2, value 0.8, beta 0.5 -> read-back 0.5;
    beta = 0 keeps 0.2 and beta = 1 gives 0.8."""
    g = _load("worked_example.json")
    dk, dv = 4, 2
    ok = True
    for beta, want in ((g["beta"], g["readback"]),
                       (0.0, g["extremes"]["beta_0_readback"]),
                       (1.0, g["extremes"]["beta_1_readback"])):
        k = np.zeros((1, 1, 1, dk)); k[..., 0] = 1.0          # normalised key e_0
        S0 = np.zeros((1, 1, dk, dv))
        S0[0, 0, 0, 0] = g["prediction"]                       # Sbar^T k = 0.2 (alpha = 1)
        S0[0, 0, 1:, :] = [[0.3, -0.7], [1.1, 0.4], [-0.2, 0.9]]  # other channels: not read by k
        S0[0, 0, 0, 1] = -0.6
        v = np.array([g["value"], 0.25]).reshape(1, 1, 1, dv)
        a = np.ones((1, 1, 1, dk))
        b = np.full((1, 1, 1), beta)
        o, _ = run(k.copy(), k, v, a, b, S0)                    # q = k reads S_t^T k
        ok &= abs(o[0, 0, 0, 0] - want) <= TOL
    return ok


def pin_diag_example(run):
    """P1 section 3.2: Diag(0.9, 0.5, 0.2) on the left keeps 90/50/20% of rows 1/2/3."""
    g = _load("diag_example.json")
    rng = np.random.default_rng(1)
    dk, dv = 3, 4
    S0 = rng.standard_normal((1, 1, dk, dv))
    a = np.array(g["alpha"]).reshape(1, 1, 1, dk)
    q = rng.standard_normal((1, 1, 1, dk))
    k = _unit(rng.standard_normal((1, 1, 1, dk)))
    v = rng.standard_normal((1, 1, 1, dv))
    b = np.zeros((1, 1, 1))
    o, st = run(q, k, v, a, b, S0)
    want = S0[0, 0] * np.array(g["kept_fraction_per_row"])[:, None]
    return np.abs(st[0, 0] - want).max() <= TOL and np.abs(o[0, 0, 0] - want.T @ q[0, 0, 0]).max() <= TOL


def pin_unit_key_closed_form(run):
    """P1 section 3.4: for a unit key, S_t^T k = (1 - beta) Sbar^T k + beta v."""
    rng = np.random.default_rng(2)
    ok = True
    for _ in range(5):
        q, k, v, a, b, S0 = _single(6, 5, 1, rng)
        o, _ = run(k.copy(), k, v, a, b, S0)
        sbar = a[0, 0, 0][:, None] * S0[0, 0]
        pred = sbar.T @ k[0, 0, 0]
        want = (1 - b[0, 0, 0]) * pred + b[0, 0, 0] * v[0, 0, 0]
        ok &= np.abs(o[0, 0, 0] - want).max() <= TOL
    return ok


def pin_beta_one_replaces(run):
    """P1 section 3.4 (beta = 1 replaces): with unit keys, S_t^T k_t = v_t at every step."""
    rng = np.random.default_rng(3)
    q, k, v, a, _, S0 = _single(8, 5, 20, rng)
    b = np.ones((1, 20, 1))
    o, _ = run(k.copy(), k, v, a, b, S0)
    return np.abs(o - v).max() <= 1e-12


def pin_identity(run):
    """P1 section 3.2 with alpha = 1, beta = 0: S is unchanged (bit-exact) and o_t = S0^T q_t."""
    rng = np.random.default_rng(4)
    T = 7
    q, k, v, _, _, S0 = _single(5, 3, T, rng)
    a = np.ones((1, T, 1, 5))
    b = np.zeros((1, T, 1))
    o, st = run(q, k, v, a, b, S0)
    ok = np.array_equal(st, S0)
    want = np.einsum("tk,kj->tj", q[0, :, 0], S0[0, 0])
    return ok and np.abs(o[0, :, 0] - want).max() <= TOL


def _brute(q, k, v, a, b, S0):
    """Dense transition matrices A_t = (I - b k k^T) Diag(a) (d_k x d_k), and
    S_t = (A_t ... A_1) S0 + sum_s (A_t ... A_{s+1}) b_s k_s v_s^T by explicit products."""
    T, dk = q.shape[1], q.shape[-1]
    A = []
    for t in range(T):
        kt = k[0, t, 0][:, None]
        A.append((np.eye(dk) - b[0, t, 0] * kt @ kt.T) @ np.diag(a[0, t, 0]))
    outs, S_t = [], None
    for t in range(T):
        # prod = A_t A_{t-1} ... A_0, built left to right
        prod = np.eye(dk)
        for s in range(t, -1, -1):
            prod = prod @ A[s]
        S_t = prod @ S0[0, 0]
        for s in range(t + 1):
            tail = np.eye(dk)
            for u in range(t, s, -1):
                tail = tail @ A[u]
            S_t = S_t + tail @ (b[0, s, 0] * np.outer(k[0, s, 0], v[0, s, 0]))
        outs.append(S_t.T @ q[0, t, 0])
    return np.array(outs), S_t


def pin_brute_force(run):
    """P1 section 3.2 update equation expanded into explicit matrix products, T <= 4,
    non-uniform alpha, beta in (0, 2), non-unit keys, square and non-square states."""
    rng = np.random.default_rng(5)
    ok = True
    for dk, dv in ((5, 3), (4, 4)):
        for T in (1, 2, 3, 4):
            q, k, v, a, b, S0 = _single(dk, dv, T, rng, unit_k=False,
                                        beta=rng.uniform(0.05, 1.95, (1, T, 1)))
            o, st = run(q, k, v, a, b, S0)
            ob, sb = _brute(q, k, v, a, b, S0)
            ok &= np.abs(o[0, :, 0] - ob).max() <= 1e-11 and np.abs(st[0, 0] - sb).max() <= 1e-11
    return ok


def pin_pure_decay(run):
    """beta = 0 over many tokens: S_T = Diag(prod_t alpha_t) S0 (per key channel)."""
    rng = np.random.default_rng(6)
    T = 200
    q, k, v, a, _, S0 = _single(6, 4, T, rng)
    a = rng.uniform(0.9, 1.0, (1, T, 1, 6))
    b = np.zeros((1, T, 1))
    _, st = run(q, k, v, a, b, S0)
    want = np.prod(a[0, :, 0], axis=0)[:, None] * S0[0, 0]
    return np.abs(st[0, 0] - want).max() <= 1e-12


def pin_gradient_step(run):
    """P2 (delta rule as optimisation): one step of gradient descent with rate beta on
    L(S) = 1/2 ||S^T k - v||^2, taken at Sbar; the gradient is obtained numerically."""
    rng = np.random.default_rng(7)
    dk, dv = 4, 3
    q, k, v, a, b, S0 = _single(dk, dv, 1, rng, unit_k=False)
    sbar = a[0, 0, 0][:, None] * S0[0, 0]
    kk, vv = k[0, 0, 0], v[0, 0, 0]

    def loss(S):
        r = S.T @ kk - vv
        return 0.5 * float(r @ r)

    grad = np.zeros_like(sbar)
    h = 1e-6
    for i in range(dk):
        for j in range(dv):
            e = np.zeros_like(sbar); e[i, j] = h
            grad[i, j] = (loss(sbar + e) - loss(sbar - e)) / (2 * h)
    want = sbar - b[0, 0, 0] * grad
    _, st = run(q, k, v, a, b, S0)
    return np.abs(st[0, 0] - want).max() <= 1e-8


def pin_householder(run):
    """P2 (reflection): alpha = 1, beta = 2, v = 0, unit k: I - 2kk^T preserves the
    Frobenius norm, and applying the same key twice returns the state."""
    rng = np.random.default_rng(8)
    dk, dv = 6, 5
    k1 = _unit(rng.standard_normal(dk))
    k = np.stack([k1, k1]).reshape(1, 2, 1, dk)
    q = rng.standard_normal((1, 2, 1, dk))
    v = np.zeros((1, 2, 1, dv))
    a = np.ones((1, 2, 1, dk))
    b = np.full((1, 2, 1), 2.0)
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, st1 = run(q[:, :1], k[:, :1], v[:, :1], a[:, :1], b[:, :1], S0)
    _, st2 = run(q, k, v, a, b, S0)
    n0, n1 = np.linalg.norm(S0), np.linalg.norm(st1)
    return abs(n0 - n1) <= 1e-12 * n0 and np.abs(st2 - S0).max() <= 1e-12


def pin_projection_contracts(run):
    """P2 (beta in [0,1] gives eigenvalues in [0,1]): with alpha = 1, v = 0 and unit
    keys, the state's norm never grows, and strictly shrinks when S^T k != 0."""
    rng = np.random.default_rng(9)
    T, dk, dv = 30, 5, 4
    q, k, _, _, b, S0 = _single(dk, dv, T, rng)
    v = np.zeros((1, T, 1, dv))
    a = np.ones((1, T, 1, dk))
    prev = np.linalg.norm(S0)
    ok = True
    for t in range(1, T + 1):
        _, st = run(q[:, :t], k[:, :t], v[:, :t], a[:, :t], b[:, :t], S0)
        cur = np.linalg.norm(st)
        ok &= cur <= prev * (1 + 1e-14) and cur < np.linalg.norm(S0)
        prev = cur
    return ok


def pin_orthonormal_memory(run):
    """P1 section 3.3 (store v at address k): alpha = 1, beta = 1, k_t = e_t: every
    value written is read back exactly at its own address afterwards."""
    rng = np.random.default_rng(10)
    dk, dv = 6, 3
    T = dk
    k = np.eye(dk).reshape(T, 1, 1, dk).transpose(1, 0, 2, 3)
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    a = np.ones((1, T, 1, dk))
    b = np.ones((1, T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, st = run(q, k, v, a, b, S0)
    return np.abs(st[0, 0] - v[0, :, 0]).max() <= 1e-12


def pin_p2_transposed_convention(run):
    """P2 writes the state as d_v x d_k (write S <- S + v k^T, read o = S q) with the
    transition Diag(alpha)(I - beta k k^T) acting from the right.  That recurrence,
    coded here in P2's own notation, must equal the oracle (P1's d_k x d_v state)."""
    rng = np.random.default_rng(11)
    T, dk, dv = 6, 5, 3
    q, k, v, a, b, S0 = _single(dk, dv, T, rng)
    Sp = S0[0, 0].T.copy()  # d_v x d_k
    outs = []
    for t in range(T):
        kt, at, bt = k[0, t, 0], a[0, t, 0], b[0, t, 0]
        Sp = Sp @ np.diag(at) @ (np.eye(dk) - bt * np.outer(kt, kt)) + bt * np.outer(v[0, t, 0], kt)
        outs.append(Sp @ q[0, t, 0])
    o, st = run(q, k, v, a, b, S0)
    return np.abs(o[0, :, 0] - np.array(outs)).max() <= 1e-12 and np.abs(st[0, 0] - Sp.T).max() <= 1e-12


PINS = [pin_worked_example, pin_diag_example, pin_unit_key_closed_form, pin_beta_one_replaces,
        pin_identity, pin_brute_force, pin_pure_decay, pin_gradient_step, pin_householder,
        pin_projection_contracts, pin_orthonormal_memory, pin_p2_transposed_convention]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    assert pin(_run(None))


def _caught(mutation):
    failed = []
    for pin in PINS:
        try:
            if not pin(_run(mutation)):
                failed.append(pin.__name__)
        except ValueError:
            failed.append(pin.__name__ + " (rejected)")
    return failed


@pytest.mark.parametrize("mutation", sorted(oracle.MUTATIONS))
def test_planted_mistake_is_caught(mutation):
    """Each plausible mistake (dropped decay, wrong sign, pre-update readout, decay on the
    wrong axis, undecayed prediction, dropped beta, readout with k) fails some pin."""
    assert _caught(mutation), f"mutation {mutation} passed every pin"


# ---------------------------------------------------------- order, layout, plumbing


def test_decay_write_order_matters_only_for_nonuniform_alpha():
    """The literal left-multiplied reading of P2's transition (write, then decay) is a
    different operator unless alpha is uniform across channels (the scalar-gate case)."""
    rng = np.random.default_rng(12)
    T, dk, dv = 12, 6, 4
    q, k, v, a, b, S0 = _single(dk, dv, T, rng)
    o1, s1 = oracle.forward(q, k, v, a, b, S0)
    o2, s2 = oracle.forward(q, k, v, a, b, S0, order="literal_p2")
    assert np.abs(o1 - o2).max() > 1e-3
    au = np.repeat(a[..., :1], dk, axis=-1)
    o1, s1 = oracle.forward(q, k, v, au, b, S0)
    o2, s2 = oracle.forward(q, k, v, au, b, S0, order="literal_p2")
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(s1 - s2).max() <= 1e-12


def test_threads_and_column_blocks_do_not_change_results():
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 2, 33, 3, 8, 12
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1, (B, T, H, dk)).astype(np.float32)
    b = rng.uniform(0, 1, (B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    ref = oracle.forward(q, k, v, a, b, S0, threads=1)
    for th, cb in ((4, 0), (3, 5), (8, 1)):
        got = oracle.forward(q, k, v, a, b, S0, threads=th, col_block=cb)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])
    sel = [5, 0, 3]
    got = oracle.forward(q, k, v, a, b, S0, heads=sel)
    assert np.array_equal(ref[0][sel], got[0]) and np.array_equal(ref[1][sel], got[1])


def test_bf16_inputs_widen_exactly():
    """Raw bf16 bit patterns are widened exactly: same result as the same values in fp64."""
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(0)
    B, T, H, dk, dv = 1, 9, 2, 8, 8
    q, k, v = (torch.randn(B, T, H, d, generator=g).to(torch.bfloat16) for d in (dk, dk, dv))
    a = torch.rand(B, T, H, dk, generator=g)
    b = torch.rand(B, T, H, generator=g)
    r1 = oracle.forward(q, k, v, a, b)
    r2 = oracle.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), a, b)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_decode_step_is_one_forward_token():
    rng = np.random.default_rng(14)
    B, H, dk, dv = 3, 2, 8, 4
    q = rng.standard_normal((B, H, dk))
    k = rng.standard_normal((B, H, dk))
    v = rng.standard_normal((B, H, dv))
    a = rng.uniform(0.5, 1, (B, H, dk))
    b = rng.uniform(0, 1, (B, H))
    S = rng.standard_normal((B, H, dk, dv))
    o_f, s_f = oracle.forward(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None], S)
    S2 = S.copy()
    o_d = oracle.decode_step(q, k, v, a, b, S2)
    assert np.array_equal(o_d.reshape(B * H, dv), o_f[:, 0]) and np.array_equal(S2.reshape(B * H, dk, dv), s_f)


def test_split_sequence_equals_one_call():
    """S0 -> S_T makes the recurrence resumable: [0, T1) then [T1, T) equals one call."""
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 1, 40, 2, 6, 5
    q = rng.standard_normal((B, T, H, dk)); k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv)); a = rng.uniform(0.5, 1, (B, T, H, dk))
    b = rng.uniform(0, 1, (B, T, H)); S0 = rng.standard_normal((B, H, dk, dv))
    o, st = oracle.forward(q, k, v, a, b, S0)
    T1 = 17
    o1, s1 = oracle.forward(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1], b[:, :T1], S0)
    o2, s2 = oracle.forward(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:], b[:, T1:], s1.reshape(B, H, dk, dv))
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(s2, st)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(16)
    S0 = rng.standard_normal((1, 2, 4, 4))
    z = np.zeros((1, 0, 2, 4))
    o, st = oracle.forward(z, z, z, z, np.zeros((1, 0, 2)), S0)
    assert o.shape == (2, 0, 4) and np.array_equal(st, S0.reshape(2, 4, 4))


# ---- the fused gate (lower-bounded decay of P1 section 3.5) ----
# Pinned by properties, not by restating the formula: each catches a different
# plausible slip (the sign of z, the -5 factor, a missing sigmoid, the e^A scale).

def test_gate_at_zero_is_half_the_bound_for_any_scale():
    z = np.zeros((1, 3, 4, 8))
    for A in (np.zeros(4), np.array([-3.0, 0.0, 1.5, 4.0])):
        assert np.allclose(oracle.gate_alpha(z, A), np.exp(-2.5), rtol=0, atol=1e-15)


def test_gate_sigmoid_symmetry_sums_to_the_bound():
    rng = np.random.default_rng(30)
    z = rng.standard_normal((2, 5, 3, 16)) * 3
    A = rng.standard_normal(3)
    s = np.log(oracle.gate_alpha(z, A)) + np.log(oracle.gate_alpha(-z, A))
    assert np.allclose(s, -5.0, rtol=0, atol=1e-12)


def test_gate_scale_is_exp_A():
    rng = np.random.default_rng(31)
    z = rng.standard_normal((1, 4, 3, 8))
    A = np.array([0.7, -1.2, 2.0])
    scaled = z * np.exp(A)[:, None]
    assert np.allclose(oracle.gate_alpha(z, A), oracle.gate_alpha(scaled, np.zeros(3)), rtol=1e-14, atol=0)


def test_gate_range_and_monotonicity():
    z = np.linspace(-40, 40, 801).reshape(1, 801, 1, 1)
    a = oracle.gate_alpha(z, np.zeros(1)).ravel()
    assert np.all(a > np.exp(-5) - 1e-15) and np.all(a <= 1.0)
    assert np.all(np.diff(a) <= 0)                          # more gate input, faster forgetting
    assert abs(a[0] - 1.0) < 1e-12 and abs(a[-1] - np.exp(-5)) < 1e-12


def test_gate_widens_bf16_exactly():
    torch = pytest.importorskip("torch")
    zt = torch.randn(1, 3, 2, 8).to(torch.bfloat16)
    A = np.array([0.3, -0.4])
    assert np.array_equal(oracle.gate_alpha(zt, A), oracle.gate_alpha(zt.double().numpy(), A))
