"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: a hand-worked example, a closed
form of a special case, a textbook reduction or an invariant of the recurrence
the OneLA review (evolve.pub) describes in "Key claims" and "Scope & Claims"
(paper Eq. 2-4). Shapes use d_v != d_k where orientation could hide a mistake.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ancestry_walk, full_state_episode, fused_inputs, prompt_state, replay_episode, unit_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _frac_array(x):
    return np.vectorize(lambda s: float(Fraction(s)), otypes=[np.float64])(np.array(x, dtype=object))


def _random_case(rng, T=4, W=5, dk=3, dv=4, parents="uniform"):
    S0 = rng.normal(0, 0.5, (dv, dk))
    q = rng.normal(size=(T, W, dk))
    k = rng.normal(size=(T, W, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(T, W, dv))
    alpha = 1 / (1 + np.exp(-rng.normal(2, 0.5, (T, W))))
    beta = 1 / (1 + np.exp(-rng.normal(0, 1, (T, W))))
    par = np.full((T, W), -1)
    for t in range(1, T):
        par[t] = rng.integers(0, W, W)
    return S0, q, k, v, alpha, beta, par


# --------------------------------------------------------- hand-worked cases
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked(case):
    S0 = _frac_array(case["S0"])
    q, k, v = (_frac_array(case[n]) for n in ("q", "k", "v"))
    alpha, beta = _frac_array(case["alpha"]), _frac_array(case["beta"])
    par = np.array(case["parents"])
    out = full_state_episode(S0, q, k, v, alpha, beta, par)
    np.testing.assert_allclose(out["o"], _frac_array(case["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["delta"], _frac_array(case["delta"]), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(out["rec_alpha"], _frac_array(case["rec_alpha"]))
    for t, table in enumerate(case["anc"]):
        assert out["anc"][t].tolist() == table
    rep = replay_episode(S0, q, k, v, alpha, beta, par)
    np.testing.assert_allclose(rep["o"], _frac_array(case["o"]), rtol=0, atol=1e-15)


# ------------------------------------------------------------- closed forms
def test_identity_alpha1_beta0():
    """alpha = 1, beta = 0: delta = 0, the state never changes, o = S0 q on any path."""
    rng = np.random.default_rng(1)
    S0, q, k, v, _, _, par = _random_case(rng, T=4, W=6, dk=5, dv=3)
    ones, zeros = np.ones((4, 6)), np.zeros((4, 6))
    out = full_state_episode(S0, q, k, v, ones, zeros, par)
    assert np.all(out["delta"] == 0.0)
    expect = np.einsum("ij,twj->twi", S0, q)
    np.testing.assert_allclose(out["o"], expect, rtol=1e-14, atol=1e-15)


def test_pure_decay_follows_parent_path():
    """beta = 0: S_t = (product of alpha along the beam's path) * S0."""
    rng = np.random.default_rng(2)
    T, W = 5, 7
    S0, q, k, v, alpha, _, par = _random_case(rng, T=T, W=W, dk=4, dv=6)
    out = full_state_episode(S0, q, k, v, alpha, np.zeros((T, W)), par)
    for t in range(1, T + 1):
        for b in range(W):
            prod, cur = alpha[t - 1, b], b
            for s in range(t, 1, -1):
                cur = par[s - 1, cur]
                prod *= alpha[s - 2, cur]
            np.testing.assert_allclose(out["o"][t - 1, b], prod * (S0 @ q[t - 1, b]), rtol=1e-13)


def test_delta_rule_product_form():
    """S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T, the usual GDN delta-rule form."""
    rng = np.random.default_rng(3)
    T, W, dk, dv = 4, 5, 6, 3
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=dk, dv=dv)
    out = full_state_episode(S0, q, k, v, alpha, beta, par, return_states=True)
    for t in range(1, T + 1):
        for b in range(W):
            prev = S0 if t == 1 else out["states"][t - 2, par[t - 1, b]]
            kk = k[t - 1, b][:, None]
            expect = (alpha[t - 1, b] * prev @ (np.eye(dk) - beta[t - 1, b] * kk @ kk.T)
                      + beta[t - 1, b] * v[t - 1, b][:, None] @ kk.T)
            np.testing.assert_allclose(out["states"][t - 1, b], expect, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(out["o"][t - 1, b], expect @ q[t - 1, b], rtol=1e-12, atol=1e-14)


def test_write_back_unit_key():
    """beta = 1 and an exactly unit key: the new state maps k_t to v_t (so q = k gives o = v)."""
    rng = np.random.default_rng(4)
    T, W, dk, dv = 4, 6, 4, 5
    S0, _, _, v, alpha, _, par = _random_case(rng, T=T, W=W, dk=dk, dv=dv)
    signs = rng.choice([-0.5, 0.5], size=(T, W, dk))   # entries +-1/2 in 4 dims: norm exactly 1
    out = full_state_episode(S0, signs, signs, v, alpha, np.ones((T, W)), par)
    np.testing.assert_allclose(out["o"], v, rtol=0, atol=1e-14)


def test_general_key_projection_closed_form():
    """S_t k_t = alpha (1 - beta k.k) S_{t-1} k_t + beta (k.k) v_t for any key."""
    rng = np.random.default_rng(5)
    T, W, dk, dv = 3, 4, 5, 2
    S0, _, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=dk, dv=dv)
    k = k * rng.uniform(0.5, 2.0, (T, W, 1))       # not unit any more
    out = full_state_episode(S0, k, k, v, alpha, beta, par, return_states=True)
    for t in range(1, T + 1):
        for b in range(W):
            prev = S0 if t == 1 else out["states"][t - 2, par[t - 1, b]]
            kt = k[t - 1, b]
            kk = kt @ kt
            expect = alpha[t - 1, b] * (1 - beta[t - 1, b] * kk) * (prev @ kt) + beta[t - 1, b] * kk * v[t - 1, b]
            np.testing.assert_allclose(out["o"][t - 1, b], expect, rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_give_outer_product_memory():
    """alpha = beta = 1, S0 = 0, orthonormal keys: S_t = sum_s v_s k_s^T (exact recall)."""
    rng = np.random.default_rng(6)
    T, dk, dv = 4, 5, 3
    keys = np.eye(dk)[rng.permutation(dk)[:T]]                # (T, dk)
    k = keys[:, None, :]
    q = rng.normal(size=(T, 1, dk))
    v = rng.normal(size=(T, 1, dv))
    par = np.full((T, 1), -1)
    par[1:] = 0
    out = full_state_episode(np.zeros((dv, dk)), q, k, v, np.ones((T, 1)), np.ones((T, 1)), par)
    for t in range(T):
        memory = sum(np.outer(v[s, 0], keys[s]) for s in range(t + 1))
        np.testing.assert_allclose(out["o"][t, 0], memory @ q[t, 0], rtol=1e-14, atol=1e-15)
    S = prompt_state(k, v, np.ones((T, 1)), np.ones((T, 1)))
    np.testing.assert_allclose(S[0], sum(np.outer(v[s, 0], keys[s]) for s in range(T)), atol=1e-15)


def test_prompt_state_matches_single_beam_chain():
    """A W = 1 decode chain and the prompt fold run the same recurrence."""
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 4, 3
    S0, q, k, v, alpha, beta, _ = _random_case(rng, T=T, W=1, dk=dk, dv=dv)
    par = np.zeros((T, 1), dtype=int)
    par[0] = -1
    out = full_state_episode(S0, q, k, v, alpha, beta, par, return_states=True)
    S = prompt_state(k, v, alpha, beta, S_init=S0[None])
    np.testing.assert_allclose(S[0], out["states"][-1, 0], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------- invariants
def test_affine_in_s0():
    rng = np.random.default_rng(8)
    S0a, q, k, v, alpha, beta, par = _random_case(rng, T=4, W=5, dk=3, dv=4)
    S0b = rng.normal(size=S0a.shape)
    f = lambda S: full_state_episode(S, q, k, v, alpha, beta, par)
    fa, fb, fab, f0 = f(S0a), f(S0b), f(S0a + S0b), f(np.zeros_like(S0a))
    for key in ("o", "delta"):
        np.testing.assert_allclose(fab[key] + f0[key], fa[key] + fb[key], rtol=1e-12, atol=1e-13)


def test_beam_relabelling_permutes_outputs():
    rng = np.random.default_rng(9)
    T, W = 4, 6
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=3, dv=5)
    perms = [rng.permutation(W) for _ in range(T)]       # new beam b is old beam perm[t][b]
    inv = [np.argsort(p) for p in perms]
    qp = np.stack([q[t][perms[t]] for t in range(T)])
    kp = np.stack([k[t][perms[t]] for t in range(T)])
    vp = np.stack([v[t][perms[t]] for t in range(T)])
    ap = np.stack([alpha[t][perms[t]] for t in range(T)])
    bp = np.stack([beta[t][perms[t]] for t in range(T)])
    pp = par.copy()
    for t in range(1, T):
        pp[t] = inv[t - 1][par[t][perms[t]]]
    a = full_state_episode(S0, q, k, v, alpha, beta, par)
    b = full_state_episode(S0, qp, kp, vp, ap, bp, pp)
    for t in range(T):
        np.testing.assert_allclose(b["o"][t], a["o"][t][perms[t]], rtol=1e-13, atol=1e-15)


# ------------------------------------------- projection replay and ancestry
@pytest.mark.parametrize("seed,T,W,dk,dv", [(10, 4, 6, 5, 3), (11, 6, 3, 2, 7), (12, 3, 9, 8, 8)])
def test_replay_equals_full_state(seed, T, W, dk, dv):
    rng = np.random.default_rng(seed)
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=dk, dv=dv)
    full = full_state_episode(S0, q, k, v, alpha, beta, par)
    rep = replay_episode(S0, q, k, v, alpha, beta, par)
    np.testing.assert_allclose(rep["o"], full["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(rep["delta"], full["delta"], rtol=0, atol=1e-12)


def test_ancestry_matches_parent_walk():
    rng = np.random.default_rng(13)
    T, W = 6, 7
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=2, dv=2)
    out = full_state_episode(S0, q, k, v, alpha, beta, par)
    for t in range(1, T + 1):
        walk = ancestry_walk(par, t, W)
        np.testing.assert_array_equal(out["anc"][t - 1], walk)
        assert walk.shape == (W, t - 1)
        if t > 1:
            # the record at depth j (0-based) was written at step j+1
            for j in range(t - 1):
                assert np.all(walk[:, j] // W == j)
            assert walk.max() < (t - 1) * W


def test_records_are_parent_independent_copies():
    """alpha and k of record rid(t, b) are exactly beam b's step-t inputs."""
    rng = np.random.default_rng(14)
    T, W = 3, 4
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=T, W=W, dk=3, dv=2)
    out = full_state_episode(S0, q, k, v, alpha, beta, par)
    np.testing.assert_array_equal(out["rec_alpha"].reshape(T, W), alpha)
    np.testing.assert_array_equal(out["rec_k"].reshape(T, W, 3), k)
    np.testing.assert_array_equal(out["rec_delta"].reshape(T, W, 2), out["delta"])


def test_out_of_range_parent_rejected():
    rng = np.random.default_rng(15)
    S0, q, k, v, alpha, beta, par = _random_case(rng, T=2, W=3, dk=2, dv=2)
    par[1, 0] = 3
    with pytest.raises(ValueError):
        full_state_episode(S0, q, k, v, alpha, beta, par)


# ------------------------------------------------------ input-side fusion
def test_fused_gates_closed_forms():
    """alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b) at
    points where they have exact values: softplus(0) = ln 2 gives
    alpha = 2^-exp(A_log); a very negative argument leaves no decay; a large
    one decays by exp(-A (a + dt_bias)); sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4."""
    H = 4
    A_log = np.array([0.0, np.log(3.0), np.log(0.5), 0.0])
    dt_bias = np.array([-2.0, 1.5, 0.25, -3.0])
    a_raw = np.array([[2.0, -1.5, -0.25, -60.0]])      # a + dt_bias = 0, 0, 0, -63
    b_raw = np.array([[0.0, np.log(3.0), -np.log(3.0), 0.0]])
    _, _, alpha, beta = fused_inputs(np.ones((1, H, 8)), np.ones((1, H, 8)), a_raw, b_raw, A_log, dt_bias)
    np.testing.assert_allclose(alpha[0, :3], [0.5, 0.125, 2 ** -0.5], rtol=1e-15)
    assert abs(alpha[0, 3] - 1.0) < 1e-20
    np.testing.assert_allclose(beta[0], [0.5, 0.75, 0.25, 0.5], rtol=1e-15)
    _, _, alpha, _ = fused_inputs(np.ones((1, 1, 8)), np.ones((1, 1, 8)), np.array([[30.0]]), np.zeros((1, 1)),
                                  np.array([np.log(2.0)]), np.array([0.5]))
    np.testing.assert_allclose(alpha[0, 0], np.exp(-2.0 * 30.5), rtol=1e-14)


def test_fused_normalisation():
    """Per-head L2 normalisation rounded to bf16: (3, 4, 0, ...) becomes the
    bf16 neighbours of (0.6, 0.8); power-of-two scaling of the raw vector
    changes nothing (eps = 0); every normalised vector has unit length to
    within bf16 rounding; heads are normalised independently."""
    x = np.zeros((1, 2, 32))
    x[0, 0, :2] = [3.0, 4.0]
    x[0, 1, 5] = -7.0
    q, _, _, _ = fused_inputs(x, x, np.zeros((1, 2)), np.zeros((1, 2)), np.zeros(2), np.zeros(2))
    assert q[0, 0, 0] == np.float32(0.6015625) and q[0, 0, 1] == np.float32(0.80078125)
    assert np.count_nonzero(q[0, 0]) == 2 and q[0, 1, 5] == -1.0 and np.count_nonzero(q[0, 1]) == 1
    rng = np.random.default_rng(5)
    raw = rng.standard_normal((50, 3, 64)).astype(np.float32)
    base, k1, _, _ = fused_inputs(raw, raw, np.zeros((50, 3)), np.zeros((50, 3)), np.zeros(3), np.zeros(3), eps=0.0)
    for scale in (2.0 ** -7, 2.0 ** 9):
        scaled, _, _, _ = fused_inputs(raw * np.float32(scale), raw, np.zeros((50, 3)), np.zeros((50, 3)),
                                       np.zeros(3), np.zeros(3), eps=0.0)
        assert np.array_equal(scaled, base)
    norms = np.linalg.norm(base.astype(np.float64), axis=-1)
    assert np.all(np.abs(norms - 1.0) <= 2.0 ** -8)
    assert np.array_equal(base, k1)


def test_unit_rows_definition():
    """The float64 normalisation: (3, 4) -> (0.6, 0.8); unit length for
    eps = 0; invariant under positive scaling (eps = 0); eps enters under the
    square root: (3, 4) with eps = 11 has norm 5 / 6."""
    x = np.array([[3.0, 4.0, 0.0]])
    np.testing.assert_allclose(unit_rows(x, eps=0.0), [[0.6, 0.8, 0.0]], rtol=0, atol=1e-16)
    np.testing.assert_allclose(unit_rows(x, eps=11.0), [[0.5, 2.0 / 3.0, 0.0]], rtol=1e-15)
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((40, 3, 64))
    u = unit_rows(raw, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(unit_rows(raw * 37.5, eps=0.0), u, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d,eps", [(32, 1e-6), (64, 0.0), (128, 1e-6)])
def test_fused_normalisation_against_float64(d, eps):
    """fused_inputs takes the bf16 rounding of the normalised q and k in
    float32 (the step's precision); against the float64 definition every
    element is one of the two bf16 values that bracket the exact value, and
    it is the exact value's nearest one wherever that is farther from their
    midpoint than the derived float32 error bound (tests/bf16_bounds.py)."""
    from bf16_bounds import check_rounded, fp32_unit_rel_bound
    from workload import bf16_bits_to_f32

    rng = np.random.default_rng(d)
    bits = (rng.standard_normal((300, 4, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raw = bf16_bits_to_f32(bits)                     # bf16-valued raw projections, as the step receives them
    q, k, _, _ = fused_inputs(raw, raw, np.zeros((300, 4)), np.zeros((300, 4)), np.zeros(4), np.zeros(4), eps=eps)
    u = unit_rows(raw, eps=eps)
    for x in (q, k):
        bracket, exact, n_band, n_diff = check_rounded(x, u, fp32_unit_rel_bound(d))
        assert bracket and exact, (n_band, n_diff)
        assert n_diff <= n_band
    # a mistake in the definition shows: without eps under the root, or with the
    # squares summed over the wrong axis, elements leave their bracket
    bad = raw / np.sqrt(np.sum(raw * raw, axis=-2, keepdims=True))
    assert not check_rounded(k, bad, fp32_unit_rel_bound(d))[0]
