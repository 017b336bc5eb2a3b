"""Pins that tie the fp64 oracle to the pages and to mathematics, not to itself.

Each pin_* function takes an oracle object (oracle.Oracle: the real build, or a build of a
deliberately broken copy of fwa_oracle.c) and raises AssertionError when the oracle violates
what the pages or the mathematics fix.  tests/test_oracle_pins.py runs every pin against the
real oracle; tests/test_oracle_mutants.py checks that every planted mistake fails at least one.

Sources: the Fast Weights Transformer guide (xdnf.cn/news/308600), sections "DPFP / projection
formula and hyper-parameters", "DPFP / normalisation", "FastWeightsAttention / update formula",
"FastWeightsAttention / module structure and source walkthrough", and "Background / fast
computation form of linear self-attention" (the sum-update form used in pin_disjoint_keys).
"""
import math
import os
from fractions import Fraction

import numpy as np

EPS = 1e-6
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- sign-pattern helpers

def _positive_positions(bits, d_k):
    """Cycle positions of relu([k, -k]) that are > 0 for the sign pattern `bits`
    (bit j set <=> k_j > 0; no k_j is zero)."""
    first = (bits[:, None] >> np.arange(d_k)[None, :]) & 1
    return np.concatenate([first, 1 - first], axis=1).astype(bool)


def _all_patterns(d_k):
    return np.arange(1 << d_k, dtype=np.int64)


def _keys_from_bits(bits, d_k, rng):
    """Vectors with the given sign patterns and magnitudes in [0.5, 2)."""
    mag = rng.uniform(0.5, 2.0, size=(len(bits), d_k))
    sign = np.where(((bits[:, None] >> np.arange(d_k)[None, :]) & 1) == 1, 1.0, -1.0)
    return sign * mag


def onehot_patterns(d_k=16):
    """All sign patterns whose shift-1 DPFP block has exactly one nonzero entry, grouped by
    the index m of that entry.  Entry j of the shift-1 block is nonzero exactly when cycle
    positions j and j-1 (mod 2*d_k) are both positive -- the roll by +1 of the pages' code."""
    bits = _all_patterns(d_k)
    pos = _positive_positions(bits, d_k)
    prev = np.concatenate([pos[:, -1:], pos[:, :-1]], axis=1)  # position j-1, cyclic
    both = pos & prev
    one = both.sum(axis=1) == 1
    m = np.argmax(both, axis=1)
    out = {}
    for b, mm in zip(bits[one], m[one]):
        out.setdefault(int(mm), []).append(int(b))
    return out


# ---------------------------------------------------------------- DPFP pins

def pin_dpfp_shape_nonneg_sum(O):
    """phi has 2*d_k*nu entries, all >= 0, summing to just below 1 (sum-normalised with an
    additive eps)."""
    rng = np.random.default_rng(11)
    for d_k, nu in [(16, 1), (16, 3), (64, 1), (64, 2), (64, 3), (8, 15), (32, 5)]:
        k = rng.standard_normal((257, d_k))
        phi = O.dpfp(k, nu)
        assert phi.shape == (257, 2 * d_k * nu), (d_k, nu, phi.shape)
        assert np.all(phi >= 0.0), (d_k, nu)
        s = phi.sum(axis=1)
        assert np.all(s < 1.0) and np.all(s > 1.0 - 1e-3), (d_k, nu, s.min(), s.max())


def pin_dpfp_eps_is_additive(O):
    """Scaling k by c scales every raw product by c^2, so with an additive eps
    (1/sum(phi(c k)) - 1) / (1/sum(phi(k)) - 1) = 1/c^2 exactly in exact arithmetic."""
    rng = np.random.default_rng(12)
    k = rng.standard_normal((64, 16))
    for c in (0.5, 0.1, 0.01):
        r_k = 1.0 / O.dpfp(k, 2).sum(axis=1) - 1.0
        r_ck = 1.0 / O.dpfp(c * k, 2).sum(axis=1) - 1.0
        np.testing.assert_allclose(r_ck / r_k, 1.0 / c ** 2, rtol=1e-6)


def pin_dpfp_onehot_roll_direction(O):
    """Sign pattern (+,+,-,+,-,+,...,+) at d_k = 16 leaves exactly one adjacent pair of
    positive cycle positions, (0, 1).  Under the roll by +i of the pages' code the surviving
    product sits at index 1 (it would sit at index 0 under the formula's literal x_j * x_{j+i});
    its value is p/(p+eps) with p = k_0 * k_1.  With nu = 2 the second block (offset 32) is
    x[j] * x[j-2]: for this pattern the positive positions j with j-2 (mod 32) positive are
    0 (paired with 30), 3, 5, ..., 15 and 20, 22, ..., 30."""
    d_k = 16
    signs = np.array([1, 1] + [(-1 if j % 2 == 0 else 1) for j in range(2, 16)], dtype=float)
    mag = np.linspace(0.7, 1.9, 16)
    k = signs * mag
    phi = O.dpfp(k[None], 1)[0]
    nz = np.flatnonzero(phi)
    assert list(nz) == [1], nz
    p = k[0] * k[1]
    assert math.isclose(phi[1], p / (p + EPS), rel_tol=1e-14), (phi[1], p / (p + EPS))
    eps_back = p * (1.0 / phi[1] - 1.0)
    assert math.isclose(eps_back, EPS, rel_tol=1e-6), eps_back
    phi2 = O.dpfp(k[None], 2)[0]
    expect2 = {1} | {32 + j for j in [0] + list(range(3, 16, 2)) + list(range(20, 31, 2))}
    assert set(np.flatnonzero(phi2)) == expect2, sorted(set(np.flatnonzero(phi2)) ^ expect2)


def pin_dpfp_hand_examples(O):
    """Worked examples derived by hand from the DPFP definition (tests/golden/dpfp_hand.txt)."""
    with open(os.path.join(GOLDEN, "dpfp_hand.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, k_s, raw_s, s_s = [x.strip() for x in line.split("|")]
            d_k, nu = (int(x) for x in head.split())
            k = np.array([float(x) for x in k_s.split()])
            raw = np.array([float(x) for x in raw_s.split()])
            S = float(s_s)
            assert len(k) == d_k and len(raw) == 2 * d_k * nu and raw.sum() == S
            phi = O.dpfp(k[None], nu)[0]
            np.testing.assert_allclose(phi, raw / (S + EPS), rtol=1e-14, atol=0)


def pin_dpfp_mask_sign_predicate(O):
    """For every sign pattern at d_k = 12 and nu = 1..3, the nonzero entries of phi are exactly
    the (i, j) whose cycle positions j and j-i are both positive, and dpfp_mask agrees."""
    d_k = 12
    rng = np.random.default_rng(13)
    bits = _all_patterns(d_k)
    k = _keys_from_bits(bits, d_k, rng)
    pos = _positive_positions(bits, d_k)
    for nu in (1, 2, 3):
        expect = np.concatenate(
            [pos & np.concatenate([pos[:, 2 * d_k - i:], pos[:, :2 * d_k - i]], axis=1)
             for i in range(1, nu + 1)], axis=1)
        got = O.dpfp(k, nu) != 0.0
        assert np.array_equal(got, expect), (nu, int((got != expect).sum()))
        assert np.array_equal(O.dpfp_mask(k, nu), expect), nu


def pin_dpfp_degenerate(O):
    """Shift d_k pairs x[j] with x[j - d_k], i.e. relu(k) with relu(-k) of the same entry, so
    its block is identically zero; d_k = 1 (only nu = 1 allowed) gives phi = 0; k = 0 and odd
    d_k with strictly alternating signs also give all-zero products, and phi = 0 / eps = 0."""
    rng = np.random.default_rng(14)
    k = rng.standard_normal((50, 4))
    phi = O.dpfp(k, 7)
    assert np.all(phi[:, 3 * 8:4 * 8] == 0.0)        # block of shift i = 4 = d_k
    assert np.all(O.dpfp(rng.standard_normal((10, 1)), 1) == 0.0)
    assert np.all(O.dpfp(np.zeros((3, 16)), 2) == 0.0)
    alt = np.array([[1.0, -2.0, 3.0]])                # cycle + - + | - + -: no adjacent pair
    assert np.all(O.dpfp(alt, 1) == 0.0)
    assert not np.any(np.isnan(O.dpfp(np.zeros((1, 5)), 4)))


def pin_dpfp_negation_rotates_blocks(O):
    """[-k, k] is [k, -k] rolled by d_k, so phi(-k) is phi(k) with every block rotated by d_k."""
    rng = np.random.default_rng(15)
    d_k, nu = 16, 3
    k = rng.standard_normal((40, d_k))
    a = O.dpfp(k, nu).reshape(40, nu, 2 * d_k)
    b = O.dpfp(-k, nu).reshape(40, nu, 2 * d_k)
    np.testing.assert_array_equal(b != 0.0, np.roll(a, d_k, axis=2) != 0.0)
    np.testing.assert_allclose(b, np.roll(a, d_k, axis=2), rtol=1e-14, atol=0)


# ---------------------------------------------------------------- sigmoid pins

def pin_sigmoid_values(O):
    assert O.sigmoid(0.0) == 0.5
    assert O.sigmoid(-math.inf) == 0.0 and O.sigmoid(math.inf) == 1.0
    assert math.isclose(O.sigmoid(math.log(3.0)), 0.75, rel_tol=1e-15)
    assert math.isclose(O.sigmoid(-math.log(3.0)), 0.25, rel_tol=1e-15)
    for x in (0.3, 2.0, 17.0, 700.0):
        assert math.isclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, rel_tol=1e-15)
    assert O.sigmoid(-745.0) > 0.0 or O.sigmoid(-745.0) == 0.0  # no overflow / NaN
    assert O.sigmoid(-800.0) == 0.0 and O.sigmoid(800.0) == 1.0


# ---------------------------------------------------------------- recurrence pins

def _rand_case(rng, B, H, T, d_k, d_v, nu, w0=True):
    q = rng.standard_normal((B, H, T, d_k))
    k = rng.standard_normal((B, H, T, d_k))
    v = rng.standard_normal((B, H, T, d_v))
    l = rng.standard_normal((B, H, T))
    W0 = 0.1 * rng.standard_normal((B, H, d_v, 2 * d_k * nu)) if w0 else None
    return q, k, v, l, W0


def pin_beta_zero_freezes_state(O):
    """beta = sigmoid(-inf) = 0 makes every write vanish: W_final = W0, y_t = W0 phi(q_t)."""
    rng = np.random.default_rng(21)
    q, k, v, l, W0 = _rand_case(rng, 2, 2, 9, 8, 5, 2)
    l[:] = -math.inf
    y, W = O.delta_forward(q, k, v, l, W0, nu=2)
    np.testing.assert_array_equal(W, W0)
    np.testing.assert_allclose(y, np.einsum("bhvd,bhtd->bhtv", W0, O.dpfp(q, 2)),
                               rtol=1e-13, atol=1e-15)


def pin_single_step_from_zero(O):
    """One step from W = 0: v_bar = 0, so W = beta v phi(k)^T and y = beta v (phi(k).phi(q))."""
    rng = np.random.default_rng(22)
    q, k, v, l, _ = _rand_case(rng, 1, 3, 1, 16, 7, 1, w0=False)
    y, W = O.delta_forward(q, k, v, l, None, nu=1)
    beta = 1.0 / (1.0 + np.exp(-l))
    fk, fq = O.dpfp(k, 1), O.dpfp(q, 1)
    W_exp = beta[:, :, 0, None, None] * v[:, :, 0, :, None] * fk[:, :, 0, None, :]
    np.testing.assert_allclose(W, W_exp, rtol=1e-13, atol=1e-16)
    y_exp = beta[:, :, 0, None] * v[:, :, 0] * np.sum(fk[:, :, 0] * fq[:, :, 0], axis=-1)[..., None]
    np.testing.assert_allclose(y[:, :, 0], y_exp, rtol=1e-12, atol=1e-16)


def pin_transition_matrix_form(O):
    """Tiny-T brute force through explicit D x D matrices:
    W_t = W_{t-1} (I - beta_t f_t f_t^T) + beta_t v_t f_t^T, y_t = W_t phi(q_t)."""
    rng = np.random.default_rng(23)
    q, k, v, l, W0 = _rand_case(rng, 1, 2, 6, 4, 3, 2)
    y, W = O.delta_forward(q, k, v, l, W0, nu=2)
    fk, fq = O.dpfp(k, 2), O.dpfp(q, 2)
    beta = 1.0 / (1.0 + np.exp(-l))
    D = fk.shape[-1]
    for h in range(2):
        Wt = W0[0, h].copy()
        for t in range(6):
            f = fk[0, h, t]
            Wt = Wt @ (np.eye(D) - beta[0, h, t] * np.outer(f, f)) + beta[0, h, t] * np.outer(v[0, h, t], f)
            np.testing.assert_allclose(y[0, h, t], Wt @ fq[0, h, t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(W[0, h], Wt, rtol=1e-12, atol=1e-14)


def pin_disjoint_keys_reduce_to_linear_attention(O):
    """Keys with pairwise disjoint DPFP supports and W = 0 at the start make every retrieval
    v_bar = 0, so the rule reduces to the pages' sum-update linear attention without the z
    normaliser: Y = tril_incl(phi(Q) phi(K)^T) diag(beta) V -- a masked matmul."""
    rng = np.random.default_rng(24)
    groups = onehot_patterns(16)
    ms = sorted(groups)[:12]
    T = len(ms)
    bits = np.array([groups[m][rng.integers(len(groups[m]))] for m in ms])
    k = _keys_from_bits(bits, 16, rng)[None, None]         # [1,1,T,16]
    q = rng.standard_normal((1, 1, T, 16))
    q[0, 0, 3] = k[0, 0, 1]                                 # a query that hits an earlier key
    v = rng.standard_normal((1, 1, T, 5))
    l = rng.standard_normal((1, 1, T))
    y, W = O.delta_forward(q, k, v, l, None, nu=1)
    fk, fq = O.dpfp(k, 1)[0, 0], O.dpfp(q, 1)[0, 0]
    assert np.count_nonzero(fk @ fk.T - np.diag(np.diag(fk @ fk.T))) == 0
    beta = 1.0 / (1.0 + np.exp(-l[0, 0]))
    Y = np.tril(fq @ fk.T) @ (beta[:, None] * v[0, 0])
    np.testing.assert_allclose(y[0, 0], Y, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(W[0, 0], (beta[:, None] * v[0, 0]).T @ fk, rtol=1e-12, atol=1e-15)


def pin_repeated_key_is_ema(O):
    """The same one-hot key f = c e_m at every step: column m of W follows
    w_t = (1 - beta_t c^2) w_{t-1} + beta_t c v_t and every other column keeps its W0 value."""
    rng = np.random.default_rng(25)
    groups = onehot_patterns(16)
    m = sorted(groups)[5]
    bits = np.array([groups[m][0]] * 20)
    k = _keys_from_bits(bits[:1], 16, rng).repeat(20, axis=0)[None, None]
    T = 20
    q = rng.standard_normal((1, 1, T, 16))
    v = rng.standard_normal((1, 1, T, 4))
    l = rng.standard_normal((1, 1, T)) + 1.0
    W0 = rng.standard_normal((1, 1, 4, 32))
    y, W = O.delta_forward(q, k, v, l, W0, nu=1)
    c = O.dpfp(k[0, 0, :1], 1)[0, m]
    beta = 1.0 / (1.0 + np.exp(-l[0, 0]))
    w = W0[0, 0, :, m].copy()
    for t in range(T):
        w = (1.0 - beta[t] * c * c) * w + beta[t] * c * v[0, 0, t]
    np.testing.assert_allclose(W[0, 0, :, m], w, rtol=1e-12, atol=1e-14)
    others = [d for d in range(32) if d != m]
    np.testing.assert_array_equal(W[0, 0][:, others], W0[0, 0][:, others])


def pin_hand_recurrence(O):
    """Two steps worked by hand (tests/golden/recurrence_hand.txt): d_k = 2, nu = 1, d_v = 1,
    k = q = [1, -2] both steps (phi = c e_0 with c = 2/(2+eps)), beta_logit = 0 (beta = 1/2),
    v = 1 then 3, W0 = 0.  Then y_1 = c^2/2, W_1 = c/2, y_2 = 2c^2 - c^4/4, W_2 = 2c - c^3/4."""
    with open(os.path.join(GOLDEN, "recurrence_hand.txt")) as f:
        rows = [ln.split("#", 1)[0].split(None, 1) for ln in f]
    rows = [r for r in rows if r]
    c = Fraction(2) / (Fraction(2) + Fraction(1, 10 ** 6))
    env = {"c": c}
    k = np.array([[[[1.0, -2.0], [1.0, -2.0]]]])
    y, W = O.delta_forward(k, k, np.array([[[[1.0], [3.0]]]]), np.zeros((1, 1, 2)), None, nu=1)
    got = {"y1": y[0, 0, 0, 0], "y2": y[0, 0, 1, 0], "W2_0": W[0, 0, 0, 0],
           "W2_1": W[0, 0, 0, 1], "W2_2": W[0, 0, 0, 2], "W2_3": W[0, 0, 0, 3]}
    for name, expr in rows:
        want = float(eval(expr, {"__builtins__": {}}, env))
        assert math.isclose(got[name], want, rel_tol=1e-14, abs_tol=0.0), (name, got[name], want)


def pin_linearity(O):
    """(y, W_final) is linear in (v, W0) jointly for fixed q, k, beta."""
    rng = np.random.default_rng(26)
    q, k, v1, l, A = _rand_case(rng, 2, 2, 17, 8, 6, 2)
    v2 = rng.standard_normal(v1.shape)
    Bm = 0.1 * rng.standard_normal(A.shape)
    y1, W1 = O.delta_forward(q, k, v1, l, A, nu=2)
    y2, W2 = O.delta_forward(q, k, v2, l, Bm, nu=2)
    y3, W3 = O.delta_forward(q, k, v1 - 2.5 * v2, l, A - 2.5 * Bm, nu=2)
    np.testing.assert_allclose(y3, y1 - 2.5 * y2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(W3, W1 - 2.5 * W2, rtol=1e-11, atol=1e-13)


def pin_contraction(O):
    """||phi||_2 <= ||phi||_1 < 1, so each step's transition I - beta f f^T has eigenvalues in
    [0, 1]: a perturbation of W0 never grows in Frobenius norm, and it shrinks over many steps."""
    rng = np.random.default_rng(27)
    q, k, v, l, W0 = _rand_case(rng, 1, 3, 200, 4, 3, 1)
    d = rng.standard_normal(W0.shape)
    _, Wa = O.delta_forward(q, k, v, l, W0, nu=1)
    _, Wb = O.delta_forward(q, k, v, l, W0 + d, nu=1)
    for h in range(3):
        n0 = np.linalg.norm(d[0, h])
        n1 = np.linalg.norm(Wb[0, h] - Wa[0, h])
        assert n1 <= n0 * (1 + 1e-12) and n1 < 0.9 * n0, (h, n0, n1)


def pin_segmentation_and_steps(O):
    """forward(T1) then forward(T2, W0 = W_final) equals forward(T1 + T2), and equals T
    successive single-token steps carrying W."""
    rng = np.random.default_rng(28)
    q, k, v, l, W0 = _rand_case(rng, 2, 3, 23, 8, 4, 2)
    y, W = O.delta_forward(q, k, v, l, W0, nu=2)
    ya, Wa = O.delta_forward(q[:, :, :10], k[:, :, :10], v[:, :, :10], l[:, :, :10], W0, nu=2)
    yb, Wb = O.delta_forward(q[:, :, 10:], k[:, :, 10:], v[:, :, 10:], l[:, :, 10:], Wa, nu=2)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=2), y, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(Wb, W, rtol=1e-13, atol=1e-15)
    Ws = W0.copy()
    for t in range(23):
        ys, Ws = O.delta_step(q[:, :, t], k[:, :, t], v[:, :, t], l[:, :, t], Ws, nu=2)
        np.testing.assert_allclose(ys, y[:, :, t], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(Ws, W, rtol=1e-13, atol=1e-15)


def pin_permutation_equivariance(O):
    """Permuting v's components permutes the rows of W and the components of y; permuting
    (batch, head) slices permutes the outputs (slices are independent)."""
    rng = np.random.default_rng(29)
    q, k, v, l, W0 = _rand_case(rng, 2, 3, 11, 8, 6, 1)
    y, W = O.delta_forward(q, k, v, l, W0, nu=1)
    pv = rng.permutation(6)
    yp, Wp = O.delta_forward(q, k, v[..., pv], l, W0[:, :, pv], nu=1)
    np.testing.assert_allclose(yp, y[..., pv], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(Wp, W[:, :, pv], rtol=1e-14, atol=1e-16)
    ph = rng.permutation(3)
    yh, Wh = O.delta_forward(q[:, ph], k[:, ph], v[:, ph], l[:, ph], W0[:, ph], nu=1)
    np.testing.assert_array_equal(yh, y[:, ph])
    np.testing.assert_array_equal(Wh, W[:, ph])


def pin_matches_numpy_twin(O):
    """Two implementations in different forms: the C oracle's literal retrieve / write / read
    loop with explicit modular indices, and the NumPy twin's index-gather DPFP, tanh-form
    sigmoid and row-wise read-before-write identity."""
    from oracle import twin
    rng = np.random.default_rng(30)
    for (B, H, T, d_k, d_v, nu) in [(1, 1, 64, 16, 16, 1), (1, 2, 40, 64, 64, 1),
                                    (2, 1, 33, 8, 5, 3)]:
        q, k, v, l, W0 = _rand_case(rng, B, H, T, d_k, d_v, nu)
        y, W = O.delta_forward(q, k, v, l, W0, nu=nu)
        y2, W2 = twin.delta_forward(q, k, v, l, W0, nu=nu)
        np.testing.assert_allclose(y, y2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(W, W2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(O.dpfp(k, nu), twin.dpfp(k, nu), rtol=0, atol=1e-15)
    for x in (-30.0, -1.5, 0.0, 0.7, 25.0):
        assert abs(O.sigmoid(x) - twin.sigmoid(x)) <= 1e-15


# ---------------------------------------------------------------- gradient pins
# The pages train the layer ([FWT] "Training experiment"), which needs the forward's gradient.
# These pins tie the oracle's reverse pass to the forward (already pinned above) and to closed
# forms, never to itself.

def _bwd_case(rng, B, H, T, d_k, d_v, nu, w0=True, dwf=True):
    """Inputs with |q|, |k| entries in [0.2, 1.5] (no DPFP kink within a finite-difference
    step), and random cotangents dy, dW_final."""
    D = 2 * d_k * nu
    mag = lambda *s: rng.uniform(0.2, 1.5, size=s) * rng.choice([-1.0, 1.0], size=s)
    q, k = mag(B, H, T, d_k), mag(B, H, T, d_k)
    v = rng.normal(size=(B, H, T, d_v))
    l = rng.normal(size=(B, H, T))
    W0 = rng.normal(size=(B, H, d_v, D)) * 0.3 if w0 else None
    dy = rng.normal(size=(B, H, T, d_v))
    dWf = rng.normal(size=(B, H, d_v, D)) if dwf else None
    return q, k, v, l, W0, dy, dWf


def _loss(O, args, nu, dy, dWf):
    y, W = O.delta_forward(*args, nu=nu)
    return float((dy * y).sum() + (0.0 if dWf is None else (dWf * W).sum()))


def pin_backward_central_differences(O):
    """Every gradient equals the central difference of the (pinned) forward, on random entries
    of every input, for nu 1 and 3, with and without W0 and dW_final, and for T = 70 across the
    reverse pass's 64-step recomputation boundary."""
    rng = np.random.default_rng(41)
    h = 1e-6
    for (B, H, T, d_k, d_v, nu, w0, dwf) in [(1, 2, 9, 4, 3, 1, True, True),
                                              (1, 1, 70, 4, 3, 3, True, False),
                                              (2, 1, 6, 8, 5, 2, False, True)]:
        q, k, v, l, W0, dy, dWf = _bwd_case(rng, B, H, T, d_k, d_v, nu, w0, dwf)
        grads = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=nu)
        args = [q, k, v, l, W0]
        for idx in range(5 if w0 else 4):
            a0 = args[idx]
            flat = rng.choice(a0.size, size=min(a0.size, 24), replace=False)
            num, ana = [], []
            for f in flat:
                i = np.unravel_index(f, a0.shape)
                ap = [x if x is None else x.copy() for x in args]
                ap[idx][i] += h
                am = [x if x is None else x.copy() for x in args]
                am[idx][i] -= h
                num.append((_loss(O, ap, nu, dy, dWf) - _loss(O, am, nu, dy, dWf)) / (2 * h))
                ana.append(grads[idx if idx < 4 else 4][i])
            num, ana = np.array(num), np.array(ana)
            scale = max(np.abs(num).max(), 1e-12)
            assert np.abs(num - ana).max() / scale < 1e-6, (idx, np.abs(num - ana).max() / scale)


def pin_backward_euler_identity(O):
    """(y, W_final) is linear in (v, W0) jointly, so L = <dy, y> + <dW_final, W_final> is
    homogeneous of degree one in them: sum(v * dv) + sum(W0 * dW0) = L exactly (up to
    rounding), over T = 150 (three recomputation segments)."""
    rng = np.random.default_rng(42)
    q, k, v, l, W0, dy, dWf = _bwd_case(rng, 2, 2, 150, 8, 6, 2)
    L = _loss(O, [q, k, v, l, W0], 2, dy, dWf)
    _, _, dv, _, dW0 = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=2)
    lhs = float((v * dv).sum() + (W0 * dW0).sum())
    assert abs(lhs - L) <= 1e-10 * max(1.0, abs(L)), (lhs, L)


def pin_backward_one_step_closed_form(O):
    """T = 1 from W0 = 0: y = beta v (f.g) and W = beta v f^T, so dv = beta ((f.g) dy +
    dW_final f), dl = beta (1 - beta) ((f.g) (dy.v) + v^T dW_final f) and
    dW0 = dW_final + dy g^T - beta (dW_final f + (f.g) dy) f^T."""
    rng = np.random.default_rng(43)
    d_k, d_v, nu = 6, 4, 2
    q, k, v, l, _, dy, dWf = _bwd_case(rng, 1, 1, 1, d_k, d_v, nu, w0=False)
    W0 = np.zeros((1, 1, d_v, 2 * d_k * nu))
    _, _, dv, dl, dW0 = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=nu)
    f, g = O.dpfp(k[0, 0, 0], nu), O.dpfp(q[0, 0, 0], nu)
    beta = 1.0 / (1.0 + math.exp(-l[0, 0, 0]))
    fg = float(f @ g)
    Gf = dWf[0, 0] @ f
    np.testing.assert_allclose(dv[0, 0, 0], beta * (fg * dy[0, 0, 0] + Gf), rtol=1e-12, atol=1e-14)
    exp_dl = beta * (1 - beta) * (fg * float(dy[0, 0, 0] @ v[0, 0, 0]) + float(v[0, 0, 0] @ Gf))
    assert abs(dl[0, 0, 0] - exp_dl) <= 1e-12 * max(1.0, abs(exp_dl))
    du = Gf + fg * dy[0, 0, 0]
    exp_dW0 = dWf[0, 0] + np.outer(dy[0, 0, 0], g) - beta * np.outer(du, f)
    np.testing.assert_allclose(dW0[0, 0], exp_dW0, rtol=1e-12, atol=1e-13)


def pin_backward_degenerate(O):
    """beta = 0 (logit -60): no write happens, so dv = 0, dk = 0, dl = 0 and dW0 = dW_final +
    sum_t dy_t phi(q_t)^T; zero key rows have zero dk (relu's derivative at 0 taken as 0) and
    leave dv of their step at beta * (dW f) = 0; d_k = 1 makes phi identically 0."""
    rng = np.random.default_rng(44)
    nu = 2
    q, k, v, l, W0, dy, dWf = _bwd_case(rng, 1, 2, 12, 4, 3, nu)
    l[:] = -60.0
    dq, dk, dv, dl, dW0 = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=nu)
    assert np.abs(dv).max() < 1e-20 and np.abs(dk).max() < 1e-18 and np.abs(dl).max() < 1e-20
    phq = O.dpfp(q, nu)
    np.testing.assert_allclose(dW0, dWf + np.einsum("bhtv,bhtd->bhvd", dy, phq), rtol=1e-12,
                               atol=1e-13)
    q, k, v, l, W0, dy, dWf = _bwd_case(rng, 1, 1, 10, 4, 3, nu)
    k[0, 0, 3] = 0.0
    k[0, 0, 7] = 0.0
    dq, dk, dv, dl, dW0 = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=nu)
    assert not dk[0, 0, 3].any() and not dk[0, 0, 7].any()
    assert dk[0, 0, 2].any() and dk[0, 0, 4].any()
    q, k, v, l, W0, dy, dWf = _bwd_case(rng, 1, 1, 5, 1, 2, 1)
    dq, dk, dv, dl, dW0 = O.delta_backward(q, k, v, l, W0, dy, dWf, nu=1)
    assert not dq.any() and not dk.any() and not dl.any()
    np.testing.assert_array_equal(dW0, dWf)


# ---------------------------------------------------------------- sum-update pins
# [FWT] "Background / fast computation form of linear self-attention": with the kernel
# phi(k)^T phi(q), causal attention sum_s v_s k(s, t) / sum_s k(s, t) becomes the W, z
# recurrence.  These pins compute the attention form directly (a masked matmul).

def pin_sum_update_is_normalised_masked_matmul(O):
    """y_t = (W0 phi(q_t) + sum_{s<=t} v_s (phi(k_s).phi(q_t))) / (z0.phi(q_t) + sum_{s<=t}
    phi(k_s).phi(q_t)); W_final = W0 + V^T Phi_K; z_final = z0 + Phi_K^T 1."""
    rng = np.random.default_rng(51)
    for (B, H, T, d_k, d_v, nu, carried) in [(1, 2, 40, 8, 5, 2, False), (2, 1, 33, 16, 4, 1, True)]:
        q, k, v, _, W0 = _rand_case(rng, B, H, T, d_k, d_v, nu)
        D = 2 * d_k * nu
        z0 = rng.uniform(0.0, 0.5, size=(B, H, D)) if carried else None
        if not carried:
            W0 = None
        y, Wf, zf = O.sum_forward(q, k, v, W0, z0, nu=nu)
        Fq, Fk = O.dpfp(q, nu), O.dpfp(k, nu)
        for b in range(B):
            for h in range(H):
                M = np.tril(Fq[b, h] @ Fk[b, h].T)
                num = M @ v[b, h]
                den = M @ np.ones(T)
                if carried:
                    num = num + Fq[b, h] @ W0[b, h].T
                    den = den + Fq[b, h] @ z0[b, h]
                np.testing.assert_allclose(y[b, h], num / den[:, None], rtol=1e-11, atol=1e-14)
                W_exp = (0 if W0 is None else W0[b, h]) + v[b, h].T @ Fk[b, h]
                z_exp = (0 if z0 is None else z0[b, h]) + Fk[b, h].sum(axis=0)
                np.testing.assert_allclose(Wf[b, h], W_exp, rtol=1e-12, atol=1e-14)
                np.testing.assert_allclose(zf[b, h], z_exp, rtol=1e-12, atol=1e-14)


def pin_sum_update_convex_and_degenerate(O):
    """From W0 = 0, z0 = 0 every output is a convex combination of the values so far (so a
    constant value sequence comes back unchanged); a zero query reads 0 (zero denominator)."""
    rng = np.random.default_rng(52)
    q, k, v, _, _ = _rand_case(rng, 1, 1, 30, 8, 3, 2)
    y, _, _ = O.sum_forward(q, k, v, nu=2)
    lo = np.minimum.accumulate(v[0, 0], axis=0)
    hi = np.maximum.accumulate(v[0, 0], axis=0)
    assert np.all(y[0, 0] >= lo - 1e-12) and np.all(y[0, 0] <= hi + 1e-12)
    c = rng.normal(size=3)
    yc, _, _ = O.sum_forward(q, k, np.broadcast_to(c, v.shape).copy(), nu=2)
    np.testing.assert_allclose(yc[0, 0], np.broadcast_to(c, (30, 3)), rtol=1e-12)
    q2 = q.copy()
    q2[0, 0, 7] = 0.0
    y2, _, _ = O.sum_forward(q2, k, v, nu=2)
    assert not y2[0, 0, 7].any()
    np.testing.assert_array_equal(np.delete(y2[0, 0], 7, axis=0), np.delete(y[0, 0], 7, axis=0))


# ---------------------------------------------------------------- projection pins
# [FWT] "FastWeightsAttention / module structure and source walkthrough": bias-free linear maps
# to heads * d (split by head) and to one beta logit per head; an output linear map with bias.

def pin_layer_projections_are_matmuls(O):
    """layer_project equals x W^T (numpy's matmul) split into the q, k, v, beta blocks and by
    head; layer_output equals residual + bo + concat_heads(y) Wo^T."""
    rng = np.random.default_rng(61)
    B, T, d_model, H, d_k, d_v = 2, 5, 24, 3, 4, 6
    x = rng.normal(size=(B, T, d_model))
    N = 2 * H * d_k + H * d_v + H
    Wm = rng.normal(size=(N, d_model))
    q, k, v, bl = O.layer_project(x, Wm, H, d_k, d_v)
    full = x @ Wm.T                                   # [B, T, N]
    split = lambda blk, d: blk.reshape(B, T, H, d).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(q, split(full[..., :H * d_k], d_k), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(k, split(full[..., H * d_k:2 * H * d_k], d_k), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(v, split(full[..., 2 * H * d_k:2 * H * d_k + H * d_v], d_v),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(bl, full[..., -H:].transpose(0, 2, 1), rtol=1e-13, atol=1e-13)
    y = rng.normal(size=(B, H, T, d_v))
    Wo = rng.normal(size=(d_model, H * d_v))
    bo = rng.normal(size=d_model)
    res = rng.normal(size=(B, T, d_model))
    cat = y.transpose(0, 2, 1, 3).reshape(B, T, H * d_v)
    np.testing.assert_allclose(O.layer_output(y, Wo, bo, res), res + bo + cat @ Wo.T, rtol=1e-13,
                               atol=1e-12)
    np.testing.assert_allclose(O.layer_output(y, Wo), cat @ Wo.T, rtol=1e-13, atol=1e-12)


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
