"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test ties an oracle function to something fixed independently of it:
numbers the pages print (tests/golden/), closed forms (the SVD form of an odd
matrix polynomial, geometric sums of the moving averages), invariants and a
library routine for a special case (scipy's polar decomposition).  A dropped
term, a wrong sign or coefficient order, a transposed operand or a moved
epsilon in the oracle fails at least one of them.
"""

import numpy as np
import pytest
import scipy.linalg
import scipy.optimize

import oracle
from oracle import MUON_COEFFS
from conftest import load_golden

A_, B_, C_ = MUON_COEFFS


def _p(s, coeffs=MUON_COEFFS):
    """Scalar odd quintic of the lemma ("About Muon: Why Not Adam", section
    "Making It Actually Run"): the polynomial acts on each singular value."""
    a, b, c = coeffs
    return a * s + b * s ** 3 + c * s ** 5


def scalar_map_via_oracle(values, iters, coeffs=MUON_COEFFS):
    """Run the *oracle's matrix iteration* on diag(values) and read back the
    diagonal.  A first iteration with coefficients (||g||, 0, 0) undoes the
    Frobenius normalisation (eps = 0), so the remaining ``iters`` iterations
    see exactly the given values."""
    g = np.asarray(values, dtype=np.float64)
    norm = np.sqrt(np.sum(g * g))
    sched = [(norm, 0.0, 0.0)] + [tuple(coeffs)] * iters
    out = oracle.newton_schulz(np.diag(g), steps=iters + 1, eps=0.0, coeffs=sched)
    return np.diag(out).copy()


def _one(s, iters=1):
    # 1x1 with the value s, through a 2x2 diagonal so s need not equal its norm
    return scalar_map_via_oracle([s, 0.5], iters)[0]


# --------------------------------------------------------------------------
# P2: the scalar map numbers printed on the page
# --------------------------------------------------------------------------

GOLD_NS = load_golden("ns_scalar_map.txt")


def _check(key, got):
    want, tol = GOLD_NS[key]
    assert abs(got - want) <= tol, (key, got, want, tol)


def test_p_at_one():
    _check("p_at_1", _one(1.0))


def test_fixed_points_and_slopes():
    f = lambda s: _one(s) - s
    lo = scipy.optimize.brentq(f, 0.8, 0.95, xtol=1e-13)
    hi = scipy.optimize.brentq(f, 1.1, 1.4, xtol=1e-13)
    _check("fixed_point_low", lo)
    _check("fixed_point_high", hi)
    h = 1e-6
    _check("slope_fixed_low", (_one(lo + h) - _one(lo - h)) / (2 * h))
    _check("slope_fixed_high", (_one(hi + h) - _one(hi - h)) / (2 * h))


def test_maximum_on_unit_interval():
    res = scipy.optimize.minimize_scalar(lambda s: -_one(s), bounds=(0.3, 0.8),
                                         method="bounded", options={"xatol": 1e-9})
    _check("max_on_unit", -res.fun)
    _check("argmax_on_unit", res.x)
    grid = np.linspace(0.01, 1.0, 100)
    assert scalar_map_via_oracle(grid, 1).max() <= -res.fun + 1e-12


def test_long_run_band():
    s = np.linspace(0.02, 1.0, 50)
    vals = scalar_map_via_oracle(s, 100)
    lo, hi = np.inf, -np.inf
    x = vals
    for _ in range(200):
        x = scalar_map_via_oracle(x, 1)
        lo, hi = min(lo, x.min()), max(hi, x.max())
    _check("band_low", lo)
    _check("band_high", hi)


def test_five_iterations_of_small_values():
    out = scalar_map_via_oracle([1e-3, 1e-4, 1.0], 5)
    _check("p5_at_1e-3", out[0])
    _check("p5_at_1e-4", out[1])


def test_slope_at_zero():
    h = 1e-7
    slope = (_one(h) - _one(-h)) / (2 * h)
    _check("slope_at_0", slope)
    # the textbook quintic's slope at 0 is 15/8
    q = (15 / 8, -10 / 8, 3 / 8)
    sq = scalar_map_via_oracle([h, 0.5], 1, q)[0] / h
    assert abs(sq - 15 / 8) < 1e-9


# --------------------------------------------------------------------------
# P1: odd-polynomial lemma -- NS = U diag(p^k(sigma/(||G||+eps))) V^T
# --------------------------------------------------------------------------

def closed_form(G, steps=5, eps=1e-7, coeffs=MUON_COEFFS):
    U, sig, Vt = np.linalg.svd(G, full_matrices=False)
    s = sig / (np.linalg.norm(G, "fro") + eps)
    sched = coeffs if np.ndim(coeffs) == 2 else [coeffs] * steps
    for c in sched:
        s = _p(s, c)
    return (U * s[None, :]) @ Vt


SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (5, 3), (16, 16), (64, 48), (48, 64)]


@pytest.mark.parametrize("shape", SHAPES)
def test_lemma_closed_form(shape):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape) * 3.0
    got = oracle.newton_schulz(G)
    want = closed_form(G)
    assert np.linalg.norm(got - want) <= 1e-12 * max(1.0, np.linalg.norm(want))


def test_lemma_rank_deficient():
    rng = np.random.default_rng(7)
    G = rng.standard_normal((32, 4)) @ rng.standard_normal((4, 32))
    got = oracle.newton_schulz(G)
    want = closed_form(G)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)
    assert np.linalg.matrix_rank(got, tol=1e-9) == 4


def test_lemma_per_iteration_schedule():
    rng = np.random.default_rng(11)
    G = rng.standard_normal((12, 20))
    sched = rng.uniform([1.0, -2.0, 0.0], [3.0, 0.0, 1.0], size=(5, 3))
    got = oracle.newton_schulz(G, steps=5, coeffs=sched)
    want = closed_form(G, coeffs=sched)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def test_rank_one():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(9)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(6)
    v /= np.linalg.norm(v)
    sigma = 2.5
    got = oracle.newton_schulz(sigma * np.outer(u, v))
    s = sigma / (sigma + 1e-7)
    for _ in range(5):
        s = _p(s)
    assert abs(s - 0.69644) < 5e-5
    assert np.allclose(got, s * np.outer(u, v), atol=1e-13)


# --------------------------------------------------------------------------
# P4, P5: transpose symmetry, the long-side Gram form, equivariance
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (1, 4), (33, 17)])
def test_transpose_symmetry(shape):
    rng = np.random.default_rng(shape[0] * 100 + shape[1])
    G = rng.standard_normal(shape)
    assert np.allclose(oracle.newton_schulz(G.T), oracle.newton_schulz(G).T, atol=1e-13)


@pytest.mark.parametrize("shape", [(9, 5), (5, 9), (8, 8)])
def test_lemma_form_on_the_long_side(shape):
    # p(X) = aX + b X X^T X + c (X X^T)^2 X written through the Gram on the
    # *long* side (the large one), the route the oracle never takes: X^T X on
    # the right for a wide or square X, X X^T on the left for a tall one.
    rng = np.random.default_rng(42 + shape[0])
    G = rng.standard_normal(shape)
    X = G / (np.linalg.norm(G, "fro") + 1e-7)
    for _ in range(5):
        if shape[0] <= shape[1]:
            S = X.T @ X
            X = A_ * X + B_ * (X @ S) + C_ * (X @ S @ S)
        else:
            S = X @ X.T
            X = A_ * X + B_ * (S @ X) + C_ * (S @ S @ X)
    assert np.allclose(oracle.newton_schulz(G), X, atol=1e-13)


def test_orthogonal_equivariance_and_scale_invariance():
    rng = np.random.default_rng(5)
    G = rng.standard_normal((10, 14))
    Q, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    R, _ = np.linalg.qr(rng.standard_normal((14, 14)))
    O = oracle.newton_schulz(G)
    assert np.allclose(oracle.newton_schulz(Q @ G @ R), Q @ O @ R, atol=1e-12)
    for alpha in (1e-2, 10.0, 1e3):
        assert np.allclose(oracle.newton_schulz(alpha * G), O, atol=1e-6)


# --------------------------------------------------------------------------
# P6: textbook convergent coefficients reach the exact polar factor
# --------------------------------------------------------------------------

@pytest.mark.parametrize("coeffs", [(1.5, -0.5, 0.0), (15 / 8, -10 / 8, 3 / 8)])
@pytest.mark.parametrize("shape", [(20, 12), (12, 20), (16, 16)])
def test_convergent_coefficients_give_polar_factor(coeffs, shape):
    rng = np.random.default_rng(shape[0] + 3 * shape[1])
    G = rng.standard_normal(shape) + 0.5 * np.eye(*shape)
    got = oracle.newton_schulz(G, steps=60, coeffs=coeffs)
    U, _ = scipy.linalg.polar(G)
    assert np.allclose(got, U, atol=1e-10)


# --------------------------------------------------------------------------
# Normalisation and the epsilon guard (P10), the shape multipliers (P7)
# --------------------------------------------------------------------------

def test_zero_matrix_maps_to_zero():
    assert np.all(oracle.newton_schulz(np.zeros((4, 6))) == 0.0)


def test_epsilon_is_added_to_the_norm():
    # G = delta u v^T with delta = eps: X0 = delta/(delta+eps) u v^T = 0.5 u v^T
    rng = np.random.default_rng(1)
    u = rng.standard_normal(5)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(8)
    v /= np.linalg.norm(v)
    got = oracle.newton_schulz(1e-7 * np.outer(u, v), eps=1e-7)
    s = 0.5
    for _ in range(5):
        s = _p(s)
    assert np.allclose(got, s * np.outer(u, v), atol=1e-12)


def test_polar_factor_frobenius_and_moonlight_rms():
    # ||U V^T||_F^2 = min(m, n); 0.2 sqrt(max(m,n)) gives entry RMS 0.2
    # ("About Muon: Why Not Adam", section "Why Muon?", scaling paragraph)
    rng = np.random.default_rng(9)
    for m, n in ((24, 96), (96, 24)):
        G = rng.standard_normal((m, n))
        O = oracle.newton_schulz(G, steps=80, coeffs=(1.5, -0.5, 0.0))
        assert abs(np.sum(O * O) - min(m, n)) < 1e-9
        rms = np.sqrt(np.mean((oracle.shape_scale(m, n, "moonlight") * O) ** 2))
        assert abs(rms - 0.2) < 1e-10


def test_jordan_and_bernstein_agree_only_when_not_shrinking():
    # "Same as Bernstein when m >= n; not when the layer shrinks."
    for m, n in ((4096, 1024), (1024, 1024), (14336, 4096)):
        assert oracle.shape_scale(m, n, "jordan") == pytest.approx(oracle.shape_scale(m, n, "bernstein"))
    for m, n in ((1024, 4096), (2048, 8192)):
        assert oracle.shape_scale(m, n, "jordan") == 1.0
        assert oracle.shape_scale(m, n, "bernstein") < 1.0
    assert oracle.shape_scale(5, 7, "none") == 1.0
    with pytest.raises(ValueError):
        oracle.shape_scale(5, 7, "spectral-ish")


# --------------------------------------------------------------------------
# P8: momentum and the Nesterov blend
# --------------------------------------------------------------------------

GOLD_AD = load_golden("adamw_pages.txt")


def test_momentum_constant_gradient_closed_form():
    mu = 0.95
    g = np.array([[1.0, -2.0], [0.5, 3.0]])
    M = np.zeros_like(g)
    for t in range(1, 30):
        M = oracle.momentum_update(M, g, mu)
        assert np.allclose(M, (1 - mu ** t) * g, atol=1e-14)
        Y = oracle.nesterov_blend(g, M, mu, True)
        assert np.allclose(Y, (1 - mu) * g + mu * (1 - mu ** t) * g, atol=1e-14)
        assert np.array_equal(oracle.nesterov_blend(g, M, mu, False), M)


def test_momentum_limits_match_heavy_ball_sums():
    # The page writes the heavy-ball sum v <- beta v + g; the optimizer keeps
    # the average M <- beta M + (1-beta) g = (1-beta) v.  Limits in units of g:
    beta = 0.9
    g = np.ones((1, 1))
    M = np.zeros_like(g)
    for _ in range(2000):
        M = oracle.momentum_update(M, g, beta)
    want, tol = GOLD_AD["heavy_ball_constant_beta0.9"]
    assert abs(M[0, 0] / (1 - beta) - want) <= tol
    M = np.zeros_like(g)
    for t in range(2001):
        M = oracle.momentum_update(M, g * (1 if t % 2 == 0 else -1), beta)
    want, tol = GOLD_AD["heavy_ball_alternating_0.9"]
    assert abs(abs(M[0, 0]) / (1 - beta) - want) <= tol


# --------------------------------------------------------------------------
# Whole Muon step: zero gradient (pure decay) and the 1x1 closed form
# --------------------------------------------------------------------------

def test_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((6, 10))
    Wn, Mn, O = oracle.muon_matrix_step(W, np.zeros_like(W), np.zeros_like(W),
                                        lr=0.02, mu=0.95, weight_decay=0.01)
    assert np.all(Mn == 0) and np.all(O == 0)
    assert np.allclose(Wn, (1 - 0.02 * 0.01) * W, rtol=0, atol=1e-15)


@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("mode,s_expected", [("moonlight", 0.2), ("jordan", 1.0), ("none", 1.0)])
def test_one_by_one_step_closed_form(nesterov, mode, s_expected):
    W, G, M = np.array([[0.3]]), np.array([[-0.7]]), np.array([[0.2]])
    mu, lr, wd = 0.9, 0.05, 0.1
    Wn, Mn, O = oracle.muon_matrix_step(W, G, M, lr=lr, mu=mu, weight_decay=wd,
                                        nesterov=nesterov, scale_mode=mode, extra_scale=1.5)
    m_new = 0.9 * 0.2 + 0.1 * -0.7
    y = 0.1 * -0.7 + 0.9 * m_new if nesterov else m_new
    s = abs(y) / (abs(y) + 1e-7)
    for _ in range(5):
        s = _p(s)
    o = np.sign(y) * s
    assert Mn[0, 0] == pytest.approx(m_new, abs=1e-15)
    assert O[0, 0] == pytest.approx(o, abs=1e-13)
    assert Wn[0, 0] == pytest.approx((1 - lr * wd) * 0.3 - lr * s_expected * 1.5 * o, abs=1e-14)


def test_muon_step_over_list_is_per_matrix():
    rng = np.random.default_rng(4)
    Ws = [rng.standard_normal(s) for s in ((4, 6), (6, 4))]
    Gs = [rng.standard_normal(w.shape) for w in Ws]
    Ms = [np.zeros_like(w) for w in Ws]
    W2, M2, O2 = oracle.muon_step(Ws, Gs, Ms, lr=0.01)
    for i in range(2):
        w, m, o = oracle.muon_matrix_step(Ws[i], Gs[i], Ms[i], lr=0.01)
        assert np.array_equal(W2[i], w) and np.array_equal(M2[i], m) and np.array_equal(O2[i], o)


# --------------------------------------------------------------------------
# P9: AdamW
# --------------------------------------------------------------------------

def test_adamw_second_moment_first_step_ratio():
    g = np.array([0.3, -2.0, 1e-3])
    for b2, key in ((0.9, "rms_first_ratio_beta2_0.9"), (0.999, "rms_first_ratio_beta2_0.999")):
        _, _, v = oracle.adamw_tensor_step(np.zeros(3), g, np.zeros(3), np.zeros(3), step=1,
                                           lr=1.0, beta2=b2, eps=0.0, weight_decay=0.0)
        want, tol = GOLD_AD[key]
        assert np.all(np.abs(np.abs(g) / np.sqrt(v) - want) <= tol)


def test_adamw_corrected_first_step_is_sign():
    g = np.array([0.3, -2.0, 5.0, -1e-2])
    lr = 3e-4
    th, m, v = oracle.adamw_tensor_step(np.zeros(4), g, np.zeros(4), np.zeros(4), step=1,
                                        lr=lr, eps=1e-12, weight_decay=0.0)
    want, tol = GOLD_AD["corrected_first_step"]
    assert np.all(np.abs(-th / lr - want * np.sign(g)) <= tol)


def test_adamw_decay_per_step():
    th0 = np.array([1.0, -2.0, 0.5])
    th, m, v = oracle.adamw_tensor_step(th0, np.zeros(3), np.zeros(3), np.zeros(3), step=1,
                                        lr=3e-4, weight_decay=0.1)
    want, tol = GOLD_AD["decay_per_step"]
    assert np.all(np.abs((th0 - th) / th0 - want) <= tol)
    assert np.all(m == 0) and np.all(v == 0)


def test_adamw_constant_gradient_identical_steps_and_geometric_mean():
    g = np.array([0.7, -0.1, 2.0])
    th = np.zeros(3)
    m = np.zeros(3)
    v = np.zeros(3)
    steps = []
    b1 = 0.9
    for t in range(1, 12):
        new, m, v = oracle.adamw_tensor_step(th, g, m, v, step=t, lr=1e-3, beta1=b1,
                                             eps=1e-12, weight_decay=0.0)
        steps.append(new - th)
        th = new
        # m_t = (1 - b1^t) g  ("Adam: las dos ideas juntas")
        assert np.allclose(m, (1 - b1 ** t) * g, atol=1e-15)
    for s in steps[1:]:
        assert np.allclose(s, steps[0], atol=1e-15)


def test_adamw_epsilon_brakes_gradients_below_it():
    # eps outside the square root: a gradient of size eps moves half a step
    eps = 1e-5
    g = np.array([eps, -eps])
    th, _, _ = oracle.adamw_tensor_step(np.zeros(2), g, np.zeros(2), np.zeros(2), step=1,
                                        lr=1.0, eps=eps, weight_decay=0.0)
    assert np.allclose(th, [-0.5, 0.5], atol=1e-12)


def test_adamw_decay_uses_old_theta_and_step_validation():
    th0 = np.array([2.0])
    g = np.array([1.0])
    th, _, _ = oracle.adamw_tensor_step(th0, g, np.zeros(1), np.zeros(1), step=1, lr=0.1,
                                        eps=0.0, weight_decay=0.5)
    assert th[0] == pytest.approx(2.0 - 0.1 * (1.0 + 0.5 * 2.0), abs=1e-15)
    with pytest.raises(ValueError):
        oracle.adamw_tensor_step(th0, g, th0, th0, step=0, lr=0.1)


# --------------------------------------------------------------------------
# QK-Clip ("The Optimizer Wars ...", "What is MuonClip?") and gradient
# clipping ("Por qué AdamW ...", "Por qué AdamW, y por qué con esos números")
# --------------------------------------------------------------------------

GOLD_QK = load_golden("qkclip_pages.txt")


def test_qk_clip_caps_every_heads_max_logit_at_tau():
    # Attention logits of head h are q.k with q = Wq_h x, k = Wk_h x'.
    # Scaling both projections by sqrt(gamma_h) scales every logit by gamma_h,
    # so after the clip each head's maximum is min(S_max^h, tau).
    tau = GOLD_QK["tau_kimi_k2"][0]
    rng = np.random.default_rng(12)
    H, dh, dm, T = 4, 8, 32, 16
    Wq = rng.standard_normal((H * dh, dm)) * 3.0
    Wk = rng.standard_normal((H * dh, dm)) * 3.0
    Wq[:dh] *= 0.05  # head 0 stays below tau
    X = rng.standard_normal((T, dm))

    def max_logits(q, k):
        out = []
        for h in range(H):
            Q = X @ q[h * dh:(h + 1) * dh].T
            K = X @ k[h * dh:(h + 1) * dh].T
            out.append(np.max(Q @ K.T))
        return np.array(out)

    S = max_logits(Wq, Wk)
    assert S[0] < tau and np.all(S[1:] > tau)
    q2 = oracle.qk_clip(Wq, S, tau, dh)
    k2 = oracle.qk_clip(Wk, S, tau, dh)
    S2 = max_logits(q2, k2)
    assert np.allclose(S2, np.minimum(S, tau), rtol=1e-12)
    assert np.array_equal(q2[:dh], Wq[:dh])


def test_qk_clip_is_a_post_update_row_scaling():
    rng = np.random.default_rng(13)
    W, G = rng.standard_normal((6, 5)), rng.standard_normal((6, 5))
    smax = np.array([50.0, 400.0, 100.0])
    Wn, Mn, O = oracle.muon_matrix_step(W, G, np.zeros_like(W), lr=0.1, weight_decay=0.1,
                                        qk_smax=smax, qk_block_rows=2, qk_tau=100.0)
    Wp, Mp, Op = oracle.muon_matrix_step(W, G, np.zeros_like(W), lr=0.1, weight_decay=0.1)
    assert np.array_equal(Mn, Mp) and np.array_equal(O, Op)
    assert np.allclose(Wn[0:2], Wp[0:2]) and np.allclose(Wn[4:6], Wp[4:6])
    assert np.allclose(Wn[2:4], 0.5 * Wp[2:4])   # sqrt(100/400)


def test_global_norm_clipping():
    want, _ = GOLD_AD["grad_clip_threshold"]
    rng = np.random.default_rng(14)
    gs = [rng.standard_normal(7) * 3.0, rng.standard_normal((3, 4)) * 3.0]
    norm = np.sqrt(sum(np.sum(g * g) for g in gs))
    assert norm > want
    cg, n = oracle.clip_by_global_norm(gs, want)
    assert n == pytest.approx(norm)
    assert np.sqrt(sum(np.sum(g * g) for g in cg)) == pytest.approx(want, rel=1e-12)
    for a, b in zip(cg, gs):
        assert np.allclose(a, b * want / norm)
    small = [g * 1e-3 for g in gs]
    cs, _ = oracle.clip_by_global_norm(small, want)
    for a, b in zip(cs, small):
        assert np.array_equal(a, b)
    # clipping happens before the moments: second step with an unclipped g2
    g1, g2 = np.array([30.0, 40.0]), np.array([0.3, -0.4])
    ts, ms, vs = oracle.adamw_step([np.zeros(2)], [g1], [np.zeros(2)], [np.zeros(2)],
                                   max_grad_norm=1.0, step=1, lr=1.0, weight_decay=0.0)
    assert np.allclose(ms[0], 0.1 * g1 / 50.0)
    ts, ms, vs = oracle.adamw_step(ts, [g2], ms, vs, max_grad_norm=1.0, step=2, lr=1.0,
                                   weight_decay=0.0)
    assert np.allclose(ms[0], 0.9 * 0.1 * g1 / 50.0 + 0.1 * g2)


# --------------------------------------------------------------------------
# bf16 storage rounding: closed-form ties and torch's conversion
# --------------------------------------------------------------------------

def test_bf16_rounding_closed_forms():
    # spacing of bf16 in [1, 2) is 2^-7; halfway cases go to the even neighbour
    h = 2.0 ** -7
    cases = {1.0: 1.0, 1.0 + h / 2: 1.0, 1.0 + 1.5 * h: 1.0 + 2 * h, 1.0 + 0.49 * h: 1.0,
             1.0 + 0.51 * h: 1.0 + h, -(1.0 + 1.5 * h): -(1.0 + 2 * h), 0.0: 0.0,
             2.0 - h / 4: 2.0, 3.0 * 2.0 ** -20: 3.0 * 2.0 ** -20,
             (1.0 + h / 2) * 2.0 ** 40: 2.0 ** 40}
    got = oracle.round_to_bf16(np.array(list(cases)))
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])
    assert oracle.round_to_bf16(np.array([-np.inf]))[0] == -np.inf


def test_bf16_rounding_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    # exact ties: float32 values whose low 16 bits are 0x8000
    bits = rng.integers(0x00800000, 0x7f000000, 20000, dtype=np.uint32)
    ties = ((bits & 0xffff0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), want)


def test_bf16_parameter_stores_the_rounded_step():
    rng = np.random.default_rng(18)
    W = oracle.round_to_bf16(rng.standard_normal((6, 9)) * 0.02)
    G = rng.standard_normal((6, 9))
    full, M, O = oracle.muon_matrix_step(W, G, np.zeros_like(W), lr=0.02)
    low, M2, O2 = oracle.muon_matrix_step(W, G, np.zeros_like(W), lr=0.02, param_dtype="bf16")
    assert np.array_equal(low, oracle.round_to_bf16(full))
    assert np.array_equal(M, M2) and np.array_equal(O, O2)
    th, m, v = oracle.adamw_tensor_step(W, G, np.zeros_like(W), np.zeros_like(W), step=1, lr=1e-3)
    th2, m2, v2 = oracle.adamw_tensor_step(W, G, np.zeros_like(W), np.zeros_like(W), step=1,
                                           lr=1e-3, param_dtype="bf16")
    assert np.array_equal(th2, oracle.round_to_bf16(th))
    assert np.array_equal(m, m2) and np.array_equal(v, v2)
