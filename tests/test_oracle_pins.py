"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every pin here is a closed form, an exact rational computation, an invariant
of the mathematics, or a brute-force definition, chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign, a transposed operand, a
wrong norm, a misplaced epsilon, a wrong scale or scatter index) fails at
least one of them.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon_oracle as mo
from oracle import same_order as so

A_, B_, C_ = (Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315"))
#: The normalization epsilon of the stated reading (added to the Frobenius norm).
EPS = 1e-7


def quintic(x: Fraction) -> Fraction:
    """The scalar map the iteration applies to each singular value, exactly."""
    return A_ * x + B_ * x ** 3 + C_ * x ** 5


def quintic_iter(x, k):
    for _ in range(k):
        x = quintic(x)
    return x


def quintic_f64(x: np.ndarray, k: int) -> np.ndarray:
    for _ in range(k):
        x = 3.4445 * x - 4.7750 * x ** 3 + 2.0315 * x ** 5
    return x


def orthonormal(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


# ---------------------------------------------------------------- momentum

@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_constant_gradient_closed_form(nesterov):
    """G constant, M0 = 0: M_t = G (1 - beta^t)/(1 - beta); U_t = G + beta M_t."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal((3, 5))
    beta = 0.9
    m = np.zeros_like(g)
    for t in range(1, 6):
        m = mo.momentum_update(g, m, beta)
        closed = g * (1 - beta ** t) / (1 - beta)
        np.testing.assert_allclose(m, closed, rtol=1e-13, atol=0)
        u = mo.orthogonalization_input(g, m, beta, nesterov)
        want = g + beta * closed if nesterov else closed
        np.testing.assert_allclose(u, want, rtol=1e-13, atol=0)


def test_beta_zero_input_is_gradient():
    g = np.arange(6.0).reshape(2, 3) - 2.5
    m = mo.momentum_update(g, np.full_like(g, 7.0), 0.0)
    assert np.array_equal(m, g)
    assert np.array_equal(mo.orthogonalization_input(g, m, 0.0, True), g)


# ---------------------------------------------------------- decay + apply

def test_zero_gradient_is_pure_decay_over_steps():
    """G = 0 => U = 0 => O = 0 (epsilon keeps 0/0 away) => W_t = W0 (1-lr wd)^t."""
    rng = np.random.default_rng(2)
    w0 = rng.standard_normal(4 * 6)
    d = [mo.MatrixDesc(offset=0, rows=4, cols=6, param_offset=0)]
    lr, wd = 0.02, 0.01
    lr32, wd32 = mo.as_f32_value(lr), mo.as_f32_value(wd)
    w = w0.astype(np.float32)
    m = np.zeros(24, np.float32)
    g = np.zeros(24, np.float32)
    for t in range(1, 4):
        p64, m64, upd = mo.muon_step(w, g, m, d, lr=lr, weight_decay=wd, beta=0.95)
        assert np.array_equal(upd[0], np.zeros((4, 6)))
        assert np.array_equal(m64, np.zeros(24))
        np.testing.assert_allclose(p64, w.astype(np.float64) * (1 - lr32 * wd32), rtol=1e-15)
        w = p64.astype(np.float32)
        np.testing.assert_allclose(p64, w0.astype(np.float32) * (1 - lr32 * wd32) ** t,
                                   rtol=1e-6)


def test_lr_zero_leaves_weights():
    rng = np.random.default_rng(3)
    w = rng.standard_normal(12).astype(np.float32)
    g = rng.standard_normal(12).astype(np.float32)
    d = [mo.MatrixDesc(0, 3, 4, 0)]
    p64, _, _ = mo.muon_step(w, g, np.zeros(12, np.float32), d, lr=0.0, weight_decay=0.5,
                             beta=0.9)
    assert np.array_equal(p64, w.astype(np.float64))


def test_decay_then_update_order_exact_1x1():
    """W, O and wd all non-zero: W1 = W (1 - lr wd) - lr O, exactly in rationals.

    Decay acts on the old weight only (decoupled decay applied in
    _compute_momentum_inputs before _apply_local_updates subtracts the
    update).  Decaying after the update, (W - lr O)(1 - lr wd), differs by
    lr^2 wd O ~ 0.04 here.  Every hyperparameter is exact in float32.
    """
    g, w0, lr, wd = 0.25, 0.5, 0.5, 0.25
    p64, _, upd = mo.muon_step(np.array([w0], np.float32), np.array([g], np.float32),
                               np.zeros(1, np.float32), [mo.MatrixDesc(0, 1, 1, 0)],
                               lr=lr, weight_decay=wd, beta=0.0, nesterov=False)
    o = quintic_iter(Fraction(g) / (Fraction(g) + Fraction(EPS)), 5)
    want = Fraction(w0) * (1 - Fraction(lr) * Fraction(wd)) - Fraction(lr) * o
    assert abs(Fraction(upd[0][0, 0]) - o) < Fraction(1, 10 ** 14)
    assert abs(Fraction(p64[0]) - want) < Fraction(1, 10 ** 14)


#: float32 roundings of the hyperparameters, written out by hand (24-bit
#: significands of 0.02, 0.1 and 0.95).
F32_OF_0_02 = float.fromhex("0x1.47ae14p-6")
F32_OF_0_1 = float.fromhex("0x1.99999ap-4")
F32_OF_0_95 = float.fromhex("0x1.e66666p-1")


def test_hyperparameters_are_float32_values():
    """The oracle works with the float32 values the device receives.

    Expected values use hand-written float32 constants, not the oracle's
    rounding helper: zero gradient and zero momentum give O = 0 and
    W1 = W (1 - lr wd) with lr = wd = fl32(0.1); zero gradient and M0 = 1 give
    M1 = fl32(0.95).  Products of two 24-bit significands are exact in float64,
    so both comparisons are exact.
    """
    assert mo.as_f32_value(0.02) == F32_OF_0_02
    assert mo.as_f32_value(0.95) == F32_OF_0_95
    d = [mo.MatrixDesc(0, 1, 1, 0)]
    p64, _, _ = mo.muon_step(np.array([1.0], np.float32), np.zeros(1, np.float32),
                             np.zeros(1, np.float32), d, lr=0.1, weight_decay=0.1, beta=0.5)
    assert p64[0] == 1.0 - F32_OF_0_1 * F32_OF_0_1
    _, m64, _ = mo.muon_step(np.array([1.0], np.float32), np.zeros(1, np.float32),
                             np.ones(1, np.float32), d, lr=0.0, weight_decay=0.0, beta=0.95)
    assert m64[0] == F32_OF_0_95


def test_update_direction_opposes_gradient_1x1():
    """1x1, W = 0, g > 0: W1 = -lr f^5(g/(g+eps)) exactly in rationals."""
    g = 0.25
    p64, _, upd = mo.muon_step(np.zeros(1, np.float32), np.array([g], np.float32),
                               np.zeros(1, np.float32), [mo.MatrixDesc(0, 1, 1, 0)],
                               lr=0.5, weight_decay=0.0, beta=0.0, nesterov=False)
    sigma = Fraction(g) / (Fraction(g) + Fraction(EPS))
    want = -Fraction(0.5) * quintic_iter(sigma, 5)
    assert p64[0] < 0
    assert abs(Fraction(p64[0]) - want) < Fraction(1, 10 ** 14)


# ---------------------------------------------------- Newton-Schulz values

def test_quintic_at_one_exact_values():
    """f(1) = a+b+c = 0.701; iterates of 1 through the quintic, exact rationals."""
    assert quintic(Fraction(1)) == Fraction("0.701")
    want = [0.701, 1.113620216, 0.720705950, 1.089974202, 0.696436409469752]
    for k, v in enumerate(want, start=1):
        assert abs(float(quintic_iter(Fraction(1), k)) - v) < 5e-10


@pytest.mark.parametrize("g", [1.0, -3.0, 1e-7, 2.5e-7])
def test_newton_schulz_1x1_exact(g):
    """1x1 input g: X0 = g/(|g|+eps) and each step is the scalar quintic.

    g = 1e-7 makes sigma = 1/2 exactly: a misplaced epsilon (inside a square
    root, or multiplied) changes the result by far more than the tolerance.
    """
    out = mo.newton_schulz(np.array([[g]]), 5)
    fg = Fraction(g)
    sigma = abs(fg) / (abs(fg) + Fraction(EPS))
    want = quintic_iter(sigma, 5) * (1 if g > 0 else -1)
    assert abs(Fraction(out[0, 0]) - want) < Fraction(1, 10 ** 13)


def test_newton_schulz_zero_matrix():
    assert np.array_equal(mo.newton_schulz(np.zeros((3, 7)), 5), np.zeros((3, 7)))


@pytest.mark.parametrize("shape", [(8, 8), (6, 10), (10, 6), (1, 5), (5, 1), (32, 48),
                                   (48, 32), (17, 3)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_newton_schulz_singular_value_closed_form(shape, steps):
    """G = P diag(s) Q^T  =>  NS(G) = scale * P diag(f^k(s/(||s||+eps))) Q^T."""
    rows, cols = shape
    k = min(rows, cols)
    rng = np.random.default_rng([rows, cols, steps])
    p = orthonormal(rng, rows, k)
    q = orthonormal(rng, cols, k)
    s = rng.uniform(0.05, 2.0, k)
    g = (p * s) @ q.T
    sigma = s / (np.sqrt(np.sum(s * s)) + EPS)
    scale = math.sqrt(max(1.0, rows / cols))
    want = scale * (p * quintic_f64(sigma, steps)) @ q.T
    got = mo.newton_schulz(g, steps)
    assert got.shape == (rows, cols)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


@pytest.mark.parametrize("shape", [(8, 8), (6, 10), (1, 5), (3, 40), (16, 48)])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_left_factor_closed_form(shape, steps):
    """U = P diag(s) Q^T (rows <= cols)  =>  the Gram form's factor is
    F = P diag(f^k(sigma) / s) P^T, sigma = s / (||s|| + eps), so that
    F U = P diag(f^k(sigma)) Q^T: the singular-value closed form of the
    iteration, reached from U U^T alone."""
    rows, cols = shape
    rng = np.random.default_rng([rows, cols, steps, 2])
    p = orthonormal(rng, rows, rows)
    q = orthonormal(rng, cols, rows)
    s = rng.uniform(0.05, 2.0, rows)
    u = (p * s) @ q.T
    sigma = s / (np.sqrt(np.sum(s * s)) + EPS)
    want = (p * (quintic_f64(sigma, steps) / s)) @ p.T
    got = mo.newton_schulz_left_factor(u @ u.T, steps)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11 * max(1.0, np.abs(want).max()))
    np.testing.assert_allclose(got @ u, (p * quintic_f64(sigma, steps)) @ q.T, rtol=0,
                               atol=1e-11)


@pytest.mark.parametrize("rank", [1, 2, 4])
def test_left_factor_matches_the_direct_iteration(rank):
    """F U against newton_schulz(U) on random 4 x 30 inputs of full and lower rank."""
    rng = np.random.default_rng([rank, 30])
    u = rng.standard_normal((4, rank)) @ rng.standard_normal((rank, 30))
    for steps in (1, 5):
        got = mo.newton_schulz_left_factor(u @ u.T, steps) @ u
        np.testing.assert_allclose(got, mo.newton_schulz(u, steps), rtol=0, atol=1e-12)


def test_shape_scale_values():
    assert mo.shape_scale(14336, 4096) == math.sqrt(3.5)
    assert mo.shape_scale(4096, 14336) == 1.0
    assert abs(mo.shape_scale(18432, 7168) - 1.603567) < 1e-6
    assert mo.shape_scale(5, 5) == 1.0


def test_rank_one_input():
    """g u v^T (unit u, v): one singular value 1/(1+eps/|g|), output f^5 u v^T."""
    rng = np.random.default_rng(4)
    u = rng.standard_normal(7)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(11)
    v /= np.linalg.norm(v)
    out = mo.newton_schulz(40.0 * np.outer(u, v), 5)
    f5 = float(quintic_iter(Fraction(40.0) / (Fraction(40.0) + Fraction(EPS)), 5))
    np.testing.assert_allclose(out, f5 * np.outer(u, v), atol=1e-14)


def test_orthogonal_input():
    """n x n orthogonal Q has ||Q||_F = sqrt(n): output f^5(1/sqrt(n)) Q."""
    rng = np.random.default_rng(5)
    n = 9
    q = orthonormal(rng, n, n)
    out = mo.newton_schulz(q, 5)
    sigma = 1.0 / (math.sqrt(n) + EPS)
    np.testing.assert_allclose(out, quintic_f64(np.array(sigma), 5) * q, atol=1e-13)


def test_output_band_for_well_conditioned_input():
    """Singular values entering within [0.005184, 1] leave 5 steps in about [0.68, 1.13]."""
    rng = np.random.default_rng(6)
    rows, cols = 16, 40
    p = orthonormal(rng, rows, rows)
    q = orthonormal(rng, cols, rows)
    s = rng.uniform(0.3, 1.0, rows)  # sigma = s/||s|| lies in [0.07, 0.34]
    out = mo.newton_schulz((p * s) @ q.T, 5)
    sv = np.linalg.svd(out, compute_uv=False)
    assert sv.min() >= 0.6818 and sv.max() <= 1.1344
    assert np.linalg.norm(out - p @ q.T, 2) <= 0.32


# ----------------------------------------------------------- invariants

def test_oddness_exact():
    g = np.random.default_rng(7).standard_normal((5, 9))
    assert np.array_equal(mo.newton_schulz(-g, 5), -mo.newton_schulz(g, 5))


def test_scale_invariance():
    g = 1e3 * np.random.default_rng(8).standard_normal((6, 11))
    np.testing.assert_allclose(mo.newton_schulz(3.7 * g, 5), mo.newton_schulz(g, 5),
                               atol=1e-9)


@pytest.mark.parametrize("shape", [(6, 11), (11, 6), (8, 8)])
def test_orthogonal_equivariance(shape):
    rng = np.random.default_rng(9)
    g = rng.standard_normal(shape)
    p = orthonormal(rng, shape[0], shape[0])
    q = orthonormal(rng, shape[1], shape[1])
    np.testing.assert_allclose(mo.newton_schulz(p @ g @ q, 5), p @ mo.newton_schulz(g, 5) @ q,
                               atol=1e-12)


@pytest.mark.parametrize("shape", [(6, 11), (13, 4)])
def test_transposition(shape):
    g = np.random.default_rng(10).standard_normal(shape)
    r, c = shape
    left = mo.newton_schulz(g.T, 5) / mo.shape_scale(c, r)
    right = (mo.newton_schulz(g, 5) / mo.shape_scale(r, c)).T
    np.testing.assert_allclose(left, right, atol=1e-12)


# ------------------------------------------------------------ flat layout

def _rand_flat(rng, n):
    return rng.standard_normal(n).astype(np.float32)


def test_descriptor_order_does_not_matter():
    rng = np.random.default_rng(11)
    descs = [mo.MatrixDesc(0, 4, 6, 0), mo.MatrixDesc(24, 7, 3, 24), mo.MatrixDesc(48, 5, 5, 48)]
    n = 73
    w, g, m = _rand_flat(rng, n), _rand_flat(rng, n), _rand_flat(rng, n)
    kw = dict(lr=0.02, weight_decay=0.01, beta=0.95)
    p1, m1, u1 = mo.muon_step(w, g, m, descs, **kw)
    p2, m2, u2 = mo.muon_step(w, g, m, descs[::-1], **kw)
    assert np.array_equal(p1, p2) and np.array_equal(m1, m2)
    assert all(np.array_equal(u1[i], u2[2 - i]) for i in range(3))
    # elements outside every descriptor are untouched
    assert np.array_equal(p1[45:48], w[45:48].astype(np.float64))


def test_sharded_scatter_equals_contiguous():
    """Splitting a matrix's destination into slices leaves the math unchanged."""
    rng = np.random.default_rng(12)
    rows, cols, shards = 6, 8, 4
    n = rows * cols
    per = n // shards
    stride = per + 5  # slices separated by gaps the step must not touch
    g, m = _rand_flat(rng, n), _rand_flat(rng, n)
    w_contig = _rand_flat(rng, n)
    w_sharded = np.full(3 + shards * stride, 123.0, np.float32)
    for k in range(shards):
        w_sharded[3 + k * stride:3 + k * stride + per] = w_contig[k * per:(k + 1) * per]
    kw = dict(lr=0.02, weight_decay=0.01, beta=0.95)
    pc, mc, uc = mo.muon_step(w_contig, g, m, [mo.MatrixDesc(0, rows, cols, 0)], **kw)
    ps, ms, us = mo.muon_step(w_sharded, g, m,
                              [mo.MatrixDesc(0, rows, cols, 3, stride, shards)], **kw)
    assert np.array_equal(mc, ms) and np.array_equal(uc[0], us[0])
    touched = np.zeros(w_sharded.size, bool)
    for k in range(shards):
        sl = slice(3 + k * stride, 3 + k * stride + per)
        assert np.array_equal(ps[sl], pc[k * per:(k + 1) * per])
        touched[sl] = True
    assert np.all(ps[~touched] == 123.0)


def test_matrices_are_independent():
    rng = np.random.default_rng(13)
    d0, d1 = mo.MatrixDesc(0, 3, 5, 0), mo.MatrixDesc(15, 5, 2, 15)
    w, g, m = _rand_flat(rng, 25), _rand_flat(rng, 25), _rand_flat(rng, 25)
    kw = dict(lr=0.1, weight_decay=0.1, beta=0.5)
    both, _, _ = mo.muon_step(w, g, m, [d0, d1], **kw)
    only0, _, _ = mo.muon_step(w, g, m, [d0], **kw)
    only1, _, _ = mo.muon_step(w, g, m, [d1], **kw)
    assert np.array_equal(both[:15], only0[:15]) and np.array_equal(both[15:], only1[15:])


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3E80, 0x8000], np.uint16)
    want = [1.0, -2.0, math.inf, 2.0 ** -133, 0.25, -0.0]
    got = mo.bf16_bits_to_f64(bits)
    assert list(got) == want
    assert math.copysign(1, got[-1]) == -1


def test_bf16_params_step_uses_exact_widening():
    w_bits = np.array([0x3F80, 0x4000, 0xBF80, 0x3F00], np.uint16)  # 1, 2, -1, 0.5
    p64, _, _ = mo.muon_step(w_bits, np.zeros(4, np.float32), np.zeros(4, np.float32),
                             [mo.MatrixDesc(0, 2, 2, 0)], lr=0.5, weight_decay=0.5, beta=0.0,
                             param_dtype="bf16")
    assert list(p64) == [0.75, 1.5, -0.75, 0.375]


# -------------------------------------------- same-order float32 reference

def round_f32(x: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational: nearest, ties to even."""
    c = np.float32(float(x))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = None
    for v in cands:
        err = abs(Fraction(float(v)) - x)
        key = (err, int(np.array(v, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def exact_front(g, m, beta, nesterov):
    b = Fraction(float(np.float32(beta)))
    m1 = round_f32(round_f32(b * Fraction(float(m))) + Fraction(float(g)))
    if not nesterov:
        return m1, m1
    u = round_f32(round_f32(b * Fraction(float(m1))) + Fraction(float(g)))
    return m1, u


@pytest.mark.parametrize("nesterov", [True, False])
def test_same_order_front_matches_exact_rounding(nesterov):
    rng = np.random.default_rng(14)
    g = (rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400))).astype(np.float32)
    m = (rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400))).astype(np.float32)
    beta = 0.95
    m1, u = so.front(g, m, beta, nesterov)
    for i in range(400):
        em1, eu = exact_front(g[i], m[i], beta, nesterov)
        assert m1[i].view(np.uint32) == em1.view(np.uint32)
        assert u[i].view(np.uint32) == eu.view(np.uint32)


def nearest_bf16_bits(x: np.float32) -> int:
    """Brute force: the nearer of the two bfloat16 neighbours, ties to even."""
    bits = int(np.array(x, np.float32).view(np.uint32))
    lo = bits >> 16
    hi = lo + 1
    val = Fraction(float(x))

    def as_frac(b):
        if (b & 0x7F80) == 0x7F80:  # rounding up reaches infinity: weigh it as 2^128
            return Fraction(2) ** 128 * (-1 if b & 0x8000 else 1)
        return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))

    flo, fhi = as_frac(lo), as_frac(hi)
    dl, dh = abs(val - flo), abs(fhi - val)
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi


def test_bf16_rounding_matches_definition():
    rng = np.random.default_rng(15)
    vals = (rng.standard_normal(2000) * np.exp(rng.uniform(-30, 30, 2000))).astype(np.float32)
    # exact ties: low 16 bits == 0x8000, with even and odd kept parts
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00008000, 0x00018000],
                    np.uint32).view(np.float32)
    vals = np.concatenate([vals, ties])
    got = so.f32_to_bf16_bits(vals)
    for v, b in zip(vals, got):
        assert int(b) == nearest_bf16_bits(v), hex(int(np.array(v).view(np.uint32)))
    special = np.array([np.inf, -np.inf, np.nan, 3.4e38], np.float32)
    sb = so.f32_to_bf16_bits(special)
    assert sb[0] == 0x7F80 and sb[1] == 0xFF80
    assert (sb[2] & 0x7F80) == 0x7F80 and (sb[2] & 0x007F) != 0
    assert sb[3] == 0x7F80  # 3.4e38 is above the largest bfloat16 + half ulp


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_same_order_apply_matches_exact_rounding(dtype):
    rng = np.random.default_rng(16)
    n = 300
    w32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w = so.f32_to_bf16_bits(w32) if dtype == "bf16" else w32
    o = rng.standard_normal(n).astype(np.float32)
    lr, wd = 0.02, 0.01
    got = so.apply(w, o, lr, wd, dtype)
    lrq = Fraction(float(np.float32(lr)))
    f = round_f32(Fraction(1) - round_f32(lrq * Fraction(float(np.float32(wd)))))
    for i in range(n):
        wv = float(so.bf16_bits_to_f32(w[i:i + 1])[0]) if dtype == "bf16" else float(w[i])
        w1 = round_f32(Fraction(wv) * Fraction(float(f)))
        wn = round_f32(Fraction(float(w1)) - round_f32(lrq * Fraction(float(o[i]))))
        if dtype == "bf16":
            assert int(got[i]) == nearest_bf16_bits(wn)
        else:
            assert got[i].view(np.uint32) == wn.view(np.uint32)
