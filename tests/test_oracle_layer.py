"""Pins for the oracle's layer products (CPU only): the forward Y = X W^T with
XP = X P, and the backward dX = D W with C += D^T (X P) [RGC, "How it works"].

Checked against things other than the oracle's own formulas: explicit loops on
tiny inputs (operand order and transposes), the derivative of the layer's
scalar loss <D, X W^T> taken by finite differences (dX is its gradient in X),
the adjoint identity that makes the sketch C the weight gradient D^T X times
P, and the rounding of exactly representable results.
"""
import numpy as np

import oracle as orc


def _bits(a):
    return orc.f32_to_bf16_rne(np.asarray(a, dtype=np.float32))


def _rand_bits(shape, seed, scale=1.0):
    return _bits(np.random.default_rng(seed).standard_normal(shape) * scale)


def test_forward_matches_loops_on_tiny_inputs():
    T, k, d, r = 3, 5, 4, 2
    x, w, p = _rand_bits((T, k), 1), _rand_bits((d, k), 2), _rand_bits((k, r), 3)
    xv, wv, pv = orc.bf16_to_f64(x), orc.bf16_to_f64(w), orc.bf16_to_f64(p)
    y, xp = orc.layer_forward(x, w, p)
    for t in range(T):
        for j in range(d):
            acc = 0.0
            for i in range(k):
                acc += xv[t, i] * wv[j, i]  # column j of Y is row j of W against row t of X
            assert y[t, j] == _bits(acc)
        for a in range(r):
            assert xp[t, a] == _bits(sum(xv[t, i] * pv[i, a] for i in range(k)))


def test_backward_matches_loops_on_tiny_inputs():
    T, k, d, r = 3, 5, 4, 2
    dd, w, xp = _rand_bits((T, d), 4), _rand_bits((d, k), 5), _rand_bits((T, r), 6)
    c0 = np.random.default_rng(7).standard_normal((d, r)).astype(np.float32)
    dv, wv, xpv = orc.bf16_to_f64(dd), orc.bf16_to_f64(w), orc.bf16_to_f64(xp)
    dx, c = orc.layer_backward(dd, w, xp, c0)
    for t in range(T):
        for i in range(k):
            assert dx[t, i] == _bits(sum(dv[t, j] * wv[j, i] for j in range(d)))
    for j in range(d):
        for a in range(r):
            assert c[j, a] == np.float32(np.float64(c0[j, a]) + sum(dv[t, j] * xpv[t, a] for t in range(T)))


def test_input_gradient_is_the_derivative_of_the_layer_loss():
    """f(X) = <D, X W^T> is linear in X, so a unit step in X[t, i] changes f by
    exactly dX[t, i] (before dX's rounding); square W (d = k) so that a
    transposed W would have the same shape and still fail."""
    T, k = 4, 6
    x, w, dd = _rand_bits((T, k), 8), _rand_bits((k, k), 9), _rand_bits((T, k), 10)
    xv, wv, dv = orc.bf16_to_f64(x), orc.bf16_to_f64(w), orc.bf16_to_f64(dd)

    def f(xm):
        return float(np.sum(dv * (xm @ wv.T)))

    dx, _ = orc.layer_backward(dd, w, None, None)
    for t in range(T):
        for i in range(k):
            e = np.zeros_like(xv)
            e[t, i] = 1.0
            assert dx[t, i] == _bits(f(xv + e) - f(xv))


def test_sketch_is_the_weight_gradient_times_p():
    """D^T (X P) = (D^T X) P: the backward's C increment is the dense weight
    gradient of f(W) = <D, X W^T> (which is D^T X, by finite differences in W)
    projected by P."""
    T, k, d, r = 5, 6, 4, 3
    x, dd, p = _rand_bits((T, k), 11), _rand_bits((T, d), 12), _rand_bits((k, r), 13)
    w = _rand_bits((d, k), 14)
    xv, dv, pv = orc.bf16_to_f64(x), orc.bf16_to_f64(dd), orc.bf16_to_f64(p)
    wv = orc.bf16_to_f64(w)
    g = np.zeros((d, k))
    for j in range(d):
        for i in range(k):
            e = np.zeros_like(wv)
            e[j, i] = 1.0
            g[j, i] = np.sum(dv * (xv @ (wv + e).T)) - np.sum(dv * (xv @ wv.T))
    # XP kept in float64 here (before its bf16 rounding) to compare sums exactly
    c_exact = dv.T @ (xv @ pv)
    np.testing.assert_allclose(c_exact, g @ pv, rtol=1e-12, atol=1e-12)
    _, xp = orc.layer_forward(x, w, p)
    _, c = orc.layer_backward(dd, w, xp, np.zeros((d, r), np.float32))
    np.testing.assert_array_equal(c, orc.accumulate(np.zeros((d, r), np.float32), dd, xp))


def test_exact_results_round_to_themselves():
    """Small-integer operands give sums that bf16 holds exactly."""
    x = _bits(np.array([[1, 2, 0, -1], [3, 0, 1, 1]], dtype=np.float32))
    w = _bits(np.array([[1, 1, 1, 1], [0, 2, 0, 0], [-1, 0, 4, 1]], dtype=np.float32))
    y, _ = orc.layer_forward(x, w, None)
    np.testing.assert_array_equal(orc.bf16_to_f64(y), [[2, 4, -2], [5, 0, 2]])
    dx, _ = orc.layer_backward(_bits(np.array([[1, 0, 1]], dtype=np.float32)), w, None, None)
    np.testing.assert_array_equal(orc.bf16_to_f64(dx), [[0, 1, 5, 2]])
