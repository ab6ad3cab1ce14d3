"""Pins of the oracle's adapted-linear forward and backward.

"QLoRA, explained", The forward pass and gradients, and The algorithm, step by step. The forward
is checked against pure-Python loops on tiny sizes and exact special cases; the backward against the
forward by finite differences (the forward is linear in X, in A and in B separately, so a central
difference is exact up to float64 rounding).
"""
import numpy as np

import oracle
from workloads import to_bf16_bits


def _bits(rng, shape, sigma):
    return to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def _f(b):
    return oracle.f32_from_bf16_bits(b).astype(np.float64)


def _small(seed=0, m=3, n=5, k=7, r=2):
    rng = np.random.default_rng(seed)
    return (_bits(rng, (m, k), 1.0), _bits(rng, (n, k), 0.5), _bits(rng, (r, k), 0.3),
            _bits(rng, (n, r), 0.3), _bits(rng, (m, n), 1.0))


def test_forward_matches_loops():
    x, w, a, b, _ = _small()
    s = 2.0
    y, u = oracle.linear_fwd(x, w, a, b, s)
    X, W, A, B = _f(x), _f(w), _f(a), _f(b)
    m, k = X.shape; n = W.shape[0]; r = A.shape[0]
    for i in range(m):
        uu = [sum(X[i, t] * A[j, t] for t in range(k)) for j in range(r)]
        for j in range(r):
            assert abs(u[i, j] - uu[j]) <= 1e-12 * (1 + abs(uu[j]))
        for o in range(n):
            ref = sum(X[i, t] * W[o, t] for t in range(k)) + s * sum(uu[j] * B[o, j] for j in range(r))
            assert abs(y[i, o] - ref) <= 1e-12 * (1 + abs(ref))


def test_backward_matches_loops():
    x, w, a, b, dy = _small(1)
    s = 0.25
    dx, da, db = oracle.linear_bwd(x, dy, w, a, b, s)
    X, W, A, B, D = _f(x), _f(w), _f(a), _f(b), _f(dy)
    m, k = X.shape; n = W.shape[0]; r = A.shape[0]
    for i in range(m):
        for t in range(k):
            ref = sum(D[i, o] * (W[o, t] + s * sum(B[o, j] * A[j, t] for j in range(r))) for o in range(n))
            assert abs(dx[i, t] - ref) <= 1e-12 * (1 + abs(ref))
    for j in range(r):
        for t in range(k):
            ref = s * sum(B[o, j] * D[i, o] * X[i, t] for o in range(n) for i in range(m))
            assert abs(da[j, t] - ref) <= 1e-12 * (1 + abs(ref))
    for o in range(n):
        for j in range(r):
            ref = s * sum(D[i, o] * X[i, t] * A[j, t] for i in range(m) for t in range(k))
            assert abs(db[o, j] - ref) <= 1e-12 * (1 + abs(ref))


def test_backward_is_the_adjoint_of_forward():
    """<dY, dy/dZ . V> = <dZ, V> for Z in {X, A, B}, by central differences of the forward."""
    rng = np.random.default_rng(3)
    m, n, k, r, s = 6, 9, 16, 4, 2.0
    X, W, A, B, D = (rng.standard_normal(sh) for sh in [(m, k), (n, k), (r, k), (n, r), (m, n)])
    dx, da, db = oracle.linear_bwd_f64(X, D, W, A, B, s)
    eps = 1e-3
    for name, Z, G in (("x", X, dx), ("a", A, da), ("b", B, db)):
        V = rng.standard_normal(Z.shape)
        args = dict(x=X, a=A, b=B)
        args[name] = Z + eps * V
        yp, _ = oracle.linear_fwd_f64(args["x"], W, args["a"], args["b"], s)
        args[name] = Z - eps * V
        ym, _ = oracle.linear_fwd_f64(args["x"], W, args["a"], args["b"], s)
        fd = np.sum(D * (yp - ym)) / (2 * eps)
        assert abs(fd - np.sum(G * V)) <= 1e-9 * (1 + abs(fd)), name


def test_no_weight_gradient_and_w_enters_dx():
    """Changing W~ changes dX by dY . dW~ and leaves dA, dB unchanged (G does not involve W~)."""
    rng = np.random.default_rng(4)
    X, W, A, B, D = (rng.standard_normal(sh) for sh in [(4, 8), (5, 8), (2, 8), (5, 2), (4, 5)])
    dW = rng.standard_normal(W.shape)
    g1 = oracle.linear_bwd_f64(X, D, W, A, B, 2.0)
    g2 = oracle.linear_bwd_f64(X, D, W + dW, A, B, 2.0)
    assert np.allclose(g2[0] - g1[0], D @ dW, atol=1e-12)
    assert np.array_equal(g1[1], g2[1]) and np.array_equal(g1[2], g2[2])


def test_special_cases():
    rng = np.random.default_rng(5)
    m, n, k, r = 4, 6, 8, 2
    w = _bits(rng, (n, k), 1.0)
    a = _bits(rng, (r, k), 1.0)
    b0 = np.zeros((n, r), np.uint16)
    # one-hot rows of X with B = 0: y rows are columns of W~, exactly
    x = np.zeros((m, k), np.uint16)
    cols = [0, 3, 5, 7]
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80                                       # bf16 1.0
    y, _ = oracle.linear_fwd(x, w, a, b0, 2.0)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], _f(w)[:, c])
    # one-hot rows of dY with B = 0: dX rows are rows of W~
    dy = np.zeros((m, n), np.uint16)
    for i in range(m):
        dy[i, i] = 0x3F80
    dx, _, _ = oracle.linear_bwd(x, dy, w, a, b0, 2.0)
    for i in range(m):
        assert np.array_equal(dx[i], _f(w)[i])
    # zero W: y is the adapter term alone
    b = _bits(rng, (n, r), 1.0)
    x = _bits(rng, (m, k), 1.0)
    y, u = oracle.linear_fwd(x, np.zeros((n, k), np.uint16), a, b, 0.5)
    assert np.allclose(y, 0.5 * (_f(x) @ _f(a).T) @ _f(b).T, rtol=0, atol=1e-12)
    # zero X: y = 0, u = 0, dA = 0 and dB = 0
    z = np.zeros((m, k), np.uint16)
    y, u = oracle.linear_fwd(z, w, a, b, 2.0)
    assert not y.any() and not u.any()
    _, da, db = oracle.linear_bwd(z, _bits(rng, (m, n), 1.0), w, a, b, 2.0)
    assert not da.any() and not db.any()


def test_sampled_backward_equals_full():
    x, w, a, b, dy = _small(6, m=9, n=12, k=16, r=4)
    full = oracle.linear_bwd(x, dy, w, a, b, 0.5)
    rows, cols, brows = [0, 5, 8], [1, 2, 15], [3, 11]
    dx, da, db = oracle.linear_bwd_sampled(x, dy, w, a, b, 0.5, rows, cols, brows)
    assert np.allclose(dx, full[0][rows], rtol=1e-13, atol=1e-13)
    assert np.allclose(da, full[1][:, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(db, full[2][brows], rtol=1e-13, atol=1e-13)
