"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle library handle (``oracle.load(path)``) so the
same checks can be run on deliberately broken builds of the oracle
(tests/test_oracle_mutants.py) to show that they catch plausible mistakes.

What the pins rest on (the pages print no numbers for a worked example, so
every expected value below is a closed form or a property of the definition):
  * hand arithmetic on 2x2 examples;
  * special cases that reduce to a library matmul (rows of unit RMS, eps = 0);
  * the closed form of a constant row, c / sqrt(c^2 + eps);
  * the normalised rows' mean square, S / (S + eps), when W = I;
  * invariants: scale law, gain folding, linearity, permutations;
  * exact rational / 50-digit brute force on tiny shapes;
  * the gate's closed forms at z = +-ln 3 (sigmoid = 3/4 and 1/4 exactly);
  * LoRA: a hand-worked 1x2 example, B = 0, and the merged-weight identity
    Act W + (Act A^T) B = Act (W + A^T B) on exactly representable inputs;
  * QKNorm + attention: a two-key closed form (scores sqrt 2 and 0), one key,
    identical keys, invariance to each key's scale (the norm removes it),
    only g_q * g_k mattering, key permutations, one-hot limits and overflow
    of large scores, 50-digit brute force.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle


def _mm(lib, X, g, W, eps):
    return oracle.rmsnorm_matmul(X, g, W, eps, lib=lib)


def _gated(lib, X, g, W1, W3, eps):
    return oracle.rmsnorm_gated_mlp(X, g, W1, W3, eps, lib=lib)


def _close(a, b, rtol=1e-12, atol=1e-14):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"max err {err.max():.3e} (worst at {np.unravel_index(np.argmax(err - lim), err.shape)})"


def pin_worked_example(lib):
    # X = [3, 4]: mean square (9 + 16) / 2 = 12.5; with eps = 12.5 the RMS is
    # sqrt(25) = 5, so the normalised row is [0.6, 0.8] and with g = [1, 2]
    # the gained row is [0.6, 1.6].
    X = np.array([[3.0, 4.0]])
    g = np.array([1.0, 2.0])
    _close(_mm(lib, X, g, np.eye(2), 12.5), [[0.6, 1.6]])
    # W rows are indexed by k: Y = [0.6*1 + 1.6*3, 0.6*2 + 1.6*4] = [5.4, 7.6].
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    _close(_mm(lib, X, g, W, 12.5), [[5.4, 7.6]])


def pin_library_matmul(lib):
    # Rows of +-1 (any sign pattern) have mean square exactly 1; with eps = 0
    # the RMS is 1 and the path reduces to (X * g) @ W, a library matmul.
    # Non-square, non-symmetric shapes catch a transposed operand or a gain
    # indexed by the wrong axis.
    rng = np.random.default_rng(11)
    for (M, K, N) in ((3, 5, 7), (4, 9, 2), (1, 1, 3), (6, 4, 4)):
        X = rng.choice([-1.0, 1.0], size=(M, K))
        g = rng.normal(1.0, 0.3, size=K)
        W = rng.normal(size=(K, N))
        _close(_mm(lib, X, g, W, 0.0), (X * g[None, :]) @ W)
        # Rows of constant magnitude c_m: the RMS is c_m, so X / RMS = sign(X).
        c = rng.uniform(0.1, 10.0, size=(M, 1))
        _close(_mm(lib, X * c, g, W, 0.0), (X * g[None, :]) @ W)


def pin_identity_weight(lib):
    # W = I, g = 1: Y is RMSNorm(X) itself; every output row has mean square
    # S / (S + eps) where S is the input row's mean square.
    rng = np.random.default_rng(12)
    M, K = 5, 8
    X = rng.normal(size=(M, K)) * rng.uniform(0.1, 3.0, size=(M, 1))
    for eps in (0.0, 0.3, 2.0):
        Y = _mm(lib, X, np.ones(K), np.eye(K), eps)
        S = np.mean(X * X, axis=1)
        _close(np.mean(Y * Y, axis=1), S / (S + eps))
        # and each output row is a positive multiple of its input row
        ratio = Y / X
        _close(ratio, np.repeat(ratio[:, :1], K, axis=1))
        assert np.all(ratio[:, 0] > 0)


def pin_constant_row(lib):
    # A row of constant value c has mean square c^2 for any K, so every
    # output is c / sqrt(c^2 + eps) * sum_k g_k W[k, n].
    rng = np.random.default_rng(13)
    K, N = 6, 5
    g = rng.normal(1.0, 0.1, size=K)
    W = rng.normal(size=(K, N))
    for c, eps, factor in ((1e-3, 1e-6, 1.0 / math.sqrt(2.0)),
                           (2.0, 0.0, 1.0),
                           (0.01, 1e-5, 0.9534625892455924),
                           (-0.5, 0.75, -0.5)):
        X = np.full((2, K), c)
        _close(_mm(lib, X, g, W, eps), np.repeat((factor * (g @ W))[None, :], 2, axis=0))


def pin_scale_law(lib):
    # Scaling a row by alpha and eps by alpha^2 leaves Y unchanged.
    rng = np.random.default_rng(14)
    M, K, N = 4, 7, 3
    X = rng.normal(size=(M, K))
    g = rng.normal(1.0, 0.1, size=K)
    W = rng.normal(size=(K, N))
    base = _mm(lib, X, g, W, 0.25)
    for alpha in (3.7, 1e-3, 256.0):
        _close(_mm(lib, alpha * X, g, W, 0.25 * alpha * alpha), base, rtol=1e-11)
    # With eps = 0 a per-row positive scale drops out; a negative one flips the row.
    s = rng.uniform(0.01, 100.0, size=(M, 1))
    _close(_mm(lib, s * X, g, W, 0.0), _mm(lib, X, g, W, 0.0), rtol=1e-11)
    _close(_mm(lib, -X, g, W, 0.0), -_mm(lib, X, g, W, 0.0), rtol=1e-11)


def pin_gain_fold(lib):
    # sum_k X g W = X (diag(g) W): the gain can move from the activation to W.
    rng = np.random.default_rng(15)
    M, K, N = 3, 6, 4
    X = rng.normal(size=(M, K))
    g = rng.normal(1.0, 0.5, size=K)
    W = rng.normal(size=(K, N))
    _close(_mm(lib, X, g, W, 0.1), _mm(lib, X, np.ones(K), g[:, None] * W, 0.1))


def pin_structure(lib):
    rng = np.random.default_rng(16)
    M, K, N = 5, 6, 4
    X = rng.normal(size=(M, K))
    g = rng.normal(1.0, 0.2, size=K)
    W1 = rng.normal(size=(K, N))
    W2 = rng.normal(size=(K, N))
    eps = 0.05
    # linear in W
    _close(_mm(lib, X, g, 2.0 * W1 - 3.0 * W2, eps),
           2.0 * _mm(lib, X, g, W1, eps) - 3.0 * _mm(lib, X, g, W2, eps), rtol=1e-11, atol=1e-12)
    # permuting rows of X permutes rows of Y
    p = rng.permutation(M)
    _close(_mm(lib, X[p], g, W1, eps), _mm(lib, X, g, W1, eps)[p])
    # a common permutation of k in X, g and W changes nothing
    q = rng.permutation(K)
    _close(_mm(lib, X[:, q], g[q], W1[q], eps), _mm(lib, X, g, W1, eps))
    # rows are independent: a single row gives the same result as in the batch
    _close(_mm(lib, X[2:3], g, W1, eps), _mm(lib, X, g, W1, eps)[2:3])
    # permuting columns of W permutes columns of Y
    r = rng.permutation(N)
    _close(_mm(lib, X, g, W1[:, r], eps), _mm(lib, X, g, W1, eps)[:, r])


def pin_zero_row(lib):
    rng = np.random.default_rng(17)
    K, N = 5, 3
    X = rng.normal(size=(3, K))
    X[1] = 0.0
    Y = _mm(lib, X, rng.normal(size=K), rng.normal(size=(K, N)), 1e-6)
    assert np.all(Y[1] == 0.0)
    assert np.all(np.isfinite(Y))


def _brute(X, g, W, eps):
    """Exact rationals for the k-sums and the mean square, 50-digit sqrt."""
    getcontext().prec = 50
    M, K = len(X), len(X[0])
    N = len(W[0])
    out = []
    for m in range(M):
        S = sum(Fraction(X[m][k]) ** 2 for k in range(K)) / K + Fraction(eps)
        rms = Decimal(S.numerator).sqrt() / Decimal(S.denominator).sqrt()
        row = []
        for n in range(N):
            num = sum(Fraction(X[m][k]) * Fraction(g[k]) * Fraction(W[k][n]) for k in range(K))
            row.append(float(Decimal(num.numerator) / Decimal(num.denominator) / rms))
        out.append(row)
    return np.array(out)


def pin_brute_force(lib):
    rng = np.random.default_rng(18)
    for _ in range(12):
        M, K, N = (int(v) for v in rng.integers(1, 6, size=3))
        X = rng.normal(size=(M, K))
        g = rng.normal(1.0, 0.3, size=K)
        W = rng.normal(size=(K, N))
        eps = float(rng.choice([0.0, 1e-6, 0.5]))
        X[0, 0] += 0.1  # keep row 0 away from zero
        _close(_mm(lib, X, g, W, eps), _brute(X.tolist(), g.tolist(), W.tolist(), eps),
               rtol=1e-13, atol=1e-15)


def pin_gated_closed_forms(lib):
    # X = [1, 1], g = 1, eps = 0: the normalised row is [1, 1] and each output
    # column's pre-activation is the column sum of the weight.
    ln3 = math.log(3.0)
    X = np.array([[1.0, 1.0]])
    g = np.ones(2)
    W1 = np.array([[ln3 / 2, 0.0, -ln3 / 2, 20.0], [ln3 / 2, 0.0, -ln3 / 2, 20.0]])
    W3 = np.array([[1.0, 2.5, 0.5, 0.25], [1.0, 2.5, 0.5, 0.25]])
    # z1 = [ln3, 0, -ln3, 40], z3 = [2, 5, 1, 0.5]; sigmoid(ln3) = 3/4,
    # sigmoid(-ln3) = 1/4, sigmoid(40) = 1 to double precision.
    want = [[0.75 * ln3 * 2.0, 0.0, -0.25 * ln3 * 1.0, 40.0 * 0.5]]
    _close(_gated(lib, X, g, W1, W3, 0.0), want)
    # W3 = W1: y = z^2 sigmoid(z)
    _close(_gated(lib, X, g, W1[:, :3], W1[:, :3], 0.0),
           [[0.75 * ln3 * ln3, 0.0, 0.25 * ln3 * ln3]])
    # The worked example of pin_worked_example gated with W3 = I:
    # z1 = [5.4, 7.6], z3 = [0.6, 1.6].
    Xw = np.array([[3.0, 4.0]])
    gw = np.array([1.0, 2.0])
    Ww = np.array([[1.0, 2.0], [3.0, 4.0]])
    _close(_gated(lib, Xw, gw, Ww, np.eye(2), 12.5),
           [[3.225432074958551, 12.153917554537914]], rtol=1e-13)
    # The gate uses the same normalised activations as the plain path.
    rng = np.random.default_rng(19)
    Xr = rng.normal(size=(3, 5))
    gr = rng.normal(1.0, 0.1, size=5)
    Wa = rng.normal(size=(5, 4))
    z = _mm(lib, Xr, gr, Wa, 1e-3)
    ones = np.zeros((5, 4))
    ones[0] = 1.0  # z3 = Nrm[:, 0] (first normalised column)
    y = _gated(lib, Xr, gr, Wa, ones, 1e-3)
    nrm0 = _mm(lib, Xr, gr, np.eye(5)[:, :1], 1e-3)
    _close(y, z / (1.0 + np.exp(-z)) * nrm0, rtol=1e-12)


def _brute_rows(X, g, eps):
    """Exact rationals for the mean square, 50-digit sqrt: (X / r) * g."""
    getcontext().prec = 50
    out = []
    for row in X:
        S = sum(Fraction(v) ** 2 for v in row) / len(row) + Fraction(eps)
        rms = Decimal(S.numerator).sqrt() / Decimal(S.denominator).sqrt()
        out.append([float(Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) / rms
                          * Decimal(Fraction(gk).numerator) / Decimal(Fraction(gk).denominator))
                    for v, gk in zip(row, g)])
    return np.array(out)


def pin_unfused_steps(lib):
    # The unfused program's pieces on their own.  Worked example: X = [3, 4],
    # eps = 12.5 -> RMS 5, normalised [0.6, 0.8], gained by g = [1, 2].
    _close(oracle.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 12.5, lib=lib),
           [[0.6, 1.6]])
    # Hand product with k-indexed rows of B: [[0,1,2],[3,4,5]] @ [[0..3],[4..7],[8..11]].
    A = np.arange(6.0).reshape(2, 3)
    B = np.arange(12.0).reshape(3, 4)
    _close(oracle.matmul(A, B, lib=lib), [[20, 23, 26, 29], [56, 68, 80, 92]])
    # Brute force: exact rationals for the rows and for integer products.
    rng = np.random.default_rng(21)
    for _ in range(8):
        M, K, N = (int(v) for v in rng.integers(1, 6, size=3))
        X = rng.normal(size=(M, K))
        X[:, 0] += 0.5
        g = rng.normal(1.0, 0.3, size=K)
        eps = float(rng.choice([0.0, 1e-6, 0.5]))
        _close(oracle.rmsnorm(X, g, eps, lib=lib), _brute_rows(X.tolist(), g.tolist(), eps),
               rtol=1e-14, atol=1e-15)
        Ai = rng.integers(-9, 10, size=(M, K))
        Bi = rng.integers(-9, 10, size=(K, N))
        want = [[sum(int(Ai[m, k]) * int(Bi[k, n]) for k in range(K)) for n in range(N)]
                for m in range(M)]
        assert np.array_equal(oracle.matmul(Ai, Bi, lib=lib), np.array(want, np.float64))
    # Gate closed forms on given activations A = [1, 1]: z1 = column sums.
    ln3 = math.log(3.0)
    W1 = np.array([[ln3 / 2, 0.0, -ln3 / 2], [ln3 / 2, 0.0, -ln3 / 2]])
    W3 = np.array([[1.0, 2.5, 0.5], [1.0, 2.5, 0.5]])
    _close(oracle.gated_matmul(np.ones((1, 2)), W1, W3, lib=lib),
           [[0.75 * ln3 * 2.0, 0.0, -0.25 * ln3 * 1.0]])
    # The pieces compose to the fused definition exactly (same operations).
    X = rng.normal(size=(4, 6))
    g = rng.normal(1.0, 0.2, size=6)
    W = rng.normal(size=(6, 5))
    W3r = rng.normal(size=(6, 5))
    n = oracle.rmsnorm(X, g, 1e-3, lib=lib)
    assert np.array_equal(oracle.matmul(n, W, lib=lib), _mm(lib, X, g, W, 1e-3))
    assert np.array_equal(oracle.gated_matmul(n, W, W3r, lib=lib), _gated(lib, X, g, W, W3r, 1e-3))


def pin_lora(lib):
    # Hand-worked: X = [3, 4], g = [1, 2], eps = 12.5 -> Nrm = [0.6, 1.6];
    # W = [[1, 0], [1, 2]] -> Nrm W = [2.2, 3.2].  Rank 1: A = [1, -1] gives
    # T = -1, B = [2, -1] adds [-2, 1].  Rank 2 adds A row [0, 1] (T = 1.6)
    # with B row [1, 1]: T B = [-2 + 1.6, 1 + 1.6].
    X, g = np.array([[3.0, 4.0]]), np.array([1.0, 2.0])
    W = np.array([[1.0, 0.0], [1.0, 2.0]])
    A, B = np.array([[1.0, -1.0], [0.0, 1.0]]), np.array([[2.0, -1.0], [1.0, 1.0]])
    _close(oracle.rmsnorm_lora(X, g, W, A[:1], B[:1], 12.5, lib=lib), [[0.2, 4.2]])
    _close(oracle.rmsnorm_lora(X, g, W, A, B, 12.5, lib=lib), [[1.8, 5.8]])
    # Without the norm, by hand: X W = [7, 8], X A^T = [-1, 4], T B = [-2 + 4, 1 + 4].
    _close(oracle.lora_matmul(X, W, A, B, lib=lib), [[9.0, 13.0]])
    rng = np.random.default_rng(33)
    for (M, K, N, R) in ((3, 8, 5, 2), (4, 6, 7, 6), (2, 5, 3, 9), (1, 1, 1, 1)):
        # B = 0: the plain fused product, bit for bit.
        Xf = rng.normal(size=(M, K))
        gf = rng.normal(1.0, 0.2, size=K)
        Wf = rng.normal(size=(K, N))
        Af = rng.normal(size=(R, K))
        assert np.array_equal(oracle.rmsnorm_lora(Xf, gf, Wf, Af, np.zeros((R, N)), 1e-3, lib=lib),
                              _mm(lib, Xf, gf, Wf, 1e-3))
        # Merged weights on exact inputs: rows of +-2^j (RMS 2^j with eps = 0),
        # small-integer g, W, A, B; every value is a short dyadic rational, so
        # both sides are exact and must agree bit for bit.  R = K (case 2)
        # tells A from A^T.
        Xi = rng.choice([-1.0, 1.0], size=(M, K)) * np.exp2(rng.integers(-3, 4, size=(M, 1)))
        gi = rng.integers(1, 4, size=K).astype(np.float64)
        Wi = rng.integers(-3, 4, size=(K, N)).astype(np.float64)
        Ai = rng.integers(-3, 4, size=(R, K)).astype(np.float64)
        Bi = rng.integers(-3, 4, size=(R, N)).astype(np.float64)
        merged = Wi + Ai.T @ Bi
        assert np.array_equal(oracle.rmsnorm_lora(Xi, gi, Wi, Ai, Bi, 0.0, lib=lib),
                              _mm(lib, Xi, gi, merged, 0.0))
        assert np.array_equal(oracle.lora_matmul(Xi, Wi, Ai, Bi, lib=lib), Xi @ merged)
        # Brute force: 50-digit rows, then exact-rational sums of the two terms.
        eps = 0.25
        nrm = _brute_rows(Xf.tolist(), gf.tolist(), eps)
        Bf = rng.normal(size=(R, N))
        T = [[sum(Fraction(nrm[m, k]) * Fraction(Af[r, k]) for k in range(K)) for r in range(R)]
             for m in range(M)]
        want = [[float(sum(Fraction(nrm[m, k]) * Fraction(Wf[k, n]) for k in range(K))
                       + sum(T[m][r] * Fraction(Bf[r, n]) for r in range(R)))
                 for n in range(N)] for m in range(M)]
        _close(oracle.rmsnorm_lora(Xf, gf, Wf, Af, Bf, eps, lib=lib), want, rtol=1e-12, atol=1e-12)


def _attn(lib, Q, K, V, gq, gk, eps):
    return oracle.qknorm_attention(Q, K, V, gq, gk, eps, lib=lib)


def _brute_attention(Q, K, V, gq, gk, eps):
    getcontext().prec = 50
    D = lambda x: Decimal(Fraction(float(x)).numerator) / Decimal(Fraction(float(x)).denominator)
    out = []
    for h in range(Q.shape[0]):
        def norm(x, g):
            S = sum(D(v) ** 2 for v in x) / len(x) + D(eps)
            r = S.sqrt()
            return [D(v) / r * D(gg) for v, gg in zip(x, g)]
        qn = norm(Q[h], gq)
        sc = []
        for s in range(K.shape[1]):
            kn = norm(K[h, s], gk)
            sc.append(sum(a * b for a, b in zip(qn, kn)) / Decimal(K.shape[2]).sqrt())
        mx = max(sc)
        e = [(x - mx).exp() for x in sc]
        den = sum(e)
        out.append([float(sum(e[s] / den * D(V[h, s, d]) for s in range(K.shape[1])))
                    for d in range(K.shape[2])])
    return np.array(out)


def pin_qknorm_attention(lib):
    # Two keys, D = 2: q = [1, 0], k0 = [1, 0], k1 = [0, 1], unit gains, eps = 0:
    # normalised q = k0 = [sqrt 2, 0], k1 = [0, sqrt 2]; scores 2 / sqrt 2 and 0.
    Q = np.array([[1.0, 0.0]])
    K = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    V = np.array([[[1.0, 2.0], [3.0, 5.0]]])
    one = np.ones(2)
    p0 = math.exp(math.sqrt(2.0)) / (math.exp(math.sqrt(2.0)) + 1.0)
    _close(_attn(lib, Q, K, V, one, one, 0.0), [[p0 * 1 + (1 - p0) * 3, p0 * 2 + (1 - p0) * 5]])
    rng = np.random.default_rng(41)
    for (BH, S, D) in ((3, 5, 8), (2, 1, 4), (4, 7, 16)):
        Q = rng.normal(size=(BH, D))
        K = rng.normal(size=(BH, S, D))
        V = rng.normal(size=(BH, S, D))
        gq = rng.normal(1.0, 0.3, size=D)
        gk = rng.normal(1.0, 0.3, size=D)
        ref = _attn(lib, Q, K, V, gq, gk, 0.0)
        # one key: the weight is exactly 1
        assert np.array_equal(_attn(lib, Q, K[:, :1], V[:, :1], gq, gk, 1e-3), V[:, 0])
        # identical keys: uniform weights, the mean of the values
        Ks = np.repeat(K[:, :1], S, axis=1)
        _close(_attn(lib, Q, Ks, V, gq, gk, 1e-3), V.mean(axis=1))
        # each key's scale (powers of two: exact) is removed by its norm (eps = 0)
        scale = np.exp2(rng.integers(-4, 5, size=(BH, S, 1)))
        assert np.array_equal(_attn(lib, Q, K * scale, V, gq, gk, 0.0), ref)
        # only the product of the gains enters the score
        _close(_attn(lib, Q, K, V, gq * gk, np.ones(D), 0.0), ref, rtol=1e-12, atol=1e-13)
        # keys (with their values) in another order
        perm = rng.permutation(S)
        _close(_attn(lib, Q, K[:, perm], V[:, perm], gq, gk, 0.0), ref, rtol=1e-12, atol=1e-13)
        # brute force at 50 digits
        eps = 0.125
        _close(_attn(lib, Q, K, V, gq, gk, eps), _brute_attention(Q, K, V, gq, gk, eps),
               rtol=1e-12, atol=1e-13)
    # One-hot limit and overflow: with gains of 40 the aligned key's score is
    # 1600 sqrt(D) above the others'; the result is that key's value, and the
    # maximum is subtracted before exp (exp(1600 sqrt 8) would overflow).
    D, S = 8, 6
    Q = rng.normal(size=(1, D))
    K = rng.normal(size=(1, S, D))
    K[0, 3] = Q[0] * 0.5
    V = rng.normal(size=(1, S, D))
    g = np.full(D, 40.0)
    _close(_attn(lib, Q, K, V, g, g, 0.0), V[:, 3], rtol=1e-12, atol=1e-12)


def _brute_plain_attention(Q, K, V):
    getcontext().prec = 50
    D = lambda x: Decimal(Fraction(float(x)).numerator) / Decimal(Fraction(float(x)).denominator)
    out = []
    for h in range(Q.shape[0]):
        sc = [sum(D(a) * D(b) for a, b in zip(Q[h], K[h, s])) / Decimal(K.shape[2]).sqrt()
              for s in range(K.shape[1])]
        mx = max(sc)
        e = [(x - mx).exp() for x in sc]
        den = sum(e)
        out.append([float(sum(e[s] / den * D(V[h, s, d]) for s in range(K.shape[1])))
                    for d in range(K.shape[2])])
    return np.array(out)


def pin_attention(lib):
    """The attention step alone (the unfused program's second kernel)."""
    # Two keys, D = 2, no normalisation: q = [1, 0], k0 = [1, 0], k1 = [0, 1]:
    # scores 1 / sqrt 2 and 0.
    Q = np.array([[1.0, 0.0]])
    K = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    V = np.array([[[1.0, 2.0], [3.0, 5.0]]])
    e = math.exp(1.0 / math.sqrt(2.0))
    p0 = e / (e + 1.0)
    _close(oracle.attention(Q, K, V, lib=lib), [[p0 * 1 + (1 - p0) * 3, p0 * 2 + (1 - p0) * 5]])
    rng = np.random.default_rng(43)
    for (BH, S, D) in ((3, 5, 8), (2, 1, 4), (4, 7, 16)):
        Q = rng.normal(size=(BH, D))
        K = rng.normal(size=(BH, S, D))
        V = rng.normal(size=(BH, S, D))
        ref = oracle.attention(Q, K, V, lib=lib)
        # one key: the weight is exactly 1
        assert np.array_equal(oracle.attention(Q, K[:, :1], V[:, :1], lib=lib), V[:, 0])
        # identical keys: the mean of the values
        _close(oracle.attention(Q, np.repeat(K[:, :1], S, axis=1), V, lib=lib), V.mean(axis=1))
        # a power-of-two scale may sit on the query or on the keys (exact)
        _close(oracle.attention(4.0 * Q, K, V, lib=lib), oracle.attention(Q, 4.0 * K, V, lib=lib),
               rtol=0, atol=0)
        # keys (with their values) in another order
        perm = rng.permutation(S)
        _close(oracle.attention(Q, K[:, perm], V[:, perm], lib=lib), ref, rtol=1e-12, atol=1e-13)
        # brute force at 50 digits
        _close(ref, _brute_plain_attention(Q, K, V), rtol=1e-12, atol=1e-13)
        # the fused definition is the unfused program: both vectors normalised as
        # rows by the RMSNorm step, then this step -- the same operations
        gq = rng.normal(1.0, 0.3, size=D)
        gk = rng.normal(1.0, 0.3, size=D)
        eps = 0.125
        qn = oracle.rmsnorm(Q, gq, eps, lib=lib)
        kn = oracle.rmsnorm(K.reshape(BH * S, D), gk, eps, lib=lib).reshape(BH, S, D)
        assert np.array_equal(oracle.attention(qn, kn, V, lib=lib),
                              oracle.qknorm_attention(Q, K, V, gq, gk, eps, lib=lib))


def _brute_prefill(Q, K, V, gq, gk, eps, causal):
    # every query row of every query head, written out per the definition:
    # its key/value head's keys (the first i + Skv - Sq + 1 under the mask)
    BHq, Sq, Dd = Q.shape
    BH, Skv = K.shape[0], K.shape[1]
    G = BHq // BH
    out = np.empty(Q.shape)
    for qh in range(BHq):
        for i in range(Sq):
            n = i + Skv - Sq + 1 if causal else Skv
            out[qh, i] = _brute_attention(Q[qh, i][None], K[qh // G, :n][None],
                                          V[qh // G, :n][None], gq, gk, eps)[0]
    return out


def pin_qknorm_attention_prefill(lib):
    """Many queries per head, grouped heads, the causal mask."""
    rng = np.random.default_rng(47)
    pre = lambda *a, **k: oracle.qknorm_attention_prefill(*a, lib=lib, **k)
    for (BH, G, Sq, Skv, D) in ((2, 1, 3, 3, 4), (1, 3, 2, 5, 8), (2, 2, 4, 6, 4)):
        Q = rng.normal(size=(BH * G, Sq, D))
        K = rng.normal(size=(BH, Skv, D))
        V = rng.normal(size=(BH, Skv, D))
        gq = rng.normal(1.0, 0.3, size=D)
        gk = rng.normal(1.0, 0.3, size=D)
        eps = 0.125
        for causal in (True, False):
            ref = pre(Q, K, V, gq, gk, eps, causal=causal)
            # brute force at 50 digits, query row by query row
            _close(ref, _brute_prefill(Q, K, V, gq, gk, eps, causal), rtol=1e-12, atol=1e-13)
        causal_ref = pre(Q, K, V, gq, gk, eps, causal=True)
        full_ref = pre(Q, K, V, gq, gk, eps, causal=False)
        Gh = np.repeat(np.arange(BH), G)
        # without the mask each query row is the single-query call on its head
        single = _attn(lib, Q.reshape(BH * G * Sq, D), np.repeat(K[Gh], Sq, axis=0),
                       np.repeat(V[Gh], Sq, axis=0), gq, gk, eps)
        assert np.array_equal(full_ref.reshape(-1, D), single)
        # the last query sees every key: mask and no mask agree there
        assert np.array_equal(causal_ref[:, -1], full_ref[:, -1])
        # under the mask, query i ignores the keys after i + Skv - Sq: changing them
        # (and their values) leaves it as it was
        K2, V2 = K.copy(), V.copy()
        K2[:, Skv - Sq + 1:] = rng.normal(size=K2[:, Skv - Sq + 1:].shape)
        V2[:, Skv - Sq + 1:] = rng.normal(size=V2[:, Skv - Sq + 1:].shape)
        assert np.array_equal(pre(Q, K2, V2, gq, gk, eps, causal=True)[:, 0], causal_ref[:, 0])
        # with one visible key the first query's output is that key's value
        if Skv == Sq:
            for qh in range(BH * G):
                assert np.array_equal(causal_ref[qh, 0], V[qh // G, 0])


ALL_PINS = [pin_worked_example, pin_library_matmul, pin_identity_weight, pin_constant_row,
            pin_scale_law, pin_gain_fold, pin_structure, pin_zero_row, pin_brute_force,
            pin_gated_closed_forms, pin_unfused_steps, pin_lora, pin_qknorm_attention,
            pin_attention, pin_qknorm_attention_prefill]
