"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each pin takes an object ``o`` with the oracle API (``sgemm_ref``,
``sgemm_ref_entries``, ``sgemm_ref_op``, ``sgemm_ref_op_entries``) so that the same pins can be run against a copy of the
oracle with a planted mistake, which at least one of them must catch.

What fixes each expected value (none is produced by the code under test):
  * hand-worked products (tests/golden), worked out on paper;
  * identity and permutation matrices: the product copies or permutes the other
    operand exactly (every other term is an exact zero);
  * (AB)^T = B^T A^T: a structural identity of the product;
  * exact rational arithmetic (Python ``fractions``) on tiny shapes;
  * integer matrices: numpy's int64 matmul is exact;
  * rank-one integer factors: C_ij = u_i w_j (s . t) in closed form;
  * all-ones operands: every entry equals K*alpha + beta*C0 exactly;
  * alpha = 0 and beta = 0: the unused operands are not read (NaN stays out);
  * IEEE 754's sign rules for zero results (alpha * (+0) with alpha < 0 is -0;
    beta * C0 alone when there is no product term);
  * the float64 library matmul on random inputs, to within float64 rounding;
  * for the transposed-operand form: its own hand-worked fixture, numpy's exact
    int64 matmul of the explicitly transposed integer operands, the float64
    library matmul, and (op(A) op(B))^T = op(B)^T op(A)^T;
  * for the 16-bit inputs: values of hand-decoded bit patterns of both formats,
    numpy's own binary16 conversion for all 65536 patterns, the bfloat16 rule
    "upper half of a binary32" for all 65536 patterns, and exact integer
    products of 16-bit integer-valued inputs;
  * the standard deviation sqrt(K/9) of a dot product of uniform[-1,1) vectors,
    which gives the "typical size 21" of entries at n = 4096 that "Writing a
    Fast Matmul in CUDA, Step by Step" reports in its "Step 1" section.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from golden_io import load_cases


def _rng(seed):
    return np.random.default_rng(seed)


def _uniform(rng, shape):
    return (rng.random(shape, dtype=np.float32) * 2 - 1).astype(np.float32)


def _bits(x):
    return np.asarray(x, dtype=np.float64).view(np.uint64)


def pin_golden(o):
    for fname in ("hand_2x2.txt", "hand_3x3.txt"):
        for c in load_cases(fname):
            Cref, _ = o.sgemm_ref(c["A"], c["B"], c["alpha"], c["beta"], c["C0"])
            assert np.array_equal(Cref, c["C"]), (fname, c["name"], Cref, c["C"])


def pin_identity(o):
    rng = _rng(1)
    for (m, k) in [(5, 7), (13, 4), (1, 9)]:
        A = _uniform(rng, (m, k))
        I = np.eye(k, dtype=np.float32)
        Cref, _ = o.sgemm_ref(A, I)
        assert np.array_equal(Cref, A.astype(np.float64)), "A*I != A"
        Il = np.eye(m, dtype=np.float32)
        Cref, _ = o.sgemm_ref(Il, A)
        assert np.array_equal(Cref, A.astype(np.float64)), "I*A != A"


def pin_permutation(o):
    rng = _rng(2)
    K, N = 9, 6
    B = _uniform(rng, (K, N))
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[np.arange(K), perm] = 1.0          # (P B)[i] = B[perm[i]]
    Cref, _ = o.sgemm_ref(P, B)
    assert np.array_equal(Cref, B[perm].astype(np.float64)), "P*B row permutation"
    permc = rng.permutation(N)
    Q = np.zeros((N, N), dtype=np.float32)
    Q[permc, np.arange(N)] = 1.0         # (B Q)[:, j] = B[:, permc[j]]
    Cref, _ = o.sgemm_ref(B, Q)
    assert np.array_equal(Cref, B[:, permc].astype(np.float64)), "B*Q column permutation"


def pin_transpose(o):
    rng = _rng(3)
    M, N, K = 7, 5, 11
    A = _uniform(rng, (M, K))
    B = _uniform(rng, (K, N))
    C1, _ = o.sgemm_ref(A, B)
    C2, _ = o.sgemm_ref(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(_bits(C1.T), _bits(C2)), "(AB)^T != B^T A^T"


def _exact(A, B, alpha, beta, C0):
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            v = Fraction(float(np.float32(alpha))) * s
            if np.float32(beta) != 0:
                v += Fraction(float(np.float32(beta))) * Fraction(float(C0[i, j]))
            out[i, j] = v
    return out


def pin_exact_rational(o):
    rng = _rng(4)
    shapes = [(0, 3, 2), (3, 0, 2), (2, 3, 0), (1, 1, 1), (2, 3, 4), (4, 1, 5),
              (3, 5, 8), (8, 8, 3), (5, 7, 6)]
    for (M, N, K) in shapes:
        for (alpha, beta) in [(1.0, 0.0), (-0.75, 1.25), (3.0, -2.0)]:
            A = _uniform(rng, (M, K))
            B = _uniform(rng, (K, N))
            C0 = _uniform(rng, (M, N))
            Cref, absab = o.sgemm_ref(A, B, alpha, beta, C0)
            ex = _exact(A, B, alpha, beta, C0)
            for i in range(M):
                for j in range(N):
                    mag = abs(alpha) * sum(abs(float(A[i, k]) * float(B[k, j])) for k in range(K))
                    mag += abs(beta) * abs(float(C0[i, j])) if beta != 0 else 0.0
                    tol = (K + 3) * 2.0 ** -52 * mag
                    err = abs(Fraction(float(Cref[i, j])) - ex[i, j])
                    assert float(err) <= tol, ((M, N, K), (i, j), float(err), tol)


def pin_integer_exact(o):
    rng = _rng(5)
    M, N, K = 19, 23, 37
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    C0 = rng.integers(-9, 10, (M, N)).astype(np.float32)
    Cref, absab = o.sgemm_ref(A, B, 1.5, -0.5, C0)
    Ai, Bi, Ci = A.astype(np.int64), B.astype(np.int64), C0.astype(np.int64)
    want = 1.5 * (Ai @ Bi).astype(np.float64) - 0.5 * Ci.astype(np.float64)
    assert np.array_equal(Cref, want), "integer product not exact"
    assert np.array_equal(absab, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)), "|A||B|"


def pin_rank_one(o):
    M, N, K = 6, 9, 8
    u = np.arange(1, M + 1, dtype=np.int64)            # rows of A scale
    s = np.array([1, -2, 3, 0, 5, -1, 2, 4], dtype=np.int64)
    t = np.array([2, 1, -1, 7, 1, 3, -2, 1], dtype=np.int64)
    w = np.arange(-4, N - 4, dtype=np.int64)
    A = np.outer(u, s).astype(np.float32)             # A[i][k] = u_i s_k
    B = np.outer(t, w).astype(np.float32)             # B[k][j] = t_k w_j
    Cref, _ = o.sgemm_ref(A, B)
    st = int(np.dot(s, t))
    want = np.outer(u, w).astype(np.float64) * st
    assert np.array_equal(Cref, want), "rank-one closed form"


def pin_all_ones(o):
    M, N, K = 5, 4, 33
    A = np.ones((M, K), np.float32)
    B = np.ones((K, N), np.float32)
    rng = _rng(6)
    C0 = rng.integers(-5, 6, (M, N)).astype(np.float32)
    Cref, _ = o.sgemm_ref(A, B, 1.5, -0.5, C0)
    assert np.array_equal(Cref, K * 1.5 - 0.5 * C0.astype(np.float64)), "ones"


def pin_scalar_special_cases(o):
    rng = _rng(7)
    M, N, K = 4, 6, 5
    A = np.full((M, K), np.nan, np.float32)
    B = np.full((K, N), np.nan, np.float32)
    C0 = _uniform(rng, (M, N))
    Cref, absab = o.sgemm_ref(A, B, 0.0, -0.5, C0)   # alpha = 0: A, B unread
    assert np.array_equal(Cref, -0.5 * C0.astype(np.float64)), "alpha = 0"
    assert np.array_equal(absab, np.zeros((M, N))), "alpha = 0 magnitude"
    A = _uniform(rng, (M, K))
    B = _uniform(rng, (K, N))
    Cn = np.full((M, N), np.nan, np.float32)
    Cref, _ = o.sgemm_ref(A, B, 1.0, 0.0, Cn)        # beta = 0: C0 unread
    assert np.all(np.isfinite(Cref)), "beta = 0 read C0"
    Cref0, _ = o.sgemm_ref(A[:, :0].copy(), B[:0, :].copy(), 2.0, 3.0, C0)  # K = 0
    assert np.array_equal(Cref0, 3.0 * C0.astype(np.float64)), "K = 0"
    Cz, _ = o.sgemm_ref(np.zeros((M, K), np.float32), B, 1.0, 1.0, C0)
    assert np.array_equal(Cz, C0.astype(np.float64)), "A = 0, beta = 1 leaves C"


def _neg_zero_where(vals, zero_mask):
    """vals with -0.0 wherever zero_mask holds."""
    out = np.asarray(vals, dtype=np.float64).copy()
    out[zero_mask] = -0.0
    return out


def pin_signed_zero(o):
    # IEEE 754 fixes the sign of a zero result: (-1) * (+0) = -0, (-0.5) * (+0)
    # = -0, (-0) + (+0) = +0 and (-0) + (-0) = -0 under round-to-nearest.  With
    # beta = 0 the result is alpha * sum alone; with no product term (alpha = 0
    # or K = 0) it is beta * C0 alone; beta = 0 with no product term is +0.
    rng = _rng(12)
    M, N, K = 6, 7, 9
    Ai = rng.integers(-4, 5, (M, K))
    Bi = rng.integers(-4, 5, (K, N))
    Ai[2] = 0                       # a zero row of A: a zero sum across row 2
    Bi[:, 4] = 0                    # a zero column of B: a zero sum down column 4
    Ai[4, :2] = [1, 1]; Ai[4, 2:] = 0
    Bi[:2, 1] = [3, -3]             # row 4, column 1: 3 - 3 cancels exactly
    A, B = Ai.astype(np.float32), Bi.astype(np.float32)
    prod = Ai @ Bi
    zero = prod == 0
    assert zero[2].all() and zero[:, 4].all() and zero[4, 1]
    nanC = np.full((M, N), np.nan, np.float32)
    want = _neg_zero_where(-prod.astype(np.float64), zero)
    Cref, _ = o.sgemm_ref(A, B, -1.0, 0.0, nanC)
    assert np.array_equal(_bits(Cref), _bits(want)), "alpha < 0, beta = 0: alpha * (+0) is -0"
    for ta, tb in _FORMS:
        Cop, _ = o.sgemm_ref_op(_stored(A, ta), _stored(B, tb), ta, tb, -1.0, 0.0, nanC)
        assert np.array_equal(_bits(Cop), _bits(want)), ("op form, beta = 0", ta, tb)
    r = np.array([2, 4, 0, 5]); c = np.array([3, 1, 4, 0])
    v, _ = o.sgemm_ref_entries(A, B, r, c, -1.0, 0.0, nanC)
    assert np.array_equal(_bits(v), _bits(want[r, c])), "entries, beta = 0"
    v, _ = o.sgemm_ref_op_entries(A, B, r, c, False, False, -1.0, 0.0, nanC)
    assert np.array_equal(_bits(v), _bits(want[r, c])), "op entries, beta = 0"

    # beta != 0: (-0) + beta * C0 with C0 = +0 is +0 for beta > 0, -0 for beta < 0.
    C0 = np.zeros((M, N), np.float32)
    for beta in (1.0, -1.0):
        Cref, _ = o.sgemm_ref(A, B, -1.0, beta, C0)
        w = -prod.astype(np.float64)
        w[zero] = 0.0 if beta > 0 else -0.0
        assert np.array_equal(_bits(Cref), _bits(w)), ("-0 + beta * (+0)", beta)

    # No product term: beta * C0 alone (-0.5 * +0 = -0); beta = 0 as well: +0.
    C0 = rng.integers(-3, 4, (M, N)).astype(np.float32)
    C0[1] = 0.0
    nanA = np.full((M, K), np.nan, np.float32)
    nanB = np.full((K, N), np.nan, np.float32)
    want = _neg_zero_where(-0.5 * C0.astype(np.float64), C0 == 0)
    Cref, _ = o.sgemm_ref(nanA, nanB, 0.0, -0.5, C0)
    assert np.array_equal(_bits(Cref), _bits(want)), "alpha = 0: beta * C0 keeps -0"
    Cref, _ = o.sgemm_ref_op(nanA, nanB, False, False, 0.0, -0.5, C0)
    assert np.array_equal(_bits(Cref), _bits(want)), "op form, alpha = 0"
    Cref, _ = o.sgemm_ref(A[:, :0].copy(), B[:0, :].copy(), 2.0, -0.5, C0)
    assert np.array_equal(_bits(Cref), _bits(want)), "K = 0: beta * C0 keeps -0"
    Cref, _ = o.sgemm_ref(nanA, nanB, 0.0, 0.0, nanC)
    assert np.array_equal(_bits(Cref), _bits(np.zeros((M, N)))), "alpha = beta = 0 is +0"


def pin_library_matmul(o):
    rng = _rng(8)
    M, N, K = 37, 29, 301
    A = _uniform(rng, (M, K))
    B = _uniform(rng, (K, N))
    C0 = _uniform(rng, (M, N))
    alpha, beta = 1.25, -0.75
    Cref, absab = o.sgemm_ref(A, B, alpha, beta, C0)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    want = alpha * (A64 @ B64) + beta * C0.astype(np.float64)
    mag = abs(alpha) * (np.abs(A64) @ np.abs(B64)) + abs(beta) * np.abs(C0)
    assert np.all(np.abs(Cref - want) <= 2 * (K + 3) * 2.0 ** -53 * mag), "vs float64 matmul"
    assert np.all(np.abs(absab - np.abs(A64) @ np.abs(B64))
                  <= 2 * K * 2.0 ** -53 * (np.abs(A64) @ np.abs(B64))), "absab"


def pin_leading_dims(o):
    rng = _rng(9)
    M, N, K = 9, 10, 12
    Ap = np.full((M, K + 5), np.nan, np.float32)
    Bp = np.full((K, N + 3), np.nan, np.float32)
    Cp = np.full((M, N + 7), np.nan, np.float32)
    Ap[:, :K] = _uniform(rng, (M, K))
    Bp[:, :N] = _uniform(rng, (K, N))
    Cp[:, :N] = _uniform(rng, (M, N))
    A, B, C0 = Ap[:, :K], Bp[:, :N], Cp[:, :N]
    C1, _ = o.sgemm_ref(A, B, 1.0, 2.0, C0)
    C2, _ = o.sgemm_ref(A.copy(), B.copy(), 1.0, 2.0, C0.copy())
    assert np.all(np.isfinite(C1)), "padding read"
    assert np.array_equal(C1, C2), "row strides change the result"


def pin_entries_match(o):
    rng = _rng(10)
    M, N, K = 17, 13, 40
    A = _uniform(rng, (M, K))
    B = _uniform(rng, (K, N))
    C0 = _uniform(rng, (M, N))
    Cref, absab = o.sgemm_ref(A, B, -1.5, 0.25, C0)
    r = rng.integers(0, M, 50)
    c = rng.integers(0, N, 50)
    v, av = o.sgemm_ref_entries(A, B, r, c, -1.5, 0.25, C0)
    assert np.array_equal(_bits(v), _bits(Cref[r, c])), "entries != full"
    assert np.array_equal(_bits(av), _bits(absab[r, c])), "entry magnitudes"


def pin_uniform_statistics(o):
    rng = _rng(11)
    M, N, K = 32, 64, 4096
    A = _uniform(rng, (M, K))
    B = _uniform(rng, (K, N))
    Cref, _ = o.sgemm_ref(A, B)
    sd = float(np.std(Cref))
    want = (K / 9.0) ** 0.5                           # about 21.3 at K = 4096
    assert abs(sd / want - 1) < 0.05, (sd, want)


_FORMS = [(False, False), (False, True), (True, False), (True, True)]


def _stored(x, trans):
    """The array whose transposed reading is x (a fresh row-major copy)."""
    return np.ascontiguousarray(x.T) if trans else x


def pin_op_golden(o):
    for c in load_cases("hand_trans.txt"):
        Cref, _ = o.sgemm_ref_op(c["A"], c["B"], c["trans_a"], c["trans_b"],
                                 c["alpha"], c["beta"], c["C0"])
        assert np.array_equal(Cref, c["C"]), (c["name"], Cref, c["C"])


def pin_op_integer_exact(o):
    # Rectangular and all different (M, N, K), so a swapped extent or index shows.
    rng = _rng(21)
    M, N, K = 7, 5, 11
    Ai = rng.integers(-4, 5, size=(M, K))
    Bi = rng.integers(-4, 5, size=(K, N))
    want = (Ai @ Bi).astype(np.float64)              # exact in int64
    for ta, tb in _FORMS:
        A = _stored(Ai.astype(np.float32), ta)
        B = _stored(Bi.astype(np.float32), tb)
        Cref, absab = o.sgemm_ref_op(A, B, ta, tb)
        assert np.array_equal(Cref, want), ("integer product", ta, tb)
        assert np.array_equal(absab, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)), ("|A||B|", ta, tb)


def pin_op_library_matmul(o):
    # Padded views (row stride larger than the width) for every stored operand.
    rng = _rng(22)
    M, N, K = 9, 6, 13
    X = _uniform(rng, (M, K))
    Y = _uniform(rng, (K, N))
    C0 = _uniform(rng, (M, N))
    want = 1.25 * (X.astype(np.float64) @ Y.astype(np.float64)) - 0.75 * C0.astype(np.float64)
    for ta, tb in _FORMS:
        A = _stored(X, ta)
        B = _stored(Y, tb)
        Ap = np.zeros((A.shape[0], A.shape[1] + 3), np.float32); Ap[:, :A.shape[1]] = A
        Bp = np.zeros((B.shape[0], B.shape[1] + 5), np.float32); Bp[:, :B.shape[1]] = B
        Cref, _ = o.sgemm_ref_op(Ap[:, :A.shape[1]], Bp[:, :B.shape[1]], ta, tb, 1.25, -0.75, C0)
        assert np.allclose(Cref, want, rtol=1e-13, atol=1e-13), ("library matmul", ta, tb)


def pin_op_transpose_identity(o):
    # C^T = op(B)^T op(A)^T: the stored B read transposed is the left operand.
    rng = _rng(23)
    M, N, K = 6, 10, 7
    X = _uniform(rng, (M, K))
    Y = _uniform(rng, (K, N))
    for ta, tb in _FORMS:
        A = _stored(X, ta)
        B = _stored(Y, tb)
        C, _ = o.sgemm_ref_op(A, B, ta, tb)
        Ct, _ = o.sgemm_ref_op(B, A, not tb, not ta)
        assert np.array_equal(_bits(C.T), _bits(Ct)), ("(AB)^T", ta, tb)


def pin_op_entries_match(o):
    rng = _rng(24)
    M, N, K = 8, 12, 9
    X = _uniform(rng, (M, K))
    Y = _uniform(rng, (K, N))
    C0 = _uniform(rng, (M, N))
    r = rng.integers(0, M, size=20)
    c = rng.integers(0, N, size=20)
    for ta, tb in _FORMS:
        A = _stored(X, ta)
        B = _stored(Y, tb)
        Cref, absab = o.sgemm_ref_op(A, B, ta, tb, 0.5, 2.0, C0)
        v, av = o.sgemm_ref_op_entries(A, B, r, c, ta, tb, 0.5, 2.0, C0)
        assert np.array_equal(_bits(v), _bits(Cref[r, c])), ("entries != full", ta, tb)
        assert np.array_equal(_bits(av), _bits(absab[r, c])), ("entry magnitudes", ta, tb)


# (pattern, value) pairs decoded by hand from the field layouts.
_BF16_HAND = [(0x0000, 0.0), (0x3F80, 1.0), (0xC000, -2.0), (0x3E80, 0.25), (0x4049, 3.140625),
              (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),
              (0x7F80, np.inf), (0xFF80, -np.inf), (0x4300, 128.0), (0xC2C8, -100.0)]
_F16_HAND = [(0x0000, 0.0), (0x3C00, 1.0), (0xC000, -2.0), (0x3555, 1365 / 4096), (0x7BFF, 65504.0),
             (0x0400, 2.0 ** -14), (0x0001, 2.0 ** -24), (0x7C00, np.inf), (0xFC00, -np.inf),
             (0x5640, 100.0), (0xD800, -128.0), (0x3800, 0.5)]


def pin_decode_hand(o):
    for kind, table in ((1, _BF16_HAND), (2, _F16_HAND)):
        bits = np.array([b for b, _ in table], np.uint16)
        got = o.decode_16(bits, kind).astype(np.float64)
        want = np.array([v for _, v in table], np.float64)
        assert np.array_equal(got, want), (kind, got, want)
        nan = o.decode_16(np.array([0x7FC0 if kind == 1 else 0x7E00], np.uint16), kind)
        assert np.isnan(nan[0])
    neg0 = o.decode_16(np.array([0x8000], np.uint16), 1)
    assert neg0[0] == 0 and np.signbit(neg0[0])


def pin_decode_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = o.decode_16(bits, 2)
    ref = bits.view(np.float16).astype(np.float32)              # numpy's binary16
    same = (f16 == ref) | (np.isnan(f16) & np.isnan(ref))
    assert same.all() and np.array_equal(np.signbit(f16), np.signbit(ref)), "binary16 decode"
    bf = o.decode_16(bits, 1)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)      # upper half of a binary32
    same = (bf == ref) | (np.isnan(bf) & np.isnan(ref))
    assert same.all() and np.array_equal(np.signbit(bf), np.signbit(ref)), "bfloat16 decode"


def _to16(x, kind):
    """Integer-valued float32 -> 16-bit patterns (exact for the small integers used)."""
    x = np.asarray(x, np.float32)
    if kind == 2:
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def pin_lowp_integer_exact(o):
    rng = _rng(31)
    M, N, K = 9, 7, 40
    Ai = rng.integers(-8, 9, size=(M, K))
    Bi = rng.integers(-8, 9, size=(K, N))
    C0 = rng.integers(-5, 6, size=(M, N)).astype(np.float32)
    want = (2 * (Ai @ Bi) - 3 * C0.astype(np.int64)).astype(np.float64)
    for kind in (1, 2):
        for ta, tb in _FORMS:
            A = _stored(_to16(Ai, kind).reshape(M, K), ta)
            B = _stored(_to16(Bi, kind).reshape(K, N), tb)
            Cref, absab = o.sgemm_ref_lowp(A, B, kind, ta, tb, 2.0, -3.0, C0)
            assert np.array_equal(Cref, want), ("lowp integer", kind, ta, tb)
            assert np.array_equal(absab, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


PINS = [pin_golden, pin_identity, pin_permutation, pin_transpose, pin_exact_rational,
        pin_integer_exact, pin_rank_one, pin_all_ones, pin_scalar_special_cases, pin_signed_zero,
        pin_library_matmul, pin_leading_dims, pin_entries_match,
        pin_uniform_statistics, pin_op_golden, pin_op_integer_exact,
        pin_op_library_matmul, pin_op_transpose_identity, pin_op_entries_match,
        pin_decode_hand, pin_decode_all_patterns, pin_lowp_integer_exact]
