"""Pins of the pure fractional-LNS oracle (BitState/HSDR brief v0.5, section
5.2; section 7 Phase A) against what the mathematics fixes, independent of
the oracle's own code:

* table entries against a 60-digit ``decimal`` evaluation of their defining
  formula, exact entries (doubling, powers of two), monotonicity, and the
  identity (1 + u)(1 - u) = 1 - u^2 between the two add tables;
* the pair add against round(N*log2|a +- b|) evaluated in ``decimal``;
* the balanced tree order, each add taken from that exact definition, and
  the leaf order of a whole row by brute force at coarse precision;
* whole rows: closed forms (single product, all-equal rows, exact
  cancellation, power-of-two scales) and the first-order rounding-error
  bounds of the reduction, same-sign (log-domain, tight) and mixed-sign
  (against the sum of magnitudes).
"""
import math
from decimal import ROUND_HALF_EVEN, Decimal, localcontext

import numpy as np
import pytest

import oracle
from bit_decode_gemv_amd import synth

PREC = 60


def _d_log2(x: Decimal) -> Decimal:
    return x.ln() / Decimal(2).ln()


def _d_pow2(y: Decimal) -> Decimal:
    return (y * Decimal(2).ln()).exp()


def _d_round(x: Decimal) -> int:
    return int(x.to_integral_value(rounding=ROUND_HALF_EVEN))


def _kp_exact(D: int, N: int) -> int:
    with localcontext() as c:
        c.prec = PREC
        return _d_round(N * _d_log2(1 + _d_pow2(Decimal(-D) / N)))


def _km_exact(D: int, N: int) -> int:
    with localcontext() as c:
        c.prec = PREC
        return _d_round(N * _d_log2(1 - _d_pow2(Decimal(-D) / N)))


def _lc_exact(n: int, N: int) -> int:
    with localcontext() as c:
        c.prec = PREC
        return _d_round(N * _d_log2(Decimal(n)))


def _add_exact(a, b, N: int):
    """round(N*log2|V|) of V = a + b, a and b given as (sign, L) with value
    sign * 2^(L/N); zero when V = 0."""
    with localcontext() as c:
        c.prec = PREC
        v = Decimal(0)
        for s, lam in (a, b):
            if s:
                v += s * _d_pow2(Decimal(lam) / N)
        if abs(v) < Decimal(10) ** (-40):     # only exact cancellation gets here
            return (0, 0)
        return (1 if v > 0 else -1, _d_round(N * _d_log2(abs(v))))


@pytest.mark.parametrize("f", [0, 1, 2, 3])
def test_tables_every_entry_small_f(f):
    tb = oracle.flns_tables(f)
    N = tb["N"]
    assert N == 8 << f
    for n in range(1, 129):
        assert tb["lc"][n] == _lc_exact(n, N), n
    for D in range(tb["kp"].size):
        assert tb["kp"][D] == _kp_exact(D, N), D
    for D in range(1, tb["km"].size):
        assert tb["km"][D] == _km_exact(D, N), D
    # the first D past each table rounds to zero
    assert _kp_exact(tb["kp"].size, N) == 0 and tb["kp"][-1] != 0
    assert _km_exact(tb["km"].size, N) == 0 and tb["km"][-1] != 0


@pytest.mark.parametrize("f", [5, 8, 12])
def test_tables_sampled_entries_large_f(f):
    tb = oracle.flns_tables(f)
    N = tb["N"]
    rng = np.random.default_rng(100 + f)
    for n in list(range(1, 20)) + list(rng.integers(20, 129, size=20)):
        assert tb["lc"][n] == _lc_exact(int(n), N), n
    nkp, nkm = tb["kp"].size, tb["km"].size
    ds = list(range(0, 12)) + list(rng.integers(0, nkp, size=60)) + list(range(nkp - 6, nkp))
    for D in ds:
        assert tb["kp"][D] == _kp_exact(int(D), N), D
    ds = list(range(1, 12)) + list(rng.integers(1, nkm, size=60)) + list(range(nkm - 6, nkm))
    for D in ds:
        assert tb["km"][D] == _km_exact(int(D), N), D
    assert _kp_exact(nkp, N) == 0 and _km_exact(nkm, N) == 0
    # no entry lies near a rounding tie, so the rounding is unambiguous
    assert tb["margin"] > 1e-9


@pytest.mark.parametrize("f", [0, 4, 8, 12])
def test_table_exact_entries_and_shape(f):
    tb = oracle.flns_tables(f)
    N, lc, kp, km = tb["N"], tb["lc"], tb["kp"], tb["km"]
    assert kp[0] == N                        # a + a = 2a: one octave up, exactly
    for m in range(8):
        assert lc[1 << m] == m * N           # 2^m identical states
    assert np.all(np.diff(kp) <= 0) and np.all(kp > 0)
    assert np.all(np.diff(km[1:]) >= 0) and np.all(km[1:] < 0)
    # analytic table lengths: kappa_plus(D) < 1/2 from D ~ N*(log2(N) + log2(2/ln 2))
    est = N * (math.log2(N) + math.log2(2 / math.log(2)))
    assert abs(kp.size - est) <= 0.02 * est + 2
    assert abs(km.size - est) <= 0.02 * est + 2


@pytest.mark.parametrize("f", [0, 3, 8])
def test_table_identity_plus_minus(f):
    """(1 + u)(1 - u) = 1 - u^2 with u = 2^(-D/N): kappa_plus(D) +
    kappa_minus(D) = kappa_minus(2D); three roundings, so within 1."""
    tb = oracle.flns_tables(f)
    kp, km = tb["kp"], tb["km"]

    def get(t, D):
        return int(t[D]) if D < t.size else 0

    for D in range(1, km.size):
        assert abs(get(kp, D) + get(km, D) - get(km, 2 * D)) <= 1, D


@pytest.mark.parametrize("f", [0, 2, 8])
def test_pair_add_is_rounded_log_of_exact_sum(f):
    N = 8 << f
    tb = oracle.flns_tables(f)
    rng = np.random.default_rng(7 + f)
    span = tb["kp"].size + 40
    cases = []
    for _ in range(300):
        la = int(rng.integers(-5 * N, 200 * N))
        d = int(rng.choice([0, 1, 2, int(rng.integers(0, span)), span + 5]))
        sa, sb = int(rng.choice([-1, 1])), int(rng.choice([-1, 1]))
        cases.append(((sa, la), (sb, la - d)))
        cases.append(((sb, la - d), (sa, la)))
    for a, b in cases:
        assert oracle.flns_add(f, a, b) == _add_exact(a, b, N), (a, b)


def test_pair_add_special_cases():
    f = 4
    N = 8 << f
    assert oracle.flns_add(f, (1, 1000), (-1, 1000)) == (0, 0)      # exact cancellation
    assert oracle.flns_add(f, (-1, 1000), (1, 1000)) == (0, 0)
    assert oracle.flns_add(f, (1, 1000), (1, 1000)) == (1, 1000 + N)
    assert oracle.flns_add(f, (-1, -7), (-1, -7)) == (-1, -7 + N)
    assert oracle.flns_add(f, (1, 123), (0, 0)) == (1, 123)          # zero is the identity
    assert oracle.flns_add(f, (0, 0), (-1, 55)) == (-1, 55)
    assert oracle.flns_add(f, (0, 0), (0, 0)) == (0, 0)
    # the larger magnitude decides the sign
    assert oracle.flns_add(f, (1, 500), (-1, 600))[0] == -1
    assert oracle.flns_add(f, (-1, 500), (1, 600))[0] == 1


@pytest.mark.parametrize("f", [0, 1])
def test_tree_order_is_balanced_pairwise(f):
    """Leaves reduced as ((v0+v1)+(v2+v3))+... with an unpaired last element
    moving up; each add from its exact definition.  Coarse f makes the
    rounding order-dependent, so a different pairing fails."""
    N = 8 << f
    rng = np.random.default_rng(11 + f)
    differs = 0
    for trial in range(200):
        n = int(rng.integers(1, 21))
        signs = rng.choice([-1, 0, 1, 1], size=n)
        lams = rng.integers(0, 6 * N, size=n)
        vals = [(int(s), int(l) if s else 0) for s, l in zip(signs, lams)]
        level = list(vals)
        while len(level) > 1:
            nxt = [_add_exact(level[i], level[i + 1], N) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        want = level[0]
        # a left-to-right chain for contrast (not the method's order)
        chain = vals[0]
        for v in vals[1:]:
            chain = _add_exact(chain, v, N)
        differs += chain != want
        assert oracle.flns_tree(f, signs, [l for _, l in vals]) == want, (trial, vals)
    assert differs > 10            # the order is observable at this precision


def _row(k, entries):
    """One row: t int8[1][k], x uint8[k] from (position, code, s1, t)."""
    t = np.zeros((1, k), dtype=np.int8)
    x = np.zeros(k, dtype=np.uint8)
    for pos, code, s1, w in entries:
        x[pos] = (s1 << 7) | code
        t[0, pos] = w
    return t, x


@pytest.mark.parametrize("f", [0, 5, 12])
def test_row_single_product(f):
    for pos, code, s1, w, sign in [(0, 74, 0, 1, 1), (300, 1, 1, 1, -1), (511, 127, 1, -1, 1),
                                   (129, 99, 0, -1, -1)]:
        t, x = _row(512, [(pos, code, s1, w)])
        assert oracle.flns_gemv(t, x, f).tolist() == [[sign, code << f]]


@pytest.mark.parametrize("f", [0, 7, 12])
def test_row_all_equal_products_is_exact(f):
    """K = 4096 products of one code c, all +: 32 tiles of 128 identical
    states fold to c + 8*7 code units each, and five levels of doubling add
    8*5: the value 4096 * 2^((c-74)/8), exactly."""
    N = 8 << f
    k = 4096
    for c in (1, 60, 74, 127):
        x = np.full(k, c, dtype=np.uint8)
        t = np.ones((1, k), dtype=np.int8)
        assert oracle.flns_gemv(t, x, f).tolist() == [[1, (c << f) + 12 * N]]
        # negative products and a power-of-two scale 2^3
        assert oracle.flns_gemv(-t, x, f, scale_d=8).tolist() == [[-1, (c << f) + 15 * N]]


def test_row_scale():
    f = 6
    N = 8 << f
    t, x = _row(256, [(3, 80, 0, 1)])
    assert oracle.flns_gemv(t, x, f, scale_d=1).tolist() == [[1, 80 << f]]
    assert oracle.flns_gemv(t, x, f, scale_d=1 << 20).tolist() == [[1, (80 << f) + 20 * N]]
    assert oracle.flns_gemv(t, x, f, scale_d=3).tolist() == [[1, (80 << f) + _lc_exact(3, N)]]
    assert oracle.flns_log_scale(f, 1000) == _lc_exact(1000, N)
    z = np.zeros((1, 256), dtype=np.int8)
    assert oracle.flns_gemv(z, x, f, scale_d=12345).tolist() == [[0, 0]]


@pytest.mark.parametrize("f", [0, 8])
def test_row_exact_cancellation(f):
    # inside one tile: the signed population is 0
    t, x = _row(256, [(5, 90, 0, 1), (17, 90, 1, 1)])
    assert oracle.flns_gemv(t, x, f).tolist() == [[0, 0]]
    # across tiles: equal and opposite tile aggregates meet in the tree
    t, x = _row(256, [(5, 90, 0, 1), (133, 90, 0, -1)])
    assert oracle.flns_gemv(t, x, f).tolist() == [[0, 0]]
    # across phases: 2 * 2^((c-74)/8) against the code c + 8 (double), opposite
    t, x = _row(256, [(0, 70, 0, 1), (1, 70, 0, 1), (200, 78, 1, 1)])
    assert oracle.flns_gemv(t, x, f).tolist() == [[0, 0]]
    # code 0 and t = 0 contribute nothing, whatever the sign bit
    t, x = _row(256, [(0, 0, 1, 1), (1, 0, 0, -1), (2, 50, 1, 0)])
    assert oracle.flns_gemv(t, x, f).tolist() == [[0, 0]]


def _exact_sum(t, x):
    """Exact S = sum_i t_i * (-1)^S1_i * 2^((c_i-74)/8) per row, in decimal,
    from the pinned integer accumulators A[p] (sum_p A[p] 2^((p-2)/8) 2^-9)."""
    acc = oracle.lns8_direct(t, x)
    out = []
    with localcontext() as c:
        c.prec = PREC
        fs = [_d_pow2(Decimal(p - 2) / 8) / 512 for p in range(8)]
        for r in range(acc.shape[0]):
            out.append(sum(int(acc[r, p]) * fs[p] for p in range(8)))
    return out


def _levels(k):
    return 4 + math.ceil(math.log2(k // 128)) + 3


@pytest.mark.parametrize("f,k", [(12, 1024), (8, 4096), (3, 1152)])
def test_row_same_sign_error_bound(f, k):
    """All products positive: every add is a same-sign add, which is
    1-Lipschitz in the log domain, so the result is within 0.5 unit per
    rounding on any root-to-leaf path (fold + tree levels) of N*log2 S."""
    N = 8 << f
    rng = np.random.default_rng(5)
    t = rng.integers(0, 2, size=(12, k)).astype(np.int8)
    code = rng.integers(1, 128, size=k)
    code[rng.random(k) < 0.05] = 0
    x = code.astype(np.uint8)
    out = oracle.flns_gemv(t, x, f)
    S = _exact_sum(t, x)
    bound = 0.5 * (_levels(k) + 1)
    with localcontext() as c:
        c.prec = PREC
        for r in range(t.shape[0]):
            assert out[r, 0] == 1
            want = (74 << f) + N * _d_log2(S[r])
            assert abs(Decimal(int(out[r, 1])) - want) <= Decimal(bound), (r, out[r], want)


@pytest.mark.parametrize("f", [6, 10])
def test_row_mixed_sign_error_bound(f):
    """Mixed signs: to first order the absolute error is at most
    eps * (sum over the nodes on each level of |node|) <= (levels + 1) * eps
    * sum_i |t_i x_i| with eps = 2^(0.5/N) - 1, here with a (1 + eps)^L
    margin; plus one rounding for the scale."""
    N = 8 << f
    k = 2048
    t, x = synth.lns8(16, k, 3)
    d = 5
    out = oracle.flns_gemv(t, x, f, scale_d=d)
    S = _exact_sum(t, x)
    mags = np.abs(t).astype(np.float64) @ np.array(
        [oracle.lns8_decode(int(b) & 127) for b in x])
    L = _levels(k) + 2
    with localcontext() as c:
        c.prec = PREC
        eps = _d_pow2(Decimal("0.5") / N) - 1
        for r in range(t.shape[0]):
            got = Decimal(0) if out[r, 0] == 0 else (
                int(out[r, 0]) * _d_pow2((Decimal(int(out[r, 1])) / (1 << f) - 74) / 8))
            err = abs(got - d * S[r])
            bound = L * eps * (1 + eps) ** L * d * Decimal(float(mags[r])) * Decimal("1.0001")
            assert err <= bound, (r, err, bound)


def _tree_exact(vals, N):
    level = list(vals)
    if not level:
        return (0, 0)
    while len(level) > 1:
        nxt = [_add_exact(level[i], level[i + 1], N) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def _row_bruteforce(t_row, x, f, order):
    """Populations per Tile128 from their definition, exact folds, exact
    adds; leaves of a phase at 16*tile + band ("tile") or T*band + tile
    ("band", a different order for contrast)."""
    N = 8 << f
    k = t_row.size
    T = k // 128
    aggs = []
    for p in range(8):
        leaves = [(0, 0)] * (16 * T)
        for j in range(T):
            for b in range(16):
                c = 8 * b + p
                if c == 0:
                    continue
                pop = 0
                for i in range(128 * j, 128 * j + 128):
                    if (x[i] & 127) == c and t_row[i] != 0:
                        pop += -1 if ((x[i] >> 7) ^ (t_row[i] < 0)) else 1
                if pop:
                    leaf = (1 if pop > 0 else -1, (c << f) + _lc_exact(abs(pop), N))
                    leaves[16 * j + b if order == "tile" else T * b + j] = leaf
        aggs.append(_tree_exact(leaves, N))
    return _tree_exact(aggs, N)


@pytest.mark.parametrize("k", [256, 384])
def test_row_leaf_order_bruteforce(k):
    """The leaf order of the per-phase tree (tile-major, band-minor, then the
    8 -> 4 -> 2 -> 1 phase tree) by brute force at f = 0, where the rounding
    order is observable."""
    f = 0
    rng = np.random.default_rng(k)
    t = rng.integers(-1, 2, size=(10, k)).astype(np.int8)
    x = ((rng.integers(0, 2, size=k) << 7) | rng.integers(0, 128, size=k)).astype(np.uint8)
    out = oracle.flns_gemv(t, x, f)
    differs = 0
    for r in range(t.shape[0]):
        want = _row_bruteforce(t[r], x, f, "tile")
        assert tuple(out[r].tolist()) == want, r
        differs += _row_bruteforce(t[r], x, f, "band") != want
    assert differs >= 1
