"""Pins of the float64 oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every check uses an independent
route (closed forms, integer or rational brute force, textbook special cases,
the page's printed constants).
"""
import itertools
import json
import math
import os
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest

from oracle import sata_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(g, n, d):
    x = g.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# Basis: counts, contents and the page's printed constants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,P", [(1, 4), (2, 3), (3, 4), (5, 5), (8, 3), (16, 4), (32, 4)])
def test_basis_counts_closed_form(d, P):
    basis = O.enumerate_basis(d, P)
    for p, (idx, mult, scale) in enumerate(basis):
        assert idx.shape == (math.comb(d + p - 1, p), p)
        assert scale == 1.0 / math.factorial(p)
    # hockey-stick identity: total over orders 0..P-1 equals C(d+P-1, P-1)
    assert sum(b[0].shape[0] for b in basis) == math.comb(d + P - 1, P - 1)


def test_page_constants():
    g = json.load(open(GOLDEN))
    e = g["minimal_basis_d64_P4"]
    assert O.basis_size(e["d_k"], e["P"]) == e["value"] == 47905
    # the state size closed form at the same point: 65 * 47905 values
    assert O.cost_model(64, 64, 4)[0] == 65 * 47905
    # the page's P=3 / P=5 figures are not the formula's: sizes come from the formula
    f = g["page_basis_sizes_not_from_formula"]
    assert O.basis_size(64, 3) == 2145 != f["P3_page"]
    assert O.basis_size(64, 5) == 814385 != f["P5_page"]


def test_full_expansion_count_matches_page():
    # the multiplicities of the order-4 rows count every index tuple of the
    # full tensor power: sum mu = 64^4, which the page calls "over 16 million"
    g = json.load(open(GOLDEN))["full_expansion_d64_p4_exceeds"]
    idx, mult, _ = O.enumerate_basis(64, 5)[4]
    total = int(mult.astype(np.int64).sum())
    assert total == 64 ** 4 > g["value"]
    assert idx.shape[0] == math.comb(67, 4) < total


@pytest.mark.parametrize("d,p", [(1, 3), (2, 4), (3, 3), (4, 4), (5, 2)])
def test_basis_contents_brute_force(d, p):
    """Every index tuple sorted gives one row; the number of tuples per row is mu."""
    idx, mult, _ = O.enumerate_basis(d, p + 1)[p]
    counts = Counter(tuple(sorted(t)) for t in itertools.product(range(d), repeat=p))
    rows = [tuple(int(x) for x in r) for r in idx]
    assert rows == sorted(counts.keys())                 # lexicographic, complete, no repeats
    assert [counts[r] for r in rows] == [int(m) for m in mult]
    assert all(all(a <= b for a, b in zip(r, r[1:])) for r in rows)


@pytest.mark.parametrize("d,p", [(2, 1), (3, 2), (3, 3), (4, 3), (4, 4), (2, 5)])
def test_phi_identity_exact_integers(d, p):
    """sum_m mu(m) q^m k^m == (q.k)^p exactly, and == the full d^p tuple sum."""
    g = _rng(100 + 10 * d + p)
    idx, mult, _ = O.enumerate_basis(d, p + 1)[p]
    for _ in range(5):
        q = [int(x) for x in g.integers(-5, 6, size=d)]
        k = [int(x) for x in g.integers(-5, 6, size=d)]
        target = sum(a * b for a, b in zip(q, k)) ** p
        brute = 0
        for t in itertools.product(range(d), repeat=p):
            term = 1
            for i in t:
                term *= q[i] * k[i]
            brute += term
        sym = 0
        for r in range(idx.shape[0]):
            mq = 1
            mk = 1
            for i in idx[r]:
                mq *= q[int(i)]
                mk *= k[int(i)]
            sym += int(mult[r]) * mq * mk
        assert brute == target
        assert sym == target


@pytest.mark.parametrize("c", [1.0, 2.0, 0.5])
def test_features_give_truncated_exponential(c):
    """phi_q(q) . phi_k(k) = sum_{p<P} (q.k/c)^p / p! for the weighted one-sided map."""
    g = _rng(7)
    d, P = 5, 4
    basis = O.enumerate_basis(d, P, c)
    q = g.standard_normal((6, d))
    k = g.standard_normal((6, d))
    lhs = np.sum(O.features_q(q, basis) * O.features_k(k, basis), axis=1)
    x = np.sum(q * k, axis=1) / c
    rhs = 1 + x + x * x / 2 + x ** 3 / 6
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)


def test_symmetric_sqrt_weighting_also_factors():
    """Splitting the weight as sqrt(w) on both sides gives the same kernel."""
    g = _rng(8)
    d, P, c = 4, 4, 1.5
    basis = O.enumerate_basis(d, P, c)
    sw = np.sqrt(O.query_weights(basis))
    q = g.standard_normal(d)
    k = g.standard_normal(d)
    lhs = np.sum(O.features_k(q, basis) * sw * O.features_k(k, basis) * sw)
    x = q @ k / c
    assert abs(lhs - sum(x ** p / math.factorial(p) for p in range(P))) < 1e-13


def test_taylor_weight_values():
    assert O.taylor_weight(1.0, 4) == pytest.approx(8.0 / 3.0, abs=1e-15)
    assert O.taylor_weight(-1.0, 3) == pytest.approx(0.5, abs=1e-15)
    xs = np.linspace(-1, 1, 11)
    np.testing.assert_allclose(O.taylor_weight(xs, 30), np.exp(xs), rtol=1e-15)
    np.testing.assert_array_equal(O.taylor_weight(xs, 1), np.ones_like(xs))


# ----------------------------------------------------------------------------
# Direct truncated-Taylor attention: special cases and exact brute force
# ----------------------------------------------------------------------------

def test_P1_is_running_mean():
    g = _rng(11)
    q, k, v = _unit(g, 50, 4), _unit(g, 50, 4), g.standard_normal((50, 3))
    out = O.direct_taylor(q, k, v, P=1)
    ref = np.cumsum(v, axis=0) / np.arange(1, 51)[:, None]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_zero_query_is_running_mean_any_P():
    g = _rng(12)
    k, v = _unit(g, 40, 6), g.standard_normal((40, 2))
    q = np.zeros((40, 6))
    for P in (2, 3, 4, 5):
        out = O.direct_taylor(q, k, v, P=P)
        ref = np.cumsum(v, axis=0) / np.arange(1, 41)[:, None]
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("c", [1.0, 3.0])
def test_P2_is_linear_attention_prefix_sums(c):
    """T_2(x) = 1 + x: out_i = (sum v + q_i^T sum k v^T / c) / (i+1 + q_i . sum k / c)."""
    g = _rng(13)
    n, d, dv = 60, 5, 4
    q, k, v = _unit(g, n, d), _unit(g, n, d), g.standard_normal((n, dv))
    out = O.direct_taylor(q, k, v, P=2, c=c)
    Skv = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)      # [n, d, dv]
    Sk = np.cumsum(k, axis=0)
    Sv = np.cumsum(v, axis=0)
    num = Sv + np.einsum("nd,nde->ne", q, Skv) / c
    den = np.arange(1, n + 1) + np.sum(q * Sk, axis=1) / c
    np.testing.assert_allclose(out, num / den[:, None], rtol=1e-12, atol=1e-13)


def test_direct_taylor_exact_rational():
    """Rational arithmetic straight from the definition on dyadic inputs."""
    g = _rng(14)
    n, d, dv, P = 7, 3, 2, 4
    for c in (1, 2):
        qi = g.integers(-8, 9, size=(n, d))
        ki = g.integers(-8, 9, size=(n, d))
        vi = g.integers(-16, 17, size=(n, dv))
        q = qi / 16.0
        k = ki / 16.0
        v = vi / 4.0
        out = O.direct_taylor(q, k, v, P=P, c=float(c))
        for i in range(n):
            num = [Fraction(0)] * dv
            den = Fraction(0)
            for j in range(i + 1):
                x = sum(Fraction(int(qi[i, a]), 16) * Fraction(int(ki[j, a]), 16) for a in range(d)) / c
                w = sum(x ** p / math.factorial(p) for p in range(P))
                den += w
                for e in range(dv):
                    num[e] += w * Fraction(int(vi[j, e]), 4)
            for e in range(dv):
                assert abs(out[i, e] - float(num[e] / den)) <= 1e-14 * max(1.0, abs(float(num[e] / den)))


def test_causality_and_inclusivity():
    """Changing a future token leaves earlier rows unchanged; row 0 equals v_0."""
    g = _rng(15)
    q, k, v = _unit(g, 30, 4), _unit(g, 30, 4), g.standard_normal((30, 3))
    out = O.direct_taylor(q, k, v, P=4)
    np.testing.assert_allclose(out[0], v[0], rtol=1e-15)
    k2, v2 = k.copy(), v.copy()
    k2[20:] = _unit(g, 10, 4)
    v2[20:] = g.standard_normal((10, 3))
    out2 = O.direct_taylor(q, k2, v2, P=4)
    np.testing.assert_array_equal(out[:20], out2[:20])
    assert np.max(np.abs(out[20:] - out2[20:])) > 1e-3


def test_rows_and_blocks_agree():
    g = _rng(16)
    q, k, v = _unit(g, 300, 8), _unit(g, 300, 8), g.standard_normal((300, 8))
    full = O.direct_taylor(q, k, v, P=3, block=64)
    rows = np.array([0, 5, 63, 64, 199, 299])
    part = O.direct_taylor(q, k, v, P=3, rows=rows, block=4)
    np.testing.assert_allclose(part, full[rows], rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------------------
# The state factorisation and the cost model
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,P", [(3, 3), (4, 4), (2, 5)])
def test_recurrence_matches_direct_and_counts_flops(d, P):
    g = _rng(20 + d + P)
    n, dv = 9, 3
    q, k, v = _unit(g, n, d), _unit(g, n, d), g.standard_normal((n, dv))
    out, ops = O.recurrent_sata(q, k, v, P)
    np.testing.assert_allclose(out, O.direct_taylor(q, k, v, P), rtol=1e-12, atol=1e-13)
    state, flops = O.cost_model(d, dv, P)
    assert np.all(ops == flops)                              # same work for every token
    assert state == (dv + 1) * O.basis_size(d, P)


def test_cost_model_page_values():
    # per-head state and FLOPs for the study's head shapes (exact integers)
    assert O.cost_model(8, 8, 3) == (405, 1780)
    assert O.cost_model(16, 16, 4) == (16473, 71364)
    assert O.cost_model(64, 64, 4) == (3113825, 12738308)
    assert O.cost_model(32, 32, 4) == (215985, 902020)


def test_cost_model_split_per_row():
    """The page total equals sum_p C_p (4 d_v + 4 + 2 p), counted row by row."""
    for d, dv, P in [(8, 8, 3), (16, 16, 4), (64, 64, 4), (32, 32, 4), (5, 7, 5)]:
        basis = O.enumerate_basis(d, P)
        per_rows = sum(idx.shape[0] * (4 * dv + 4 + 2 * p) for p, (idx, _, _) in enumerate(basis))
        assert O.cost_model(d, dv, P)[1] == per_rows


def test_direct_state_readout_matches_direct():
    g = _rng(30)
    n, d, dv, P, c = 40, 4, 3, 4, 1.25
    q, k, v = _unit(g, n, d), _unit(g, n, d), g.standard_normal((n, dv))
    basis = O.enumerate_basis(d, P, c)
    ref = O.direct_taylor(q, k, v, P, c)
    for i in (0, 1, 17, n - 1):
        S, z = O.direct_state(k[:i + 1], v[:i + 1], basis, block=7)
        np.testing.assert_allclose(O.state_readout(q[i], S, z, basis)[0], ref[i], rtol=1e-12, atol=1e-13)


def test_direct_state_brute_force():
    g = _rng(31)
    n, d, dv, P = 6, 3, 2, 4
    k, v = g.standard_normal((n, d)), g.standard_normal((n, dv))
    basis = O.enumerate_basis(d, P)
    S, z = O.direct_state(k, v, basis)
    r = 0
    for idx, _, _ in basis:
        for row in idx:
            mono = [math.prod(float(k[j, int(i)]) for i in row) for j in range(n)]
            assert z[r] == pytest.approx(sum(mono), rel=1e-13, abs=1e-14)
            for e in range(dv):
                assert S[r, e] == pytest.approx(sum(m * v[j, e] for j, m in enumerate(mono)), rel=1e-13, abs=1e-14)
            r += 1


# ----------------------------------------------------------------------------
# Truncation error against exact softmax (reported, not gated)
# ----------------------------------------------------------------------------

def test_softmax_stable_matches_naive():
    g = _rng(40)
    q, k, v = _unit(g, 30, 4), _unit(g, 30, 4), g.standard_normal((30, 3))
    out = O.exact_softmax(q, k, v, c=0.5)
    for i in range(30):
        e = np.exp(k[:i + 1] @ q[i] / 0.5)
        np.testing.assert_allclose(out[i], e @ v[:i + 1] / e.sum(), rtol=1e-13)


def test_truncation_error_bound_and_decrease():
    w = W.WORKLOADS["tiny_d8_n256"]
    q, k, v = (a[0, 0].astype(np.float64) for a in W.workload_inputs(w))
    sm = O.exact_softmax(q, k, v)
    errs = []
    for P in range(1, 7):
        t = O.direct_taylor(q, k, v, P)
        delta = O.taylor_delta(q, k, P)
        if P >= 3:
            assert np.all(delta < 1)
        for i in range(0, 256, 17):
            if delta[i] >= 1:          # the bound needs every weight ratio within (0, 2)
                continue
            spread = np.max(np.abs(v[:i + 1] - sm[i][None, :]), axis=0)
            bound = delta[i] / (1 - delta[i]) * spread
            assert np.all(np.abs(t[i] - sm[i]) <= bound * (1 + 1e-9) + 1e-15)
        errs.append(np.max(np.abs(t - sm)))
    assert all(a > b for a, b in zip(errs, errs[1:]))


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5])
def test_taylor_delta_exact_values(P):
    """delta at logits of +-1 and 1/2 against the partial sums of e written as
    exact fractions (T_P(1) = 1, 2, 5/2, 8/3, 65/24; T_P(-1) = 1, 0, 1/2, 1/3,
    3/8), with math.e / math.exp as the exponential; the max runs over the
    keys j <= i only."""
    t_plus = [Fraction(1), Fraction(2), Fraction(5, 2), Fraction(8, 3), Fraction(65, 24)][P - 1]
    t_minus = [Fraction(1), Fraction(0), Fraction(1, 2), Fraction(1, 3), Fraction(3, 8)][P - 1]
    t_half = sum(Fraction(1, 2 ** p * math.factorial(p)) for p in range(P))
    d_plus = abs(1.0 - float(t_plus) / math.e)
    d_minus = abs(1.0 - float(t_minus) * math.e)
    d_half = abs(1.0 - float(t_half) / math.exp(0.5))
    q = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    k = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 5.0]])   # row 2's own key: x = 5
    got = O.taylor_delta(q[:2], k[:2], P)
    np.testing.assert_allclose(got, [d_plus, max(d_plus, d_minus)], rtol=1e-13, atol=1e-15)
    # c = 2 halves every logit; a later key never enters an earlier row
    got = O.taylor_delta(q, k, P, c=2.0, rows=[0])
    np.testing.assert_allclose(got, [d_half], rtol=1e-13, atol=1e-15)
    # a zero logit is exact for every P
    assert O.taylor_delta(np.array([[0.0, 1.0]]), np.array([[1.0, 0.0]]), P)[0] == 0.0


def test_denominator_positive_on_unit_rows():
    # |x| <= 1 for unit rows; T_3 >= 1/2 and T_4 >= 1/3 there
    xs = np.linspace(-1.01, 1.01, 2001)
    assert np.min(O.taylor_weight(xs, 3)) >= 0.5 - 1e-12
    assert np.min(O.taylor_weight(xs, 4)) >= 1.0 / 3.0 - 0.01


# ----------------------------------------------------------------------------
# Error metric and the seeded inputs
# ----------------------------------------------------------------------------

def test_row_normwise_error():
    ref = np.array([[1.0, -2.0], [0.5, 0.25]])
    out = np.array([[1.1, -2.0], [0.5, 0.30]])
    assert O.row_normwise_error(out, ref) == pytest.approx(0.1)
    assert O.global_normwise_error(out, ref) == pytest.approx(0.05)


def test_bf16_rounding_matches_torch():
    import torch
    g = _rng(50)
    x = np.concatenate([g.standard_normal(10000), g.standard_normal(100) * 1e-30,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8])])
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert np.all(W.bf16_bits(ours).astype(np.uint32) << 16 == ours.view(np.uint32))


def test_inputs_recipe():
    w = W.WORKLOADS["tiny_d8_n256"]
    q, k, v = W.workload_inputs(w)
    assert q.shape == (1, 1, 256, 8) and v.shape == (1, 1, 256, 8)
    np.testing.assert_allclose(np.linalg.norm(q.astype(np.float64), axis=-1), 1.0, rtol=1e-6)
    q2, _, _ = W.workload_inputs(w)
    np.testing.assert_array_equal(q, q2)
    rows = W.sampled_rows(1 << 20)
    assert rows.shape == (64,) and rows[0] == 0 and rows[-1] == (1 << 20) - 1
    assert len(set(rows.tolist())) == 64
