"""Plain, slow float64 CPU oracle for causal symmetry-aware Taylor attention (SATA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library: no kernels, headers, tables or helpers.  It depends only on
numpy and the Python standard library.

What it computes, and where each definition comes from
(SATA page = the blog.hotdry.top summary of "symmetry-aware Taylor
approximation for constant-cost attention"; MoA page = the agents-report.net
summary of memory-optimal attention with a Mathematics of Arrays framework):

* ``taylor_weight`` -- exp(x) truncated to the P terms of orders 0..P-1
  (SATA page, section "Core insight: symmetric tensor decomposition": the
  softmax kernel is the exponential of the query-key dot product, expanded as
  a Taylor series; section "Precision/efficiency trade-off parameter": P is
  the truncation order).
* ``direct_taylor`` -- causal attention with those weights, written straight
  from the definition: out_i = sum_{j<=i} T_P(q_i.k_j/c) v_j / sum_{j<=i} T_P(q_i.k_j/c).
  The sum includes j = i: the section "Engineering of constant compute cost"
  maps the current token's key into the state before the output is formed.
* ``enumerate_basis`` -- the minimal basis of the order-p symmetric tensor:
  all multisets i1 <= ... <= ip over [0, d_K) (section "Core insight"),
  with the multinomial multiplicity mu(m) = p!/prod(count!) and the order
  scale 1/(p! c^p).  Rows are ordered by p, then lexicographically.
* ``direct_state`` -- the fixed-size state of section "Engineering of constant
  compute cost": S_m = sum_j phi_m(k_j) v_j and z_m = sum_j phi_m(k_j), with
  phi_m the unweighted monomial prod_r k[i_r].
* ``state_readout`` -- out = sum_m w_m phi_m(q) S_m / sum_m w_m phi_m(q) z_m
  with w_m = mu(m)/(p! c^p) (the weights sit on the query side).
* ``recurrent_sata`` -- the token-by-token recurrence of section "Engineering
  of constant compute cost", with an operation counter, for tiny inputs.
* ``cost_model`` -- the closed-form state size and per-token FLOP count of the
  same section.
* ``exact_softmax`` -- causal, max-subtracted (numerically stable) softmax
  attention, as in the MoA page's section "DNF derivation".  Report only.
* ``taylor_delta`` -- per-row truncation factor used by the Taylor-remainder
  bound that relates the truncated result to exact softmax.

Readings where the pages are silent or garbled (kept in the design notes):
P counts terms (orders 0..P-1); the causal sum is inclusive; the logit scale
is exp(q.k/c) with c a parameter; weights sit on the query side; rows are
0-based multisets ordered by p, then lexicographically.
"""
from __future__ import annotations

import itertools
import math
from collections import Counter
from fractions import Fraction

import numpy as np


# ----------------------------------------------------------------------------
# Truncated exponential
# ----------------------------------------------------------------------------

def taylor_weight(x, P: int):
    """T_P(x) = sum_{p=0}^{P-1} x^p / p!  (float64, elementwise)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.zeros_like(x)
    for p in range(P):
        w = w + x ** p / math.factorial(p)
    return w


# ----------------------------------------------------------------------------
# Direct causal truncated-Taylor attention (the result definition)
# ----------------------------------------------------------------------------

def direct_taylor(q, k, v, P: int, c: float = 1.0, rows=None, block: int = 1024,
                  return_den: bool = False):
    """Causal truncated-Taylor attention of one head, float64.

    q, k: [n, d_k]; v: [n, d_v].  rows: optional sorted query indices to
    evaluate (default: all n).  Returns out [len(rows), d_v] (and den).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    den = np.empty(rows.shape[0], dtype=np.float64)
    for s in range(0, rows.shape[0], block):
        r = rows[s:s + block]
        jmax = int(r.max()) + 1
        x = (q[r] @ k[:jmax].T) / c                      # [b, jmax]
        w = taylor_weight(x, P)
        w[np.arange(jmax)[None, :] > r[:, None]] = 0.0    # causal, inclusive of j = i
        num = w @ v[:jmax]
        dd = w.sum(axis=1)
        if np.any(dd <= 0):
            raise FloatingPointError("non-positive truncated-Taylor denominator")
        out[s:s + block] = num / dd[:, None]
        den[s:s + block] = dd
    return (out, den) if return_den else out


# ----------------------------------------------------------------------------
# Exact causal softmax (report only)
# ----------------------------------------------------------------------------

def exact_softmax(q, k, v, c: float = 1.0, rows=None, block: int = 1024):
    """Causal softmax attention with max subtraction, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    for s in range(0, rows.shape[0], block):
        r = rows[s:s + block]
        jmax = int(r.max()) + 1
        x = (q[r] @ k[:jmax].T) / c
        mask = np.arange(jmax)[None, :] > r[:, None]
        x[mask] = -np.inf
        m = x.max(axis=1, keepdims=True)
        e = np.exp(x - m)
        out[s:s + block] = (e @ v[:jmax]) / e.sum(axis=1)[:, None]
    return out


def taylor_delta(q, k, P: int, c: float = 1.0, rows=None):
    """delta_i = max_{j<=i} |1 - T_P(x_ij)/exp(x_ij)| per query row.

    With it the truncated output differs from softmax by at most
    delta/(1-delta) * max_{j<=i} |v_j - out_softmax_i| per component.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    res = np.empty(rows.shape[0])
    for t, i in enumerate(rows):
        x = (k[:i + 1] @ q[i]) / c
        res[t] = np.max(np.abs(1.0 - taylor_weight(x, P) / np.exp(x)))
    return res


# ----------------------------------------------------------------------------
# Minimal symmetric basis
# ----------------------------------------------------------------------------

def enumerate_basis(d: int, P: int, c: float = 1.0):
    """Per order p = 0..P-1: (idx int32 [C_p, p], mult uint32 [C_p], scale float64).

    idx rows are the multisets i1 <= ... <= ip over [0, d) in lexicographic
    order; mult is p!/prod(count_i!); scale is 1/(p! c^p).
    """
    out = []
    for p in range(P):
        rows = list(itertools.combinations_with_replacement(range(d), p))
        idx = np.array(rows, dtype=np.int32).reshape(len(rows), p)
        mult = np.empty(len(rows), dtype=np.uint32)
        for r, m in enumerate(rows):
            denom = 1
            for cnt in Counter(m).values():
                denom *= math.factorial(cnt)
            mult[r] = math.factorial(p) // denom
        scale = 1.0 / (math.factorial(p) * float(c) ** p)
        out.append((idx, mult, scale))
    return out


def basis_size(d: int, P: int) -> int:
    """Total number of basis rows over orders 0..P-1 (counted, not closed form)."""
    return sum(idx.shape[0] for idx, _, _ in enumerate_basis(d, P))


def monomials(x, idx):
    """prod_r x[..., idx[:, r]] for each basis row; x [..., d] -> [..., C_p]."""
    x = np.asarray(x, dtype=np.float64)
    res = np.ones(x.shape[:-1] + (idx.shape[0],), dtype=np.float64)
    for r in range(idx.shape[1]):
        res = res * x[..., idx[:, r]]
    return res


def query_weights(basis):
    """w_m = mu(m) * scale_p for every row, concatenated over orders."""
    return np.concatenate([mult.astype(np.float64) * scale for _, mult, scale in basis])


def features_k(x, basis):
    """Unweighted monomials of every row, concatenated over orders: [..., D]."""
    return np.concatenate([monomials(x, idx) for idx, _, _ in basis], axis=-1)


def features_q(x, basis):
    """Weighted query features w_m * prod_r x[i_r]: [..., D]."""
    return features_k(x, basis) * query_weights(basis)


# ----------------------------------------------------------------------------
# The fixed-size state and its readout
# ----------------------------------------------------------------------------

def direct_state(k, v, basis, block: int = 1024):
    """S [D, d_v] = sum_j phi(k_j) v_j^T and z [D] = sum_j phi(k_j), float64."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    D = sum(idx.shape[0] for idx, _, _ in basis)
    S = np.zeros((D, v.shape[1]))
    z = np.zeros(D)
    for s in range(0, k.shape[0], block):
        f = features_k(k[s:s + block], basis)     # [b, D]
        S += f.T @ v[s:s + block]
        z += f.sum(axis=0)
    return S, z


def state_readout(q, S, z, basis):
    """out = phi_q(q) S / phi_q(q) z for query rows q [m, d]."""
    f = features_q(np.atleast_2d(q), basis)
    return (f @ S) / (f @ z)[:, None]


# ----------------------------------------------------------------------------
# Token-by-token recurrence with an operation counter (tiny inputs only)
# ----------------------------------------------------------------------------

def recurrent_sata(q, k, v, P: int, c: float = 1.0):
    """Per-token recurrence over the minimal basis, counting every multiply/add.

    Each token: build phi(k) and the weighted phi(q) for every basis row (p
    multiplies each, starting from the row's constant), add phi(k) [v, 1] into
    the state (one multiply and one add per value column and for z), then read
    out num = phi(q) S and den = phi(q) z (one multiply and one add each).
    Returns (out [n, d_v], per-token op counts [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    dv = v.shape[1]
    basis = enumerate_basis(d, P, c)
    rows = []
    for idx, mult, scale in basis:
        for r in range(idx.shape[0]):
            rows.append((tuple(int(t) for t in idx[r]), float(mult[r]) * scale))
    S = [[0.0] * dv for _ in rows]
    z = [0.0] * len(rows)
    out = np.zeros((n, dv))
    ops = np.zeros(n, dtype=np.int64)
    for t in range(n):
        cnt = 0
        num = [0.0] * dv
        den = 0.0
        for m, (mi, w) in enumerate(rows):
            fk = 1.0
            fq = w
            for i in mi:
                fk *= k[t, i]; cnt += 1
                fq *= q[t, i]; cnt += 1
            for col in range(dv):
                S[m][col] += fk * v[t, col]; cnt += 2
            z[m] += fk * 1.0; cnt += 2
            for col in range(dv):
                num[col] += fq * S[m][col]; cnt += 2
            den += fq * z[m]; cnt += 2
        out[t] = np.array(num) / den
        ops[t] = cnt
    return out, ops


# ----------------------------------------------------------------------------
# Closed-form cost model (section "Engineering of constant compute cost")
# ----------------------------------------------------------------------------

def cost_model(d_k: int, d_v: int, P: int):
    """(state values per head, FLOPs per token per head), exact integers.

    State: (d_v + 1) * C(d_k + P - 1, P - 1).
    FLOPs: (4 d_v + 2 (P d_k + 1)/(d_k + 1) + 2) * C(d_k + P - 1, P - 1).
    Neither depends on the sequence length.
    """
    D = math.comb(d_k + P - 1, P - 1)
    flops = (Fraction(4 * d_v) + Fraction(2 * (P * d_k + 1), d_k + 1) + 2) * D
    if flops.denominator != 1:
        raise ArithmeticError("FLOP count is not an integer")
    return (d_v + 1) * D, int(flops)


# ----------------------------------------------------------------------------
# Error metrics used by the parity gates
# ----------------------------------------------------------------------------

def row_normwise_error(out, ref):
    """max over rows of ||o_i - r_i||_inf / ||r_i||_inf."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    o = out.reshape(-1, out.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.max(np.abs(o - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    return float(np.max(num / den))


def global_normwise_error(out, ref):
    """||O - R||_inf / ||R||_inf over the whole array."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(out - ref)) / np.max(np.abs(ref)))
