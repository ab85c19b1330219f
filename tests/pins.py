"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
AssertionError when the handle disagrees with the pages.  The same functions
run against the real oracle (tests/test_oracle_pins.py) and against copies of
it with planted mistakes (tests/test_oracle_mutants.py), which must fail at
least one pin each.

Expected values come from the pages' printed numbers (tests/golden/*.json),
from closed forms, or from library routines (scipy.special.softmax /
logsumexp, numpy.searchsorted) applied to the same inputs; never from the
oracle itself.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy import special, stats

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def grid(M):
    """Stratified uniforms (m + 1/2) / M, exact in fp32 for M a power of two
    or a small integer grid used below."""
    return ((np.arange(M, dtype=np.float64) + 0.5) / M).astype(np.float32)


def logits_of(p):
    """fp32 logits whose softmax at T=1 is p up to fp32 rounding (-inf where
    p is 0)."""
    p = np.asarray(p, np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


def softmax_T(l, T):
    return special.softmax(np.asarray(l, np.float64) / T, axis=-1)


# --------------------------------------------------------------------------
# Row statistics
# --------------------------------------------------------------------------

def pin_stats_logsumexp(o):
    """m is the exact row max; m/T + log Z equals scipy's logsumexp(l/T)."""
    rng = np.random.default_rng(11)
    for T in (1.0, 0.6, 1.7):
        l32 = (rng.standard_normal((7, 513)) * 3).astype(np.float32)
        l32[2, 100:200] = -np.inf
        m, z = o.softmax_stats(l32, T)
        assert np.array_equal(m, l32.max(axis=1).astype(np.float64))
        lse = special.logsumexp(l32.astype(np.float64) / T, axis=1)
        np.testing.assert_allclose(m / T + np.log(z), lse, rtol=1e-13, atol=1e-13)
        f = (rng.standard_normal((3, 300)) * 4).astype(np.float32)
        bits = (f.view(np.uint32) >> 16).astype(np.uint16)     # valid bf16 values
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        m, z = o.softmax_stats(bits, T)
        assert np.array_equal(m, vals.max(axis=1))
        np.testing.assert_allclose(m / T + np.log(z), special.logsumexp(vals / T, axis=1),
                                   rtol=1e-13, atol=1e-13)


def pin_stats_closed_forms(o):
    """Constant row: Z = V.  Two-level row {a x n, b x (V-n)}: Z = n +
    (V-n) exp((b-a)/T)."""
    V = 1000
    m, z = o.softmax_stats(np.full((1, V), 2.5, np.float32), 0.8)
    assert m[0] == 2.5 and z[0] == float(V)
    row = np.full((1, V), -1.0, np.float32)
    row[0, :37] = 3.0
    for T in (1.0, 0.8, 2.0):
        m, z = o.softmax_stats(row, T)
        assert m[0] == 3.0
        assert abs(z[0] - (37 + (V - 37) * np.exp(-4.0 / T))) < 1e-10 * z[0]


# --------------------------------------------------------------------------
# One position: accept test and residual, the pages' worked pairs
# --------------------------------------------------------------------------

def _one_position_laws(o, p, q, M, T=1.0):
    """Measure, through the oracle with stratified uniforms, the accept
    probability of every draft token and the residual law.

    Returns (a, h): a[x] = fraction of u in the grid that accepts draft x;
    h = token histogram of the final draw after a rejection."""
    V = len(p)
    lt = np.stack([logits_of(p), logits_of(p)])[None]        # [1, 2, V]
    ld = logits_of(q)[None, None]                              # [1, 1, V]
    u = grid(M)
    a = np.zeros(V)
    for x in range(V):
        tgt = np.repeat(lt, M, axis=0)
        drf = np.repeat(ld, M, axis=0)
        toks = np.full((M, 1), x, np.int32)
        uni = np.stack([u, np.full(M, 0.5, np.float32)], axis=1)
        r = o.verify(tgt, drf, toks, uni, T)
        a[x] = np.mean(r["num_accepted"] == 1)
    # Residual law: draft the token with the smallest p/q (a sure rejection
    # at u = 1 - 2^-24) and sweep the final uniform.
    ratios = np.where(np.asarray(q) > 0, np.asarray(p) / np.maximum(q, 1e-300), np.inf)
    x = int(np.argmin(ratios))
    tgt = np.repeat(lt, M, axis=0)
    drf = np.repeat(ld, M, axis=0)
    toks = np.full((M, 1), x, np.int32)
    uni = np.stack([np.full(M, 1 - 2**-24, np.float32), u], axis=1)
    r = o.verify(tgt, drf, toks, uni, T)
    assert np.all(r["num_accepted"] == 0)
    h = np.bincount(r["out_tokens"][:, 0], minlength=V)[:V] / M
    return a, h


def pin_check_your_understanding(o):
    """3.5 Speculative Decoding, 'Check your understanding': beta = 0.7,
    residual (1, 0, 0), P(a) = 0.3 + 0.3 * 1 = 0.6."""
    g = golden("check_your_understanding.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    M = 4096
    a, h = _one_position_laws(o, p, q, M)
    beta = float(np.dot(q, a))
    assert abs(beta - g["acceptance_beta"]) < 2.0 / M, beta
    np.testing.assert_allclose(h, g["residual"], atol=2.0 / M)
    law = q * a + np.dot(q, 1 - a) * h
    assert abs(law[0] - g["p_emit_a"]) < 3.0 / M
    np.testing.assert_allclose(law, p, atol=3.0 / M)


def pin_single_position_experiment(o):
    """246 Speculative Decoding, 3.2: accept rate sum min(p, q) = 0.55,
    residual (2/3, 1/3, 0, 0, 0, 0); emitted law = p.  The printed empirical
    accept rate (0.551 at N = 200000) lies within 3 sigma of 0.55."""
    g = golden("single_position_experiment.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    M = 4096
    a, h = _one_position_laws(o, p, q, M)
    beta = float(np.dot(q, a))
    assert abs(beta - 0.55) < 2.0 / M, beta
    np.testing.assert_allclose(h, [2 / 3, 1 / 3, 0, 0, 0, 0], atol=2.0 / M)
    law = q * a + np.dot(q, 1 - a) * h
    np.testing.assert_allclose(law, p, atol=3.0 / M)
    sigma = np.sqrt(0.55 * 0.45 / g["samples"])
    assert abs(g["printed_accept_rate"] - beta) < 3 * sigma + 0.0005 + 2.0 / M


def pin_single_position_chisquare(o):
    """Random drafts x ~ q and random uniforms: the emitted token passes a
    chi-square test against p (246 Speculative Decoding, 3.2 experiment,
    redone through the oracle)."""
    g = golden("single_position_experiment.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    N = 200_000
    rng = np.random.default_rng(12345)
    lt = np.stack([logits_of(p), logits_of(p)])
    tgt = np.ascontiguousarray(np.broadcast_to(lt, (N, 2, 6)))
    drf = np.ascontiguousarray(np.broadcast_to(logits_of(q), (N, 1, 6)))
    toks = rng.choice(6, size=(N, 1), p=q).astype(np.int32)
    uni = rng.random((N, 2), dtype=np.float32)
    r = o.verify(tgt, drf, toks, uni, 1.0)
    counts = np.bincount(r["out_tokens"][:, 0], minlength=6)
    chi = stats.chisquare(counts, N * p)
    assert chi.pvalue > 1e-3, (counts / N, chi)
    acc = np.mean(r["num_accepted"])
    assert abs(acc - 0.55) < 4 * np.sqrt(0.55 * 0.45 / N)


# --------------------------------------------------------------------------
# Several positions: per-position laws, bonus row, uniform indexing
# --------------------------------------------------------------------------

def _rows(seed, K, V, T):
    rng = np.random.default_rng(seed)
    lt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    ld = (lt[:K] + rng.standard_normal((K, V)) * 1.2).astype(np.float32)
    return lt, ld, softmax_T(lt, T), softmax_T(ld, T)


def pin_multi_position_exact(o):
    """K=3, V=5, T=0.7.  Forcing acceptance before position i with u = 0,
    the accept probability at i is min(1, P_i/Q_i), the residual law after a
    rejection at i is max(0, P_i - Q_i)/S (drawn with uniforms[k]), the bonus
    law is P_k, and the law of the token emitted at i is P_i
    (3.5 Speculative Decoding, 'The algorithm (one step)' and 'Proof')."""
    K, V, T, M = 3, 5, 0.7, 2048
    lt, ld, P, Q = _rows(5, K, V, T)
    u = grid(M)
    base_t = np.repeat(lt[None], M, axis=0)
    base_d = np.repeat(ld[None], M, axis=0)
    for i in range(K):
        a = np.zeros(V)
        for x in range(V):
            toks = np.zeros((M, K), np.int32)
            toks[:, i] = x
            uni = np.zeros((M, K + 1), np.float32)
            uni[:, i] = u
            uni[:, K] = 0.5
            r = o.verify(base_t, base_d, toks, uni, T)
            assert np.all(r["num_accepted"] >= i)
            a[x] = np.mean(r["num_accepted"] > i)
            np.testing.assert_allclose(r["accept_prob"][0, i], min(1.0, P[i, x] / Q[i, x]),
                                       rtol=1e-6)
        np.testing.assert_allclose(a, np.minimum(1.0, P[i] / Q[i]), atol=1.0 / M)
        x = int(np.argmin(P[i] / Q[i]))
        toks = np.zeros((M, K), np.int32)
        toks[:, i] = x
        uni = np.zeros((M, K + 1), np.float32)
        uni[:, i] = 1 - 2**-24
        uni[:, i + 1:K] = 0.25          # unused by the step
        uni[:, K] = u
        r = o.verify(base_t, base_d, toks, uni, T)
        assert np.all(r["num_accepted"] == i)
        h = np.bincount(r["out_tokens"][:, i], minlength=V)[:V] / M
        res = np.maximum(P[i] - Q[i], 0)
        np.testing.assert_allclose(h, res / res.sum(), atol=2.0 / M)
        law = Q[i] * a + np.dot(Q[i], 1 - a) * h
        np.testing.assert_allclose(law, P[i], atol=3.0 / M)
    toks = np.zeros((M, K), np.int32)
    uni = np.zeros((M, K + 1), np.float32)
    uni[:, K] = u
    r = o.verify(base_t, base_d, toks, uni, T)
    assert np.all(r["num_accepted"] == K)
    h = np.bincount(r["out_tokens"][:, K], minlength=V)[:V] / M
    np.testing.assert_allclose(h, P[K], atol=2.0 / M)


def pin_multi_position_chisquare(o):
    """Fixed rows, drafts x_i ~ Q_i, random uniforms: given position i is
    reached, the emitted token there passes a chi-square test against P_i."""
    K, V, T, N = 3, 6, 0.9, 120_000
    lt, ld, P, Q = _rows(9, K, V, T)
    rng = np.random.default_rng(99)
    toks = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1).astype(np.int32)
    uni = rng.random((N, K + 1), dtype=np.float32)
    tgt = np.ascontiguousarray(np.broadcast_to(lt, (N, K + 1, V)))
    drf = np.ascontiguousarray(np.broadcast_to(ld, (N, K, V)))
    r = o.verify(tgt, drf, toks, uni, T)
    n = r["num_accepted"]
    for i in range(K + 1):
        reached = n >= i
        counts = np.bincount(r["out_tokens"][reached, i], minlength=V)[:V]
        exp = reached.sum() * P[i]
        keep = exp >= 5
        c = np.append(counts[keep], counts[~keep].sum())
        e = np.append(exp[keep], exp[~keep].sum())
        if e[-1] == 0:
            c, e = c[:-1], e[:-1]
        assert stats.chisquare(c, e).pvalue > 1e-3, (i, counts, exp)


def pin_k0_is_inverse_cdf(o):
    """k_b = 0 reduces to plain inverse-CDF sampling from p_1 (the bonus draw
    with no drafts): token = searchsorted(cumsum(p), u * sum(p), 'right')."""
    rng = np.random.default_rng(3)
    V, T, N = 777, 1.3, 4000
    lt = (rng.standard_normal((1, 1, V)) * 2).astype(np.float32)
    tgt = np.repeat(lt, N, axis=0)
    u = rng.random((N, 1), dtype=np.float32)
    r = o.verify(tgt, None, np.zeros((N, 0), np.int32), u, T)
    P = softmax_T(lt[0, 0], T)
    c = np.cumsum(P)
    ref = np.searchsorted(c, u[:, 0].astype(np.float64) * c[-1], side="right")
    safe = np.min(np.abs(c[None, :] / c[-1] - u.astype(np.float64)), axis=1) > 1e-9
    assert safe.mean() > 0.99
    assert np.array_equal(r["out_tokens"][safe, 0], ref[safe])
    assert np.all(r["num_accepted"] == 0)


def pin_identity(o):
    """q = p accepts every draft (246 Speculative Decoding, 3.4: noise 0.0
    gives acceptance 1 and k+1 tokens per call)."""
    rng = np.random.default_rng(4)
    B, K, V = 64, 4, 300
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = lt[:, :K].copy()
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    r = o.verify(lt, ld, toks, uni, 0.9)
    assert np.all(r["num_accepted"] == K)
    assert np.array_equal(r["out_tokens"][:, :K], toks)
    assert np.all(r["accept_prob"] == 1.0)


def pin_disjoint_support(o):
    """Disjoint supports: every draft is rejected at the first position and
    the replacement is drawn from p_1 itself."""
    V, M, T = 6, 4096, 1.0
    p = np.array([0.5, 0.3, 0.2, 0, 0, 0])
    q = np.array([0, 0, 0, 0.25, 0.75, 0])
    lt = np.stack([logits_of(p), logits_of(p)])[None]
    ld = logits_of(q)[None, None]
    tgt = np.repeat(lt, M, axis=0)
    drf = np.repeat(ld, M, axis=0)
    toks = np.full((M, 1), 4, np.int32)
    uni = np.stack([np.full(M, 0.0, np.float32), grid(M)], axis=1)
    r = o.verify(tgt, drf, toks, uni, T)
    assert np.all(r["num_accepted"] == 0)
    assert np.all(r["accept_prob"][:, 0] == 0.0)
    h = np.bincount(r["out_tokens"][:, 0], minlength=V) / M
    np.testing.assert_allclose(h, p, atol=2.0 / M)


def pin_strict_comparisons(o):
    """Readings: accept iff u < ratio (strict), and the draw is the smallest t
    with u*S < C_t (strict).  With one-hot drafts and p = (1/2, 1/2) both
    thresholds are exactly 1/2."""
    lt = np.zeros((2, 2, 2), np.float32)          # p = (0.5, 0.5) exactly
    toks = np.zeros((2, 1), np.int32)
    uni = np.array([[0.5, 0.5], [0.5 - 2**-24, 0.5]], np.float32)
    r = o.verify(lt, None, toks, uni, 1.0)
    assert list(r["num_accepted"]) == [0, 1]
    # After the rejection at u = 1/2 the one-hot residual is (0, 1).
    assert r["out_tokens"][0, 0] == 1
    # k = 0: the bonus draw from (1/2, 1/2) at u = 1/2 lands on token 1,
    # just below 1/2 on token 0.
    lt0 = np.zeros((2, 1, 2), np.float32)
    r = o.verify(lt0, None, np.zeros((2, 0), np.int32),
                 np.array([[0.5], [0.5 - 2**-24]], np.float32), 1.0)
    assert list(r["out_tokens"][:, 0]) == [1, 0]


def pin_q_zero_accepts(o):
    """A draft token with q = 0 gets ratio 1 and is accepted (246 Speculative
    Decoding, 3.1)."""
    lt = np.zeros((1, 2, 4), np.float32)
    ld = np.array([[[0.0, 0.0, -np.inf, 0.0]]], np.float32)
    r = o.verify(lt, ld, np.array([[2]], np.int32), np.array([[0.999, 0.3]], np.float32), 1.0)
    assert r["num_accepted"][0] == 1 and r["accept_prob"][0, 0] == 1.0
    assert r["out_tokens"][0, 0] == 2


def pin_one_hot_drafts(o):
    """One-hot drafts: accept probability p(x); the residual is p with x
    removed and renormalised (3.5 Speculative Decoding, 'Proof', greedy
    remark and the n-gram row of 'Choosing a draft')."""
    V, M, T = 5, 4096, 0.8
    lt, _, P, _ = _rows(21, 1, V, T)
    tgt = np.repeat(lt[None], M, axis=0)
    x = 2
    uni = np.stack([grid(M), np.full(M, 0.5, np.float32)], axis=1)
    r = o.verify(tgt, None, np.full((M, 1), x, np.int32), uni, T)
    assert abs(np.mean(r["num_accepted"] == 1) - P[0, x]) < 1.0 / M
    uni = np.stack([np.full(M, 1 - 2**-24, np.float32), grid(M)], axis=1)
    r = o.verify(tgt, None, np.full((M, 1), x, np.int32), uni, T)
    h = np.bincount(r["out_tokens"][:, 0], minlength=V) / M
    res = P[0].copy()
    res[x] = 0
    np.testing.assert_allclose(h, res / res.sum(), atol=2.0 / M)


# --------------------------------------------------------------------------
# Expected tokens per step: the closed form through the oracle
# --------------------------------------------------------------------------

def closed_form(alpha, k):
    return (1 - alpha ** (k + 1)) / (1 - alpha)


def pin_closed_form_printed_values(o=None):
    """The closed form reproduces every value the pages print (to their
    printed precision)."""
    for c in golden("tokens_per_step.json")["cases"]:
        v = closed_form(c["alpha"], c["k"])
        assert round(v, c["decimals"]) == round(c["value"], c["decimals"]) or \
            abs(v - c["value"]) <= 0.5 * 10 ** -c["decimals"] + 1e-9, (c, v)


def _mean_emitted_grid(o, alpha, M, k):
    """Exact mean tokens per step over the full product grid of accept
    uniforms: one-hot drafts whose target probability is alpha (V = 2), and a
    grid of M values per position on which exactly alpha*M values accept."""
    lt = logits_of([alpha, 1 - alpha])
    u = grid(M)
    mesh = np.stack(np.meshgrid(*([u] * k), indexing="ij"), axis=-1).reshape(-1, k)
    N = mesh.shape[0]
    tgt = np.ascontiguousarray(np.broadcast_to(lt, (N, k + 1, 2)))
    uni = np.concatenate([mesh, np.full((N, 1), 0.5, np.float32)], axis=1)
    r = o.verify(tgt, None, np.zeros((N, k), np.int32), uni, 1.0)
    return float(np.mean(r["num_accepted"] + 1))


def pin_closed_form_through_oracle(o):
    """Independent acceptance with probability alpha at each position gives
    (1 - alpha^(k+1)) / (1 - alpha) tokens per step (3.5 Speculative
    Decoding, 'Expected tokens per step'; 246 Speculative Decoding, 2.4;
    Speculative Decoding from First Principles)."""
    for alpha, M, k in ((0.7, 20, 3), (0.6, 5, 3), (0.8, 5, 4), (0.8, 5, 8), (0.7, 10, 5)):
        got = _mean_emitted_grid(o, alpha, M, k)
        assert abs(got - closed_form(alpha, k)) < 1e-9, (alpha, k, got)
    # alpha = 0.7, k = 8 ("about 3.2") with random uniforms.
    rng = np.random.default_rng(8)
    N, k = 200_000, 8
    tgt = np.ascontiguousarray(np.broadcast_to(logits_of([0.7, 0.3]), (N, k + 1, 2)))
    r = o.verify(tgt, None, np.zeros((N, k), np.int32),
                 rng.random((N, k + 1), dtype=np.float32), 1.0)
    e = r["num_accepted"] + 1.0
    assert abs(e.mean() - closed_form(0.7, 8)) < 4 * e.std() / np.sqrt(N)
    assert e.min() >= 1 and e.max() <= k + 1


# --------------------------------------------------------------------------
# Ragged k, invariants
# --------------------------------------------------------------------------

def pin_ragged_equals_truncated(o):
    """A request with k_b < K gives the same result as the same request
    alone with K = k_b (padded rows are never read: they hold NaN)."""
    rng = np.random.default_rng(6)
    B, K, V, T = 12, 5, 200, 0.6
    kp = rng.integers(0, K + 1, size=B).astype(np.int32)
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    for b in range(B):
        lt[b, kp[b] + 1:] = np.nan
        ld[b, kp[b]:] = np.nan
        uni[b, kp[b]] = rng.random(dtype=np.float32)
    r = o.verify(lt, ld, toks, uni, T, k_per_req=kp)
    for b in range(B):
        kb = int(kp[b])
        rb = o.verify(lt[b:b + 1, :kb + 1], ld[b:b + 1, :kb], toks[b:b + 1, :kb],
                      uni[b:b + 1, :kb + 1], T)
        assert r["num_accepted"][b] == rb["num_accepted"][0]
        assert np.array_equal(r["out_tokens"][b, :kb + 1], rb["out_tokens"][0])
        assert np.all(r["out_tokens"][b, kb + 1:] == -1)
        assert np.all(r["accept_prob"][b, kb:] == -1.0)


def pin_invariants(o):
    """Every step emits between 1 and k+1 tokens; the accepted prefix is the
    drafts; a replacement after a rejection is never the rejected draft."""
    rng = np.random.default_rng(7)
    B, K, V, T = 500, 6, 50, 1.0
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    Q = softmax_T(ld, T)
    toks = np.array([[rng.choice(V, p=Q[b, i]) for i in range(K)] for b in range(B)], np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    r = o.verify(lt, ld, toks, uni, T)
    n = r["num_accepted"]
    assert n.min() >= 0 and n.max() <= K
    for b in range(B):
        out = r["out_tokens"][b]
        assert np.array_equal(out[:n[b]], toks[b, :n[b]])
        assert 0 <= out[n[b]] < V
        assert np.all(out[n[b] + 1:] == -1)
        if n[b] < K:
            assert out[n[b]] != toks[b, n[b]]


# --------------------------------------------------------------------------
# Greedy
# --------------------------------------------------------------------------

def pin_greedy_worked_trace(o):
    """3.5 Speculative Decoding, 'Worked example': drafts (Paris, ., It, is),
    target argmax (Paris, ., The, -, -) emit Paris, ., The; no bonus."""
    g = golden("worked_greedy_trace.json")
    voc = g["vocabulary"]
    V = len(voc)
    rng = np.random.default_rng(1)
    lt = rng.standard_normal((1, 5, V)).astype(np.float32)
    for i, w in enumerate(g["target_argmax"]):
        tok = voc[w] if w is not None else voc["<other>"]
        lt[0, i, tok] = 10.0
    drafts = np.array([[voc[w] for w in g["drafts"]]], np.int32)
    r = o.verify_greedy(lt, drafts)
    assert r["num_accepted"][0] == g["num_accepted"]
    emitted = [int(t) for t in r["out_tokens"][0] if t >= 0]
    assert emitted == [voc[w] for w in g["emitted"]]


def pin_greedy_ties_and_bonus(o):
    """Ties go to the lowest id; when all drafts match, the argmax of the row
    after the last draft is emitted as the extra token."""
    lt = np.zeros((1, 3, 10), np.float32)
    lt[0, 0, [3, 7]] = 5.0
    lt[0, 1, [8, 2, 9]] = 4.0
    lt[0, 2, [6, 1]] = 2.0
    r = o.verify_greedy(lt, np.array([[3, 2]], np.int32))
    assert r["num_accepted"][0] == 2 and list(r["out_tokens"][0]) == [3, 2, 1]
    r = o.verify_greedy(lt, np.array([[7, 2]], np.int32))
    assert r["num_accepted"][0] == 0 and list(r["out_tokens"][0]) == [3, -1, -1]
    bits = np.zeros((1, 2, 4), np.uint16)
    bits[0, 0] = [0x4000, 0x4040, 0x4040, 0x3F80]       # 2, 3, 3, 1
    bits[0, 1] = [0xFF80, 0xC000, 0xBF80, 0xBF80]       # -inf, -2, -1, -1
    r = o.verify_greedy(bits, np.array([[1]], np.int32))
    assert list(r["out_tokens"][0]) == [1, 2]


def pin_greedy_equals_argmax_decoding(o):
    """Greedy verification reproduces plain argmax decoding token for token
    (3.5 Speculative Decoding, 'Proof', greedy remark; Speculative Decoding
    from First Principles, 'The output does not change').  Toy model: a
    V x V table of next-token logits (a Markov chain over V = 1000 ids);
    drafts come from a noisy argmax."""
    rng = np.random.default_rng(2024)
    V, K, n_tokens = 1000, 4, 10_000
    table = (rng.standard_normal((V, V)) * 2).astype(np.float32)
    table_am = np.argmax(table, axis=1)
    plain = [0]
    while len(plain) < n_tokens + 1:
        plain.append(int(table_am[plain[-1]]))
    seq, steps = [0], 0
    while len(seq) < n_tokens + 1:
        ctx = seq[-1]
        drafts, c = [], ctx
        for _ in range(K):
            c = int(table_am[c]) if rng.random() < 0.75 else int(rng.integers(V))
            drafts.append(c)
        rows = table[[ctx] + drafts][None]
        r = o.verify_greedy(rows, np.array([drafts], np.int32))
        n = int(r["num_accepted"][0])
        seq.extend(int(t) for t in r["out_tokens"][0, :n + 1])
        steps += 1
    assert seq[:n_tokens + 1] == plain[:n_tokens + 1]
    assert steps < n_tokens / 1.5


# --------------------------------------------------------------------------
# End to end: the toy Markov chain of 3.5 Speculative Decoding, 'Code'
# --------------------------------------------------------------------------

def pin_markov_chain_third_token(o):
    """V = 6, k = 4: a target chain and a draft 0.7 * target + 0.3 * other;
    drafts are sampled autoregressively from the draft chain, the oracle
    verifies, and the frequency of the third generated token from start
    token 0 passes a chi-square test against the third power of the target
    chain (3.5 Speculative Decoding, 'Code')."""
    rng = np.random.default_rng(0)
    V, k, N = 6, 4, 40_000

    def chain(sharp):
        x = np.exp(rng.standard_normal((V, V)) * sharp)
        return x / x.sum(1, keepdims=True)

    Pt = chain(2.0)
    Pd = 0.7 * Pt + 0.3 * chain(2.0)
    Lt, Ld = logits_of(Pt), logits_of(Pd)
    cdf_d = np.cumsum(Pd, axis=1)
    seqs = [[] for _ in range(N)]
    prev = np.zeros(N, np.int64)
    active = np.arange(N)
    while active.size:
        n = active.size
        drafts = np.empty((n, k), np.int32)
        ctx = prev[active].copy()
        for i in range(k):
            u = rng.random(n)
            nxt = (u[:, None] < cdf_d[ctx]).argmax(axis=1)
            drafts[:, i] = nxt
            ctx = nxt
        rows_t = np.concatenate([prev[active][:, None], drafts], axis=1)
        tgt = Lt[rows_t]
        drf = Ld[rows_t[:, :k]]
        r = o.verify(tgt, drf, drafts, rng.random((n, k + 1), dtype=np.float32), 1.0)
        still = []
        for j, b in enumerate(active):
            m = int(r["num_accepted"][j]) + 1
            seqs[b].extend(int(t) for t in r["out_tokens"][j, :m])
            prev[b] = seqs[b][-1]
            if len(seqs[b]) < 3:
                still.append(b)
        active = np.array(still, np.int64)
    counts = np.bincount([s[2] for s in seqs], minlength=V)
    exact = np.linalg.matrix_power(Pt, 3)[0]
    assert stats.chisquare(counts, N * exact).pvalue > 1e-3, (counts / N, exact)


def _counters_for_alpha(num, den):
    """One-position counters whose tested/accepted ratio is num/den."""
    return np.array([[den], [den], [num]], np.uint64)


def pin_speedup_table_and_choice(o):
    """3.5 Speculative Decoding, 'Worked example' (alpha = 0.8, c = 0.05):
    the speedup of every k the table prints, to its two decimals, and the
    table's best k (8) chosen over k = 1..10."""
    g = golden("speedup_choosing_k.json")
    cnt = _counters_for_alpha(4, 5)
    for case in g["cases"]:
        k, at, ad, sp = o.choose_k(cnt, g["c"], case["k"], case["k"])
        assert k == case["k"] and abs(at - g["alpha"]) < 1e-15
        assert round(sp, case["decimals"]) == case["speedup"], (case, sp)
    k, _, _, sp = o.choose_k(cnt, g["c"], 1, 10)
    assert k == g["best_printed_k"], k
    # 'Speedup: each step costs T(1 + 4 x 0.05) = 1.2 T, so speedup = 3.36 / 1.2 = 2.8'
    assert abs(o.choose_k(cnt, g["c"], 4, 4)[3] - 3.3616 / 1.2) < 1e-12
    # A dearer draft shifts the optimum to a smaller k ('with a separate 1B
    # draft model (c perhaps 0.1-0.2) the optimum shifts to smaller k').
    assert o.choose_k(cnt, 0.15, 1, 10)[0] < k
    # alpha = 0: one token per step whatever k, so the cheapest k; alpha = 1:
    # k + 1 tokens per step, so the largest k while c < 1.
    assert o.choose_k(_counters_for_alpha(0, 7), 0.05, 1, 10)[0] == 1
    assert o.choose_k(_counters_for_alpha(7, 7), 0.05, 1, 10)[0] == 10
    # Reading: on equal speedups the smaller k (fewer draft passes).  With
    # alpha = 0 and free drafts every k gives exactly one token per pass.
    assert o.choose_k(_counters_for_alpha(0, 7), 0.0, 2, 9)[0] == 2


def pin_acceptance_count_identities(o):
    """Per-position counters against identities that hold for any step:
    sum_i drafted_i = sum_b k_b; sum_i accepted_i = sum_b n_b; every
    request tests its accepted positions plus the one it rejects, so
    sum_i tested_i = sum_b (n_b + [n_b < k_b]); accepted_i <= tested_i <=
    drafted_i; position 0 is tested by every request that drafts; position
    i+1 is tested by the requests that accepted i and drafted i+1.  Counters
    accumulate across calls."""
    rng = np.random.default_rng(31)
    K = 7
    for trial in range(20):
        B = int(rng.integers(1, 40))
        kp = rng.integers(0, K + 1, size=B).astype(np.int32)
        n = np.array([rng.integers(0, k + 1) for k in kp], np.int32)
        c = o.acceptance_counts(n, K, kp)
        d, t, a = (c[r].astype(np.int64) for r in range(3))
        assert d.sum() == kp.sum() and a.sum() == n.sum()
        assert t.sum() == (n + (n < kp)).sum()
        assert np.all(a <= t) and np.all(t <= d)
        assert t[0] == np.count_nonzero(kp > 0)
        for i in range(K - 1):
            assert t[i + 1] == np.count_nonzero((n > i) & (kp > i + 1))
        c2 = o.acceptance_counts(n, K, kp, c.copy())
        assert np.array_equal(c2, 2 * c)
    # k_per_req omitted means k_b = K for every request.
    n = np.array([0, K, 3], np.int32)
    assert np.array_equal(o.acceptance_counts(n, K), o.acceptance_counts(n, K, np.full(3, K, np.int32)))


def pin_alpha_test_estimates_alpha(o):
    """Draws from the pages' simplifying model -- each draft accepted
    independently with probability alpha, the step stopping at the first
    rejection -- give alpha_test = accepted / tested within sampling error
    of alpha, while the engine ratio accepted / drafted stays below it (the
    positions after a rejection are drafted but never tested)."""
    rng = np.random.default_rng(47)
    K, B = 6, 20000
    for alpha in (0.3, 0.6, 0.85):
        acc = rng.random((B, K)) < alpha
        n = np.where(acc.all(axis=1), K, np.argmin(acc, axis=1)).astype(np.int32)
        c = o.acceptance_counts(n, K)
        _, at, ad, _ = o.choose_k(c, 0.0, 1, 1)
        tested = float(c[1].sum())
        assert abs(at - alpha) < 4.0 * np.sqrt(alpha * (1 - alpha) / tested), (alpha, at)
        assert ad < alpha - 0.01, (alpha, ad)


def _ngram_by_rfind(ctx, n_min, n_max, K):
    """The drafter's reading restated with str.rfind: one code point per
    token; the haystack stops one token short of the end, so a match can
    not be the suffix itself."""
    s = "".join(chr(0x100 + int(t)) for t in ctx)
    L = len(ctx)
    for n in range(n_max, n_min - 1, -1):
        if n > L - 1:
            continue
        idx = s[:L - 1].rfind(s[L - n:])
        if idx >= 0:
            e = idx + n - 1
            prop = [int(t) for t in ctx[e + 1:e + 1 + K]]
            return prop + [-1] * (K - len(prop)), len(prop)
    return [-1] * K, 0


def pin_ngram_drafter(o):
    """n-gram / prompt lookup: find the last few tokens earlier in the
    context and propose what followed them (3.5 Speculative Decoding,
    'Choosing a draft'; Mathematical Foundations, 'Non-Parametric Drafters';
    First Principles, 'Four kinds of drafter').  Hand cases for each reading,
    then random copy-heavy contexts against str.rfind."""
    def run(tokens, n_min, n_max, K):
        ctx = np.array([tokens], np.int32)
        d, k = o.ngram_propose(ctx, np.array([len(tokens)], np.int32), n_min, n_max, K)
        return list(d[0][:k[0]]), int(k[0]), list(d[0])
    # 'the cat sat on the mat . the cat' -> 'sat on the'
    w = "the cat sat on the mat . the cat".split()
    ids = {t: i for i, t in enumerate(dict.fromkeys(w))}
    prop, k, _ = run([ids[t] for t in w], 1, 4, 3)
    assert [list(ids)[i] for i in prop] == ["sat", "on", "the"] and k == 3
    # No earlier occurrence: no drafts, padding -1.
    assert run([1, 2, 3, 4], 1, 3, 3) == ([], 0, [-1, -1, -1])
    # The latest occurrence wins: ... 5 7 | ... 5 8 | 5  -> propose 8.
    assert run([5, 7, 9, 5, 8, 9, 5], 1, 1, 1)[0] == [8]
    # A longer match beats a later shorter one: suffix (3, 4); (3, 4) occurs
    # early (followed by 10), 4 alone occurs late (followed by 11).
    assert run([3, 4, 10, 4, 11, 3, 4], 1, 2, 1)[0] == [10]
    # n_min: a length-1 match is ignored when n_min = 2.
    assert run([7, 1, 2, 9, 7], 2, 3, 2)[1] == 0
    # Cut at the end of the context, running into the suffix: 6 6 6 -> 6 6.
    assert run([6, 6, 6], 1, 2, 4)[0] == [6]
    assert run([1, 6, 6, 6], 1, 1, 4)[0] == [6]
    rng = np.random.default_rng(77)
    for _ in range(300):
        L = int(rng.integers(1, 60))
        base = rng.integers(0, 6, size=L).astype(np.int32)
        # Copy a random segment to the end now and then (copy-heavy text).
        if L > 8 and rng.random() < 0.5:
            a = int(rng.integers(0, L - 4))
            m = int(rng.integers(2, 5))
            base[L - m:] = base[a:a + m]
        n_min = int(rng.integers(1, 4))
        n_max = n_min + int(rng.integers(0, 4))
        K = int(rng.integers(1, 6))
        _, k, d = run(list(base), n_min, n_max, K)
        ref, kr = _ngram_by_rfind(base, n_min, n_max, K)
        assert (d, k) == (ref, kr), (list(base), n_min, n_max, K)


def _tree_logits(B, N, V, argmax_rows, rng=None):
    """Logits whose row r has its maximum at argmax_rows[b][r] (lower,
    distinct values elsewhere)."""
    rng = rng or np.random.default_rng(0)
    t = rng.random((B, N + 1, V)).astype(np.float32)
    for b in range(B):
        for r, a in enumerate(argmax_rows[b]):
            t[b, r, a] = 2.0
    return t


def pin_tree_verify_page_trees(o):
    """The pages' trees: 3.5 Speculative Decoding, 'Tree verification'
    (flattened [a, b, a1, a2, b1, b2]) and Mathematical Foundations,
    'Tree-Based Verification' (its drawn topology): the longest
    root-to-leaf path whose tokens match the target's argmax after their
    parent is kept, then the argmax after its last node."""
    V = 16
    a, b, a1, a2, b1, b2 = 1, 2, 3, 4, 5, 6
    tok = np.array([[a, b, a1, a2, b1, b2]], np.int32)
    par = np.array([[-1, -1, 0, 0, 1, 1]], np.int32)
    # rows: 0 root, then after a, b, a1, a2, b1, b2
    cases = [
        ([a, a2, 0, 0, 11, 0, 0], [a, a2, 11], [0, 3]),   # a then a2, bonus 11
        ([b, 0, b1, 0, 0, 12, 0], [b, b1, 12], [1, 4]),   # b then b1, bonus 12
        ([b, a1, 9, 0, 0, 0, 0], [b, 9], [1]),            # b, then none of b1 / b2
        ([7, a1, b1, 0, 0, 0, 0], [7], []),                # root argmax drafted nowhere
    ]
    for rows, want, path in cases:
        r = o.tree_verify_greedy(_tree_logits(1, 6, V, [rows]), tok, par)
        n = int(r["num_accepted"][0])
        assert list(r["out_tokens"][0][:n + 1]) == want and n == len(want) - 1, (rows, r)
        assert list(r["path_nodes"][0][:n]) == path and np.all(r["out_tokens"][0][n + 1:] == -1)
    # The Mathematical Foundations tree (A_1, B_1, C_1 under the root; A_2
    # and A_3 under A_1, B_2 under B_1, C_2 under C_1), flattened breadth
    # first as [A1, B1, C1, A2, A3, B2, C2].
    A1, B1, C1, A2, A3, B2, C2 = 1, 2, 3, 4, 5, 6, 7
    tok = np.array([[A1, B1, C1, A2, A3, B2, C2]], np.int32)
    par = np.array([[-1, -1, -1, 0, 0, 1, 2]], np.int32)
    rows = [C1, 0, 0, C2, 0, 0, 0, 13]                     # root -> C1, after C1 -> C2, after C2 -> 13
    r = o.tree_verify_greedy(_tree_logits(1, 7, V, [rows]), tok, par)
    assert list(r["out_tokens"][0][:3]) == [C1, C2, 13] and list(r["path_nodes"][0][:2]) == [2, 6]


def pin_tree_chain_is_linear_greedy(o):
    """A tree that is one chain (parent[n] = n - 1) is the linear greedy
    verify of the same drafts (pinned by the worked example and by plain
    argmax decoding)."""
    rng = np.random.default_rng(8)
    B, N, V = 30, 6, 7
    t = rng.standard_normal((B, N + 1, V)).astype(np.float32)
    am = t.argmax(axis=2)
    tok = np.where(rng.random((B, N)) < 0.75, am[:, :N], rng.integers(0, V, (B, N))).astype(np.int32)
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    r = o.tree_verify_greedy(t, tok, par)
    g = o.verify_greedy(t, tok)
    assert np.array_equal(r["out_tokens"], g["out_tokens"])
    assert np.array_equal(r["num_accepted"], g["num_accepted"])


def pin_tree_best_of_paths(o):
    """Brute force on random small trees: the kept length is the longest
    accepted prefix over all root-to-leaf paths, each path checked as a
    linear greedy verify of its own rows; on equal lengths the path whose
    last node comes first in the flattened order (only repeated sibling
    tokens make several paths pass)."""
    rng = np.random.default_rng(12)
    for trial in range(200):
        N = int(rng.integers(1, 9))
        V = int(rng.integers(2, 5))          # few ids: many repeated siblings
        par = np.array([int(rng.integers(-1, n)) for n in range(N)], np.int32)
        tok = rng.integers(0, V, N).astype(np.int32)
        t = rng.standard_normal((1, N + 1, V)).astype(np.float32)
        r = o.tree_verify_greedy(t, tok[None], par[None])
        best_len, best_end = 0, -1
        leaves = [n for n in range(N) if n not in set(par.tolist())]
        for leaf in leaves:
            chain = []
            n = leaf
            while n >= 0:
                chain.append(n)
                n = int(par[n])
            chain = chain[::-1]
            rows = np.stack([t[0, 0]] + [t[0, n + 1] for n in chain])
            g = o.verify_greedy(rows[None], tok[chain][None])
            ln = int(g["num_accepted"][0])
            end = chain[ln - 1] if ln > 0 else -1
            if ln > best_len or (ln == best_len and ln > 0 and end < best_end):
                best_len, best_end = ln, end
        assert int(r["num_accepted"][0]) == best_len, (trial, par, tok)
        if best_len:
            assert int(r["path_nodes"][0][best_len - 1]) == best_end
        bonus_row = t[0, best_end + 1]
        assert int(r["out_tokens"][0][best_len]) == int(np.argmax(bonus_row))


def pin_tree_mask_page(o):
    """The mask printed under 3.5 Speculative Decoding, 'Tree verification'
    for [a, b, a1, a2, b1, b2], and its equal position indices at equal
    depth (tests/golden/tree_mask_page.json)."""
    with open(os.path.join(GOLDEN, "tree_mask_page.json")) as f:
        g = json.load(f)
    par = np.array([g["parents"]], np.int32)
    mask, depth = o.tree_mask(par)
    assert np.array_equal(mask[0], np.array(g["mask"], np.uint8)), mask[0]
    idx = {n: i for i, n in enumerate(g["nodes"])}
    for group in g["equal_positions"]:
        assert len({int(depth[0, idx[n]]) for n in group}) == 1
    assert depth[0, idx["a"]] < depth[0, idx["a1"]]


def pin_tree_mask_properties(o):
    """Closed forms and invariants: a chain gives the causal lower-triangular
    mask with positions 1..N; a star (every node under the root) gives the
    identity; on random trees the attended set of a node is a chain (any two
    attended nodes are nested), closed under 'attended by what it attends
    to', contains the node and its parent, and has as many members as the
    node's depth; padded rows and columns are empty."""
    N = 9
    chain = np.arange(-1, N - 1, dtype=np.int32)[None]
    m, d = o.tree_mask(chain)
    assert np.array_equal(m[0], np.tril(np.ones((N, N), np.uint8))) and list(d[0]) == list(range(1, N + 1))
    m, d = o.tree_mask(np.full((1, N), -1, np.int32))
    assert np.array_equal(m[0], np.eye(N, dtype=np.uint8)) and np.all(d == 1)
    rng = np.random.default_rng(21)
    B = 40
    par = np.array([[int(rng.integers(-1, n)) for n in range(N)] for _ in range(B)], np.int32)
    nn = rng.integers(0, N + 1, B).astype(np.int32)
    m, d = o.tree_mask(par, nn)
    for b in range(B):
        n = int(nn[b])
        assert not m[b, n:, :].any() and not m[b, :, n:].any() and np.all(d[b, n:] == -1)
        mb = m[b, :n, :n].astype(bool)
        for i in range(n):
            att = np.flatnonzero(mb[i])
            assert mb[i, i] and (par[b, i] < 0 or mb[i, par[b, i]])
            assert len(att) == d[b, i]
            for j in att:
                assert np.all(mb[i] >= mb[j])            # closed: what j attends to, i does
                for k in att:
                    assert mb[j, k] or mb[k, j]           # nested: one chain
            assert not mb[i, i + 1:].any()


# --------------------------------------------------------------------------
# Processed distributions (top-k, then top-p, after temperature)
# --------------------------------------------------------------------------

def _processed_brute(l, T, top_k, top_p):
    """The processed law of one row by brute force over upper sets: the
    top-k survivors are the smallest upper set {l >= v} holding at least
    top_k tokens; top-p keeps the smallest upper set of survivors holding at
    least top_p of their mass.  Returns the renormalised law."""
    l = np.asarray(l, np.float64)
    V = len(l)
    vals = sorted(set(l.tolist()), reverse=True)
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        v = max(v for v in vals if np.count_nonzero(l >= v) >= top_k)
        keep = l >= v
    if top_p < 1:
        w = np.where(keep, softmax_T(np.where(keep, l, -np.inf), T), 0.0)
        for v in vals:
            up = keep & (l >= v)
            if w[up].sum() >= top_p:
                keep = up
                break
    return np.where(keep, softmax_T(np.where(keep, l, -np.inf), T), 0.0)


def pin_processed_floor_closed_forms(o):
    """Hand-computed cases: l = (0, 1, 2, 3).  At T = 1 the law is
    e^l / sum = (0.032, 0.087, 0.237, 0.644): top-p 0.6 keeps {3}; 0.7 keeps
    {2, 3}; 0.9 keeps {1, 2, 3}; top-k 2 keeps {2, 3}; top-k 3 then top-p
    0.9 renormalises over {1, 2, 3} = (0.090, 0.245, 0.665) and keeps {2, 3}
    (0.910).  At T = 2 the law is (0.102, 0.167, 0.276, 0.455): top-p 0.4
    keeps {3}, 0.7 keeps {2, 3}.  Ties at the cut are kept: (1, 1, 1, 0)
    with top-k 1 or top-p 0.1 keeps the three 1s.  No filter: -inf."""
    l = np.array([[0, 1, 2, 3]], np.float32)
    cases = [(1.0, 0, 1.0, -np.inf), (1.0, 0, 0.6, 3), (1.0, 0, 0.7, 2), (1.0, 0, 0.9, 1),
             (1.0, 2, 1.0, 2), (1.0, 3, 0.9, 2), (1.0, 4, 1.0, -np.inf), (1.0, 0, 0.6438, 3),
             (1.0, 0, 0.6440, 2), (2.0, 0, 0.4, 3), (2.0, 0, 0.7, 2), (2.0, 1, 0.3, 3)]
    for T, k, p, want in cases:
        fl, _ = o.sampling_floor(l, T, k, p)
        assert fl[0] == want, (T, k, p, fl[0])
    ties = np.array([[1, 1, 1, 0]], np.float32)
    assert o.sampling_floor(ties, 1.0, 1, 1.0)[0][0] == 1.0
    assert o.sampling_floor(ties, 1.0, 0, 0.1)[0][0] == 1.0
    # bf16 bits of the same values give the same floors.
    bits = (l.view(np.uint32) >> 16).astype(np.uint16)
    assert o.sampling_floor(bits, 1.0, 3, 0.9)[0][0] == 2.0
    # -inf logits count in the top-k ranks but carry no mass.
    li = np.array([[0.5, -np.inf, -np.inf, 2.0]], np.float32)
    assert o.sampling_floor(li, 1.0, 3, 1.0)[0][0] == -np.inf
    assert o.sampling_floor(li, 1.0, 0, 0.99)[0][0] == 0.5


def pin_processed_boundary_is_inclusive(o):
    """The top-p cut keeps the smallest set whose mass reaches top_p: a set
    holding exactly top_p is enough.  With l = (0, -1, -2) and top_p = 1/Z,
    the top token alone holds exactly top_p * Z whenever that product rounds
    to 1 in fp64 (checked here): the floor is then 0, not -1."""
    import math
    found = 0
    for d in np.linspace(0.5, 3.0, 200):
        z = 1.0 + math.exp(-d) + math.exp(-2 * d)
        p = 1.0 / z
        if p * z != 1.0 or not (np.float32(-d) == -d and np.float32(-2 * d) == -2 * d):
            continue
        l = np.array([[0.0, -d, -2 * d]], np.float32)
        fl, mg = o.sampling_floor(l, 1.0, 0, p)
        assert fl[0] == 0.0 and mg[0] == 0.0, (d, fl, mg)
        found += 1
    assert found > 0


def pin_processed_law_exact(o):
    """With the same processing on both sides (3.5 Speculative Decoding,
    'Common pitfalls'), the emitted token is distributed exactly as the
    processed target law P': by stratified uniforms, the accept probability
    of every draft token the processed draft can propose is min(1, P'/Q'),
    the residual law is max(0, P' - Q') normalised, and the emitted law is
    P' (P' and Q' by brute force over upper sets)."""
    V, T, M = 7, 0.9, 1024
    rng = np.random.default_rng(19)
    u = grid(M)
    for top_k, top_p in [(3, 1.0), (0, 0.8), (5, 0.7), (2, 0.95), (6, 0.5)]:
        lt = (rng.standard_normal((1, 2, V)) * 1.5).astype(np.float32)
        ld = (lt[:, :1] + rng.standard_normal((1, 1, V)) * 0.8).astype(np.float32)
        P = _processed_brute(lt[0, 0], T, top_k, top_p)
        Q = _processed_brute(ld[0, 0], T, top_k, top_p)
        a = np.zeros(V)
        tgt = np.repeat(lt, M, axis=0)
        drf = np.repeat(ld, M, axis=0)
        for x in np.flatnonzero(Q > 0):
            uni = np.stack([u, np.full(M, 0.5, np.float32)], axis=1)
            r = o.verify_processed(tgt, drf, np.full((M, 1), x, np.int32), uni, T, top_k, top_p)
            a[x] = np.mean(r["num_accepted"] == 1)
        ok = Q > 0
        np.testing.assert_allclose(a[ok], np.minimum(1.0, P[ok] / Q[ok]), atol=1.0 / M)
        x = int(np.flatnonzero(ok)[np.argmin(P[ok] / Q[ok])])
        uni = np.stack([np.full(M, 1 - 2**-24, np.float32), u], axis=1)
        r = o.verify_processed(tgt, drf, np.full((M, 1), x, np.int32), uni, T, top_k, top_p)
        res = np.maximum(P - Q, 0)
        if res.sum() > 0 and a[x] < 1:
            assert np.all(r["num_accepted"] == 0)
            h = np.bincount(r["out_tokens"][:, 0], minlength=V)[:V] / M
            np.testing.assert_allclose(h, res / res.sum(), atol=2.0 / M)
            law = Q * a + np.dot(Q, 1 - a) * h
            np.testing.assert_allclose(law, P, atol=3.0 / M)
        # Bonus after an accepted draft: the processed law of the last row.
        Pk = _processed_brute(lt[0, 1], T, top_k, top_p)
        xs = int(np.argmax(np.where(ok, P / np.maximum(Q, 1e-300), -1)))
        uni = np.stack([np.zeros(M, np.float32), u], axis=1)
        r = o.verify_processed(tgt, drf, np.full((M, 1), xs, np.int32), uni, T, top_k, top_p)
        assert np.all(r["num_accepted"] == 1)
        h = np.bincount(r["out_tokens"][:, 1], minlength=V)[:V] / M
        np.testing.assert_allclose(h, Pk, atol=2.0 / M)


def pin_top_k_one_is_greedy(o):
    """top-k = 1 leaves each side a point mass at its argmax, so the
    stochastic step with any uniforms is the greedy step on the drafts'
    argmaxes ('Proof', greedy remark); a vanishing top-p does the same."""
    rng = np.random.default_rng(23)
    B, K, V = 60, 4, 50
    lt = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    ld = np.where(rng.random((B, K, 1)) < 0.6, lt[:, :K], rng.standard_normal((B, K, V))).astype(np.float32)
    toks = ld.argmax(axis=-1).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    g = o.verify_greedy(lt, toks)
    for k, p in ((1, 1.0), (0, 1e-9), (1, 0.5)):
        r = o.verify_processed(lt, ld, toks, uni, 1.3, k, p)
        assert np.array_equal(r["out_tokens"], g["out_tokens"])
        assert np.array_equal(r["num_accepted"], g["num_accepted"])


def pin_no_processing_is_plain_verify(o):
    """top-k off (0 or >= V) and top-p = 1 leave the step unchanged."""
    rng = np.random.default_rng(29)
    B, K, V, T = 40, 3, 64, 0.8
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, (B, K)).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    ref = o.verify(lt, ld, toks, uni, T)
    for k in (0, V, V + 5):
        r = o.verify_processed(lt, ld, toks, uni, T, k, 1.0)
        assert np.array_equal(r["out_tokens"], ref["out_tokens"])
        assert np.array_equal(r["num_accepted"], ref["num_accepted"])
        assert np.all(np.isneginf(r["target_floor"]))


ALL_PINS = [
    pin_stats_logsumexp, pin_stats_closed_forms,
    pin_check_your_understanding, pin_single_position_experiment,
    pin_single_position_chisquare, pin_multi_position_exact,
    pin_multi_position_chisquare, pin_k0_is_inverse_cdf, pin_identity,
    pin_disjoint_support, pin_strict_comparisons, pin_q_zero_accepts,
    pin_one_hot_drafts, pin_closed_form_printed_values,
    pin_closed_form_through_oracle, pin_ragged_equals_truncated,
    pin_invariants, pin_greedy_worked_trace, pin_greedy_ties_and_bonus,
    pin_greedy_equals_argmax_decoding, pin_markov_chain_third_token,
    pin_speedup_table_and_choice, pin_acceptance_count_identities,
    pin_alpha_test_estimates_alpha, pin_ngram_drafter, pin_tree_verify_page_trees,
    pin_tree_chain_is_linear_greedy, pin_tree_best_of_paths, pin_tree_mask_page,
    pin_tree_mask_properties, pin_processed_floor_closed_forms, pin_processed_boundary_is_inclusive,
    pin_processed_law_exact, pin_top_k_one_is_greedy, pin_no_processing_is_plain_verify,
]
