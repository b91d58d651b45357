"""Pins for the oracle's typical acceptance.

The rule (vibeengines.com "Medusa, explained", section "Typical acceptance";
pofe.ai "Medusa and EAGLE ...", "Typical acceptance"; infra-guide "5.3
Medusa、EAGLE 与 MTP", section 9.1): a drafted token passes iff the target's
probability of it exceeds min(eps, delta * exp(-H)). Checked against:
  * SciPy's softmax and entropy (library routines) for p and H;
  * closed forms: a flat row has H = ln V and p = 1 / V; a two-level row has
    a closed-form p and H;
  * the greedy rule, which typical acceptance must reproduce exactly when the
    floor is 1/2 and every target distribution has a token above 1/2 (then
    "p > 1/2" holds for the argmax and for nothing else);
  * the pages' extremes: with eps = delta = 0 every candidate passes; with
    high thresholds only near-argmax tokens pass;
  * brute force over every tree with up to 6 nodes, enumerating root paths
    and judging each edge with SciPy's p and H;
  * the pages' qualitative claim that the floor drops as entropy rises;
  * monotonicity: raising eps or delta never lengthens the accepted path.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from tests.test_oracle_tree import all_trees
from workloads import bf16_bits_to_f32, generate, target_logits


def one_seq(parents, tok, logits):
    n = len(parents)
    return (np.asarray(logits, dtype=np.float64)[None], np.asarray(tok, dtype=np.int32)[None],
            np.asarray(parents, dtype=np.int32)[None], np.array([n], dtype=np.int32))


def test_distribution_matches_scipy():
    rng = np.random.default_rng(11)
    for V, scale in ((7, 1.0), (1000, 3.0), (32000, 2.0)):
        x = rng.standard_normal(V) * scale
        p, H, am = oracle.next_token_distribution(x)
        ref = scipy.special.softmax(x)
        assert np.allclose(p, ref, rtol=1e-12, atol=0)
        assert abs(H - scipy.stats.entropy(ref)) < 1e-10
        assert am == int(np.argmax(ref))


def test_flat_row_closed_form():
    for V in (1, 2, 5, 32000):
        p, H, am = oracle.next_token_distribution(np.full(V, 3.25))
        assert np.allclose(p, 1.0 / V, rtol=1e-14)
        assert abs(H - math.log(V)) < 1e-12
        assert am == 0     # all equal: lowest index


def test_two_level_row_closed_form():
    # k tokens at logit a, V - k at 0: p_hi = e^a / (k e^a + V - k)
    V, k, a = 1000, 3, 5.0
    x = np.zeros(V)
    hi = [10, 400, 999]
    x[hi] = a
    p, H, am = oracle.next_token_distribution(x)
    Z = k * math.exp(a) + (V - k)
    p_hi, p_lo = math.exp(a) / Z, 1.0 / Z
    assert np.allclose(p[hi], p_hi, rtol=1e-13)
    assert abs(p[0] - p_lo) < 1e-16
    assert abs(H - (-k * p_hi * math.log(p_hi) - (V - k) * p_lo * math.log(p_lo))) < 1e-12
    assert am == 10


def test_argmax_ties_go_to_lowest_index():
    x = np.array([0.0, 2.0, -1.0, 2.0, 2.0])
    assert oracle.next_token_distribution(x)[2] == 1


def test_reduces_to_greedy_when_every_distribution_is_peaked():
    # floor = min(0.5, 1e6 exp(-H)) = 0.5 for any H below ln(2e6); a token
    # passes iff p > 0.5, which only the argmax can have.
    w = generate(3)
    rng = np.random.default_rng(5)
    V = 2000
    logits = rng.standard_normal((w.B, w.n_max, V))
    peak = rng.integers(0, V, size=(w.B, w.n_max))
    for b in range(w.B):
        for i in range(w.n_max):
            logits[b, i, peak[b, i]] = 12.0        # p(peak) > 0.99
    # candidates: either the parent's peak token or some other token
    tok = rng.integers(0, V, size=(w.B, w.n_max)).astype(np.int32)
    for b in range(w.B):
        for c in range(1, int(w.n_nodes[b])):
            if rng.random() < 0.7:
                tok[b, c] = peak[b, w.parents[b, c]]
    H, pt, am, acc, path, bonus, toks = oracle.typical_accept(logits, tok, w.parents, w.n_nodes, 0.5, 1e6)
    assert (am[:, 0] == peak[:, 0]).all()
    g_acc, g_path, g_bonus, g_toks = oracle.accept(tok, am, w.parents, w.n_nodes)
    assert (acc == g_acc).all() and (path == g_path).all()
    assert (bonus == g_bonus).all() and (toks == g_toks).all()
    assert len(set(acc.tolist())) > 1


def test_zero_thresholds_accept_every_candidate():
    # the pages: with eps and delta near zero almost any candidate passes
    w = generate(3)
    x = bf16_bits_to_f32(target_logits(w)).astype(np.float64)
    H, pt, am, acc, path, bonus, toks = oracle.typical_accept(x, w.tok, w.parents, w.n_nodes, 0.0, 0.0)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        dep = oracle.tree_depth([int(v) for v in w.parents[b, :n]])
        deepest = max(dep)
        assert acc[b] == deepest
        e = dep.index(deepest)                 # lowest index at that depth
        assert path[b, :deepest + 1].tolist() == oracle.ancestors_or_self(
            [int(v) for v in w.parents[b, :n]], e)
        assert bonus[b] == am[b, e]


def test_high_thresholds_stop_at_the_root():
    # a floor of 1 can never be exceeded: only the root (the target's own
    # token) is kept and the step is one plain decode step
    w = generate(3)
    x = bf16_bits_to_f32(target_logits(w)).astype(np.float64)
    H, pt, am, acc, path, bonus, toks = oracle.typical_accept(x, w.tok, w.parents, w.n_nodes, 1.0, 1e9)
    assert (acc == 0).all()
    assert (path[:, 0] == 0).all() and (path[:, 1:] == -1).all()
    assert (bonus == am[:, 0]).all()


def scipy_edge_passes(logits_parent, token, eps, delta):
    p = scipy.special.softmax(logits_parent)
    H = scipy.stats.entropy(p)
    prob = p[token] if 0 <= token < len(p) else 0.0
    return prob > min(eps, delta * math.exp(-H))


@pytest.mark.parametrize("n", range(1, 7))
def test_brute_force_small_trees(n):
    rng = np.random.default_rng(100 + n)
    V = 12
    for parents in all_trees(n):
        logits = rng.standard_normal((n, V)) * rng.uniform(0.3, 3.0)
        tok = rng.integers(0, V, size=n).astype(np.int32)
        eps, delta = rng.uniform(0.02, 0.4), rng.uniform(0.1, 2.0)
        lg, tk, par, nn = one_seq(parents, tok, logits)
        H, pt, am, acc, path, bonus, toks = oracle.typical_accept(lg, tk, par, nn, eps, delta)
        # enumerate every root path; keep the deepest whose every edge passes
        best = None
        for e in range(n):
            p = [e]
            while parents[p[-1]] != -1:
                p.append(parents[p[-1]])
            p.reverse()
            if all(scipy_edge_passes(logits[p[k - 1]], tok[p[k]], eps, delta) for k in range(1, len(p))):
                if best is None or len(p) > len(best):
                    best = p
        assert acc[0] == len(best) - 1
        assert path[0, :len(best)].tolist() == best
        assert bonus[0] == int(np.argmax(logits[best[-1]]))
        assert toks[0, :len(best)].tolist() == [int(tok[a]) for a in best[1:]] + [bonus[0]]


def test_floor_drops_as_entropy_rises():
    # the same candidate probability 0.05 fails under a confident target and
    # passes under an uncertain one (eps = 0.09, delta = 0.3)
    V = 32000
    confident = np.full(V, -30.0)
    confident[0], confident[1] = math.log(0.95), math.log(0.05)
    uncertain = np.zeros(V)
    uncertain[1] = math.log(0.05 * (V - 1) / 0.95)     # p(token 1) = 0.05
    for row, expect in ((confident, 0), (uncertain, 1)):
        logits = np.stack([row, np.zeros(V)])
        lg, tk, par, nn = one_seq([-1, 0], [0, 1], logits)
        H, pt, am, acc, path, bonus, toks = oracle.typical_accept(lg, tk, par, nn, 0.09, 0.3)
        assert abs(pt[0, 1] - 0.05) < 1e-6
        assert acc[0] == expect


def test_monotone_in_thresholds():
    w = generate(3, seed=9)
    x = bf16_bits_to_f32(target_logits(w)).astype(np.float64)
    prev = None
    for eps, delta in ((0.0, 0.0), (0.01, 0.1), (0.05, 0.3), (0.09, 0.3), (0.2, 1.0), (0.5, 5.0), (1.0, 10.0)):
        acc = oracle.typical_accept(x, w.tok, w.parents, w.n_nodes, eps, delta)[3]
        if prev is not None:
            assert (acc <= prev).all()
        prev = acc


def test_padding_skipped_and_out_of_range_tokens():
    V = 10
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((3, 4, V))
    parents = np.array([[-1, 0, 1, -1], [-1, 0, 0, 1], [-1, 0, -1, -1]], dtype=np.int32)
    n_nodes = np.array([3, 4, 0], dtype=np.int32)
    tok = np.array([[1, -2, 3, 0], [4, V, int(np.argmax(logits[1, 0])), 7], [0, 0, 0, 0]], dtype=np.int32)
    err = np.array([0, 0, 0], dtype=np.int32)
    H, pt, am, acc, path, bonus, toks = oracle.typical_accept(logits, tok, parents, n_nodes, 0.0, 0.0, err)
    assert pt[0, 1] == 0.0 and pt[1, 1] == 0.0          # ids outside [0, V)
    assert acc.tolist() == [0, 1, -1]                   # p = 0 never passes, even at floor 0
    assert path[1, :2].tolist() == [0, 2]
    assert (am[0, 3:] == -1).all() and (H[0, 3:] == 0).all() and (pt[0, 3:] == 0).all()
    assert (am[2] == -1).all() and (path[2] == -1).all() and bonus[2] == -1
    err = np.array([0, 2, 0], dtype=np.int32)
    acc2 = oracle.typical_accept(logits, tok, parents, n_nodes, 0.0, 0.0, err)[3]
    assert acc2.tolist() == [0, -1, -1]
