"""Pins for the oracle's chain speculative sampling (robertz.co "Drafters
...", section "Why the answer does not change": keep with probability
min(1, p/q), else draw from the target with the draft subtracted; the output
is then distributed exactly as sampling from the target alone).

Checked against: that distribution claim itself, by exact enumeration of the
first emitted token's law over a grid of draws (a wrong residual or keep rule
breaks it) and by Monte Carlo over whole chains; closed cases (draft equal to
target keeps everything; a draft token the target rules out is always
rejected; u = 0 keeps every token the target allows); inverse-CDF draws
against numpy's own cumulative sums on hand cases.
"""
import numpy as np
import pytest

import oracle


def test_inverse_cdf_hand_cases():
    w = np.array([0.0, 1.0, 3.0, 0.0, 4.0])
    assert oracle.inverse_cdf(w, 0.0) == 1
    assert oracle.inverse_cdf(w, 0.124) == 1
    assert oracle.inverse_cdf(w, 0.126) == 2
    assert oracle.inverse_cdf(w, 0.5) == 4
    assert oracle.inverse_cdf(w, 0.999999) == 4


@pytest.mark.parametrize("seed", range(4))
def test_first_token_law_equals_the_target(seed):
    # P(first emitted token = y) summed over the keep/reject branches equals
    # p_0(y): enumerate u on a fine grid for both draws
    rng = np.random.default_rng(seed)
    V = 6
    pl = rng.standard_normal((2, V)) * 1.5
    ql = rng.standard_normal((1, V)) * 1.5
    p0, q0 = oracle.softmax64(pl[0]), oracle.softmax64(ql[0])
    law = np.zeros(V)
    grid = (np.arange(400) + 0.5) / 400
    for x in range(V):                       # the draft token, drawn from q
        for ua in grid:
            for ur in grid[::8]:
                acc, toks, _, _ = oracle.speculative_sample(pl, ql, np.array([x]), np.array([ua]), ur)
                law[toks[0]] += q0[x] / (len(grid) * len(grid[::8]))
    assert np.abs(law - p0).max() < 0.01


def test_monte_carlo_chain_matches_target_sampling():
    rng = np.random.default_rng(7)
    V, L, trials = 5, 3, 20000
    pl = rng.standard_normal((L + 1, V))
    ql = rng.standard_normal((L, V))
    p = [oracle.softmax64(r) for r in pl]
    q = [oracle.softmax64(r) for r in ql]
    counts = np.zeros(V)
    for _ in range(trials):
        draft = np.array([rng.choice(V, p=q[i]) for i in range(L)])
        acc, toks, _, _ = oracle.speculative_sample(pl, ql, draft, rng.random(L), rng.random())
        counts[toks[0]] += 1
    sd = np.sqrt(trials * p[0] * (1 - p[0]))
    assert (np.abs(counts - trials * p[0]) < 4 * sd).all()


def test_equal_draft_keeps_everything_and_samples_the_bonus():
    rng = np.random.default_rng(1)
    V, L = 7, 4
    pl = rng.standard_normal((L + 1, V))
    draft = rng.integers(0, V, L)
    acc, toks, pt, qt = oracle.speculative_sample(pl, pl[:L], draft, rng.random(L), 0.3)
    assert acc == L
    assert toks[:L].tolist() == draft.tolist()
    c = np.cumsum(oracle.softmax64(pl[L]))
    assert toks[L] == int(np.argmax(c > 0.3 * c[-1]))
    assert np.allclose(pt, qt)


def test_token_the_target_rules_out_is_rejected():
    V = 4
    pl = np.array([[0.0, -200.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    ql = np.array([[0.0, 5.0, 0.0, 0.0]])
    for ua in (1e-6, 0.5, 0.999):
        acc, toks, _, _ = oracle.speculative_sample(pl, ql, np.array([1]), np.array([ua]), 0.5)
        assert acc == 0
    # the residual max(0, p - q) puts no mass on token 1
    assert toks[0] != 1 and toks[1] == -1


def test_u_zero_keeps_what_the_target_allows():
    rng = np.random.default_rng(3)
    V, L = 9, 5
    pl = rng.standard_normal((L + 1, V))
    ql = rng.standard_normal((L, V)) * 3
    draft = rng.integers(0, V, L)
    acc, toks, _, _ = oracle.speculative_sample(pl, ql, draft, np.zeros(L), 0.5)
    assert acc == L


def test_softmax64_equals_scipy_softmax():
    """oracle.softmax64 against scipy.special.softmax (a library routine):
    flat, peaked, very large and very negative logits, a single entry, and
    ties; also sums to one and is invariant to a shift."""
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    rows = [rng.normal(size=32000), 30.0 * rng.normal(size=1001), rng.normal(size=7) + 1e4,
            rng.normal(size=9) - 1e4, np.array([3.5]), np.zeros(5), np.array([2.0, 2.0, -1.0, 2.0])]
    for x in rows:
        got = oracle.softmax64(x)
        ref = softmax(np.asarray(x, dtype=np.float64))
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)
        assert abs(got.sum() - 1.0) < 1e-12
        assert np.allclose(oracle.softmax64(x + 123.25), got, rtol=1e-12, atol=1e-300)
    # a plausible mistake (no max shift, or a missing normalisation) fails
    x = rows[2]
    assert not np.all(np.isfinite(np.exp(x)))
