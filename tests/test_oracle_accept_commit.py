"""Pins for the oracle's greedy acceptance and KV commit.

Acceptance is checked against (a) the tiny workload's forced outcome,
(b) brute force over every tree with up to 7 nodes and every match pattern,
by enumerating root paths (a different algorithm from the oracle's parent
recursion), and (c) the expected tokens per step printed on the pages
(pofe.ai "Medusa and EAGLE ...", section "Medusa: heads, losses and trees",
worked example; vibeengines.com "Medusa, explained"), by Monte Carlo.
Commit is checked against hand-derived slot moves and against an ascending
sequential copy, which is a valid in-place order because path[d] >= d.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_tree import all_trees
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_workload_forced_path():
    w = generate(1)
    acc, path, bonus, toks = oracle.accept(w.tok, w.tgt, w.parents, w.n_nodes)
    assert acc.tolist() == [2]
    assert path[0].tolist() == [0, 1, 3, -1, -1]
    assert bonus[0] == w.tgt[0, 3]
    assert toks[0].tolist() == [w.tok[0, 1], w.tok[0, 3], w.tgt[0, 3], -1, -1]


def brute_force_accept(parents, tok, tgt):
    """Longest root path whose every drafted token equals the target's choice
    at its parent; ties go to the lowest endpoint index."""
    n = len(parents)
    best = None
    for e in range(n):
        path = [e]
        while parents[path[-1]] != -1:
            path.append(parents[path[-1]])
        path.reverse()
        if all(tok[path[k]] == tgt[path[k - 1]] for k in range(1, len(path))):
            if best is None or len(path) > len(best):
                best = path
    return best


@pytest.mark.parametrize("n", range(1, 8))
def test_accept_brute_force_all_trees_all_patterns(n):
    for parents in all_trees(n):
        for bits in range(1 << max(0, n - 1)):
            tgt = np.array([1000 + i for i in range(n)], dtype=np.int32)
            tok = np.zeros(n, dtype=np.int32)
            tok[0] = 7
            for i in range(1, n):
                hit = (bits >> (i - 1)) & 1
                tok[i] = tgt[parents[i]] if hit else 5000 + i
            acc, path, bonus, toks = oracle.accept(
                tok[None], tgt[None], np.array([parents], dtype=np.int32), np.array([n], dtype=np.int32))
            ref = brute_force_accept(parents, tok, tgt)
            assert acc[0] == len(ref) - 1
            assert path[0, :len(ref)].tolist() == ref and (path[0, len(ref):] == -1).all()
            assert bonus[0] == tgt[ref[-1]]
            assert toks[0, :len(ref)].tolist() == [int(tok[a]) for a in ref[1:]] + [int(tgt[ref[-1]])]


def build_regular_tree(shape):
    """Root, then shape[0] children, each with shape[1] children, and so on."""
    parents, level = [-1], [0]
    for s in shape:
        nxt = []
        for p in level:
            for _ in range(s):
                nxt.append(len(parents))
                parents.append(p)
        level = nxt
    return parents


def test_expected_tokens_per_step_match_pages():
    cases = json.load(open(os.path.join(GOLDEN, "acceptance_closed_forms.json")))["cases"]
    rng = np.random.default_rng(2024)
    trials = 40000
    for case in cases:
        parents = build_regular_tree(case["shape"])
        n = len(parents)
        assert n - 1 == case["candidates"]
        depth = oracle.tree_depth(parents)
        children = [[c for c in range(n) if parents[c] == p] for p in range(n)]
        P = np.tile(np.array(parents, dtype=np.int32), (trials, 1))
        tok = np.tile(np.arange(n, dtype=np.int32) + 100, (trials, 1))
        tgt = np.full((trials, n), 9, dtype=np.int32)   # 9 is no candidate
        for p in range(n):
            kids = children[p]
            if not kids:
                continue
            rate = case["hit_rates"][depth[p]]
            hit = rng.random(trials) < rate
            which = rng.integers(0, len(kids), size=trials)
            tgt[:, p] = np.where(hit, np.array(kids)[which] + 100, 9)
        acc = oracle.accept(tok, tgt, P, np.full(trials, n, dtype=np.int32))[0]
        tokens = acc + 1
        mean, se = tokens.mean(), tokens.std() / np.sqrt(trials)
        assert abs(mean - case["tokens_per_step_exact"]) < 4 * se, (case, mean, se)
        assert abs(case["tokens_per_step_exact"] - case["tokens_per_step_printed"]) < 0.05


def test_single_node_is_plain_decode_and_errors_skip():
    P = np.array([[-1, -1], [-1, 0], [-1, 0]], dtype=np.int32)
    nn = np.array([1, 0, 2], dtype=np.int32)
    tok = np.array([[5, 0], [5, 6], [5, 6]], dtype=np.int32)
    tgt = np.array([[42, 0], [6, 0], [6, 0]], dtype=np.int32)
    err = np.array([0, 0, 2], dtype=np.int32)
    acc, path, bonus, toks = oracle.accept(tok, tgt, P, nn, err_in=err)
    assert acc.tolist() == [0, -1, -1]
    assert path.tolist() == [[0, -1], [-1, -1], [-1, -1]]
    assert bonus.tolist() == [42, -1, -1]
    assert toks.tolist() == [[42, -1], [-1, -1], [-1, -1]]


# ------------------------------------------------------------------ commit

def test_commit_tiny_workload_slots():
    w = generate(1)
    kc, vc = w.f64("k_cache"), w.f64("v_cache")
    acc, path, bonus, toks = oracle.accept(w.tok, w.tgt, w.parents, w.n_nodes)
    k2, v2, plen = oracle.commit(kc, vc, w.prefix_len, acc, path)
    assert plen.tolist() == [67]
    for d, node in enumerate([0, 1, 3]):
        assert np.array_equal(k2[0, :, 64 + d], kc[0, :, 64 + node])
        assert np.array_equal(v2[0, :, 64 + d], vc[0, :, 64 + node])
    assert np.array_equal(k2[0, :, :64], kc[0, :, :64])
    assert np.array_equal(k2[0, :, 67:], kc[0, :, 67:])


def sequential_commit(k, v, P, path, L):
    k, v = np.array(k, copy=True), np.array(v, copy=True)
    for d in range(L + 1):
        k[:, P + d] = k[:, P + path[d]]
        v[:, P + d] = v[:, P + path[d]]
    return k, v


@pytest.mark.parametrize("path", [[0], [0, 1, 2, 3], [0, 2, 3], [0, 2, 5, 6], [0, 3, 4, 7]])
def test_commit_equals_ascending_copy(path):
    rng = np.random.default_rng(len(path))
    Hkv, cap, D, P = 2, 20, 4, 6
    k = rng.standard_normal((1, Hkv, cap, D))
    v = rng.standard_normal((1, Hkv, cap, D))
    L = len(path) - 1
    pp = np.full((1, 8), -1, dtype=np.int32)
    pp[0, :L + 1] = path
    k2, v2, plen = oracle.commit(k, v, np.array([P]), np.array([L]), pp)
    ks, vs = sequential_commit(k[0], v[0], P, path, L)
    assert np.array_equal(k2[0], ks) and np.array_equal(v2[0], vs)
    assert plen[0] == P + L + 1
    if path == list(range(L + 1)):
        assert np.array_equal(k2, k)   # chain fully accepted: nothing moves


def test_commit_skips_negative_accept_len():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 1, 10, 4))
    v = rng.standard_normal((2, 1, 10, 4))
    pp = np.array([[0, 2, -1], [-1, -1, -1]], dtype=np.int32)
    k2, v2, plen = oracle.commit(k, v, np.array([3, 4]), np.array([1, -1]), pp)
    assert plen.tolist() == [5, 4]
    assert np.array_equal(k2[1], k[1]) and np.array_equal(v2[1], v[1])
    assert np.array_equal(k2[0, :, 4], k[0, :, 5])
