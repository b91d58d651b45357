"""Pins for the oracle's tree set-up (mask, depth, ancestor words, validity).

The oracle walks parent links; the checks here use the worked tree printed on
the infra-guide page "5.3 Medusa、EAGLE 与 MTP" (section 8), a transitive
closure computed by Warshall's algorithm, and shape invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_trees(n):
    """Every parents-first tree on n nodes: parents[i] ranges over [0, i)."""
    if n == 0:
        yield []
        return
    for rest in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(rest)


def warshall_closure(parents):
    """Reflexive-transitive closure of the child->parent relation."""
    n = len(parents)
    R = np.eye(n, dtype=bool)
    for i, p in enumerate(parents):
        if p >= 0:
            R[i, p] = True
    for k in range(n):
        R = R | (R[:, [k]] & R[[k], :])
    return R.astype(np.uint8)


def test_worked_tree_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "worked_tree.json")))
    par = g["parents"]
    mask = oracle.tree_mask(par)
    depth = oracle.tree_depth(par)
    # the page's own assertions
    assert list(mask[4]) == g["page_checks"]["mask_row_4"]
    assert depth[1] == g["page_checks"]["depth_1"] and depth[2] == g["page_checks"]["depth_2"]
    # the page's statement about what a lower-triangular mask leaks to node 4
    causal = np.tril(np.ones((5, 5), dtype=np.uint8))
    leaks = [[j for j in range(5) if causal[i, j] and not mask[i, j]] for i in range(5)]
    assert leaks[4] == g["page_checks"]["node_4_causal_leaks"]
    # the hand-derived rest of the figure
    assert mask.tolist() == g["mask"]
    assert depth == g["depth"]
    assert leaks == g["causal_leaks"]
    words = oracle.ancestor_words(par, 5)[:, 0].tolist()
    assert words == g["ancestor_words_lsb_first"]


@pytest.mark.parametrize("n", range(1, 8))
def test_all_small_trees_against_warshall(n):
    count = 0
    for par in all_trees(n):
        count += 1
        R = warshall_closure(par)
        assert (oracle.tree_mask(par) == R).all(), par
        # depth = number of proper ancestors = row popcount - 1
        assert oracle.tree_depth(par) == [int(r.sum()) - 1 for r in R], par
        words = oracle.ancestor_words(par, n)[:, 0]
        for i in range(n):
            assert int(words[i]) == sum(1 << j for j in range(n) if R[i, j])
    assert count == max(1, __import__("math").factorial(n - 1))


def test_chain_and_star_shapes():
    n = 9
    chain = [-1] + list(range(n - 1))
    assert (oracle.tree_mask(chain) == np.tril(np.ones((n, n), dtype=np.uint8))).all()
    assert oracle.tree_depth(chain) == list(range(n))
    star = [-1] + [0] * (n - 1)
    assert oracle.tree_depth(star) == [0] + [1] * (n - 1)
    m = oracle.tree_mask(star)
    assert (m[1:, 1:] == np.eye(n - 1, dtype=np.uint8)).all() and (m[:, 0] == 1).all()


@pytest.mark.parametrize("par", [
    [0, 0, 1],          # root not -1
    [-1, 1, 0],         # node 1 is its own parent
    [-1, 0, 3, 0],      # parent after child
    [-1, 0, -1],        # second root
    [-1, -2, 0],        # parent below -1
])
def test_invalid_trees_rejected(par):
    assert not oracle.tree_is_valid(par)
    P = np.array([par], dtype=np.int32)
    anc, depth, err = oracle.build_tree(P, np.array([len(par)], dtype=np.int32))
    assert err[0] == oracle.ERR_BAD_TREE
    assert (anc == 0).all() and (depth == 0).all()


def test_build_tree_batch_padding_and_empty():
    P = np.full((3, 6), -1, dtype=np.int32)
    P[0, :5] = [-1, 0, 0, 1, 2]
    P[1, :1] = [-1]
    P[2, :6] = [-1, 0, 1, 2, 3, 4]
    nn = np.array([5, 0, 6], dtype=np.int32)
    anc, depth, err = oracle.build_tree(P, nn)
    assert err.tolist() == [0, 0, 0]
    assert anc[0].tolist() == [1, 3, 5, 11, 21, 0]
    assert (anc[1] == 0).all() and (depth[1] == 0).all()
    assert depth[2].tolist() == [0, 1, 2, 3, 4, 5]
    assert anc[2].tolist() == [(1 << (i + 1)) - 1 for i in range(6)]
