"""Pins for the oracle's EAGLE-2 draft tree (infra-guide "5.3 Medusa、EAGLE
与 MTP", section 5.2: a node's value is the product of the draft's
confidences on its path; expansion grows the best nodes, the rerank keeps the
best of all).

Checked against: the workload generator's own EAGLE-2 procedure
(workloads.configs.eagle_dynamic_tree, written for the inputs and fed the
same confidences through its random draws); hand-built closed cases (a chain;
equal confidences, where values fall with depth only and ties go to the
earlier node); the global top-(n-1) property over every created node,
recomputed by an enumeration of the expansion; ancestor closure and
parents-first order; clamping of confidences outside [0, 1].
"""
import numpy as np
import pytest

import oracle
from workloads import draft_proposals
from workloads.configs import eagle_dynamic_tree


class ScriptedDraws:
    """Stands in for the generator's random stream: hands out, in order, the
    stick-breaking fractions that reproduce a given confidence table."""

    def __init__(self, conf):
        self.fracs = []
        S, K, M = conf.shape
        layer = 1                      # the root
        for s in range(S):
            grown = min(K, layer)      # rows of step s the expansion uses
            layer = grown * M
            for k in range(grown):
                left = 1.0
                for c in range(M):
                    x = float(conf[s, k, c])
                    self.fracs.append(x / left if left > 0 else 0.0)
                    left -= x
        self.pos = 0

    def next_frac(self, _rng):
        f = self.fracs[self.pos]
        self.pos += 1
        return f


def generator_tree(conf, n):
    """The workload generator's EAGLE-2 tree for the same confidences."""
    S, K, M = conf.shape
    draws = ScriptedDraws(conf)
    t = eagle_dynamic_tree(None, n, S, K, n_children=lambda r: M, first_frac=draws.next_frac,
                           other_frac=draws.next_frac)
    return t.parents


@pytest.mark.parametrize("seed", range(6))
def test_matches_the_workload_generator(seed):
    conf, cand, root = draft_proposals(1, 6, 8, 8, seed=seed)
    # the generator consumes a layer's fractions in value order, which is
    # the order of this table's rows (k = rank)
    par, tok, val, n = oracle.eagle2_tree(conf[0], cand[0], root[0], 60)
    want = generator_tree(conf[0].astype(np.float64), 60)
    assert n == 60
    assert par[:n].tolist() == want


def enumerate_expansion(conf):
    """Every created node as (value, parent, depth), by expanding each layer's
    best K (argsort with ties to the earlier node)."""
    S, K, M = conf.shape
    nodes = [(np.float32(1.0), -1, 0)]
    layer = [0]
    for s in range(S):
        vals = np.array([nodes[i][0] for i in layer], dtype=np.float32)
        best = [layer[j] for j in np.lexsort((np.arange(len(layer)), -vals))[:K]]
        new = []
        for k, p in enumerate(best):
            for c in range(M):
                nodes.append((np.float32(nodes[p][0] * np.float32(min(max(conf[s, k, c], 0.0), 1.0))), p,
                              nodes[p][2] + 1))
                new.append(len(nodes) - 1)
        layer = new
    return nodes


@pytest.mark.parametrize("S,K,M,n", [(6, 8, 8, 60), (7, 4, 3, 32), (3, 2, 5, 64), (5, 3, 2, 10)])
def test_keeps_the_best_nodes_closed_and_parents_first(S, K, M, n):
    conf, cand, root = draft_proposals(1, S, K, M, seed=S * 100 + n)
    par, tok, val, kept = oracle.eagle2_tree(conf[0], cand[0], root[0], n)
    nodes = enumerate_expansion(conf[0])
    assert kept == min(n, len(nodes))
    # parents first, depth non-decreasing, values match the path products
    depth = [0] * kept
    for i in range(1, kept):
        assert 0 <= par[i] < i
        depth[i] = depth[par[i]] + 1
        assert val[i] <= val[par[i]]
    assert depth == sorted(depth)
    # the kept values are the n - 1 best of every created node
    all_vals = sorted((float(v) for v, _, _ in nodes[1:]), reverse=True)
    assert sorted((float(v) for v in val[1:kept]), reverse=True) == all_vals[:kept - 1]
    assert (par[kept:] == -1).all() and (tok[kept:] == -1).all()


def test_chain_closed_form():
    conf = np.full((5, 1, 1), 0.5, dtype=np.float32)
    cand = np.arange(5, dtype=np.int32).reshape(5, 1, 1) + 100
    par, tok, val, n = oracle.eagle2_tree(conf, cand, 7, 10)
    assert n == 6
    assert par[:6].tolist() == [-1, 0, 1, 2, 3, 4]
    assert tok[:6].tolist() == [7, 100, 101, 102, 103, 104]
    assert val[:6].tolist() == [1.0, 0.5, 0.25, 0.125, 0.0625, 0.03125]


def test_equal_confidences_closed_form():
    # values fall with depth only; ties go to the earlier node, so step 2
    # grows nodes 3 and 4, and the rerank keeps the first n - 1 created
    conf = np.full((3, 2, 2), 0.5, dtype=np.float32)
    cand = np.arange(12, dtype=np.int32).reshape(3, 2, 2)
    par, tok, val, n = oracle.eagle2_tree(conf, cand, 99, 8)
    assert n == 8
    assert par[:8].tolist() == [-1, 0, 0, 1, 1, 2, 2, 3]
    assert tok[:8].tolist() == [99, 0, 1, 4, 5, 6, 7, 8]
    par, tok, val, n = oracle.eagle2_tree(conf, cand, 99, 64)
    assert n == 11      # 1 + 2 + 4 + 4 created
    assert par[:11].tolist() == [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4]


def test_confidences_are_clamped():
    conf = np.array([[[1.5, np.nan, -0.2]]], dtype=np.float32)
    cand = np.array([[[1, 2, 3]]], dtype=np.int32)
    par, tok, val, n = oracle.eagle2_tree(conf, cand, 0, 4)
    assert val[:4].tolist() == [1.0, 1.0, 0.0, 0.0]
    assert par[:4].tolist() == [-1, 0, 0, 0]
