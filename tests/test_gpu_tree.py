"""tv_build_tree on the GPU against the oracle, bit for bit: every
parents-first tree with up to seven nodes (the infra-guide "5.3" section 8
construction: a parent precedes its child), padded into a short and a
64-node row, and each way a parents array can fail to be such a tree."""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.test_oracle_tree import all_trees

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_build(parents: np.ndarray, n_nodes: np.ndarray):
    anc, depth, err = tv.build_tree(torch.from_numpy(parents).to(DEV), torch.from_numpy(n_nodes).to(DEV))
    torch.cuda.synchronize()
    return anc.cpu().numpy().view(np.uint64), depth.cpu().numpy(), err.cpu().numpy()


@pytest.mark.parametrize("n_max", [7, 64])
def test_every_tree_up_to_seven_nodes(n_max):
    print(f"[gpu] build_tree over all trees with n <= 7, n_max={n_max}", flush=True)
    trees = [t for n in range(0, 8) for t in all_trees(n)]
    assert len(trees) == 1 + 1 + 1 + 2 + 6 + 24 + 120 + 720
    B = len(trees)
    parents = np.full((B, n_max), -1, dtype=np.int32)
    n_nodes = np.zeros(B, dtype=np.int32)
    for b, t in enumerate(trees):
        parents[b, :len(t)] = t
        n_nodes[b] = len(t)
    # padding entries hold arbitrary values (they must be ignored)
    rng = np.random.default_rng(n_max)
    for b, t in enumerate(trees):
        parents[b, len(t):] = rng.integers(-3, n_max + 3, size=n_max - len(t))
    got = _gpu_build(parents, n_nodes)
    ref = oracle.build_tree(parents, n_nodes)
    for name, g, r in zip(("anc", "depth", "err"), got, ref):
        assert np.array_equal(g, r), name
    assert (got[2] == 0).all()


def test_every_invalid_form():
    """root not -1; a second root; a parent below -1; a node its own parent;
    a parent after its child; a parent beyond the row; n_nodes < 0 and
    n_nodes > n_max; next to valid trees in the same batch."""
    print("[gpu] build_tree invalid forms", flush=True)
    n_max = 8
    good = [-1, 0, 0, 1, 1, 2, 5, 3]
    cases = []
    def case(mod, n=n_max):
        p = list(good)
        mod(p)
        cases.append((p, n))
    case(lambda p: None)                              # valid
    case(lambda p: p.__setitem__(0, 0))              # root with a parent
    case(lambda p: p.__setitem__(0, 3))              # root pointing forward
    case(lambda p: p.__setitem__(3, -1))             # a second root
    case(lambda p: p.__setitem__(2, -5))             # parent below -1
    case(lambda p: p.__setitem__(4, 4))              # its own parent
    case(lambda p: p.__setitem__(4, 6))              # parent after the child
    case(lambda p: p.__setitem__(7, 40))             # parent beyond the row
    case(lambda p: None, n=-1)                       # negative node count
    case(lambda p: None, n=n_max + 1)                # more nodes than the row
    case(lambda p: p.__setitem__(7, 9), n=7)         # bad entry only in the padding: valid
    case(lambda p: None, n=0)                        # inactive slot: valid, empty
    parents = np.array([c[0] for c in cases], dtype=np.int32)
    n_nodes = np.array([c[1] for c in cases], dtype=np.int32)
    got = _gpu_build(parents, n_nodes)
    ref = oracle.build_tree(parents, n_nodes)
    for name, g, r in zip(("anc", "depth", "err"), got, ref):
        assert np.array_equal(g, r), name
    assert got[2].tolist() == [0, 2, 2, 2, 2, 2, 2, 2, 2, 2, 0, 0]
