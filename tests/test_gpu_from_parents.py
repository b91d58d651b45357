"""tv_tree_attention_from_parents: the attention kernel builds the tree
itself. Everything it writes (out, anc, depth, err and the cache after the
tree append) must equal, bit for bit, tv_build_tree followed by
tv_tree_attention on the same inputs; the separate calls are themselves
checked against the oracle in test_gpu_parity.py and test_gpu_tree.py, and
the small cases here are checked against the oracle directly as well."""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.gpu_util import attention_error, tolerance, upload
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def both(w, parents=None, n_nodes=None, plen=None):
    """The separate calls and the combined one, each on its own copy of the
    caches; returns the two result dicts (device tensors)."""
    res = []
    for combined in (False, True):
        d = upload(w, DEV)
        par = d["parents"] if parents is None else parents
        n = d["n_nodes"] if n_nodes is None else n_nodes
        P = d["prefix_len"] if plen is None else plen
        if combined:
            out, anc, depth, err = tv.tree_attention_from_parents(d["q"], d["k_new"], d["v_new"], d["k_cache"],
                                                                  d["v_cache"], P, n, par, rope_theta=w.rope_theta)
        else:
            anc, depth, err = tv.build_tree(par, n)
            out = tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], P, n, anc, depth,
                                    err, rope_theta=w.rope_theta)
        torch.cuda.synchronize()
        res.append(dict(out=out, anc=anc, depth=depth, err=err, k=d["k_cache"], v=d["v_cache"]))
    return res


def assert_same(sep, com, what=""):
    for key in ("anc", "depth", "err"):
        assert torch.equal(sep[key], com[key]), f"{what} {key} differs: {sep[key].cpu()} vs {com[key].cpu()}"
    for key in ("out", "k", "v"):
        diff = (bits(sep[key]) != bits(com[key]))
        assert not diff.any(), f"{what} {key} differs at {diff.nonzero()[:8].tolist()}"


CASES = [
    (1, {}),                            # fp32: two launches
    (2, dict(prefix=300)),
    (3, dict(B=3, prefix=150)),
    (3, dict(B=2, prefix=1100)),        # fused split merge
    (4, dict(B=2, prefix=200)),         # two row blocks
    (5, dict(B=6, prefix=(16, 300))),   # ragged prefixes
    (2, dict(prefix=0)),
    (5, dict(B=3, prefix=(1, 70), n=7)),
    (3, dict(B=3, prefix=150, D=64)),   # bf16 head dim 64: two launches
]


@pytest.mark.parametrize("cfg,over", CASES, ids=[f"cfg{c}-{i}" for i, (c, _) in enumerate(CASES)])
def test_small_cases_equal_separate_calls_and_oracle(cfg, over):
    print(f"[gpu] from_parents small cfg={cfg} {over}", flush=True)
    w = generate(cfg, **over)
    sep, com = both(w)
    assert_same(sep, com, f"cfg{cfg}")
    ref_anc, ref_depth, ref_err = oracle.build_tree(w.parents, w.n_nodes)
    assert np.array_equal(com["anc"].cpu().numpy().view(np.uint64), ref_anc)
    assert np.array_equal(com["depth"].cpu().numpy(), ref_depth)
    got = com["out"].float().cpu().numpy().astype(np.float64)
    for b in range(w.B):
        inp = w.oracle_inputs(b)
        out, _, _, _ = oracle.tree_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                                             inp["prefix_len"], inp["n_nodes"], inp["parents"], w.rope_theta, 0.0,
                                             err_in=ref_err[b:b + 1])
        e = attention_error(w.dtype, got[b], out[0])
        assert e <= tolerance(w.dtype), (b, e)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_workloads_equal_separate_calls(cfg):
    # the launch configurations the bench times: fused merge (3), separate
    # merge with ragged prefixes (5), one split with the append kernel (4),
    # 32-row query tiles (2, 5)
    print(f"[gpu] from_parents full cfg={cfg}", flush=True)
    w = generate(cfg)
    sep, com = both(w)
    assert_same(sep, com, f"cfg{cfg}")


def test_invalid_trees_and_capacity_like_build_tree():
    """Every invalid form tv_build_tree flags, a node count out of range, a
    tree past the cache capacity, an empty slot, a single node and valid
    trees, in one batch: err, anc, depth and the zero rows as the separate
    calls give them."""
    print("[gpu] from_parents invalid forms", flush=True)
    w = generate(3, B=10, prefix=40)
    w.parents[1, 0] = 0                 # root with a parent
    w.parents[2, 9] = -1                # a second root
    w.parents[3, 5] = 7                 # parent after child
    w.parents[4, 6] = -3                # parent below -1
    w.parents[5, 4] = 4                 # own parent
    w.n_nodes[6] = 0                    # empty slot
    w.n_nodes[7] = 1                    # plain decode
    w.parents[7, 1:] = -1
    w.prefix_len[8] = w.cap - 10        # past the capacity
    d = upload(w, DEV)
    n = d["n_nodes"].clone()
    n[9] = w.n_max + 1                  # node count above n_max
    sep, com = both(w, n_nodes=n)
    assert_same(sep, com, "invalid batch")
    assert com["err"].cpu().tolist() == [0, 2, 2, 2, 2, 2, 0, 0, 3, 2]
    out = com["out"].float()
    for b in (1, 2, 3, 4, 5, 6, 8, 9):
        assert (out[b] == 0).all(), b


def test_node_count_below_zero():
    w = generate(2, B=2, prefix=70)
    d = upload(w, DEV)
    n = d["n_nodes"].clone()
    n[1] = -1
    sep, com = both(w, n_nodes=n)
    assert_same(sep, com, "negative count")
    assert com["err"].cpu().tolist() == [0, 2]


def test_deep_chain_and_wide_star():
    w = generate(2, B=2, prefix=130)
    w.parents[0] = [-1] + list(range(63))
    w.parents[1] = [-1] + [0] * 63
    sep, com = both(w)
    assert_same(sep, com, "chain and star")
    assert com["depth"].cpu()[0, 63].item() == 63


def test_repeated_calls_are_identical():
    w = generate(3, B=4, prefix=1100)
    d = upload(w, DEV)
    outs = []
    for _ in range(4):
        out, anc, depth, err = tv.tree_attention_from_parents(d["q"], d["k_new"], d["v_new"], d["k_cache"],
                                                              d["v_cache"], d["prefix_len"], d["n_nodes"],
                                                              d["parents"], rope_theta=w.rope_theta)
        outs.append(bits(out).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
