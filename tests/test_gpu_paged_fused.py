"""The paged fused calls (tv_tree_attention_paged_from_parents,
tv_accept_commit_paged) against the separate paged calls (tv_build_tree,
tv_tree_attention_paged, tv_accept, tv_commit_paged) on the same inputs,
through the C ABI: outputs, anc, depth, err, accept outputs, new prefix
lengths and both page pools (after the attention's append and after the
commit) bit for bit. The separate paged calls are checked against the dense
calls and the oracle in test_gpu_paged.py."""
import numpy as np
import pytest
import torch

import tree_attention_verification_tv_amd as tv
from tests.gpu_util import upload
from tests.test_gpu_paged import share_prefix_data, shuffled_table
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def run_both(w, bt, n_pages, corrupt=None, corrupt_after_attention=None):
    """corrupt: (b, block, value) written into the table before both steps;
    corrupt_after_attention: the same, between the attention and the commit."""
    d = upload(w, DEV)
    k_pool, v_pool = tv.pages_from_dense(d["k_cache"], d["v_cache"], bt, n_pages)
    free = torch.ones(n_pages, dtype=torch.bool, device=DEV)
    free[bt.reshape(-1).long()] = False
    k_pool[free] = 7.0
    v_pool[free] = -3.0
    if corrupt is not None:
        b, j, val = corrupt
        bt[b, j] = val
    res = {}
    for fused in (False, True):
        kp, vp = k_pool.clone(), v_pool.clone()
        if fused:
            out, anc, depth, err = tv.tree_attention_paged_from_parents(
                d["q"], d["k_new"], d["v_new"], kp, vp, bt, d["prefix_len"], d["n_nodes"], d["parents"],
                rope_theta=w.rope_theta)
        else:
            anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
            out = tv.tree_attention_paged(d["q"], d["k_new"], d["v_new"], kp, vp, bt, d["prefix_len"],
                                          d["n_nodes"], anc, depth, err, rope_theta=w.rope_theta)
        torch.cuda.synchronize()
        r = dict(out=out.clone(), anc=anc.clone(), depth=depth.clone(), err=err.clone(), k_attn=kp.clone(),
                 v_attn=vp.clone())
        btc = bt.clone()
        if corrupt_after_attention is not None:
            b, j, val = corrupt_after_attention
            btc[b, j] = val
        if fused:
            acc, path, bonus, toks, pl = tv.accept_commit_paged(d["tok"], d["tgt"], d["parents"], anc, depth,
                                                               d["n_nodes"], err, kp, vp, btc, d["prefix_len"])
        else:
            acc, path, bonus, toks = tv.accept(d["tok"], d["tgt"], d["parents"], anc, depth, d["n_nodes"], err)
            pl = tv.commit_paged(kp, vp, btc, d["prefix_len"], acc, path)
        torch.cuda.synchronize()
        r.update(acc=acc, path=path, bonus=bonus, toks=toks, pl=pl, k=kp, v=vp)
        res["fused" if fused else "sep"] = r
    res["free"] = free
    res["pools0"] = (k_pool, v_pool)
    return res


def assert_same(res):
    s, f = res["sep"], res["fused"]
    for key in ("anc", "depth", "err", "acc", "path", "bonus", "toks", "pl"):
        assert torch.equal(s[key], f[key]), (key, s[key].cpu(), f[key].cpu())
    for key in ("out", "k_attn", "v_attn", "k", "v"):
        diff = bits(s[key]) != bits(f[key])
        assert not diff.any(), (key, diff.nonzero()[:8].tolist())
    free = res["free"]
    for key, i in (("k", 0), ("v", 1)):
        assert torch.equal(bits(f[key][free]), bits(res["pools0"][i][free]))


SMALL = [(3, dict(B=3, prefix=150)), (5, dict(B=6, prefix=(16, 300))), (2, dict(prefix=300)),
         (4, dict(B=2, prefix=200)), (3, dict(B=2, prefix=1100))]


@pytest.mark.parametrize("cfg,over", SMALL, ids=[f"cfg{c}-{i}" for i, (c, _) in enumerate(SMALL)])
def test_small_equal_separate_calls(cfg, over):
    print(f"[gpu] paged fused small cfg={cfg} {over}", flush=True)
    w = generate(cfg, **over)
    bt, n_pages = shuffled_table(w, np.random.default_rng(cfg))
    assert_same(run_both(w, bt, n_pages))


@pytest.mark.parametrize("cfg,share", [(3, 0), (5, 0), (4, 0), (3, 4)])
def test_full_size_equal_separate_calls(cfg, share):
    print(f"[gpu] paged fused full cfg={cfg} share={share}", flush=True)
    w = generate(cfg)
    if share:
        share_prefix_data(w, share)
    bt, n_pages = shuffled_table(w, np.random.default_rng(10 + cfg), share=share)
    assert_same(run_both(w, bt, n_pages))


def test_bad_page_and_bad_trees():
    """A page outside the pools in one sequence, a bad tree, a tree past the
    capacity, an empty slot and a single node in one batch: err and every
    output as the separate calls give them."""
    print("[gpu] paged fused invalid forms", flush=True)
    w = generate(3, B=7, prefix=300)
    w.parents[2, 5] = 7                  # parent after child
    w.prefix_len[3] = w.cap - 10         # past the capacity
    w.n_nodes[4] = 0
    w.n_nodes[5] = 1
    w.parents[5, 1:] = -1
    bt, n_pages = shuffled_table(w, np.random.default_rng(5))
    res = run_both(w, bt, n_pages, corrupt=(1, 2, n_pages + 4))
    assert_same(res)
    assert res["fused"]["err"].cpu().tolist() == [0, tv.TV_ERR_BAD_PAGE, tv.TV_ERR_BAD_TREE, tv.TV_ERR_CAPACITY,
                                                  0, 0, 0]


def test_bad_page_found_by_the_commit():
    """A table entry of the block the accepted path moves into, made invalid
    after the attention: both commits leave that sequence unchanged."""
    print("[gpu] paged fused commit bad page", flush=True)
    w = generate(3, B=3, prefix=300)
    bt, n_pages = shuffled_table(w, np.random.default_rng(6))
    P = int(w.prefix_len[1])
    res = run_both(w, bt, n_pages, corrupt_after_attention=(1, P // tv.PAGE, n_pages + 9))
    assert_same(res)
    assert int(res["fused"]["pl"][1]) == P
    assert int(res["fused"]["pl"][0]) > int(w.prefix_len[0])
