"""GPU parity of the paged-KV calls (tv_tree_attention_paged, tv_commit_paged)
through the C ABI.

A paged cache stands for the dense cache its block table gathers (infra-guide
"5.3 Medusa、EAGLE 与 MTP", section 8, names the block table of a paged cache
as what a real implementation adds). The paged calls do the same arithmetic as
the dense ones, so on the same logical cache their outputs and the caches they
leave must equal the dense calls' bit for bit; the dense path is itself
checked against the oracle elsewhere, and small cases are compared with the
oracle here too. Pages no sequence references must stay untouched; a table
entry outside the pools must flag the sequence (TV_ERR_BAD_PAGE), zero its
rows and touch nothing.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.gpu_util import attention_error, host_f64, tolerance, upload
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def shuffled_table(w, rng, extra=5, share=0):
    """A random page for every block of every sequence (pages drawn without
    replacement from B * max_pages + extra); with share > 0, sequences 2k and
    2k + 1 share their first `share` pages."""
    mp = w.cap // tv.PAGE
    n_pages = w.B * mp + extra
    bt = rng.permutation(n_pages)[:w.B * mp].reshape(w.B, mp).astype(np.int32)
    for b in range(1, w.B, 2):
        bt[b, :share] = bt[b - 1, :share]
    return torch.from_numpy(bt).to(DEV), n_pages


def share_prefix_data(w, share):
    """Makes sequence 2k + 1's first `share` blocks hold sequence 2k's data
    (a shared page holds one content), for prefixes that cover them."""
    for b in range(1, w.B, 2):
        s = share * tv.PAGE
        assert min(w.prefix_len[b], w.prefix_len[b - 1]) >= s
        w.k_cache[b, :, :s] = w.k_cache[b - 1, :, :s]
        w.v_cache[b, :, :s] = w.v_cache[b - 1, :, :s]


def run_both(w, bt, n_pages, corrupt=None):
    """The dense step and the paged step on the same logical inputs; returns
    host copies of both steps' outputs, caches (as dense) and the pools."""
    d = upload(w, DEV)
    k_pool, v_pool = tv.pages_from_dense(d["k_cache"], d["v_cache"], bt, n_pages)
    free = torch.ones(n_pages, dtype=torch.bool, device=DEV)
    free[bt.reshape(-1).long()] = False
    # unreferenced pages hold a marker pattern that must survive
    k_pool[free] = 7.0
    v_pool[free] = -3.0
    if corrupt is not None:
        b, j, val = corrupt
        bt[b, j] = val
    pools0 = (k_pool.clone(), v_pool.clone())
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    err_p = err.clone()
    out_d = tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"],
                              d["n_nodes"], anc, depth, err, rope_theta=w.rope_theta)
    out_p = tv.tree_attention_paged(d["q"], d["k_new"], d["v_new"], k_pool, v_pool, bt, d["prefix_len"],
                                    d["n_nodes"], anc, depth, err_p, rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    res = dict(out_d=out_d.clone(), out_p=out_p.clone(), err_d=err.clone(), err_p=err_p.clone())
    res["k_attn_d"], res["v_attn_d"] = d["k_cache"].clone(), d["v_cache"].clone()
    res["pools_attn"] = (k_pool.clone(), v_pool.clone())
    acc_d, path_d, _, _ = tv.accept(d["tok"], d["tgt"], d["parents"], anc, depth, d["n_nodes"], err)
    acc_p, path_p, _, _ = tv.accept(d["tok"], d["tgt"], d["parents"], anc, depth, d["n_nodes"], err_p)
    pl_d = tv.commit(d["k_cache"], d["v_cache"], d["prefix_len"], acc_d, path_d)
    pl_p = tv.commit_paged(k_pool, v_pool, bt, d["prefix_len"], acc_p, path_p)
    torch.cuda.synchronize()
    res.update(k_d=d["k_cache"], v_d=d["v_cache"], k_pool=k_pool, v_pool=v_pool, pools0=pools0, free=free,
               pl_d=pl_d, pl_p=pl_p, acc_d=acc_d, acc_p=acc_p)
    return res


def check_equal_to_dense(res, bt, skip=()):
    live = [b for b in range(res["out_d"].shape[0]) if b not in skip]
    assert torch.equal(res["out_p"][live].view(torch.int16), res["out_d"][live].view(torch.int16))
    assert torch.equal(res["err_p"][live], res["err_d"][live])
    # caches after the attention (tree appended) and after the commit
    # (only the checked sequences' rows of the table are gathered: a row
    # with an entry outside the pools is never used as an index)
    bt_live = bt[live].contiguous()
    for (kp, vp), kd, vd in ((res["pools_attn"], res["k_attn_d"], res["v_attn_d"]),
                             ((res["k_pool"], res["v_pool"]), res["k_d"], res["v_d"])):
        kg, vg = tv.dense_from_pages(kp, vp, bt_live)
        assert torch.equal(kg.view(torch.int16), kd[live].view(torch.int16))
        assert torch.equal(vg.view(torch.int16), vd[live].view(torch.int16))
    assert torch.equal(res["pl_p"][live], res["pl_d"][live])
    # pages no sequence references are untouched
    free = res["free"]
    assert torch.equal(res["k_pool"][free].view(torch.int16), res["pools0"][0][free].view(torch.int16))
    assert torch.equal(res["v_pool"][free].view(torch.int16), res["pools0"][1][free].view(torch.int16))


def test_small_paged_against_oracle_and_dense():
    # the tree straddles two pages (P % 64 = 12, n = 60), pages shuffled
    print("[gpu] paged small", flush=True)
    w = generate(3, B=3, prefix=1100)
    rng = np.random.default_rng(1)
    bt, n_pages = shuffled_table(w, rng)
    res = run_both(w, bt, n_pages)
    check_equal_to_dense(res, bt)
    # and the oracle, on every row
    inp = w.oracle_inputs()
    out, kc, vc, e = oracle.tree_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                                           inp["prefix_len"], inp["n_nodes"], inp["parents"], w.rope_theta, 0.0)
    got = host_f64(res["out_p"])
    assert attention_error(w.dtype, got, out) <= tolerance(w.dtype)


@pytest.mark.parametrize("cfg,share", [(3, 0), (5, 4), (4, 0)])
def test_full_size_paged_equals_dense(cfg, share):
    # headline; ragged batch with shared prefix pages; 129 blocks per sequence
    print(f"[gpu] paged full cfg={cfg} share={share}", flush=True)
    w = generate(cfg)
    if share:
        share_prefix_data(w, share)
    rng = np.random.default_rng(cfg)
    bt, n_pages = shuffled_table(w, rng, share=share)
    res = run_both(w, bt, n_pages)
    check_equal_to_dense(res, bt)


def test_bad_page_flags_the_sequence_only():
    print("[gpu] paged bad page", flush=True)
    w = generate(3, B=3, prefix=1100)
    rng = np.random.default_rng(2)
    bt, n_pages = shuffled_table(w, rng)
    good_page = int(bt[1, 3])
    res = run_both(w, bt, n_pages, corrupt=(1, 3, n_pages + 5))
    assert int(res["err_p"][1]) == tv.TV_ERR_BAD_PAGE
    assert int(res["acc_p"][1]) == -1
    assert not res["out_p"][1].any()
    check_equal_to_dense(res, bt, skip=(1,))
    # the flagged sequence's pages (including the one it should have named)
    # are as the table-building left them
    pages = [int(x) for x in bt[1] if 0 <= int(x) < n_pages] + [good_page]
    for pg in pages:
        assert torch.equal(res["k_pool"][pg].view(torch.int16), res["pools0"][0][pg].view(torch.int16))
        assert torch.equal(res["v_pool"][pg].view(torch.int16), res["pools0"][1][pg].view(torch.int16))


def test_paged_is_deterministic():
    print("[gpu] paged determinism", flush=True)
    w = generate(5)
    rng = np.random.default_rng(3)
    bt, n_pages = shuffled_table(w, rng)
    d = upload(w, DEV)
    k_pool, v_pool = tv.pages_from_dense(d["k_cache"], d["v_cache"], bt, n_pages)
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    outs = []
    for _ in range(4):
        o = tv.tree_attention_paged(d["q"], d["k_new"], d["v_new"], k_pool, v_pool, bt, d["prefix_len"],
                                    d["n_nodes"], anc, depth, err, rope_theta=w.rope_theta)
        outs.append(o.view(torch.int16).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_paged_ragged_trees_against_oracle_and_dense():
    """Per-request tree boundaries with a paged cache (infra-guide "5.3"
    section 8 names both): trees of 60, 17, 1 and 0 nodes and a tree that is
    not parents-first, in one batch over shuffled pages; paged equals dense
    bit for bit, and every row of the live sequences matches the oracle."""
    print("[gpu] paged ragged trees", flush=True)
    w = generate(3, B=5, prefix=1100)
    w.n_nodes[:] = [60, 17, 1, 0, 60]
    for b in range(w.B):
        w.parents[b, w.n_nodes[b]:] = -1
    w.parents[4, 5] = 7                       # a parent after its child
    rng = np.random.default_rng(11)
    bt, n_pages = shuffled_table(w, rng)
    res = run_both(w, bt, n_pages)
    check_equal_to_dense(res, bt)
    assert res["err_p"].cpu().tolist() == [0, 0, 0, 0, tv.TV_ERR_BAD_TREE]
    assert res["acc_p"].cpu().tolist()[3:] == [-1, -1]
    inp = w.oracle_inputs()
    ref_anc, ref_depth, ref_err = oracle.build_tree(w.parents, w.n_nodes)
    out, kc, vc, e = oracle.tree_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                                           inp["prefix_len"], inp["n_nodes"], inp["parents"], w.rope_theta, 0.0,
                                           err_in=ref_err)
    got = host_f64(res["out_p"])
    assert attention_error(w.dtype, got, out) <= tolerance(w.dtype)
    assert not got[3].any() and not got[4].any()
