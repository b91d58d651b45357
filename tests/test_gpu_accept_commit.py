"""The fused accept + commit call (tv_accept_commit) against the separate
tv_accept and tv_commit on the same inputs, through the C ABI: accept
outputs, committed caches and new prefix lengths bit for bit, and the
commit against the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.gpu_util import upload
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _prepare(w):
    d = upload(w, DEV)
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    # the attention appends the tree KV (the state commit works on)
    tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"], d["n_nodes"],
                      anc, depth, err, rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    return d, anc, depth, err


def _compare(w, alias=False):
    d, anc, depth, err = _prepare(w)
    k0, v0 = d["k_cache"].clone(), d["v_cache"].clone()
    # separate calls
    acc, path, bonus, toks = tv.accept(d["tok"], d["tgt"], d["parents"], anc, depth, d["n_nodes"], err)
    plen_sep = tv.commit(d["k_cache"], d["v_cache"], d["prefix_len"], acc, path)
    # fused call on a copy of the pre-commit caches
    kf, vf = k0.clone(), v0.clone()
    plen_in = d["prefix_len"].clone()
    r = tv.accept_commit(d["tok"], d["tgt"], d["parents"], anc, depth, d["n_nodes"], err, kf, vf, plen_in,
                         prefix_len_out=plen_in if alias else None)
    torch.cuda.synchronize()
    for a, b_, name in ((r[0], acc, "accept_len"), (r[1], path, "path"), (r[2], bonus, "bonus"),
                        (r[3], toks, "out_tokens"), (r[4], plen_sep, "prefix_len_out")):
        assert torch.equal(a, b_), name
    assert torch.equal(_bits(kf), _bits(d["k_cache"])), "K cache"
    assert torch.equal(_bits(vf), _bits(d["v_cache"])), "V cache"
    # the commit is the oracle's copy of the library's post-attention cache
    kb = _bits(k0).cpu().numpy()
    vb = _bits(tv.v_cache_rows(v0)).cpu().numpy()
    k_exp, v_exp, plen = oracle.commit(kb, vb, w.prefix_len, r[0].cpu().numpy(), r[1].cpu().numpy())
    assert np.array_equal(r[4].cpu().numpy(), plen)
    assert np.array_equal(_bits(kf).cpu().numpy(), k_exp)
    assert np.array_equal(_bits(tv.v_cache_rows(vf)).cpu().numpy(), v_exp)
    return r


CASES = [(3, {}), (5, {}), (1, {}), (2, dict(prefix=300)), (4, dict(B=2, prefix=200)), (3, dict(D=64, prefix=150))]


@pytest.mark.parametrize("cfg,over", CASES, ids=[f"cfg{c}" + ("-d64" if o.get("D") == 64 else "") for c, o in CASES])
@pytest.mark.parametrize("alias", [False, True])
def test_fused_equals_separate(cfg, over, alias):
    print(f"[gpu] accept+commit cfg={cfg} {over} alias={alias}", flush=True)
    r = _compare(generate(cfg, **over), alias=alias)
    print(f"  accepted {r[0].cpu().tolist()[:8]}", flush=True)


def test_fused_edge_batch():
    """A normal tree, a single node, an inactive slot, a bad tree, a tree
    over the capacity and no prefix in one batch."""
    print("[gpu] accept+commit edge batch", flush=True)
    w = generate(3, B=6, prefix=40)
    w.n_nodes[1] = 1
    w.parents[1, 1:] = -1
    w.n_nodes[2] = 0
    w.parents[3, 5] = 7
    w.prefix_len[4] = w.cap - 10
    w.prefix_len[5] = 0
    r = _compare(w)
    assert r[0].cpu().tolist()[2:5] == [-1, -1, -1]


def test_fused_deep_chain():
    """A 64-node chain fully accepted (path of 64 slots) and a star."""
    print("[gpu] accept+commit deep chain", flush=True)
    w = generate(2, B=2, prefix=130)
    w.parents[0] = [-1] + list(range(63))
    w.parents[1] = [-1] + [0] * 63
    w.tgt[0, :63] = w.tok[0, 1:]
    r = _compare(w)
    assert r[0][0].item() == 63
