"""Pins for the oracle's RoPE and tree-masked attention.

RoPE is checked against its complex-number form, a hand rotation, and the
relative-position property. Attention is checked against
torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, with
the visibility mask taken from a Warshall closure (not from the oracle), and
against the invariants the pages state: a chain-shaped tree is plain causal
attention, siblings never see each other (infra-guide "5.3 Medusa、EAGLE 与
MTP", sections 3.1 and 8), and positions follow depth (section 3.2).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_tree import all_trees, warshall_closure


# ---------------------------------------------------------------- RoPE pins

def rope_complex(x, pos, theta):
    """Rotary embedding as multiplication of z_d = x_d + i x_{d+D/2} by a phase."""
    D = x.shape[-1]
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = np.array([theta ** (-2.0 * d / D) for d in range(half)])
    z = z * np.exp(1j * pos * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_hand_rotation():
    # D = 2: one pair, frequency 1, so position pi/2 turns (1, 0) into (0, 1)
    out = oracle.rope(np.array([1.0, 0.0]), math.pi / 2, 10000.0)
    assert np.allclose(out, [0.0, 1.0], atol=1e-15)
    out = oracle.rope(np.array([0.0, 1.0]), math.pi / 2, 10000.0)
    assert np.allclose(out, [-1.0, 0.0], atol=1e-15)


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_rope_complex_form_and_properties(D):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((3, D))
    for pos in [0, 1, 7, 4099, 8255]:
        r = oracle.rope(x, pos, 10000.0)
        assert np.allclose(r, rope_complex(x, pos, 10000.0), rtol=0, atol=1e-11)
        assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    assert np.array_equal(oracle.rope(x, 0, 10000.0), x)
    assert np.array_equal(oracle.rope(x, 123, 0.0), x)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    a = oracle.rope(q, 70, 10000.0) @ oracle.rope(k, 64, 10000.0)
    b = oracle.rope(q, 70 + 4000, 10000.0) @ oracle.rope(k, 64 + 4000, 10000.0)
    assert abs(a - b) < 1e-10


# ---------------------------------------------------------- attention pins

def make_case(rng, parents, P, Hq, Hkv, D, cap_extra=0):
    n = len(parents)
    B = 1
    return dict(
        parents=np.array([parents], dtype=np.int32),
        n_nodes=np.array([n], dtype=np.int32),
        prefix_len=np.array([P], dtype=np.int32),
        q=rng.standard_normal((B, n, Hq, D)),
        k_new=rng.standard_normal((B, n, Hkv, D)),
        v_new=rng.standard_normal((B, n, Hkv, D)),
        k_cache=rng.standard_normal((B, Hkv, P + n + cap_extra, D)),
        v_cache=rng.standard_normal((B, Hkv, P + n + cap_extra, D)),
    )


def run_oracle(c, theta=10000.0, scale=0.0):
    return oracle.tree_attention(c["q"], c["k_new"], c["v_new"], c["k_cache"], c["v_cache"],
                                 c["prefix_len"], c["n_nodes"], c["parents"], theta, scale)


def sdpa_reference(c, vis, theta=10000.0):
    """Library attention over [prefix; rotated tree keys] with mask [1..1 | vis]."""
    P = int(c["prefix_len"][0])
    n = int(c["n_nodes"][0])
    Hq, Hkv = c["q"].shape[2], c["k_new"].shape[2]
    G = Hq // Hkv
    depth = [int(r.sum()) - 1 for r in vis]
    qr = np.stack([oracle.rope(c["q"][0, i], P + depth[i], theta) for i in range(n)])   # n,Hq,D
    kr = np.stack([oracle.rope(c["k_new"][0, i], P + depth[i], theta) for i in range(n)])  # n,Hkv,D
    K = np.concatenate([c["k_cache"][0, :, :P, :], kr.transpose(1, 0, 2)], axis=1)   # Hkv, P+n, D
    V = np.concatenate([c["v_cache"][0, :, :P, :], c["v_new"][0].transpose(1, 0, 2)], axis=1)
    K = np.repeat(K, G, axis=0)
    V = np.repeat(V, G, axis=0)
    mask = np.concatenate([np.ones((n, P), dtype=bool), vis.astype(bool)], axis=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr.transpose(1, 0, 2)).unsqueeze(0),
        torch.from_numpy(K).unsqueeze(0), torch.from_numpy(V).unsqueeze(0),
        attn_mask=torch.from_numpy(mask))
    return out[0].numpy().transpose(1, 0, 2)   # n, Hq, D


@pytest.mark.parametrize("seed,parents,P,Hq,Hkv,D", [
    (0, [-1, 0, 0, 1, 2], 64, 4, 4, 64),
    (1, [-1, 0, 0, 1, 2], 0, 2, 1, 16),
    (2, [-1, 0, 1, 1, 0, 4, 2, 6, 3], 37, 8, 2, 32),
    (3, [-1], 19, 4, 2, 8),
])
def test_tree_attention_matches_library_sdpa(seed, parents, P, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    c = make_case(rng, parents, P, Hq, Hkv, D)
    out, kc, vc, err = run_oracle(c)
    ref = sdpa_reference(c, warshall_closure(parents))
    assert err[0] == 0
    assert np.allclose(out[0], ref, rtol=0, atol=1e-12)


def test_all_trees_n5_match_library_sdpa():
    rng = np.random.default_rng(5)
    for parents in all_trees(5):
        c = make_case(rng, parents, 7, 2, 1, 8)
        out = run_oracle(c)[0]
        assert np.allclose(out[0], sdpa_reference(c, warshall_closure(parents)), atol=1e-12)


def test_chain_tree_is_plain_causal_attention():
    # a chain of n nodes = n ordinary decode positions after the prefix
    rng = np.random.default_rng(11)
    n, P, H, D = 6, 21, 3, 16
    c = make_case(rng, [-1] + list(range(n - 1)), P, H, H, D)
    out = run_oracle(c)[0][0]
    qr = np.stack([oracle.rope(c["q"][0, i], P + i, 10000.0) for i in range(n)])
    kr = np.stack([oracle.rope(c["k_new"][0, i], P + i, 10000.0) for i in range(n)])
    K = np.concatenate([c["k_cache"][0, :, :P, :], kr.transpose(1, 0, 2)], axis=1)
    V = np.concatenate([c["v_cache"][0, :, :P, :], c["v_new"][0].transpose(1, 0, 2)], axis=1)
    # is_causal over the full (P+n)-long sequence; keep the last n query rows
    Qfull = np.zeros((H, P + n, D))
    Qfull[:, P:, :] = qr.transpose(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qfull), torch.from_numpy(K), torch.from_numpy(V), is_causal=True)
    ref = ref.numpy()[:, P:, :].transpose(1, 0, 2)
    assert np.allclose(out, ref, atol=1e-12)


def test_single_key_and_equal_keys_closed_forms():
    # P = 0, one node: softmax over one key is 1, so the output is that value
    rng = np.random.default_rng(3)
    c = make_case(rng, [-1], 0, 2, 1, 8)
    out = run_oracle(c)[0]
    for h in range(2):
        assert np.allclose(out[0, 0, h], c["v_new"][0, 0, 0], atol=1e-15)
    # two identical keys (prefix key = rotated root key) -> mean of the two values
    c = make_case(rng, [-1], 1, 1, 1, 8)
    c["k_cache"][0, 0, 0] = oracle.rope(c["k_new"][0, 0, 0], 1, 10000.0)
    out = run_oracle(c)[0]
    assert np.allclose(out[0, 0, 0], 0.5 * (c["v_cache"][0, 0, 0] + c["v_new"][0, 0, 0]), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(4)
    parents = [-1, 0, 0, 1, 2, 2]
    c = make_case(rng, parents, 13, 8, 2, 16)
    out = run_oracle(c)[0]
    m = dict(c)
    for key in ("k_new", "v_new"):
        m[key] = np.repeat(c[key], 4, axis=2)
    for key in ("k_cache", "v_cache"):
        m[key] = np.repeat(c[key], 4, axis=1)
    assert np.allclose(out, run_oracle(m)[0], atol=1e-13)


def test_non_ancestors_do_not_matter():
    rng = np.random.default_rng(6)
    parents = [-1, 0, 0, 1, 2, 1, 3]
    c = make_case(rng, parents, 9, 4, 2, 16)
    base = run_oracle(c)[0]
    vis = warshall_closure(parents)
    for j in range(len(parents)):
        d = {k: np.array(v, copy=True) for k, v in c.items()}
        d["q"][0, j] += 5.0
        d["k_new"][0, j] += 5.0
        d["v_new"][0, j] -= 3.0
        out = run_oracle(d)[0]
        for i in range(len(parents)):
            if i != j and not vis[i, j]:
                assert np.array_equal(out[0, i], base[0, i]), (i, j)
            elif vis[i, j]:
                assert not np.allclose(out[0, i], base[0, i])


def test_sibling_relabelling_permutes_outputs():
    rng = np.random.default_rng(8)
    parents = [-1, 0, 0, 1, 2]
    c = make_case(rng, parents, 10, 2, 2, 8)
    out = run_oracle(c)[0]
    # swap nodes 1<->2 and 3<->4: parents become [-1, 0, 0, 2, 1]... relabel map
    perm = [0, 2, 1, 4, 3]          # new index -> old index
    new_par = [-1, 0, 0, 1, 2]      # node 1(new)=2(old) has child 3(new)=4(old)
    d = dict(c)
    for key in ("q", "k_new", "v_new"):
        d[key] = c[key][:, perm]
    d["parents"] = np.array([new_par], dtype=np.int32)
    out2 = run_oracle(d)[0]
    assert np.allclose(out2[0], out[0][perm], atol=1e-13)


def test_cache_append_and_capacity_error():
    rng = np.random.default_rng(9)
    parents = [-1, 0, 1]
    c = make_case(rng, parents, 5, 2, 2, 8, cap_extra=2)
    out, kc, vc, err = run_oracle(c)
    depth = [0, 1, 2]
    for a in range(3):
        for g in range(2):
            assert np.allclose(kc[0, g, 5 + a], oracle.rope(c["k_new"][0, a, g], 5 + depth[a], 1e4))
            assert np.array_equal(vc[0, g, 5 + a], c["v_new"][0, a, g])
    assert np.array_equal(kc[0, :, :5], c["k_cache"][0, :, :5])
    assert np.array_equal(kc[0, :, 8:], c["k_cache"][0, :, 8:])
    # prefix so long that the tree does not fit: error, outputs zero, cache untouched
    c["prefix_len"] = np.array([9], dtype=np.int32)
    out, kc, vc, err = run_oracle(c)
    assert err[0] == oracle.ERR_CAPACITY
    assert (out == 0).all() and np.array_equal(kc, c["k_cache"])
