"""Pins for the oracle's paged-KV view (infra-guide "5.3 Medusa、EAGLE 与 MTP",
section 8: a real implementation adds the paged KV block table).

A paged cache stands for the dense per-sequence cache whose slot s is page
block_table[b][s // 64], offset s % 64. Checked by: an identity table is a
plain reshape of the pools; relabelling pages (pool and table permuted
together) changes nothing; scatter undoes gather on referenced pages and
leaves unreferenced ones alone; sequences may share read-only prefix pages;
and paged attention / commit, computed on the gathered cache, equal the dense
oracle on the same logical cache.
"""
import numpy as np

import oracle
from workloads import generate


def rand_pools(rng, n_pages, Hkv=2, D=8):
    return (rng.standard_normal((n_pages, Hkv, oracle.PAGE, D)),
            rng.standard_normal((n_pages, Hkv, oracle.PAGE, D)))


def test_identity_table_is_a_reshape():
    rng = np.random.default_rng(0)
    kp, vp = rand_pools(rng, 6)
    bt = np.arange(6, dtype=np.int32).reshape(2, 3)
    k, v = oracle.gather_pages(kp, vp, bt)
    # sequence b's slots are pages 3b, 3b+1, 3b+2 laid end to end
    for b in range(2):
        want = np.concatenate([kp[3 * b + j] for j in range(3)], axis=1)
        assert np.array_equal(k[b], want)
        assert np.array_equal(v[b], np.concatenate([vp[3 * b + j] for j in range(3)], axis=1))
    assert k.shape == (2, 2, 3 * 64, 8)
    assert k[1, 0, 64 + 5, 3] == kp[4, 0, 5, 3]


def test_relabelling_pages_changes_nothing():
    rng = np.random.default_rng(1)
    kp, vp = rand_pools(rng, 10)
    bt = rng.permutation(10)[:8].reshape(2, 4).astype(np.int32)
    perm = rng.permutation(10)            # new label of each page
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    bt2 = perm[bt].astype(np.int32)
    a = oracle.gather_pages(kp, vp, bt)
    b = oracle.gather_pages(kp2, vp2, bt2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_scatter_inverts_gather_and_keeps_free_pages():
    rng = np.random.default_rng(2)
    kp, vp = rand_pools(rng, 9)
    bt = np.array([[4, 0, 7], [2, 8, 5]], dtype=np.int32)     # pages 1, 3, 6 free
    k, v = oracle.gather_pages(kp, vp, bt)
    kq, vq = oracle.scatter_pages(k, v, bt, kp, vp)
    assert np.array_equal(kq, kp) and np.array_equal(vq, vp)
    k2 = k + 1.0
    kq, vq = oracle.scatter_pages(k2, v, bt, kp, vp)
    for pg in (1, 3, 6):
        assert np.array_equal(kq[pg], kp[pg])
    assert np.array_equal(kq[7], kp[7] + 1.0)


def test_shared_prefix_pages():
    rng = np.random.default_rng(3)
    kp, vp = rand_pools(rng, 5)
    bt = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)      # first two pages shared
    k, v = oracle.gather_pages(kp, vp, bt)
    assert np.array_equal(k[0, :, :128], k[1, :, :128])
    assert not np.array_equal(k[0, :, 128:], k[1, :, 128:])


def test_paged_step_equals_dense_step():
    # a small workload whose logical cache is scattered over shuffled pages
    w = generate(3, B=2, prefix=150, n=20, max_depth=4, Hq=8, Hkv=2, D=16)
    inp = w.oracle_inputs()
    cap = w.cap
    pages_per_seq = cap // oracle.PAGE
    rng = np.random.default_rng(4)
    n_pages = w.B * pages_per_seq + 3
    bt = rng.permutation(n_pages)[:w.B * pages_per_seq].reshape(w.B, pages_per_seq).astype(np.int32)
    kp = rng.standard_normal((n_pages, w.Hkv, oracle.PAGE, w.D))
    vp = rng.standard_normal((n_pages, w.Hkv, oracle.PAGE, w.D))
    kp, vp = oracle.scatter_pages(inp["k_cache"], inp["v_cache"], bt, kp, vp)
    kd, vd = oracle.gather_pages(kp, vp, bt)
    assert np.array_equal(kd, inp["k_cache"]) and np.array_equal(vd, inp["v_cache"])
    paged = dict(inp, k_cache=kd, v_cache=vd)
    r_dense = oracle.verify_step(inp)
    r_paged = oracle.verify_step(paged)
    for key in ("out", "accept_len", "path", "k_cache", "v_cache", "prefix_len_out"):
        assert np.array_equal(r_dense[key], r_paged[key]), key
    # written back, the committed cache lands in the same pages
    kq, vq = oracle.scatter_pages(r_paged["k_cache"], r_paged["v_cache"], bt, kp, vp)
    kg, vg = oracle.gather_pages(kq, vq, bt)
    assert np.array_equal(kg, r_dense["k_cache"]) and np.array_equal(vg, r_dense["v_cache"])
