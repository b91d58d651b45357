"""GPU parity for typical acceptance (tv_accept_typical through the C ABI)
against the CPU oracle.

Bit-exact: target argmax per node, accepted length, path, bonus token and
emitted tokens. Floating point: entropy within 1e-4 nats and the candidate
probability within 1e-4 relative (fp32 sums of 2^u over up to 128k terms, a
few ulp each, give a few 1e-6; the rest is margin). The accept decision is a
float comparison, so every test first checks, on the oracle side only, that
no edge lies within 1e-3 relative of its floor: there both precisions must
decide alike.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.gpu_util import to_dev
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, generate, target_logits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H_ABS_TOL = 1e-4
P_REL_TOL = 1e-4
MARGIN = 1e-3


def logits_f64(x: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def run_typical(w, logits_host, eps, delta, err=None, tok=None):
    parents = to_dev(w.parents, "i32", DEV)
    n_nodes = to_dev(w.n_nodes, "i32", DEV)
    tok_d = to_dev(w.tok if tok is None else tok, "i32", DEV)
    logits = to_dev(logits_host, "bf16" if logits_host.dtype == np.uint16 else "f32", DEV)
    anc, depth, err_d = tv.build_tree(parents, n_nodes)
    if err is not None:
        err_d = to_dev(err, "i32", DEV)
    acc, path, bonus, toks, H, pt, am = tv.accept_typical(logits, tok_d, parents, anc, depth, n_nodes,
                                                          err_d, epsilon=eps, delta=delta)
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), path=path.cpu().numpy(), bonus=bonus.cpu().numpy(),
                out_tokens=toks.cpu().numpy(), entropy=H.cpu().numpy().astype(np.float64),
                p_tok=pt.cpu().numpy().astype(np.float64), argmax=am.cpu().numpy())


def check_typical(w, logits_host, eps, delta, err=None, tok=None):
    tok = w.tok if tok is None else tok
    x = logits_f64(logits_host)
    H, pt, am, acc, path, bonus, toks = oracle.typical_accept(x, tok, w.parents, w.n_nodes, eps, delta,
                                                              err_in=err)
    # no edge so close to its floor that the two precisions could disagree
    for b in range(w.B):
        if err is not None and err[b] != 0:
            continue
        for c in range(1, int(w.n_nodes[b])):
            if pt[b, c] == 0.0:      # token outside the vocabulary: exactly 0 on both sides
                continue
            assert pt[b, c] > 1e-30   # well inside fp32's normal range
            floor = min(eps, delta * math.exp(-H[b, w.parents[b, c]]))
            assert abs(pt[b, c] - floor) > MARGIN * max(pt[b, c], floor), (b, c, pt[b, c], floor)
    got = run_typical(w, logits_host, eps, delta, err=err, tok=tok)
    assert np.array_equal(got["argmax"], am)
    assert np.abs(got["entropy"] - H).max() <= H_ABS_TOL
    assert (np.abs(got["p_tok"] - pt) <= P_REL_TOL * pt + 1e-30).all()
    assert np.array_equal(got["accept_len"], acc)
    assert np.array_equal(got["path"], path)
    assert np.array_equal(got["bonus"], bonus)
    assert np.array_equal(got["out_tokens"], toks)
    return got, acc


@pytest.mark.parametrize("eps,delta", [(0.09, 0.3), (0.2, 2.0), (0.5, 1e6), (0.0, 0.0)])
def test_full_size_bf16_eagle_trees(eps, delta):
    # 8 sequences x 60-node EAGLE-2-style trees, 32000-token vocabulary
    w = generate(3)
    L = target_logits(w)
    _, acc = check_typical(w, L, eps, delta)
    print(f"eps={eps} delta={delta} accept_len={acc.tolist()}", flush=True)


@pytest.mark.parametrize("V,dtype", [(32000, "f32"), (1001, "f32"), (1003, "bf16"), (5, "bf16"),
                                     (1, "f32"), (128256, "bf16")])
def test_vocab_sizes_and_paths(V, dtype):
    # 16-byte rows take the vector path; 1001 fp32 and 1003 bf16 the element path
    w = generate(3, B=2 if V > 100000 else 3, seed=21)
    w = dataclasses.replace(w, tok=(w.tok % V).astype(np.int32))
    L = target_logits(w, vocab=V, dtype=dtype, seed=4)
    check_typical(w, L, 0.09, 0.3)


def test_padding_skipped_sequences_and_foreign_tokens():
    w = generate(3, B=4, seed=33)
    n_nodes = w.n_nodes.copy()
    n_nodes[1], n_nodes[2] = 17, 0
    parents = w.parents.copy()
    parents[1, 17:] = -1
    w = dataclasses.replace(w, n_nodes=n_nodes, parents=parents)
    tok = w.tok.copy()
    tok[0, 3], tok[0, 7], tok[1, 2] = -3, 32000 + 7, 2 ** 31 - 1
    L = target_logits(w, seed=5)
    err = np.array([0, 0, 0, 2], dtype=np.int32)
    got, acc = check_typical(w, L, 0.0, 0.0, err=err, tok=tok)
    assert got["p_tok"][0, 3] == 0.0 and got["p_tok"][0, 7] == 0.0 and got["p_tok"][1, 2] == 0.0
    assert acc[2] == -1 and acc[3] == -1
    assert (got["argmax"][1, 17:] == -1).all() and (got["argmax"][3] == -1).all()


def test_argmax_ties_take_the_lowest_token():
    # equal maxima in one chunk, in one thread's later batch, and in other threads
    w = generate(3, B=2, seed=8)
    V = 32000
    L = target_logits(w, seed=6)
    x = bf16_bits_to_f32(L)
    top = f32_to_bf16_bits(np.array([x.max() + 8.0], dtype=np.float32))[0]
    for i in range(w.n_max):
        L[0, i, [20000, 3616, 3617, 100 + i]] = top          # lowest: 100 + i
        L[1, i, [3617, 20001, 3616 + 16384]] = top           # lowest: 3617
    got, _ = check_typical(w, L, 0.09, 0.3)
    live0, live1 = int(w.n_nodes[0]), int(w.n_nodes[1])
    assert got["argmax"][0, :live0].tolist() == [100 + i for i in range(live0)]
    assert (got["argmax"][1, :live1] == 3617).all()


def test_greedy_limit_matches_the_greedy_kernel():
    # floor 1/2 with every distribution peaked above 1/2: typical == greedy,
    # on the GPU as in the oracle
    w = generate(3, seed=12)
    rng = np.random.default_rng(2)
    V = 32000
    x = rng.standard_normal((w.B, w.n_max, V)).astype(np.float32)
    peak = rng.integers(0, V, size=(w.B, w.n_max))
    tok = w.tok.copy()
    for b in range(w.B):
        x[b, np.arange(w.n_max), peak[b]] = 14.0
        for c in range(1, int(w.n_nodes[b])):
            if rng.random() < 0.75:
                tok[b, c] = peak[b, w.parents[b, c]]
    L = f32_to_bf16_bits(x)
    got, acc = check_typical(w, L, 0.5, 1e6, tok=tok)
    parents = to_dev(w.parents, "i32", DEV)
    n_nodes = to_dev(w.n_nodes, "i32", DEV)
    anc, depth, err = tv.build_tree(parents, n_nodes)
    g = tv.accept(to_dev(tok, "i32", DEV), to_dev(got["argmax"], "i32", DEV), parents, anc, depth,
                  n_nodes, err)
    torch.cuda.synchronize()
    assert np.array_equal(g[0].cpu().numpy(), acc)
    assert np.array_equal(g[1].cpu().numpy(), got["path"])
    assert np.array_equal(g[2].cpu().numpy(), got["bonus"])
