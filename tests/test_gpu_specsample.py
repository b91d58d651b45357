"""GPU parity of chain speculative sampling (tv_speculative_sample through
the C ABI) against the CPU oracle (robertz.co "Drafters ...", section "Why
the answer does not change").

Exact: the kept count and the kept tokens; the keep test compares floats
computed in fp32 on the GPU and fp64 in the oracle, so each case first
checks, on the oracle side only, that every keep test is at least 0.1% from
its threshold. The drawn token must equal the oracle's when u * total lies
more than 1e-4 of the total inside the oracle's interval for it; otherwise
(a draw among many tiny weights, where fp32 sums legitimately disagree) it
must be a token of positive weight whose interval reaches u * total within
that tolerance. p(x) and q(x) agree within 1e-4 relative. A law test checks on the GPU that the first emitted
token is distributed as the target's first distribution.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_tv_amd as tv
from tests.gpu_util import to_dev
from workloads import bf16_bits_to_f32, speculative_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def f64(x):
    return (bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def run(p, q, draft, u_acc, u_res):
    dt = "bf16" if p.dtype == np.uint16 else "f32"
    out = tv.speculative_sample(to_dev(p, dt, DEV), to_dev(q, dt, DEV), to_dev(draft, "i32", DEV),
                                to_dev(u_acc, "f32", DEV), to_dev(u_res, "f32", DEV))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check(p, q, draft, u_acc, u_res):
    pf, qf = f64(p), f64(q)
    B, L = draft.shape
    acc, toks, pt, qt = run(p, q, draft, u_acc, u_res)
    for b in range(B):
        j, t, ptr, qtr = oracle.speculative_sample(pf[b], qf[b], draft[b], u_acc[b].astype(np.float64),
                                                   float(u_res[b]))
        for i in range(min(j + 1, L)):
            a, c = float(u_acc[b, i]) * qtr[i], ptr[i]
            assert abs(a - c) > 1e-3 * max(a, c), (b, i, a, c)
        w = np.maximum(oracle.softmax64(pf[b, j]) - oracle.softmax64(qf[b, j]), 0) if j < L else \
            oracle.softmax64(pf[b, L])
        cdf = np.cumsum(w)
        W = cdf[-1]
        tt = float(u_res[b]) * W
        assert acc[b] == j, b
        # everything but the drawn token is unique; the drawn token is unique
        # when u * total sits well inside its interval of the cumulative
        # distribution, else any token whose interval reaches it within the
        # fp32 error of the sums is a correct draw
        want, got = toks[b].copy(), toks[b].copy()
        y_ref, y = int(t[j]), int(toks[b, j])
        want[j] = got[j] = 0
        t_ref = t.copy()
        t_ref[j] = 0
        assert np.array_equal(got, t_ref), b
        lo_ref = cdf[y_ref - 1] if y_ref > 0 else 0.0
        tol = 1e-4 * W
        if tt - lo_ref > tol and cdf[y_ref] - tt > tol:
            assert y == y_ref, (b, y, y_ref)
        else:
            lo = cdf[y - 1] if y > 0 else 0.0
            assert w[y] > 0 and lo - tol <= tt < cdf[y] + tol, (b, y, y_ref)
        assert np.allclose(pt[b, :j + (j < L)], ptr[:j + (j < L)], rtol=1e-4, atol=0)
        assert np.allclose(qt[b, :j + (j < L)], qtr[:j + (j < L)], rtol=1e-4, atol=0)
    return acc


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_full_size_bf16(seed):
    print(f"[gpu] speculative sampling B=8 L=5 V=32000 seed={seed}", flush=True)
    acc = check(*speculative_inputs(8, 5, seed=seed))
    print(f"  kept {acc.tolist()}", flush=True)


@pytest.mark.parametrize("V,dtype,L", [(1001, "f32", 3), (1003, "bf16", 7), (32000, "f32", 1), (128256, "bf16", 2)])
def test_vocab_sizes(V, dtype, L):
    check(*speculative_inputs(4, L, V=V, dtype=dtype, seed=V + L))


def test_equal_draft_keeps_all_and_draws_the_bonus():
    p, q, draft, u_acc, u_res = speculative_inputs(6, 4, V=5000, dtype="f32", seed=11)
    q = np.ascontiguousarray(p[:, :4])
    acc = check(p, q, draft, u_acc, u_res)
    assert (acc == 4).all()


def test_first_token_law_matches_the_target():
    # 20000 sequences with the same logits and fresh draws: the first
    # emitted token is distributed as softmax(p_0)
    print("[gpu] speculative sampling law", flush=True)
    rng = np.random.default_rng(5)
    V, B = 6, 20000
    p1 = rng.standard_normal((2, V)).astype(np.float32)
    q1 = rng.standard_normal((1, V)).astype(np.float32)
    q0 = oracle.softmax64(q1[0])
    p = np.ascontiguousarray(np.broadcast_to(p1, (B, 2, V)))
    q = np.ascontiguousarray(np.broadcast_to(q1, (B, 1, V)))
    draft = rng.choice(V, size=(B, 1), p=q0).astype(np.int32)
    acc, toks, _, _ = run(p, q, draft, rng.random((B, 1)).astype(np.float32), rng.random(B).astype(np.float32))
    counts = np.bincount(toks[:, 0], minlength=V)
    p0 = oracle.softmax64(p1[0])
    sd = np.sqrt(B * p0 * (1 - p0))
    assert (np.abs(counts - B * p0) < 4 * sd).all(), (counts, B * p0)
