"""GPU parity of the second attention path (fp32 inputs at head dim 64 or
128, bf16 inputs at head dim 64): the tree-append kernel, then the
flash-attention kernel with key slices, against the oracle on every row,
with the same bounds as test_gpu_parity.py. The cases reach what that path
does differently from the head-dim-128 bf16 kernel: rounds of key slices
(an odd and an even count, slices past the last tile, a ragged last tile),
several row blocks of a KV head, the slices' merge, and its softmax
reference (raised only when a tile's max exceeds it by more than 8 log2
units; set from the first visible key)."""
import numpy as np
import pytest
import torch

import tree_attention_verification_tv_amd as tv
from tests.gpu_util import run_step, upload
from tests.test_gpu_parity import check_commit, check_step
from workloads import f32_to_bf16_bits, generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # bf16, head dim 64: 18 tiles (5 rounds of 4 slices, the last with two
    # idle slices), ragged prefixes, four row blocks per KV head
    (3, dict(B=3, prefix=(900, 1100), D=64)),
    # bf16, head dim 64, one KV head per query head (64 rows: one row block)
    (2, dict(prefix=700, D=64)),
    # fp32, head dim 64: 12 tiles = 6 rounds of 2 slices
    (1, dict(B=2, prefix=700)),
    # fp32, head dim 128, grouped heads: 5 tiles (one slice), two row blocks
    (1, dict(D=128, Hq=8, Hkv=2, B=2, prefix=(250, 300))),
    # prefixes that end a tile exactly, one shorter than a tile, none
    (3, dict(B=3, prefix=64, D=64, plen=[64, 10, 0])),
]


@pytest.mark.parametrize("cfg,over", CASES, ids=[f"cfg{c}-{i}" for i, (c, _) in enumerate(CASES)])
def test_against_oracle(cfg, over):
    print(f"[gpu] second path cfg={cfg} {over}", flush=True)
    over = dict(over)
    plen = over.pop("plen", None)
    w = generate(cfg, **over)
    if plen is not None:
        w.prefix_len[:] = plen
    d = upload(w, DEV)
    res = run_step(w, d)
    worst = check_step(w, res)
    check_commit(w, res, d["k_cache"], d["v_cache"])
    print(f"  attention error {worst:.3g}", flush=True)


@pytest.mark.parametrize("cfg", [3, 1])
def test_edge_cases_batch(cfg):
    """A normal tree, a single node, an inactive slot, a bad tree, a tree past
    the capacity and a sequence with no prefix in one batch."""
    print(f"[gpu] second path edge batch cfg={cfg}", flush=True)
    w = generate(cfg, B=6, prefix=40, D=64)
    w.n_nodes[1] = 1
    w.parents[1, 1:] = -1
    w.n_nodes[2] = 0
    w.parents[3, 3] = 4                 # parent after child: bad tree
    w.prefix_len[4] = w.cap - 2         # past the capacity
    w.prefix_len[5] = 0
    d = upload(w, DEV)
    res = run_step(w, d)
    assert res["err"].tolist() == [0, 0, 0, 2, 3, 0]
    check_step(w, res)
    check_commit(w, res, d["k_cache"], d["v_cache"])
    for b in (2, 3, 4):
        assert (res["out"][b] == 0).all(), b


def test_deep_chain_and_wide_star():
    print("[gpu] second path chain and star", flush=True)
    w = generate(2, B=2, prefix=130, D=64)
    w.parents[0] = [-1] + list(range(63))
    w.parents[1] = [-1] + [0] * 63
    d = upload(w, DEV)
    res = run_step(w, d)
    check_step(w, res)
    check_commit(w, res, d["k_cache"], d["v_cache"])


@pytest.mark.parametrize("cfg", [3, 1])
def test_scores_rising_across_tiles(cfg):
    """RoPE off; one KV head's queries are aligned with prefix keys whose
    magnitude grows with the slot, so later tiles' maxima exceed the
    reference by more than 8 log2 units and the running sums are rescaled
    (several times, and in every key slice). bf16: scores 0 .. ~58 log2
    units along the slots (~6 per tile); fp32: 0 .. ~17 (~2 per tile, two or
    three rescales), since an fp32 score of magnitude s carries an absolute
    rounding error of order s * 2^-24 * sqrt(D), which at s ~ 40 already
    spends the 1e-5 relative bound."""
    print(f"[gpu] second path rising scores cfg={cfg}", flush=True)
    w = generate(cfg, B=2, prefix=600, D=64)
    w.rope_theta = 0.0
    G = w.Hq // w.Hkv
    g = 1
    top = 10.0 if w.dtype == "bf16" else 3.0
    ramp = np.linspace(0.0, top, w.cap, dtype=np.float32)[:, None] * np.ones((1, w.D), dtype=np.float32)
    if w.dtype == "bf16":
        w.k_cache[:, g] = f32_to_bf16_bits(ramp[None])
        w.q[:, :, g * G:(g + 1) * G] = f32_to_bf16_bits(np.full((w.B, w.n_max, G, w.D), 0.5, dtype=np.float32))
    else:
        w.k_cache[:, g] = ramp[None]
        w.q[:, :, g * G:(g + 1) * G] = 0.5
    d = upload(w, DEV)
    res = run_step(w, d)
    check_step(w, res)
    check_commit(w, res, d["k_cache"], d["v_cache"])


@pytest.mark.parametrize("cfg", [3, 1])
def test_uniformly_low_scores(cfg):
    """Every score about -115 log2 units (RoPE off, queries -0.2, keys +50,
    head dim 64): the reference is set from the first visible key, so
    nothing underflows; ragged short prefixes."""
    print(f"[gpu] second path low scores cfg={cfg}", flush=True)
    w = generate(cfg, B=4, prefix=300, D=64)
    w.rope_theta = 0.0
    w.prefix_len[:] = [0, 5, 130, 300]
    if w.dtype == "bf16":
        w.q[:] = f32_to_bf16_bits(np.full(w.q.shape, -0.2, dtype=np.float32))
        w.k_cache[:] = f32_to_bf16_bits(np.full(w.k_cache.shape, 50.0, dtype=np.float32))
        w.k_new[:] = f32_to_bf16_bits(np.full(w.k_new.shape, 50.0, dtype=np.float32))
    else:
        w.q[:] = -0.2
        w.k_cache[:] = 50.0
        w.k_new[:] = 50.0
    d = upload(w, DEV)
    res = run_step(w, d)
    check_step(w, res)
    check_commit(w, res, d["k_cache"], d["v_cache"])
    assert np.isfinite(res["out"]).all() and np.abs(res["out"]).max() > 0.0


def test_repeated_calls_are_identical():
    w = generate(3, B=3, prefix=900, D=64)
    d = upload(w, DEV)
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    outs = []
    for _ in range(4):
        o = tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"],
                              d["n_nodes"], anc, depth, err, rope_theta=w.rope_theta)
        outs.append(o.view(torch.int16).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert not torch.equal(outs[0], torch.zeros_like(outs[0]))
