"""The allocation-free attention entry point (tv_tree_attention_noalloc)
against the allocating one (tv_tree_attention) through the C ABI: same
outputs and the same appended cache, bit for bit, on calls in a row (the
headline batch, then a smaller one, then the ragged serving batch, whose
unfused split plan uses the most scratch, then fp32), and the host-side
rejection of shapes beyond the static scratch."""
import ctypes

import numpy as np
import pytest
import torch

import tree_attention_verification_tv_amd as tv
from tree_attention_verification_tv_amd import _lib
from tests.gpu_util import upload
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(w, noalloc: bool):
    d = upload(w, DEV)
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    out = torch.empty_like(d["q"])
    if noalloc:
        tv.tree_attention_noalloc(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"],
                                  d["n_nodes"], anc, depth, err, out, rope_theta=w.rope_theta)
    else:
        a = tv.attn_args(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"],
                         d["n_nodes"], anc, depth, err, out, w.rope_theta)
        ws = tv.new_workspace(tv.tree_attention_workspace_size(a), DEV)
        tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"], d["n_nodes"],
                          anc, depth, err, rope_theta=w.rope_theta, out=out, workspace=ws)
    torch.cuda.synchronize()
    return out, d["k_cache"], d["v_cache"], err


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CALLS = [(3, {}), (3, dict(B=2, prefix=1100)), (5, {}), (1, {})]


@pytest.mark.parametrize("cfg,over", CALLS, ids=["headline", "smaller", "serving", "fp32"])
def test_noalloc_equals_allocating_entry_point(cfg, over):
    print(f"[gpu] allocation-free attention cfg={cfg} {over}", flush=True)
    w = generate(cfg, **over)
    ref = _run(w, noalloc=False)
    got = _run(w, noalloc=True)
    # the same kernels and plan: identical bits (so within any tolerance)
    assert torch.equal(_bits(got[0]), _bits(ref[0])), "attention output"
    assert torch.equal(_bits(got[1]), _bits(ref[1])), "K cache after the tree append"
    assert torch.equal(_bits(got[2]), _bits(ref[2])), "V cache after the tree append"
    assert torch.equal(got[3], ref[3]), "error codes"
    err = float((got[0].float() - ref[0].float()).abs().max())
    assert err <= (2e-2 if w.dtype == "bf16" else 0.0)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A plan whose workspace exceeds the static scratch is refused on the
    host (no device work): 32 sequences x 8 KV heads x two row blocks of
    256 rows, two key splits (about 71 MB of partials)."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    a = _lib.TvAttnArgs()
    for name in ("q", "k_new", "v_new", "k_cache", "v_cache", "prefix_len", "n_nodes", "anc", "depth", "err", "out"):
        setattr(a, name, fake.value)
    a.B, a.n_max, a.Hq, a.Hkv, a.D, a.cap, a.dtype = 32, 64, 64, 8, 128, 4096, _lib.TV_BF16
    a.rope_theta, a.softmax_scale = 10000.0, 0.0
    assert lib.tv_tree_attention_workspace_size(ctypes.byref(a)) > 48 << 20
    assert lib.tv_tree_attention_noalloc(ctypes.byref(a), None) == _lib.TV_ERR_SCRATCH
