"""Helpers for the GPU parity tests: upload a workload, run one verification
step through the library, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tree_attention_verification_tv_amd as tv

BF16_ABS_TOL = 2e-2      # max abs error, bf16 inputs, fp32 accumulation
F32_ROW_REL_TOL = 1e-5   # max over rows of ||gpu - ref||_inf / ||ref||_inf, fp32 inputs


def to_dev(a: np.ndarray, dtype: str, dev) -> torch.Tensor:
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and a.dtype == np.uint16:
        x = x.view(torch.int16).view(torch.bfloat16)
    return x.to(dev)


def upload(w, dev="cuda:0") -> dict:
    """Device copies of a workload; V goes to the library's blocked layout."""
    d = {}
    for name in ("parents", "n_nodes", "prefix_len", "tok", "tgt", "q", "k_new", "v_new",
                 "k_cache", "v_cache"):
        d[name] = to_dev(getattr(w, name), w.dtype, dev)
    d["v_cache"] = tv.v_cache_blocked(d["v_cache"])
    return d


def run_step(w, d: dict, parents_override=None, n_nodes_override=None, prefix_override=None):
    """Tree set-up, attention, accept, commit; returns host copies of every
    intermediate plus the device caches."""
    parents = d["parents"] if parents_override is None else parents_override
    n_nodes = d["n_nodes"] if n_nodes_override is None else n_nodes_override
    plen = d["prefix_len"] if prefix_override is None else prefix_override
    anc, depth, err = tv.build_tree(parents, n_nodes)
    out = tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], plen,
                            n_nodes, anc, depth, err, rope_theta=w.rope_theta)
    k_after_attn = d["k_cache"].clone()
    v_after_attn = tv.v_cache_rows(d["v_cache"])
    acc, path, bonus, toks = tv.accept(d["tok"], d["tgt"], parents, anc, depth, n_nodes, err)
    new_plen = tv.commit(d["k_cache"], d["v_cache"], plen, acc, path)
    torch.cuda.synchronize()
    return dict(anc=anc.cpu().numpy().view(np.uint64), depth=depth.cpu().numpy(),
                err=err.cpu().numpy(), out=out.float().cpu().numpy().astype(np.float64),
                k_after_attn=k_after_attn, v_after_attn=v_after_attn,
                accept_len=acc.cpu().numpy(), path=path.cpu().numpy(), bonus=bonus.cpu().numpy(),
                out_tokens=toks.cpu().numpy(), prefix_len_out=new_plen.cpu().numpy())


def attention_error(dtype: str, got: np.ndarray, ref: np.ndarray) -> float:
    """Max abs error (bf16) or max row-relative error (fp32); a non-finite
    output counts as an infinite error."""
    if not np.isfinite(got).all():
        return float("inf")
    if dtype == "f32":
        num = np.abs(got - ref).max(axis=-1)
        den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
        return float((num / den).max())
    return float(np.abs(got - ref).max())


def tolerance(dtype: str) -> float:
    return F32_ROW_REL_TOL if dtype == "f32" else BF16_ABS_TOL


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
