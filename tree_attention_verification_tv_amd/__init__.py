"""Draft-tree verification for self-speculative decoding on MI355X (gfx950).

Thin Python binding of libtv.so (include/tv.h). Each function checks and
marshals torch tensors (device memory, current HIP stream) and calls the C
ABI; every step of the verification runs in the HIP kernels. There is no CPU
fallback: if the library is not built, the calls raise.

Step order for one verification pass of one layer:
    anc, depth, err = build_tree(parents, n_nodes)
    out = tree_attention(q, k_new, v_new, k_cache, v_cache, prefix_len,
                         n_nodes, anc, depth, err)
    accept_len, path, bonus, tokens = accept(cand_tok, tgt_argmax, parents,
                                             anc, depth, n_nodes, err)
      (or, from the target's logits: accept_typical(logits, cand_tok, parents,
       anc, depth, n_nodes, err, epsilon=..., delta=...))
    new_prefix_len = commit(k_cache, v_cache, prefix_len, accept_len, path)
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (PAGE, TV_BF16, TV_ERR_BAD_PAGE, TV_ERR_BAD_TREE, TV_ERR_CAPACITY, TV_F32,  # noqa: F401
                   TV_MAX_NODES, TvAttnArgs, TvError, TvPagedKv)

__all__ = ["build_tree", "tree_attention", "tree_attention_from_parents", "tree_attention_paged_from_parents",
           "tree_attention_noalloc", "accept_commit", "accept_commit_paged", "tree_attention_workspace_size",
           "new_workspace", "accept", "accept_typical", "commit", "eagle2_tree", "speculative_sample",
           "tree_attention_paged", "commit_paged", "pages_from_dense", "dense_from_pages", "TV_ERR_BAD_PAGE", "PAGE",
           "version", "TvError", "TV_ERR_BAD_TREE", "TV_ERR_CAPACITY", "attn_args",
           "v_cache_blocked", "v_cache_rows", "v_cache_layout", "V_BLOCK"]

V_BLOCK = 64   # slots per block of the V cache


def v_cache_blocked(v_rows: torch.Tensor) -> torch.Tensor:
    """Layout helper: V cache [B, Hkv, cap, D] (slot-major) -> the library's
    blocked layout [B, Hkv, cap/64, D, 64]. cap must be a multiple of 64."""
    B, H, cap, D = v_rows.shape
    if cap % V_BLOCK:
        raise ValueError("cap must be a multiple of 64")
    return v_rows.reshape(B, H, cap // V_BLOCK, V_BLOCK, D).transpose(-1, -2).contiguous()


def v_cache_rows(v_blocked: torch.Tensor) -> torch.Tensor:
    """Inverse of v_cache_blocked: [B, Hkv, cap/64, D, 64] -> [B, Hkv, cap, D]."""
    B, H, nb, D, blk = v_blocked.shape
    return v_blocked.transpose(-1, -2).reshape(B, H, nb * blk, D).contiguous()


def pages_from_dense(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                     num_pages: int, k_pool=None, v_pool=None):
    """Layout helper: writes dense caches (K [B, Hkv, cap, D], V blocked
    [B, Hkv, cap/64, D, 64]) into page pools K [num_pages, Hkv, 64, D] and
    V [num_pages, Hkv, D, 64] at the pages block_table [B, cap/64] names;
    pages no entry names are zero (or keep k_pool / v_pool's contents)."""
    B, H, cap, D = k_cache.shape
    mp = cap // PAGE
    if tuple(block_table.shape) != (B, mp):
        raise ValueError("block_table must be [B, cap/64]")
    if k_pool is None:
        k_pool = torch.zeros((num_pages, H, PAGE, D), dtype=k_cache.dtype, device=k_cache.device)
    if v_pool is None:
        v_pool = torch.zeros((num_pages, H, D, PAGE), dtype=v_cache.dtype, device=v_cache.device)
    idx = block_table.reshape(-1).long()
    k_pool.index_copy_(0, idx, k_cache.reshape(B, H, mp, PAGE, D).permute(0, 2, 1, 3, 4).reshape(B * mp, H, PAGE, D))
    v_pool.index_copy_(0, idx, v_cache.permute(0, 2, 1, 3, 4).reshape(B * mp, H, D, PAGE))
    return k_pool, v_pool


def dense_from_pages(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor):
    """Inverse of pages_from_dense: the dense caches (K [B, Hkv, cap, D], V
    blocked [B, Hkv, cap/64, D, 64]) that the pools and table stand for."""
    B, mp = block_table.shape
    idx = block_table.reshape(-1).long()
    _, H, _, D = k_pool.shape
    k = k_pool[idx].reshape(B, mp, H, PAGE, D).permute(0, 2, 1, 3, 4).reshape(B, H, mp * PAGE, D)
    v = v_pool[idx].reshape(B, mp, H, D, PAGE).permute(0, 2, 1, 3, 4).contiguous()
    return k.contiguous(), v


def version() -> str:
    return _lib.load().tv_version().decode()


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_DTYPES = {torch.float32: TV_F32, torch.bfloat16: TV_BF16}


def build_tree(parents: torch.Tensor, n_nodes: torch.Tensor, anc=None, depth=None, err=None,
               stream=None):
    """parents [B, n_max] int32, n_nodes [B] int32 -> (anc uint64 as int64
    [B, n_max], depth int32 [B, n_max], err int32 [B])."""
    lib = _lib.load()
    _dev(parents, "parents", torch.int32)
    _dev(n_nodes, "n_nodes", torch.int32)
    B, n_max = parents.shape
    dev = parents.device
    anc = torch.empty((B, n_max), dtype=torch.int64, device=dev) if anc is None else _dev(anc, "anc", torch.int64)
    depth = torch.empty((B, n_max), dtype=torch.int32, device=dev) if depth is None else _dev(depth, "depth", torch.int32)
    err = torch.empty((B,), dtype=torch.int32, device=dev) if err is None else _dev(err, "err", torch.int32)
    _lib.check("tv_build_tree", lib.tv_build_tree(_ptr(parents), _ptr(n_nodes), B, n_max, _ptr(anc),
                                                  _ptr(depth), _ptr(err), _stream(stream)))
    return anc, depth, err


def attn_args(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err, out,
              rope_theta=10000.0, softmax_scale=0.0, workspace=None, block_table=None) -> TvAttnArgs:
    """Checks the tensors of one tree_attention call and fills tv_attn_args
    (with block_table, k_cache and v_cache are the page pools)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float32 or bfloat16 (got {q.dtype})")
    dt = q.dtype
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("out", out)):
        _dev(t, name, dt)
    for name, t in (("prefix_len", prefix_len), ("n_nodes", n_nodes), ("depth", depth), ("err", err)):
        _dev(t, name, torch.int32)
    _dev(anc, "anc", torch.int64)
    B, n_max, Hq, D = q.shape
    Hkv = k_new.shape[2]
    if tuple(k_new.shape) != (B, n_max, Hkv, D) or tuple(v_new.shape) != (B, n_max, Hkv, D):
        raise ValueError("k_new / v_new must be [B, n_max, Hkv, D]")
    if block_table is None:
        cap = k_cache.shape[2]
        if cap % V_BLOCK:
            raise ValueError("cache capacity must be a multiple of 64")
        if tuple(k_cache.shape) != (B, Hkv, cap, D):
            raise ValueError("k_cache must be [B, Hkv, cap, D]")
        if tuple(v_cache.shape) != (B, Hkv, cap // V_BLOCK, D, V_BLOCK):
            raise ValueError("v_cache must be [B, Hkv, cap/64, D, 64] (see v_cache_blocked)")
    else:
        _dev(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        cap = block_table.shape[1] * PAGE
        n_pages = k_cache.shape[0]
        if tuple(k_cache.shape) != (n_pages, Hkv, PAGE, D):
            raise ValueError("k_pool must be [num_pages, Hkv, 64, D]")
        if tuple(v_cache.shape) != (n_pages, Hkv, D, PAGE):
            raise ValueError("v_pool must be [num_pages, Hkv, D, 64]")
    if tuple(out.shape) != (B, n_max, Hq, D):
        raise ValueError("out must be [B, n_max, Hq, D]")
    if tuple(anc.shape) != (B, n_max) or tuple(depth.shape) != (B, n_max):
        raise ValueError("anc / depth must be [B, n_max]")
    if prefix_len.numel() != B or n_nodes.numel() != B or err.numel() != B:
        raise ValueError("prefix_len / n_nodes / err must have B entries")
    a = TvAttnArgs()
    a.q, a.k_new, a.v_new = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr()
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.prefix_len, a.n_nodes = prefix_len.data_ptr(), n_nodes.data_ptr()
    a.anc, a.depth, a.err, a.out = anc.data_ptr(), depth.data_ptr(), err.data_ptr(), out.data_ptr()
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    else:
        a.workspace, a.workspace_bytes = None, 0
    a.B, a.n_max, a.Hq, a.Hkv, a.D, a.cap = B, n_max, Hq, Hkv, D, cap
    a.dtype = _DTYPES[dt]
    a.rope_theta = float(rope_theta)
    a.softmax_scale = float(softmax_scale)
    return a


def tree_attention_workspace_size(args: TvAttnArgs) -> int:
    return int(_lib.load().tv_tree_attention_workspace_size(ctypes.byref(args)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace for tree_attention: zero-filled, as the library requires
    before its first use (the calls leave its synchronisation words zero)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


_WORKSPACES: dict = {}


def _default_workspace(device, need: int, stream=None) -> torch.Tensor:
    """Per-device workspace shared by calls that pass none (calls on one
    device must then not overlap on different streams). When the kernels
    run on a stream other than the current one, the tensor is recorded on
    that stream, so that replacing it by a larger one cannot hand its memory
    to other work while the kernels still use it."""
    key = torch.device(device).index
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        ws = new_workspace(need, device)
        _WORKSPACES[key] = ws
    if stream is not None and stream != torch.cuda.current_stream(ws.device):
        ws.record_stream(stream)
    return ws


def tree_attention(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err,
                   rope_theta=10000.0, softmax_scale=0.0, out=None, workspace=None, stream=None):
    """Tree-masked attention of every node over prefix + ancestors; appends
    the rotated tree K and raw tree V to cache slots [P, P + n). Returns out
    [B, n_max, Hq, D] in the dtype of q."""
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    a = attn_args(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err, out,
                  rope_theta, softmax_scale, workspace)
    need = tree_attention_workspace_size(a)
    if need > a.workspace_bytes:
        if workspace is not None:
            raise ValueError(f"workspace holds {a.workspace_bytes} bytes, {need} needed")
        workspace = _default_workspace(q.device, need, stream)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check("tv_tree_attention", lib.tv_tree_attention(ctypes.byref(a), _stream(stream)))
    return out


def tree_attention_from_parents(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, parents,
                                rope_theta=10000.0, softmax_scale=0.0, out=None, workspace=None, stream=None):
    """build_tree and tree_attention in one launch (bf16; fp32 takes two):
    returns (out, anc, depth, err), bit for bit those of the two calls."""
    lib = _lib.load()
    _dev(parents, "parents", torch.int32)
    B, n_max = q.shape[0], q.shape[1]
    if tuple(parents.shape) != (B, n_max):
        raise ValueError("parents must be [B, n_max]")
    dev = q.device
    anc = torch.empty(B, n_max, dtype=torch.int64, device=dev)
    depth = torch.empty(B, n_max, dtype=torch.int32, device=dev)
    err = torch.empty(B, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    a = attn_args(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err, out,
                  rope_theta, softmax_scale, workspace)
    need = tree_attention_workspace_size(a)
    if need > a.workspace_bytes:
        if workspace is not None:
            raise ValueError(f"workspace holds {a.workspace_bytes} bytes, {need} needed")
        workspace = _default_workspace(q.device, need, stream)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check("tv_tree_attention_from_parents",
               lib.tv_tree_attention_from_parents(ctypes.byref(a), ctypes.c_void_p(parents.data_ptr()),
                                                  ctypes.c_void_p(anc.data_ptr()), ctypes.c_void_p(depth.data_ptr()),
                                                  _stream(stream)))
    return out, anc, depth, err


def tree_attention_noalloc(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err, out,
                           rope_theta=10000.0, softmax_scale=0.0, stream=None):
    """tree_attention through the allocation-free entry point: the library's
    static per-device scratch replaces the workspace, and out must be given
    (nothing is allocated). Calls on one device must not overlap."""
    lib = _lib.load()
    a = attn_args(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, anc, depth, err, out,
                  rope_theta, softmax_scale)
    _lib.check("tv_tree_attention_noalloc", lib.tv_tree_attention_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def paged_kv(block_table: torch.Tensor, k_pool: torch.Tensor) -> TvPagedKv:
    """tv_paged_kv for a block table [B, max_pages] over pools of k_pool's size."""
    _dev(block_table, "block_table", torch.int32)
    pk = TvPagedKv()
    pk.block_table = block_table.data_ptr()
    pk.max_pages = block_table.shape[1]
    pk.num_pages = k_pool.shape[0]
    return pk


def tree_attention_paged(q, k_new, v_new, k_pool, v_pool, block_table, prefix_len, n_nodes, anc, depth,
                         err, rope_theta=10000.0, softmax_scale=0.0, out=None, workspace=None,
                         stream=None):
    """tree_attention over a paged cache: k_pool [num_pages, Hkv, 64, D],
    v_pool [num_pages, Hkv, D, 64], block_table [B, max_pages] int32 (logical
    slot s of sequence b is slot s % 64 of page block_table[b, s // 64]).
    Appends the tree KV through the table; returns out [B, n_max, Hq, D]."""
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    a = attn_args(q, k_new, v_new, k_pool, v_pool, prefix_len, n_nodes, anc, depth, err, out,
                  rope_theta, softmax_scale, workspace, block_table=block_table)
    pk = paged_kv(block_table, k_pool)
    need = tree_attention_workspace_size(a)
    if need > a.workspace_bytes:
        if workspace is not None:
            raise ValueError(f"workspace holds {a.workspace_bytes} bytes, {need} needed")
        workspace = _default_workspace(q.device, need, stream)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check("tv_tree_attention_paged",
               lib.tv_tree_attention_paged(ctypes.byref(a), ctypes.byref(pk), _stream(stream)))
    return out


def tree_attention_paged_from_parents(q, k_new, v_new, k_pool, v_pool, block_table, prefix_len, n_nodes, parents,
                                      rope_theta=10000.0, softmax_scale=0.0, out=None, workspace=None, stream=None):
    """build_tree and tree_attention_paged in one launch: returns
    (out, anc, depth, err), bit for bit those of the two calls."""
    lib = _lib.load()
    _dev(parents, "parents", torch.int32)
    B, n_max = q.shape[0], q.shape[1]
    if tuple(parents.shape) != (B, n_max):
        raise ValueError("parents must be [B, n_max]")
    dev = q.device
    anc = torch.empty(B, n_max, dtype=torch.int64, device=dev)
    depth = torch.empty(B, n_max, dtype=torch.int32, device=dev)
    err = torch.empty(B, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(q)
    a = attn_args(q, k_new, v_new, k_pool, v_pool, prefix_len, n_nodes, anc, depth, err, out,
                  rope_theta, softmax_scale, workspace, block_table=block_table)
    pk = paged_kv(block_table, k_pool)
    need = tree_attention_workspace_size(a)
    if need > a.workspace_bytes:
        if workspace is not None:
            raise ValueError(f"workspace holds {a.workspace_bytes} bytes, {need} needed")
        workspace = _default_workspace(q.device, need, stream)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check("tv_tree_attention_paged_from_parents",
               lib.tv_tree_attention_paged_from_parents(ctypes.byref(a), ctypes.byref(pk),
                                                        ctypes.c_void_p(parents.data_ptr()),
                                                        ctypes.c_void_p(anc.data_ptr()),
                                                        ctypes.c_void_p(depth.data_ptr()), _stream(stream)))
    return out, anc, depth, err


def commit_paged(k_pool, v_pool, block_table, prefix_len_in, accept_len, path, prefix_len_out=None,
                 stream=None):
    """commit over a paged cache (layout as tree_attention_paged)."""
    lib = _lib.load()
    if k_pool.dtype not in _DTYPES:
        raise ValueError("pools must be float32 or bfloat16")
    _dev(k_pool, "k_pool", k_pool.dtype)
    _dev(v_pool, "v_pool", k_pool.dtype)
    for name, t in (("prefix_len_in", prefix_len_in), ("accept_len", accept_len), ("path", path)):
        _dev(t, name, torch.int32)
    n_pages, Hkv, _, D = k_pool.shape
    if tuple(v_pool.shape) != (n_pages, Hkv, D, PAGE):
        raise ValueError("v_pool must be [num_pages, Hkv, D, 64]")
    pk = paged_kv(block_table, k_pool)
    B, n_max = path.shape
    if prefix_len_out is None:
        prefix_len_out = torch.empty_like(prefix_len_in)
    _dev(prefix_len_out, "prefix_len_out", torch.int32)
    _lib.check("tv_commit_paged", lib.tv_commit_paged(_ptr(k_pool), _ptr(v_pool), ctypes.byref(pk), B, Hkv, D,
                                                      _DTYPES[k_pool.dtype], _ptr(prefix_len_in),
                                                      _ptr(accept_len), _ptr(path), n_max,
                                                      _ptr(prefix_len_out), _stream(stream)))
    return prefix_len_out


def accept(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err=None, accept_len=None, path=None,
           bonus=None, out_tokens=None, want_tokens=True, stream=None):
    """Greedy longest accepted path -> (accept_len [B], path [B, n_max],
    bonus [B], out_tokens [B, n_max] or None), all int32."""
    lib = _lib.load()
    for name, t in (("cand_tok", cand_tok), ("tgt_argmax", tgt_argmax), ("parents", parents),
                    ("depth", depth), ("n_nodes", n_nodes)):
        _dev(t, name, torch.int32)
    _dev(anc, "anc", torch.int64)
    if err is not None:
        _dev(err, "err", torch.int32)
    B, n_max = parents.shape
    dev = parents.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev) if path is None else path
    bonus = torch.empty(B, dtype=torch.int32, device=dev) if bonus is None else bonus
    if want_tokens and out_tokens is None:
        out_tokens = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    _lib.check("tv_accept", lib.tv_accept(_ptr(cand_tok), _ptr(tgt_argmax), _ptr(parents), _ptr(anc),
                                          _ptr(depth), _ptr(n_nodes), _ptr(err), B, n_max,
                                          _ptr(accept_len), _ptr(path), _ptr(bonus), _ptr(out_tokens),
                                          _stream(stream)))
    return accept_len, path, bonus, out_tokens


def eagle2_tree(conf, cand, root_tok, n_max: int, stream=None):
    """EAGLE-2 dynamic draft tree from the draft's proposals: conf [B, S, K, M]
    float32, cand [B, S, K, M] int32, root_tok [B] int32 -> (parents, tokens
    [B, n_max] int32, values [B, n_max] float32, n_nodes [B] int32), the
    parents-first tree that build_tree takes."""
    lib = _lib.load()
    _dev(conf, "conf", torch.float32)
    _dev(cand, "cand", torch.int32)
    _dev(root_tok, "root_tok", torch.int32)
    if conf.dim() != 4 or tuple(cand.shape) != tuple(conf.shape):
        raise ValueError("conf and cand must be [B, S, K, M]")
    B, S, K, M = conf.shape
    if root_tok.numel() != B:
        raise ValueError("root_tok must have B entries")
    dev = conf.device
    parents = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    tokens = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    values = torch.empty((B, n_max), dtype=torch.float32, device=dev)
    n_nodes = torch.empty(B, dtype=torch.int32, device=dev)
    _lib.check("tv_eagle2_tree", lib.tv_eagle2_tree(_ptr(conf), _ptr(cand), _ptr(root_tok), B, S, K, M, n_max,
                                                    _ptr(parents), _ptr(tokens), _ptr(values), _ptr(n_nodes),
                                                    _stream(stream)))
    return parents, tokens, values, n_nodes


def speculative_sample(p_logits, q_logits, draft, u_acc, u_res, stream=None):
    """Chain speculative sampling: p_logits [B, L+1, V], q_logits [B, L, V]
    (float32 or bfloat16, same dtype), draft [B, L] int32, u_acc [B, L] and
    u_res [B] float32 uniform draws -> (accept_len [B], tokens [B, L+1],
    p_tok [B, L], q_tok [B, L])."""
    lib = _lib.load()
    if p_logits.dtype not in _DTYPES:
        raise ValueError("logits must be float32 or bfloat16")
    _dev(p_logits, "p_logits", p_logits.dtype)
    _dev(q_logits, "q_logits", p_logits.dtype)
    _dev(draft, "draft", torch.int32)
    _dev(u_acc, "u_acc", torch.float32)
    _dev(u_res, "u_res", torch.float32)
    B, L = draft.shape
    V = p_logits.shape[-1]
    if tuple(p_logits.shape) != (B, L + 1, V) or tuple(q_logits.shape) != (B, L, V):
        raise ValueError("p_logits must be [B, L+1, V] and q_logits [B, L, V]")
    if tuple(u_acc.shape) != (B, L) or u_res.numel() != B:
        raise ValueError("u_acc must be [B, L] and u_res [B]")
    dev = draft.device
    ws = torch.empty(max(1, int(lib.tv_speculative_sample_workspace_size(B, L))), dtype=torch.uint8, device=dev)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    tokens = torch.empty((B, L + 1), dtype=torch.int32, device=dev)
    p_tok = torch.empty((B, L), dtype=torch.float32, device=dev)
    q_tok = torch.empty((B, L), dtype=torch.float32, device=dev)
    _lib.check("tv_speculative_sample", lib.tv_speculative_sample(
        _ptr(p_logits), _ptr(q_logits), _DTYPES[p_logits.dtype], V, _ptr(draft), _ptr(u_acc), _ptr(u_res), B, L,
        _ptr(p_tok), _ptr(q_tok), _ptr(accept_len), _ptr(tokens), _ptr(ws), ws.numel(), _stream(stream)))
    return accept_len, tokens, p_tok, q_tok


def accept_typical(logits, cand_tok, parents, anc, depth, n_nodes, err=None, *, epsilon: float,
                   delta: float, want_tokens=True, stream=None):
    """Typical acceptance from the target's logits [B, n_max, V] (float32 or
    bfloat16): a drafted token passes iff its probability under its parent's
    distribution exceeds min(epsilon, delta * exp(-H(parent))).

    Returns (accept_len [B], path [B, n_max], bonus [B], out_tokens [B, n_max]
    or None, entropy [B, n_max] float32, p_tok [B, n_max] float32,
    tgt_argmax [B, n_max] int32)."""
    lib = _lib.load()
    if logits.dtype not in _DTYPES:
        raise ValueError(f"logits must be float32 or bfloat16 (got {logits.dtype})")
    _dev(logits, "logits", logits.dtype)
    for name, t in (("cand_tok", cand_tok), ("parents", parents), ("depth", depth), ("n_nodes", n_nodes)):
        _dev(t, name, torch.int32)
    _dev(anc, "anc", torch.int64)
    if err is not None:
        _dev(err, "err", torch.int32)
    B, n_max = parents.shape
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (B, n_max):
        raise ValueError("logits must be [B, n_max, V]")
    V = logits.shape[2]
    dev = parents.device
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    accept_len, bonus = torch.empty(B, **i32), torch.empty(B, **i32)
    path, tgt_argmax = torch.empty((B, n_max), **i32), torch.empty((B, n_max), **i32)
    entropy, p_tok = torch.empty((B, n_max), **f32), torch.empty((B, n_max), **f32)
    out_tokens = torch.empty((B, n_max), **i32) if want_tokens else None
    _lib.check("tv_accept_typical", lib.tv_accept_typical(
        _ptr(logits), _DTYPES[logits.dtype], V, _ptr(cand_tok), _ptr(parents), _ptr(anc), _ptr(depth),
        _ptr(n_nodes), _ptr(err), B, n_max, float(epsilon), float(delta), _ptr(entropy), _ptr(p_tok),
        _ptr(tgt_argmax), _ptr(accept_len), _ptr(path), _ptr(bonus), _ptr(out_tokens), _stream(stream)))
    return accept_len, path, bonus, out_tokens, entropy, p_tok, tgt_argmax


def v_cache_layout(src, to_rows=False, out=None, stream=None):
    """tv_v_cache_layout on the GPU: a V cache in rows [..., cap, D] ->
    blocked [..., cap/64, D, 64] (to_rows False), or blocked -> rows
    (to_rows True); the leading dims ([B, Hkv], or [num_pages, Hkv] with
    cap 64) flatten to n. Returns out (allocated when None)."""
    lib = _lib.load()
    if src.dtype not in _DTYPES:
        raise ValueError("V cache must be float32 or bfloat16")
    _dev(src, "src", src.dtype)
    if to_rows:
        if src.dim() < 3 or src.shape[-1] != V_BLOCK:
            raise ValueError("blocked V must be [..., cap/64, D, 64]")
        lead, nb, D = tuple(src.shape[:-3]), src.shape[-3], src.shape[-2]
        cap, shape = nb * V_BLOCK, tuple(src.shape[:-3]) + (nb * V_BLOCK, src.shape[-2])
    else:
        if src.dim() < 2 or src.shape[-2] % V_BLOCK:
            raise ValueError("V rows must be [..., cap, D] with cap a multiple of 64")
        lead, cap, D = tuple(src.shape[:-2]), src.shape[-2], src.shape[-1]
        shape = lead + (cap // V_BLOCK, D, V_BLOCK)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    _dev(out, "out", src.dtype)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {list(shape)}")
    n = 1
    for x in lead:
        n *= x
    _lib.check("tv_v_cache_layout", lib.tv_v_cache_layout(_ptr(src), _ptr(out), n, cap, D, _DTYPES[src.dtype],
                                                          1 if to_rows else 0, _stream(stream)))
    return out


def commit(k_cache, v_cache, prefix_len_in, accept_len, path, prefix_len_out=None, stream=None):
    """Moves the accepted path's KV to slots [P, P + L + 1) in place (k_cache
    [B, Hkv, cap, D], v_cache [B, Hkv, cap/64, D, 64]); returns the new prefix
    lengths (prefix_len_out, which may be prefix_len_in)."""
    lib = _lib.load()
    if k_cache.dtype not in _DTYPES:
        raise ValueError("cache must be float32 or bfloat16")
    _dev(k_cache, "k_cache", k_cache.dtype)
    _dev(v_cache, "v_cache", k_cache.dtype)
    for name, t in (("prefix_len_in", prefix_len_in), ("accept_len", accept_len), ("path", path)):
        _dev(t, name, torch.int32)
    B, Hkv, cap, D = k_cache.shape
    if tuple(v_cache.shape) != (B, Hkv, cap // V_BLOCK, D, V_BLOCK):
        raise ValueError("v_cache must be [B, Hkv, cap/64, D, 64]")
    n_max = path.shape[1]
    if prefix_len_out is None:
        prefix_len_out = torch.empty_like(prefix_len_in)
    _dev(prefix_len_out, "prefix_len_out", torch.int32)
    _lib.check("tv_commit", lib.tv_commit(_ptr(k_cache), _ptr(v_cache), B, Hkv, cap, D,
                                          _DTYPES[k_cache.dtype], _ptr(prefix_len_in), _ptr(accept_len),
                                          _ptr(path), n_max, _ptr(prefix_len_out), _stream(stream)))
    return prefix_len_out


def accept_commit(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err, k_cache, v_cache, prefix_len_in,
                  prefix_len_out=None, want_tokens=True, stream=None):
    """accept followed by commit in one launch (dense cache): returns
    (accept_len, path, bonus, out_tokens or None, prefix_len_out)."""
    lib = _lib.load()
    for name, t in (("cand_tok", cand_tok), ("tgt_argmax", tgt_argmax), ("parents", parents),
                    ("depth", depth), ("n_nodes", n_nodes), ("prefix_len_in", prefix_len_in)):
        _dev(t, name, torch.int32)
    _dev(anc, "anc", torch.int64)
    if err is not None:
        _dev(err, "err", torch.int32)
    if k_cache.dtype not in _DTYPES:
        raise ValueError("cache must be float32 or bfloat16")
    _dev(k_cache, "k_cache", k_cache.dtype)
    _dev(v_cache, "v_cache", k_cache.dtype)
    B, n_max = parents.shape
    Bc, Hkv, cap, D = k_cache.shape
    if Bc != B or tuple(v_cache.shape) != (B, Hkv, cap // V_BLOCK, D, V_BLOCK):
        raise ValueError("k_cache must be [B, Hkv, cap, D] and v_cache [B, Hkv, cap/64, D, 64]")
    dev = parents.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    out_tokens = torch.empty((B, n_max), dtype=torch.int32, device=dev) if want_tokens else None
    if prefix_len_out is None:
        prefix_len_out = torch.empty_like(prefix_len_in)
    _dev(prefix_len_out, "prefix_len_out", torch.int32)
    _lib.check("tv_accept_commit", lib.tv_accept_commit(
        _ptr(cand_tok), _ptr(tgt_argmax), _ptr(parents), _ptr(anc), _ptr(depth), _ptr(n_nodes), _ptr(err), B, n_max,
        _ptr(accept_len), _ptr(path), _ptr(bonus), _ptr(out_tokens), _ptr(k_cache), _ptr(v_cache), Hkv, cap, D,
        _DTYPES[k_cache.dtype], _ptr(prefix_len_in), _ptr(prefix_len_out), _stream(stream)))
    return accept_len, path, bonus, out_tokens, prefix_len_out


def accept_commit_paged(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err, k_pool, v_pool, block_table,
                        prefix_len_in, prefix_len_out=None, want_tokens=True, stream=None):
    """accept followed by commit_paged in one launch (pools and table as
    tree_attention_paged): returns (accept_len, path, bonus, out_tokens or
    None, prefix_len_out)."""
    lib = _lib.load()
    for name, t in (("cand_tok", cand_tok), ("tgt_argmax", tgt_argmax), ("parents", parents),
                    ("depth", depth), ("n_nodes", n_nodes), ("prefix_len_in", prefix_len_in)):
        _dev(t, name, torch.int32)
    _dev(anc, "anc", torch.int64)
    if err is not None:
        _dev(err, "err", torch.int32)
    if k_pool.dtype not in _DTYPES:
        raise ValueError("pools must be float32 or bfloat16")
    _dev(k_pool, "k_pool", k_pool.dtype)
    _dev(v_pool, "v_pool", k_pool.dtype)
    n_pages, Hkv, _, D = k_pool.shape
    if tuple(v_pool.shape) != (n_pages, Hkv, D, PAGE):
        raise ValueError("v_pool must be [num_pages, Hkv, D, 64]")
    pk = paged_kv(block_table, k_pool)
    B, n_max = parents.shape
    dev = parents.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    out_tokens = torch.empty((B, n_max), dtype=torch.int32, device=dev) if want_tokens else None
    if prefix_len_out is None:
        prefix_len_out = torch.empty_like(prefix_len_in)
    _dev(prefix_len_out, "prefix_len_out", torch.int32)
    _lib.check("tv_accept_commit_paged", lib.tv_accept_commit_paged(
        _ptr(cand_tok), _ptr(tgt_argmax), _ptr(parents), _ptr(anc), _ptr(depth), _ptr(n_nodes), _ptr(err), B, n_max,
        _ptr(accept_len), _ptr(path), _ptr(bonus), _ptr(out_tokens), _ptr(k_pool), _ptr(v_pool), ctypes.byref(pk),
        Hkv, D, _DTYPES[k_pool.dtype], _ptr(prefix_len_in), _ptr(prefix_len_out), _stream(stream)))
    return accept_len, path, bonus, out_tokens, prefix_len_out
