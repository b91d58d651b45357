"""The C ABI library: it loads, exports every symbol include/tv.h declares,
and rejects bad arguments on the host before any device call."""
import ctypes
import os
import re

import pytest

from tree_attention_verification_tv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libtv.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_calls():
    names = declared_functions()
    for must in ("tv_build_tree", "tv_tree_attention", "tv_accept", "tv_commit", "tv_accept_typical",
                 "tv_tree_attention_paged", "tv_commit_paged", "tv_eagle2_tree", "tv_speculative_sample",
                 "tv_tree_attention_paged_from_parents", "tv_accept_commit_paged", "tv_v_cache_layout"):
        assert must in names


def test_every_declared_symbol_is_exported_and_bound():
    lib = _lib.load()
    names = declared_functions()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.tv_version().decode().startswith("tv ")
    for code in range(8):
        assert lib.tv_status_string(code)
    assert lib.tv_status_string(_lib.TV_ERR_SCRATCH).decode().startswith("shapes need more scratch")
    assert lib.tv_status_string(_lib.TV_ERR_BAD_PAGE).decode().startswith("block table")
    assert lib.tv_status_string(_lib.TV_ERR_CAPACITY).decode().startswith("prefix")


def test_struct_layout_matches_header_order():
    # pointers first, then size_t, then the int32 / float fields
    offs = [f[0] for f in _lib.TvAttnArgs._fields_]
    assert offs[0] == "q" and offs[-1] == "softmax_scale"
    assert ctypes.sizeof(_lib.TvAttnArgs) == 12 * 8 + 8 + 7 * 4 + 2 * 4 + 4  # padded to 8


def test_host_validation_without_device():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its checks
    null = None
    # build_tree
    assert lib.tv_build_tree(fake, fake, -1, 5, fake, fake, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_build_tree(fake, fake, 1, 0, fake, fake, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_build_tree(fake, fake, 1, 65, fake, fake, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_build_tree(null, fake, 1, 5, fake, fake, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_build_tree(null, null, 0, 5, null, null, null, null) == _lib.TV_OK   # empty batch
    # accept
    assert lib.tv_accept(fake, fake, fake, fake, fake, fake, null, 1, 70, fake, fake, fake, null,
                         null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_accept(fake, fake, fake, fake, fake, fake, null, 1, 5, null, fake, fake, null,
                         null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_accept(null, null, null, null, null, null, null, 0, 5, null, null, null, null,
                         null) == _lib.TV_OK
    # typical acceptance: B, n_max, vocab, dtype, thresholds, pointers
    def typ(B=1, n_max=5, V=32000, dtype=_lib.TV_BF16, eps=0.09, delta=0.3, logits=fake, ent=fake):
        return lib.tv_accept_typical(logits, dtype, V, fake, fake, fake, fake, fake, null, B, n_max,
                                     eps, delta, ent, fake, fake, fake, fake, fake, null, null)
    assert typ(B=-1) == _lib.TV_ERR_INVALID_ARG
    assert typ(B=70000) == _lib.TV_ERR_INVALID_ARG
    assert typ(n_max=0) == _lib.TV_ERR_INVALID_ARG
    assert typ(n_max=65) == _lib.TV_ERR_INVALID_ARG
    assert typ(V=0) == _lib.TV_ERR_INVALID_ARG
    assert typ(dtype=3) == _lib.TV_ERR_INVALID_ARG
    assert typ(eps=float("nan")) == _lib.TV_ERR_INVALID_ARG
    assert typ(delta=float("nan")) == _lib.TV_ERR_INVALID_ARG
    assert typ(logits=null) == _lib.TV_ERR_INVALID_ARG
    assert typ(ent=null) == _lib.TV_ERR_INVALID_ARG
    assert typ(B=0, logits=null, ent=null) == _lib.TV_OK
    # commit
    assert lib.tv_commit(fake, fake, 1, 0, 10, 128, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit(fake, fake, 1, 2, 4, 128, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit(fake, fake, 1, 2, 100, 128, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit(fake, fake, 1, 2, 64, 96, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_UNSUPPORTED
    assert lib.tv_commit(fake, fake, 1, 2, 64, 128, 7, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit(null, fake, 1, 2, 64, 128, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG


def attn(**kw):
    a = _lib.TvAttnArgs()
    for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "prefix_len", "n_nodes", "anc", "depth",
              "err", "out"):
        setattr(a, f, 0x1000)
    a.B, a.n_max, a.Hq, a.Hkv, a.D, a.cap, a.dtype = 8, 60, 32, 8, 128, 4160, _lib.TV_BF16
    a.rope_theta, a.softmax_scale = 10000.0, 0.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_attention_host_validation_and_workspace():
    lib = _lib.load()
    run = lambda a: lib.tv_tree_attention(ctypes.byref(a), None)   # noqa: E731
    assert lib.tv_tree_attention(None, None) == _lib.TV_ERR_INVALID_ARG
    assert run(attn(Hq=30)) == _lib.TV_ERR_INVALID_ARG           # Hq % Hkv
    assert run(attn(n_max=65)) == _lib.TV_ERR_INVALID_ARG
    assert run(attn(cap=10)) == _lib.TV_ERR_INVALID_ARG
    assert run(attn(cap=4156)) == _lib.TV_ERR_INVALID_ARG        # V blocks of 64 slots
    assert run(attn(D=96)) == _lib.TV_ERR_UNSUPPORTED            # head dim 64 or 128
    assert run(attn(dtype=_lib.TV_F32, D=96)) == _lib.TV_ERR_UNSUPPORTED
    assert run(attn(dtype=9)) == _lib.TV_ERR_INVALID_ARG
    assert run(attn(q=None)) == _lib.TV_ERR_INVALID_ARG
    assert run(attn(B=0)) == _lib.TV_OK
    # the headline shape splits the prefix, so it needs a workspace
    need = lib.tv_tree_attention_workspace_size(ctypes.byref(attn()))
    assert need > 0
    assert run(attn(workspace=0x1000, workspace_bytes=need - 1)) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_workspace_size(ctypes.byref(attn(dtype=_lib.TV_F32))) == 0
    assert lib.tv_tree_attention_workspace_size(ctypes.byref(attn(Hq=30))) == 0


def test_paged_host_validation():
    lib = _lib.load()
    null = None

    def pk(max_pages=65, num_pages=100, table=0x2000):
        p = _lib.TvPagedKv()
        p.block_table, p.max_pages, p.num_pages = table, max_pages, num_pages
        return p

    def call(a, p):
        return lib.tv_tree_attention_paged(ctypes.byref(a), None if p is None else ctypes.byref(p), null)
    ok_args = attn(cap=65 * 64, workspace=0x3000, workspace_bytes=1 << 40)
    assert call(ok_args, None) == _lib.TV_ERR_INVALID_ARG                    # no table struct
    assert call(ok_args, pk(table=0)) == _lib.TV_ERR_INVALID_ARG            # null table
    assert call(ok_args, pk(max_pages=0)) == _lib.TV_ERR_INVALID_ARG
    assert call(ok_args, pk(num_pages=0)) == _lib.TV_ERR_INVALID_ARG
    assert call(attn(cap=64 * 64), pk()) == _lib.TV_ERR_INVALID_ARG        # cap != 64 max_pages
    assert call(attn(cap=300 * 64), pk(max_pages=300)) == _lib.TV_ERR_UNSUPPORTED   # > 256 pages
    assert call(attn(cap=65 * 64, dtype=_lib.TV_F32, D=64), pk()) == _lib.TV_ERR_UNSUPPORTED
    assert call(attn(cap=65 * 64, B=0), pk()) == _lib.TV_OK
    fake = ctypes.c_void_p(0x1000)
    p = pk()
    assert lib.tv_commit_paged(fake, fake, None, 1, 2, 128, 1, fake, fake, fake, 5, fake, null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit_paged(fake, fake, ctypes.byref(pk(table=0)), 1, 2, 128, 1, fake, fake, fake, 5, fake,
                               null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit_paged(fake, fake, ctypes.byref(p), 1, 2, 96, 1, fake, fake, fake, 5, fake,
                               null) == _lib.TV_ERR_UNSUPPORTED
    assert lib.tv_commit_paged(null, fake, ctypes.byref(p), 1, 2, 128, 1, fake, fake, fake, 5, fake,
                               null) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_commit_paged(null, null, ctypes.byref(p), 0, 2, 128, 1, null, null, null, 5, null,
                               null) == _lib.TV_OK


def test_eagle2_tree_host_validation():
    lib = _lib.load()
    f, null = ctypes.c_void_p(0x1000), None

    def call(B=2, S=6, K=8, M=8, n=60, conf=f):
        return lib.tv_eagle2_tree(conf, f, f, B, S, K, M, n, f, f, f, f, null)
    assert call(B=-1) == _lib.TV_ERR_INVALID_ARG
    assert call(S=0) == _lib.TV_ERR_INVALID_ARG
    assert call(K=0) == _lib.TV_ERR_INVALID_ARG
    assert call(M=0) == _lib.TV_ERR_INVALID_ARG
    assert call(n=0) == _lib.TV_ERR_INVALID_ARG
    assert call(n=65) == _lib.TV_ERR_INVALID_ARG
    assert call(S=7, K=8, M=10) == _lib.TV_ERR_UNSUPPORTED      # 560 proposals > 512
    assert call(conf=null) == _lib.TV_ERR_INVALID_ARG
    assert call(B=0, conf=null) == _lib.TV_OK


def test_speculative_sample_host_validation():
    lib = _lib.load()
    f, null = ctypes.c_void_p(0x1000), None
    ws = lib.tv_speculative_sample_workspace_size(8, 5)
    assert ws == 8 * 11 * 2 * 4
    assert lib.tv_speculative_sample_workspace_size(0, 5) == 0

    def call(B=8, L=5, V=32000, dtype=_lib.TV_BF16, p=f, wsb=ws):
        return lib.tv_speculative_sample(p, f, dtype, V, f, f, f, B, L, f, f, f, f, f, wsb, null)
    assert call(B=-1) == _lib.TV_ERR_INVALID_ARG
    assert call(L=0) == _lib.TV_ERR_INVALID_ARG
    assert call(L=65) == _lib.TV_ERR_INVALID_ARG
    assert call(V=0) == _lib.TV_ERR_INVALID_ARG
    assert call(dtype=9) == _lib.TV_ERR_INVALID_ARG
    assert call(p=null) == _lib.TV_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == _lib.TV_ERR_INVALID_ARG
    assert call(B=0, p=null) == _lib.TV_OK


def test_noalloc_host_validation_without_device():
    """The allocation-free attention entry point checks like tv_tree_attention
    and refuses, before any device call, shapes whose workspace exceeds its
    static scratch."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)

    def args(**kw):
        a = _lib.TvAttnArgs()
        for name in ("q", "k_new", "v_new", "k_cache", "v_cache", "prefix_len", "n_nodes", "anc", "depth",
                     "err", "out"):
            setattr(a, name, fake.value)
        a.B, a.n_max, a.Hq, a.Hkv, a.D, a.cap, a.dtype = 8, 60, 32, 8, 128, 4160, _lib.TV_BF16
        a.rope_theta, a.softmax_scale = 10000.0, 0.0
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    assert lib.tv_tree_attention_noalloc(None, None) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_noalloc(ctypes.byref(args(n_max=0)), None) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_noalloc(ctypes.byref(args(Hq=30)), None) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_noalloc(ctypes.byref(args(cap=4100)), None) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_noalloc(ctypes.byref(args(q=None)), None) == _lib.TV_ERR_INVALID_ARG
    assert lib.tv_tree_attention_noalloc(ctypes.byref(args(B=0, q=None)), None) == _lib.TV_OK
    # 32 sequences x 8 KV heads x two row blocks, two key splits: about 68 MiB
    big = args(B=32, n_max=64, Hq=64, cap=4096)
    assert lib.tv_tree_attention_workspace_size(ctypes.byref(big)) > 48 << 20
    assert lib.tv_tree_attention_noalloc(ctypes.byref(big), None) == _lib.TV_ERR_SCRATCH


def test_accept_commit_host_validation_without_device():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    null = None

    def call(B=1, n_max=5, Hkv=8, cap=128, D=128, dtype=_lib.TV_BF16, k=fake, plen_out=fake):
        return lib.tv_accept_commit(fake, fake, fake, fake, fake, fake, null, B, n_max, fake, fake, fake, null, k,
                                    fake, Hkv, cap, D, dtype, fake, plen_out, null)
    assert call(B=-1) == _lib.TV_ERR_INVALID_ARG
    assert call(n_max=0) == _lib.TV_ERR_INVALID_ARG
    assert call(n_max=65) == _lib.TV_ERR_INVALID_ARG
    assert call(Hkv=0) == _lib.TV_ERR_INVALID_ARG
    assert call(cap=100) == _lib.TV_ERR_INVALID_ARG
    assert call(cap=4) == _lib.TV_ERR_INVALID_ARG
    assert call(dtype=7) == _lib.TV_ERR_INVALID_ARG
    assert call(D=96) == _lib.TV_ERR_UNSUPPORTED
    assert call(k=None) == _lib.TV_ERR_INVALID_ARG
    assert call(plen_out=None) == _lib.TV_ERR_INVALID_ARG
    assert call(B=0, k=None) == _lib.TV_OK


def test_paged_fused_host_validation_without_device():
    """tv_tree_attention_paged_from_parents and tv_accept_commit_paged: the
    checks of their separate calls, no device needed."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    null = None

    def pk(max_pages=65, num_pages=100, table=0x2000):
        p = _lib.TvPagedKv()
        p.block_table, p.max_pages, p.num_pages = table, max_pages, num_pages
        return p

    def attn_call(a, p, parents=fake, anc=fake, depth=fake):
        return lib.tv_tree_attention_paged_from_parents(ctypes.byref(a), None if p is None else ctypes.byref(p),
                                                        parents, anc, depth, null)
    ok_args = attn(cap=65 * 64, workspace=0x3000, workspace_bytes=1 << 40)
    assert attn_call(ok_args, None) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(ok_args, pk(table=0)) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(ok_args, pk(num_pages=0)) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(attn(cap=64 * 64), pk()) == _lib.TV_ERR_INVALID_ARG          # cap != 64 max_pages
    assert attn_call(attn(cap=300 * 64), pk(max_pages=300)) == _lib.TV_ERR_UNSUPPORTED
    assert attn_call(attn(cap=65 * 64, dtype=_lib.TV_F32, D=64), pk()) == _lib.TV_ERR_UNSUPPORTED
    assert attn_call(ok_args, pk(), parents=None) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(ok_args, pk(), anc=None) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(ok_args, pk(), depth=None) == _lib.TV_ERR_INVALID_ARG
    assert attn_call(attn(cap=65 * 64, B=0), pk(), parents=None) == _lib.TV_OK

    def ac_call(p, B=1, n_max=5, Hkv=8, D=128, dtype=_lib.TV_BF16, k=fake, plen_out=fake):
        return lib.tv_accept_commit_paged(fake, fake, fake, fake, fake, fake, null, B, n_max, fake, fake, fake, null,
                                          k, fake, None if p is None else ctypes.byref(p), Hkv, D, dtype, fake,
                                          plen_out, null)
    assert ac_call(None) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(table=0)) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(max_pages=0)) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(num_pages=0)) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), B=-1) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), n_max=65) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(max_pages=1, num_pages=1), n_max=65) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), Hkv=0) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), dtype=7) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), D=96) == _lib.TV_ERR_UNSUPPORTED
    assert ac_call(pk(max_pages=300)) == _lib.TV_ERR_UNSUPPORTED
    assert ac_call(pk(), k=None) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), plen_out=None) == _lib.TV_ERR_INVALID_ARG
    assert ac_call(pk(), B=0, k=None) == _lib.TV_OK


def test_v_cache_layout_host_validation_without_device():
    """Every rejection of tv_v_cache_layout happens before any HIP call; no
    case below reaches a launch (a call that passes every check would)."""
    lib = _lib.load()
    a, b = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000000)   # never dereferenced
    BF16, F32 = _lib.TV_BF16, _lib.TV_F32

    def call(src=a, dst=b, n=16, cap=128, D=128, dtype=BF16, to_rows=0):
        return lib.tv_v_cache_layout(src, dst, n, cap, D, dtype, to_rows, None)
    assert call(n=-1) == _lib.TV_ERR_INVALID_ARG
    assert call(cap=0) == _lib.TV_ERR_INVALID_ARG
    assert call(cap=100) == _lib.TV_ERR_INVALID_ARG
    assert call(to_rows=2) == _lib.TV_ERR_INVALID_ARG
    assert call(dtype=7) == _lib.TV_ERR_INVALID_ARG
    assert call(D=96) == _lib.TV_ERR_UNSUPPORTED
    assert call(n=0) == _lib.TV_OK                                   # nothing to do, no launch
    assert call(n=1 << 31, cap=64) == _lib.TV_ERR_UNSUPPORTED         # more than 2^31 - 1 blocks
    assert call(src=None) == _lib.TV_ERR_INVALID_ARG
    assert call(dst=None) == _lib.TV_ERR_INVALID_ARG
    assert call(src=ctypes.c_void_p(0x10008)) == _lib.TV_ERR_INVALID_ARG   # not 16-byte aligned
    assert call(dst=a) == _lib.TV_ERR_INVALID_ARG                     # in place
    # 16 * 128 * 128 bf16 = 512 KiB: a buffer starting inside the other overlaps it
    assert call(dst=ctypes.c_void_p(0x10000 + 0x7fff0)) == _lib.TV_ERR_INVALID_ARG
    assert call(src=ctypes.c_void_p(0x20000000 + 0x70000), dtype=F32) == _lib.TV_ERR_INVALID_ARG


def test_no_kernel_spills_registers():
    """Every kernel of the built library has a zero private segment: no
    register spills. The attention kernels issue register loads from inline
    assembly and wait for them by hand, so a spill between such a load and
    its wait would store a value that has not arrived (the build refuses
    such a library; this checks the library that is there)."""
    from tree_attention_verification_tv_amd.build import kernel_private_segments
    seg = kernel_private_segments(_lib.LIB_PATH)
    assert sum("attn_bf16_kernel" in k for k in seg) == 16, sorted(seg)
    assert len(seg) >= 50, len(seg)
    assert {k: v for k, v in seg.items() if v} == {}
