"""tv_v_cache_layout on the GPU, through the C ABI: rows [n][cap][D] <->
blocked [n][cap/64][D][64], bit for bit against the addressing formula the
header states (checked element by element with NumPy index arithmetic) and
against the torch layout helpers; both dtypes, both head dims, dense caches
and page pools (cap 64), arbitrary bit patterns (NaNs included), and the
attention reading a cache converted by the library."""
import numpy as np
import pytest
import torch

import tree_attention_verification_tv_amd as tv
from tests.gpu_util import upload
from workloads import generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_bits(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    if dtype == torch.bfloat16:
        x = torch.randint(-32768, 32768, shape, dtype=torch.int32, generator=g).to(torch.int16)
        return x.view(torch.bfloat16).to(DEV)
    x = torch.randint(-(1 << 31), 1 << 31, shape, dtype=torch.int64, generator=g).to(torch.int32)
    return x.view(torch.float32).to(DEV)


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def check_formula(rows, blocked):
    """blocked holds rows[n, s, d] at flat index n*cap*D + ((s//64)*D + d)*64 + s%64."""
    r = bits(rows).cpu().numpy()
    bl = bits(blocked).cpu().numpy().reshape(-1)
    n, cap, D = r.shape[0] * (r.shape[1] if r.ndim == 4 else 1), r.shape[-2], r.shape[-1]
    r = r.reshape(n, cap, D)
    i, s, d = np.meshgrid(np.arange(n), np.arange(cap), np.arange(D), indexing="ij")
    flat = i * cap * D + ((s // 64) * D + d) * 64 + s % 64
    assert np.array_equal(bl[flat], r)


CASES = [(torch.bfloat16, 128, (3, 2, 192)), (torch.bfloat16, 64, (2, 3, 128)), (torch.float32, 128, (2, 2, 256)),
         (torch.float32, 64, (1, 5, 64)), (torch.bfloat16, 128, (37, 8, 64))]   # the last: a page pool


@pytest.mark.parametrize("dtype,D,lead_cap", CASES, ids=[f"{str(c[0])[6:]}-d{c[1]}-{c[2]}" for c in CASES])
def test_against_formula_and_helpers(dtype, D, lead_cap):
    print(f"[gpu] v cache layout {dtype} D={D} {lead_cap}", flush=True)
    a, b, cap = lead_cap
    rows = random_bits((a, b, cap, D), dtype, seed=cap + D)
    blocked = tv.v_cache_layout(rows)
    torch.cuda.synchronize()
    assert tuple(blocked.shape) == (a, b, cap // 64, D, 64)
    check_formula(rows, blocked)
    assert torch.equal(bits(blocked), bits(tv.v_cache_blocked(rows)))
    back = tv.v_cache_layout(blocked, to_rows=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(back), bits(rows))
    assert torch.equal(bits(back), bits(tv.v_cache_rows(blocked)))


def test_into_given_output_and_stream():
    """out= is written in place and nothing else; a side stream is honoured."""
    rows = random_bits((2, 2, 128, 128), torch.bfloat16, seed=5)
    out = torch.full((2, 2, 2, 128, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r = tv.v_cache_layout(rows, out=out, stream=s)
    s.synchronize()
    assert r.data_ptr() == out.data_ptr()
    assert torch.equal(bits(out), bits(tv.v_cache_blocked(rows)))


def test_headline_cache_and_attention():
    """The headline's V cache (8 sequences x 8 KV heads, 4096-token
    prefixes) in rows, converted by the library, gives the attention the same
    bytes as the torch helper; reports the conversion's bandwidth."""
    print("[gpu] v cache layout, headline cache", flush=True)
    w = generate(3)
    d = upload(w, DEV)
    rows = tv.v_cache_rows(d["v_cache"])
    blocked = tv.v_cache_layout(rows)
    torch.cuda.synchronize()
    assert torch.equal(bits(blocked), bits(d["v_cache"]))
    back = tv.v_cache_layout(blocked, to_rows=True)
    for _ in range(3):
        tv.v_cache_layout(rows, out=blocked)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        tv.v_cache_layout(rows, out=blocked)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 20
    nbytes = 2 * rows.numel() * rows.element_size()
    print(f"  {rows.numel() * 2 / 1e6:.1f} MB cache: {us:.1f} us per conversion, {nbytes / us / 1e3:.0f} GB/s", flush=True)
    assert torch.equal(bits(back), bits(rows))
    anc, depth, err = tv.build_tree(d["parents"], d["n_nodes"])
    kc = d["k_cache"].clone()
    out1 = tv.tree_attention(d["q"], d["k_new"], d["v_new"], kc, blocked, d["prefix_len"], d["n_nodes"], anc, depth,
                             err.clone(), rope_theta=w.rope_theta)
    out2 = tv.tree_attention(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["prefix_len"],
                             d["n_nodes"], anc, depth, err.clone(), rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(out2))
