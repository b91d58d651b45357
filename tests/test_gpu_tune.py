"""GPU parity of the bf16 attention under launch plans the automatic choice
does not take on the test workloads (TV_ATTN_TUNE: wavefronts per workgroup,
query tiles per wavefront, key splits). The library reads the override once
per process, so each plan runs in a child process of its own, one at a
time, on the same small cases as the full-parity tests, against the oracle
at the same tolerance. Results do not depend on the plan beyond rounding
order."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (cfg, overrides) from the full-parity list: 64, 240 and 512 rows per KV
# head, a ragged tail and ragged prefixes
CASES = [(2, dict(prefix=300)), (3, dict(B=2, prefix=1100)), (4, dict(B=2, prefix=200)),
         (5, dict(B=6, prefix=(16, 300)))]
# fused=0: the separate merge kernel on plans the automatic choice merges in
# the kernel; splits=2 / 4: the fused merge with two and four splits;
# fused=2: the fused merge in which only the last split to arrive merges;
# splits=3 / 6: split counts that do not divide the merge's items (the last
# range takes the rest); splits 6 and 8 with fused=1: the fused merge for
# five to eight splits (without fused=1 the merge kernel serves them)
# waves=8: eight wavefronts of one 32-row tile each (two per SIMD), also
# through the tree-building and paged instances; spin=0: the fused merge's
# hand-off of ranges to the last arrival (see HANDOFF below)
PLANS = ["waves=2,qt=1", "waves=2,qt=1,splits=1", "waves=4,qt=1,splits=8", "qt=2,splits=2", "splits=1",
         "splits=16", "fused=0", "splits=2", "waves=4,qt=1,splits=4", "splits=4,fused=0",
         "waves=8", "waves=8,splits=1", "waves=8,fused=0", "waves=8,splits=16",
         "fused=2", "splits=2,fused=2", "waves=4,qt=1,splits=4,fused=2",
         "splits=3", "splits=6,fused=1", "waves=2,qt=1,splits=8,fused=1",
         "spin=0", "splits=2,spin=0", "splits=3,spin=0", "waves=2,qt=1,splits=8,fused=1,spin=0"]
# the extra checks an eight-wavefront or give-up plan runs (the tree built
# in the kernel, invalid trees, the paged instances)
EIGHT = 3


def child_main(plan: str) -> None:
    sys.path.insert(0, ROOT)
    from tests.test_gpu_parity import test_small_workloads_full_parity, test_uniformly_low_scores_with_empty_splits
    for cfg, over in CASES:
        test_small_workloads_full_parity(cfg, over)
        print(f"ok plan={plan} cfg={cfg} {over}", flush=True)
    test_uniformly_low_scores_with_empty_splits()
    print(f"ok plan={plan} low scores", flush=True)
    if "waves=8" in plan or "spin=0" in plan:
        from tests.test_gpu_from_parents import test_invalid_trees_and_capacity_like_build_tree, \
            test_small_cases_equal_separate_calls_and_oracle
        from tests.test_gpu_paged import test_paged_ragged_trees_against_oracle_and_dense
        for cfg, over in CASES:
            test_small_cases_equal_separate_calls_and_oracle(cfg, over)
        print(f"ok plan={plan} tree built in the kernel", flush=True)
        test_invalid_trees_and_capacity_like_build_tree()
        print(f"ok plan={plan} invalid trees", flush=True)
        test_paged_ragged_trees_against_oracle_and_dense()
        print(f"ok plan={plan} paged", flush=True)


# The fused merge's hand-off: with spin=0 every split that is not the last to
# arrive looks at the arrival count once and, unless every split has
# arrived, leaves its range to the last arrival, which merges every range
# still unclaimed; the default wait never does so on these grids. The
# result is the same merge in the same split order, so every output bit
# must equal the default wait's: (default-wait plan, hand-off plan) pairs
# with four, two and three fused splits.
HANDOFF = [("", "spin=0"), ("splits=2", "splits=2,spin=0"), ("splits=3", "splits=3,spin=0")]
# full-size headline shape (dense and paged, tree built in the kernel), and
# two small ones with 64 and 128 rows per KV head
DIGEST_CASES = [(3, {}), (2, dict(prefix=1100)), (5, dict(B=6, prefix=(16, 300)))]


def child_digest(plan: str) -> None:
    """Prints one digest line per case: the outputs, anc, depth, err and the
    caches after the append, dense and paged."""
    sys.path.insert(0, ROOT)
    import hashlib

    import numpy as np
    import torch

    import tree_attention_verification_tv_amd as tv
    from tests.gpu_util import upload
    from tests.test_gpu_paged import shuffled_table
    from workloads import generate
    for cfg, over in DIGEST_CASES:
        w = generate(cfg, **over)
        d = upload(w, "cuda:0")
        bt, n_pages = shuffled_table(w, np.random.default_rng(cfg))
        k_pool, v_pool = tv.pages_from_dense(d["k_cache"], d["v_cache"], bt, n_pages)
        res = tv.tree_attention_from_parents(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                             d["prefix_len"], d["n_nodes"], d["parents"], rope_theta=w.rope_theta)
        res_p = tv.tree_attention_paged_from_parents(d["q"], d["k_new"], d["v_new"], k_pool, v_pool, bt,
                                                     d["prefix_len"], d["n_nodes"], d["parents"],
                                                     rope_theta=w.rope_theta)
        torch.cuda.synchronize()
        h = hashlib.sha256()
        for t in list(res) + list(res_p) + [d["k_cache"], d["v_cache"], k_pool, v_pool]:
            h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        assert torch.equal(res[0].view(torch.int16), res_p[0].view(torch.int16)), cfg
        print(f"digest cfg={cfg} {h.hexdigest()[:24]}", flush=True)


def run_child(plan: str, *args: str) -> str:
    env = dict(os.environ, TV_ATTN_TUNE=plan)
    r = subprocess.run([sys.executable, "-u", "-m", "tests.test_gpu_tune", plan, *args], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stdout


@pytest.mark.parametrize("base,handoff", HANDOFF, ids=[h for _, h in HANDOFF])
def test_fused_merge_handoff_bit_identical(base, handoff):
    print(f"[gpu] fused merge hand-off {handoff!r} against {base!r}", flush=True)
    a = [l for l in run_child(base, "--digest").splitlines() if l.startswith("digest")]
    b = [l for l in run_child(handoff, "--digest").splitlines() if l.startswith("digest")]
    assert len(a) == len(DIGEST_CASES) and a == b, (a, b)


@pytest.mark.parametrize("plan", PLANS)
def test_plan_parity(plan):
    print(f"[gpu] attention plan {plan}", flush=True)
    out = run_child(plan)
    assert out.count("ok plan=") == len(CASES) + 1 + (EIGHT if "waves=8" in plan or "spin=0" in plan else 0)


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[2] == "--digest":
        child_digest(sys.argv[1])
    else:
        child_main(sys.argv[1])
