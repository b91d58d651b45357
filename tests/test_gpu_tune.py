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
# through the tree-building and paged instances
PLANS = ["waves=2,qt=1", "waves=2,qt=1,splits=1", "waves=4,qt=1,splits=8", "qt=2,splits=2", "splits=1",
         "splits=16", "fused=0", "splits=2", "waves=4,qt=1,splits=4", "splits=4,fused=0",
         "waves=8", "waves=8,splits=1", "waves=8,fused=0", "waves=8,splits=16",
         "fused=2", "splits=2,fused=2", "waves=4,qt=1,splits=4,fused=2",
         "splits=3", "splits=6,fused=1", "waves=2,qt=1,splits=8,fused=1"]
# the extra checks an eight-wavefront plan runs
EIGHT = 3


def child_main(plan: str) -> None:
    sys.path.insert(0, ROOT)
    from tests.test_gpu_parity import test_small_workloads_full_parity, test_uniformly_low_scores_with_empty_splits
    for cfg, over in CASES:
        test_small_workloads_full_parity(cfg, over)
        print(f"ok plan={plan} cfg={cfg} {over}", flush=True)
    test_uniformly_low_scores_with_empty_splits()
    print(f"ok plan={plan} low scores", flush=True)
    if "waves=8" in plan:
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


@pytest.mark.parametrize("plan", PLANS)
def test_plan_parity(plan):
    print(f"[gpu] attention plan {plan}", flush=True)
    env = dict(os.environ, TV_ATTN_TUNE=plan)
    r = subprocess.run([sys.executable, "-u", "-m", "tests.test_gpu_tune", plan], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.count("ok plan=") == len(CASES) + 1 + (EIGHT if "waves=8" in plan else 0)


if __name__ == "__main__":
    child_main(sys.argv[1])
