"""Host-side pieces of bench.py: the algorithmic byte and flop counts its
roofline divides by, and the choice of bound (no GPU needed)."""
import bench
from workloads import generate


def test_flops_of_the_worked_tree_by_hand():
    # parents [-1, 0, 0, 1, 2]: depths 0, 1, 1, 2, 2, so 1 + 2 + 2 + 3 + 3 = 11
    # tree keys over the five nodes, plus 64 prefix keys each; 4 heads, D = 64,
    # 4 D flops per (row, key)
    w = generate(1)
    assert bench.algorithmic_flops(w) == 4 * 64 * 4 * (64 * 5 + 11)


def test_bytes_of_the_headline_by_hand():
    # 8 sequences x 8 KV heads x 4096 slots x 128 dims x (K, V) x 2 bytes, plus
    # per node: queries (32 heads) read and output written, tree K/V (8 heads)
    # read and appended
    w = generate(3)
    nodes = int(w.n_nodes.sum())
    expect = 8 * 8 * 4096 * 128 * 2 * 2 + nodes * 128 * 2 * (32 * 2 + 8 * 2 * 2)
    assert bench.algorithmic_bytes(w)["total"] == expect == 146014208


def test_bound_follows_the_ridge():
    # the headline (~221 flop/B) sits below the ridge of 2500 TFLOP/s over
    # 8000 GB/s (312.5 flop/B); the 16-sequence, 64-query-head layer (~475
    # flop/B) above it; fp32 never prices against the matrix cores
    for cfg, bound in ((1, "hbm"), (2, "hbm"), (3, "hbm"), (4, "mfma"), (5, "hbm")):
        w = generate(cfg)
        ab = bench.algorithmic_bytes(w)["total"]
        assert bench.roofline_bound(w, ab, bench.algorithmic_flops(w)) == bound, cfg
