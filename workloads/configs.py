"""Workload definitions and their seeded generators.

Five workloads, shaped like the settings the pages discuss (no dataset is
used; every value is drawn from a seeded generator):

  1 tiny-f32       fp32, batch 1, prefix 64, the five-node tree of the
                   infra-guide page "5.3 Medusa、EAGLE 与 MTP" section 8,
                   4 q heads = 4 kv heads, head dim 64.
  2 medusa-b1      bf16, Vicuna-7B-shaped attention (32 = 32 heads, dim 128),
                   prefix 1024, a 64-node Medusa-style static sparse tree
                   (pofe.ai "Medusa and EAGLE ...", section "Medusa: heads,
                   losses and trees"; vibeengines.com "Medusa, explained",
                   step 5), agreement 0.6 per child.
  3 eagle2-gqa-b8  bf16, Llama-3-8B-shaped GQA (32 q / 8 kv heads, dim 128),
                   batch 8, prefix 4096, per-sequence 60-node EAGLE-2-style
                   dynamic trees ranked by path confidence (infra-guide
                   section 5.2), acceptance chance of a node = its path
                   confidence.
  4 l70b-gqa-b16   bf16, Llama-2-70B-shaped (64 q / 8 kv heads, dim 128),
                   batch 16, prefix 8192, one 64-node static tree shared by
                   all sequences, agreement 0.7 at depth 1 decaying x0.8.
  5 serving-b64    bf16, 32 q / 8 kv heads, dim 128, batch 64, prefixes
                   uniform in [512, 4096], 32-node deep EAGLE-3-style trees
                   (1-3 children per expanded node, depth <= 7).

Random streams: ``SeedSequence(seed).spawn(9)`` gives independent PCG64
generators for tree, lengths, tokens, target, q, k_new, v_new, k_cache and
v_cache, so changing one part of a workload leaves the others unchanged.

bf16 tensors are drawn as float32 N(0, 1) and rounded to bf16 (round to
nearest even) here, once; both the library and the oracle then see the same
bits.
"""
from __future__ import annotations

import dataclasses
import heapq
from typing import Optional

import numpy as np

VOCAB = 32000


CONFIGS = {
    1: dict(name="tiny-f32-worked-tree", dtype="f32", B=1, Hq=4, Hkv=4, D=64,
            prefix=64, n=5, max_depth=2, tree="worked", rope_theta=10000.0),
    2: dict(name="vicuna7b-medusa-b1", dtype="bf16", B=1, Hq=32, Hkv=32, D=128,
            prefix=1024, n=64, max_depth=5, tree="medusa", agree=0.6,
            rope_theta=10000.0),
    3: dict(name="llama3-8b-gqa-eagle2-b8", dtype="bf16", B=8, Hq=32, Hkv=8, D=128,
            prefix=4096, n=60, max_depth=6, tree="eagle2", rope_theta=10000.0),
    4: dict(name="llama2-70b-gqa-b16", dtype="bf16", B=16, Hq=64, Hkv=8, D=128,
            prefix=8192, n=64, max_depth=5, tree="medusa-shared", agree=0.7,
            agree_decay=0.8, rope_theta=10000.0),
    5: dict(name="serving-b64-ragged", dtype="bf16", B=64, Hq=32, Hkv=8, D=128,
            prefix=(512, 4096), n=32, max_depth=7, tree="eagle3", rope_theta=10000.0),
}


# ---------------------------------------------------------------------------
# bf16 helpers (storage conversion only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Tree shapes
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Tree:
    parents: list          # flattened, parents first
    rank: list             # rank of each node among its siblings (0 = best)
    children: list         # children of each node (flattened indices), by rank
    # For dynamic trees: all children created during expansion (kept or not),
    # with their confidences, used to draw the target's choice.
    created_conf: Optional[list] = None   # per kept node: list of (conf, kept_index or -1)


def worked_tree() -> Tree:
    """The five-node tree of the infra-guide page, section 8."""
    parents = [-1, 0, 0, 1, 2]
    return Tree(parents=parents, rank=[0, 0, 1, 0, 0],
                children=[[1, 2], [3], [4], [], []])


def medusa_static_tree(rng: np.random.Generator, n: int, max_depth: int, top_k: int = 10,
                       base=(0.6, 0.4, 0.3, 0.25, 0.2, 0.15, 0.1)) -> Tree:
    """A Medusa-style sparse tree: depth d holds head d's top-k choices.

    Synthetic hit rate of rank r at depth d: a_d * (1 - a_d)^r * U(0.8, 1.2),
    with a = 0.6, 0.4, 0.3 (the per-head rates of pofe.ai's worked example)
    continuing to decay. A path's value is the product of the rates along it;
    the n - 1 best paths are kept (best-first), which makes the child count
    fall with depth. Flattened by (depth, parent index, rank).
    """
    h = [[base[d] * (1 - base[d]) ** r * rng.uniform(0.8, 1.2) for r in range(top_k)]
         for d in range(max_depth)]
    heap = [(-h[0][r], (r,)) for r in range(top_k)]
    heapq.heapify(heap)
    chosen = []
    while len(chosen) < n - 1:
        negv, path = heapq.heappop(heap)
        chosen.append(path)
        if len(path) < max_depth:
            for r in range(top_k):
                heapq.heappush(heap, (negv * h[len(path)][r], path + (r,)))
    index = {(): 0}
    parents, rank = [-1], [0]
    children = [[]]
    for depth in range(1, max_depth + 1):
        level = [p for p in chosen if len(p) == depth]
        level.sort(key=lambda p: (index[p[:-1]], p[-1]))
        for p in level:
            i = len(parents)
            index[p] = i
            parents.append(index[p[:-1]])
            rank.append(p[-1])
            children.append([])
            children[index[p[:-1]]].append(i)
    return Tree(parents=parents, rank=rank, children=children)


def eagle_dynamic_tree(rng: np.random.Generator, n: int, max_depth: int, k_expand: int,
                       n_children, first_frac, other_frac) -> Tree:
    """An EAGLE-2-style dynamic tree (infra-guide "5.3 ...", section 5.2).

    Each expansion step gives children to the k_expand nodes of the newest
    layer with the highest path confidence. A child's confidence is a
    stick-breaking share of the probability mass its parent has left, so
    siblings sum to at most 1 like a draft softmax; its path confidence is the
    product of confidences from the root. After max_depth steps every created
    node is reranked by path confidence and the best n - 1 are kept with the
    root. Path confidence falls strictly along a path, so the kept set is
    closed under ancestors. Flattened by (depth, creation order).
    """
    while True:
        par, dep, val, conf = [-1], [0], [1.0], [1.0]
        kids = [[]]
        frontier = [0]
        for _ in range(max_depth):
            expand = sorted(frontier, key=lambda i: -val[i])[:k_expand]
            frontier = []
            for p in expand:
                m = n_children(rng)
                remaining = 1.0
                for c in range(m):
                    frac = first_frac(rng) if c == 0 else other_frac(rng)
                    cf = remaining * frac
                    remaining -= cf
                    j = len(par)
                    par.append(p)
                    dep.append(dep[p] + 1)
                    val.append(val[p] * cf)
                    conf.append(cf)
                    kids.append([])
                    kids[p].append(j)
                    frontier.append(j)
        if len(par) >= n:
            break
    keep = sorted(range(1, len(par)), key=lambda i: -val[i])[: n - 1]
    keep = [0] + sorted(keep, key=lambda i: (dep[i], i))
    new_index = {old: new for new, old in enumerate(keep)}
    parents = [-1] + [new_index[par[old]] for old in keep[1:]]
    rank, children, created = [], [], []
    for old in keep:
        p = par[old]
        rank.append(0 if p == -1 else kids[p].index(old))
        children.append([new_index[c] for c in kids[old] if c in new_index])
        created.append([(conf[c], new_index.get(c, -1)) for c in kids[old]])
    return Tree(parents=parents, rank=rank, children=children, created_conf=created)


# ---------------------------------------------------------------------------
# Tokens and targets
# ---------------------------------------------------------------------------

def _draw_tokens(rng: np.random.Generator, tree: Tree, n_created: Optional[list] = None) -> np.ndarray:
    """Candidate token ids; siblings are distinct, as top-k choices are."""
    n = len(tree.parents)
    tok = np.zeros(n, dtype=np.int32)
    tok[0] = rng.integers(0, VOCAB)
    for p in range(n):
        kids = tree.children[p]
        if kids:
            ids = rng.choice(VOCAB, size=len(kids), replace=False)
            for c, t in zip(kids, ids):
                tok[c] = t
    return tok


def _non_child_token(rng: np.random.Generator, avoid) -> int:
    while True:
        t = int(rng.integers(0, VOCAB))
        if t not in avoid:
            return t


def _targets_independent(rng, tree: Tree, tok, p_agree) -> np.ndarray:
    """Each child of p agrees with probability p_agree(depth of child); the
    target's choice at p is the lowest-rank agreeing child, else a token that
    is no child of p."""
    n = len(tree.parents)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[tree.parents[i]] + 1
    tgt = np.zeros(n, dtype=np.int32)
    for p in range(n):
        kids = sorted(tree.children[p], key=lambda c: tree.rank[c])
        chosen = None
        for c in kids:
            if rng.random() < p_agree(depth[c]) and chosen is None:
                chosen = c
        if chosen is not None:
            tgt[p] = tok[chosen]
        else:
            tgt[p] = _non_child_token(rng, {int(tok[c]) for c in kids})
    return tgt


def _targets_by_confidence(rng, tree: Tree, tok) -> np.ndarray:
    """The target's choice at p is a draw over every child p created during
    expansion, each with its confidence; the leftover mass picks a token that
    is no kept child of p. A kept node is then accepted with probability equal
    to its path confidence."""
    n = len(tree.parents)
    tgt = np.zeros(n, dtype=np.int32)
    for p in range(n):
        avoid = {int(tok[c]) for c in tree.children[p]}
        u = rng.random()
        acc = 0.0
        pick = None
        for cf, kept in tree.created_conf[p]:
            acc += cf
            if u < acc:
                pick = kept
                break
        if pick is not None and pick >= 0:
            tgt[p] = tok[pick]
        else:
            tgt[p] = _non_child_token(rng, avoid)
    return tgt


# ---------------------------------------------------------------------------
# Workload container
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    cfg: int
    name: str
    dtype: str             # "f32" or "bf16"
    B: int
    n_max: int
    Hq: int
    Hkv: int
    D: int
    cap: int
    rope_theta: float
    parents: np.ndarray    # [B, n_max] int32, padding = -1
    n_nodes: np.ndarray    # [B] int32
    prefix_len: np.ndarray  # [B] int32
    tok: np.ndarray        # [B, n_max] int32
    tgt: np.ndarray        # [B, n_max] int32
    q: np.ndarray          # [B, n_max, Hq, D]  float32 or uint16 bf16 bits
    k_new: np.ndarray      # [B, n_max, Hkv, D]
    v_new: np.ndarray      # [B, n_max, Hkv, D]
    k_cache: np.ndarray    # [B, Hkv, cap, D]
    v_cache: np.ndarray    # [B, Hkv, cap, D]

    def f64(self, name: str, b: Optional[int] = None) -> np.ndarray:
        """Exact float64 view of a tensor (optionally one sequence only)."""
        a = getattr(self, name)
        if b is not None:
            a = a[b:b + 1]
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def oracle_inputs(self, b: Optional[int] = None) -> dict:
        """The float64 / int arrays the oracle takes (all or one sequence)."""
        sl = slice(None) if b is None else slice(b, b + 1)
        return dict(parents=self.parents[sl], n_nodes=self.n_nodes[sl],
                    prefix_len=self.prefix_len[sl], tok=self.tok[sl], tgt=self.tgt[sl],
                    q=self.f64("q", b), k_new=self.f64("k_new", b), v_new=self.f64("v_new", b),
                    k_cache=self.f64("k_cache", b), v_cache=self.f64("v_cache", b),
                    rope_theta=self.rope_theta, softmax_scale=0.0)

    @property
    def total_nodes(self) -> int:
        return int(self.n_nodes.sum())


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def generate(cfg: int, seed: Optional[int] = None, **over) -> Workload:
    """Draw workload ``cfg`` (1..5) from ``seed`` (default: the config number).

    Keyword overrides (B, prefix, Hq, Hkv, D, n, max_depth, dtype, cap_extra)
    shrink or reshape a workload for tests; the tree and token procedures stay
    those of the config.
    """
    c = dict(CONFIGS[cfg])
    c.update({k: v for k, v in over.items() if k in c or k in ("cap_extra",)})
    seed = cfg if seed is None else seed
    ss = np.random.SeedSequence(seed)
    r_tree, r_len, r_tok, r_tgt, r_q, r_k, r_v, r_kc, r_vc = [
        np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(9)]
    B, n_max, Hq, Hkv, D = c["B"], c["n"], c["Hq"], c["Hkv"], c["D"]
    max_depth = c["max_depth"]

    # trees
    trees = []
    kind = c["tree"]
    if kind == "worked":
        trees = [worked_tree() for _ in range(B)]
    elif kind == "medusa":
        trees = [medusa_static_tree(r_tree, n_max, max_depth) for _ in range(B)]
    elif kind == "medusa-shared":
        t = medusa_static_tree(r_tree, n_max, max_depth)
        trees = [t] * B
    elif kind == "eagle2":
        trees = [eagle_dynamic_tree(r_tree, n_max, max_depth, k_expand=8,
                                    n_children=lambda r: 8,
                                    first_frac=lambda r: r.beta(2, 2),
                                    other_frac=lambda r: r.beta(2, 2)) for _ in range(B)]
    elif kind == "eagle3":
        trees = [eagle_dynamic_tree(r_tree, n_max, max_depth, k_expand=4,
                                    n_children=lambda r: int(r.integers(1, 4)),
                                    first_frac=lambda r: r.beta(8, 2),
                                    other_frac=lambda r: r.beta(2, 2)) for _ in range(B)]
    else:
        raise ValueError(kind)

    parents = np.full((B, n_max), -1, dtype=np.int32)
    n_nodes = np.zeros(B, dtype=np.int32)
    tok = np.zeros((B, n_max), dtype=np.int32)
    tgt = np.zeros((B, n_max), dtype=np.int32)
    for b, t in enumerate(trees):
        n = len(t.parents)
        parents[b, :n] = t.parents
        n_nodes[b] = n
        tk = _draw_tokens(r_tok, t)
        if kind == "worked":
            tg = r_tgt.integers(0, VOCAB, size=n).astype(np.int32)
            tg[0] = tk[1]   # the target's choice after the root is node 1's token
            tg[1] = tk[3]   # and after node 1 it is node 3's token
        elif kind == "medusa":
            tg = _targets_independent(r_tgt, t, tk, lambda d: c["agree"])
        elif kind == "medusa-shared":
            a, dec = c["agree"], c["agree_decay"]
            tg = _targets_independent(r_tgt, t, tk, lambda d: a * dec ** (d - 1))
        else:
            tg = _targets_by_confidence(r_tgt, t, tk)
        tok[b, :n] = tk
        tgt[b, :n] = tg

    # prefix lengths and cache capacity
    pre = c["prefix"]
    if isinstance(pre, tuple):
        prefix_len = r_len.integers(pre[0], pre[1] + 1, size=B).astype(np.int32)
    else:
        prefix_len = np.full(B, pre, dtype=np.int32)
    cap = int(prefix_len.max()) + n_max + int(c.get("cap_extra", 0))
    cap = -(-cap // 64) * 64     # the library keeps V in blocks of 64 slots

    dt = c["dtype"]
    q = _normal(r_q, (B, n_max, Hq, D), dt)
    k_new = _normal(r_k, (B, n_max, Hkv, D), dt)
    v_new = _normal(r_v, (B, n_max, Hkv, D), dt)
    k_cache = _normal(r_kc, (B, Hkv, cap, D), dt)
    v_cache = _normal(r_vc, (B, Hkv, cap, D), dt)
    return Workload(cfg=cfg, name=c["name"], dtype=dt, B=B, n_max=n_max, Hq=Hq, Hkv=Hkv,
                    D=D, cap=cap, rope_theta=float(c["rope_theta"]), parents=parents,
                    n_nodes=n_nodes, prefix_len=prefix_len, tok=tok, tgt=tgt, q=q,
                    k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache)


def target_logits(w: Workload, vocab: int = VOCAB, dtype: Optional[str] = None,
                  seed: Optional[int] = None) -> np.ndarray:
    """Synthetic target logits [B, n_max, vocab] for typical acceptance.

    Row (b, i) stands for the target model's next-token logits at node i of
    sequence b. Base logits are tau * N(0, 1) with tau ~ U(0.5, 3) per row, so
    rows range from nearly flat to peaked. Each child c of node i gets, at its
    own token, the planted logit ln(vocab) + tau^2 / 2 + s with s ~ U(-9, 3):
    ln(vocab) + tau^2 / 2 is the log of the expected sum of exp over the base
    row, so s is roughly the child's log-odds against the rest of the
    vocabulary and children range from hopeless to near-certain. Rows of
    padding nodes are base logits only. Drawn from a stream of its own
    (``seed``, default the workload's config number), then rounded to bf16
    bits when the dtype (default the workload's) is bf16.
    """
    dt = w.dtype if dtype is None else dtype
    seed = w.cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x7A])))
    B, n_max = w.B, w.n_max
    tau = rng.uniform(0.5, 3.0, size=(B, n_max)).astype(np.float32)
    x = rng.standard_normal(size=(B, n_max, vocab), dtype=np.float32)
    x *= tau[:, :, None]
    base = np.float32(np.log(vocab)) + 0.5 * tau * tau
    for b in range(B):
        n = int(w.n_nodes[b])
        for c in range(1, n):
            p = int(w.parents[b, c])
            t = int(w.tok[b, c])
            if 0 <= t < vocab:
                x[b, p, t] = base[b, p] + np.float32(rng.uniform(-9.0, 3.0))
    return f32_to_bf16_bits(x) if dt == "bf16" else x


def draft_proposals(B: int, S: int, K: int, M: int, seed: int = 0):
    """Synthetic draft proposals for building EAGLE-2 trees: for each sequence,
    expansion step s and expanded node k, M children with confidences drawn by
    stick-breaking (fraction ~ Beta(2, 2) of the mass left, so siblings sum
    to at most 1 like a draft softmax), sorted best first as a top-M would be,
    and M distinct token ids. Returns (conf [B][S][K][M] float32,
    cand [B][S][K][M] int32, root_tok [B] int32)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xE2])))
    frac = rng.beta(2.0, 2.0, size=(B, S, K, M))
    left = np.cumprod(np.concatenate([np.ones((B, S, K, 1)), 1.0 - frac[..., :-1]], axis=-1), axis=-1)
    conf = -np.sort(-(left * frac), axis=-1)
    cand = np.empty((B, S, K, M), dtype=np.int32)
    for idx in np.ndindex(B, S, K):
        cand[idx] = rng.choice(VOCAB, size=M, replace=False)
    root = rng.integers(0, VOCAB, size=B).astype(np.int32)
    return conf.astype(np.float32), cand, root


def speculative_inputs(B: int, L: int, V: int = VOCAB, dtype: str = "bf16", seed: int = 0):
    """Synthetic inputs for chain speculative sampling: target logits
    [B][L+1][V] (tau * N(0, 1), tau ~ U(0.5, 3) per row, plus a few boosted
    tokens so rows range from flat to peaked), draft logits [B][L][V] (the
    target's row plus N(0, sigma^2) noise, sigma ~ U(0.2, 1.5) per row: a
    drafter that mostly agrees), drafted tokens (the draft row's top token,
    or with probability 0.3 one of its next seven, ranked by logit), and the
    uniform draws u_acc [B][L], u_res [B]. Logits rounded to bf16 bits when
    dtype is bf16."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x5B])))
    tau = rng.uniform(0.5, 3.0, size=(B, L + 1, 1)).astype(np.float32)
    p = rng.standard_normal((B, L + 1, V), dtype=np.float32) * tau
    for idx in np.ndindex(B, L + 1):
        hot = rng.choice(V, size=4, replace=False)
        p[idx][hot] += rng.uniform(2.0, 8.0, size=4).astype(np.float32) * tau[idx][0]
    sig = rng.uniform(0.2, 1.5, size=(B, L, 1)).astype(np.float32)
    q = p[:, :L] + rng.standard_normal((B, L, V), dtype=np.float32) * sig
    if dtype == "bf16":
        p, q = bf16_bits_to_f32(f32_to_bf16_bits(p)), bf16_bits_to_f32(f32_to_bf16_bits(q))
    draft = np.empty((B, L), dtype=np.int32)
    for idx in np.ndindex(B, L):
        order = np.argsort(-q[idx], kind="stable")[:8]
        draft[idx] = order[0] if rng.random() >= 0.3 else order[rng.integers(1, 8)]
    u_acc = rng.random((B, L)).astype(np.float32)
    u_res = rng.random(B).astype(np.float32)
    if dtype == "bf16":
        p, q = f32_to_bf16_bits(p), f32_to_bf16_bits(q)
    return p, q, draft, u_acc, u_res
