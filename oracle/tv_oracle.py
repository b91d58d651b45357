"""CPU oracle for draft-tree verification (test infrastructure only).

This module is the plain, slow, float64 statement of what one tree-verification
step computes. It exists to check the HIP library, never to serve results:
only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it. It shares no code, table or helper with the HIP path.

Sources (web pages, cited by title and section):
  [MEDUSA-EAGLE]  "Medusa and EAGLE: self-speculative decoding heads, explained"
                  (pofe.ai), sections "Medusa: heads, losses and trees" and
                  "Typical acceptance".
  [MEDUSA-EXPL]   "Medusa, explained" (vibeengines.com), procedure steps 6-7.
  [INFRA-5.3]     "5.3 Medusa、EAGLE 与 MTP" (infra-guide), sections 3.1, 3.2,
                  8 and 9.2.
  [DRAFTERS]      "Drafters: draft models, Medusa, EAGLE, MTP, DFlash, DSpark"
                  (robertz.co), section "Why the answer does not change".
  [MEDUSA-EXPL] also defines typical acceptance (section "Typical
  acceptance"), as do [MEDUSA-EAGLE] ("Typical acceptance") and [INFRA-5.3]
  section 9.1.

Readings of points the pages leave open are listed with each function.

Conventions shared by every function here:
  * a tree is a ``parents`` list; node 0 is the root (parent -1) and every
    other node's parent has a smaller index;
  * ``n_nodes[b]`` nodes are live in sequence b, the rest of the row is padding;
  * error codes: 0 ok, 2 bad tree, 3 cache capacity exceeded.
"""
from __future__ import annotations

import math

import numpy as np

ERR_OK = 0
ERR_BAD_TREE = 2
ERR_CAPACITY = 3


# ---------------------------------------------------------------------------
# Tree structure: visibility mask and depth position ids
# ---------------------------------------------------------------------------

def tree_is_valid(parents) -> bool:
    """A tree is usable iff it is laid out parents-first.

    [INFRA-5.3] section 8 requires every parent to come before its child in the
    flattened array; section 3.1 has exactly one root. Reading: node 0 must be
    the root (-1) and every other node's parent lies in [0, i).
    """
    n = len(parents)
    if n == 0:
        return True
    if parents[0] != -1:
        return False
    return all(0 <= parents[i] < i for i in range(1, n))


def ancestors_or_self(parents, i) -> list:
    """Nodes on the path root..i, in increasing index order (= increasing depth).

    Found by walking parent links upward from i, the way [INFRA-5.3] section 8
    marks visibility, then reversing.
    """
    path = []
    cur = i
    while cur != -1:
        path.append(cur)
        cur = parents[cur]
    path.reverse()
    return path


def tree_depth(parents) -> list:
    """Depth of each node: the root is 0, a child is one deeper than its parent.

    [INFRA-5.3] section 3.2 and [MEDUSA-EXPL] step 6: siblings share a position,
    so the position id offset of a node is its depth in the tree.
    """
    depth = [0] * len(parents)
    for i, p in enumerate(parents):
        depth[i] = 0 if p == -1 else depth[p] + 1
    return depth


def tree_mask(parents) -> np.ndarray:
    """n x n visibility matrix: row i has a 1 at i and at each ancestor of i.

    [INFRA-5.3] section 3.1: a node sees the shared prefix and its own
    ancestors only; siblings and other branches stay hidden. The prefix part is
    not stored here (every node sees all of it).
    """
    n = len(parents)
    mask = np.zeros((n, n), dtype=np.uint8)
    for i in range(n):
        for j in ancestors_or_self(parents, i):
            mask[i, j] = 1
    return mask


def ancestor_words(parents, n_max: int) -> np.ndarray:
    """Mask rows packed as 64-bit words, bit j of word j//64 = mask[i][j].

    The packing (least significant bit first, one word per 64 nodes) is this
    library's storage choice for the mask of [INFRA-5.3] section 3.1.
    """
    w = (n_max + 63) // 64
    out = np.zeros((n_max, w), dtype=np.uint64)
    mask = tree_mask(parents)
    for i in range(len(parents)):
        for j in range(len(parents)):
            if mask[i, j]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def build_tree(parents_bn: np.ndarray, n_nodes: np.ndarray):
    """Batched tree set-up: ancestor words, depths and a per-sequence status.

    Padding nodes (index >= n_nodes[b]) and every node of an invalid tree get
    ancestor word 0 and depth 0. Returns (anc [B,n_max] uint64, depth [B,n_max]
    int32, err [B] int32).
    """
    B, n_max = parents_bn.shape
    if n_max > 64:
        raise ValueError("one ancestor word per node: n_max <= 64")
    anc = np.zeros((B, n_max), dtype=np.uint64)
    depth = np.zeros((B, n_max), dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        par = [int(x) for x in parents_bn[b, :n]]
        if n < 0 or n > n_max or not tree_is_valid(par):
            err[b] = ERR_BAD_TREE
            continue
        if n == 0:
            continue
        anc[b, :n] = ancestor_words(par, n)[:, 0]
        depth[b, :n] = tree_depth(par)
    return anc, depth, err


# ---------------------------------------------------------------------------
# Rotary position embedding at depth-based positions
# ---------------------------------------------------------------------------

def rope(x: np.ndarray, pos: float, theta: float) -> np.ndarray:
    """Rotary embedding of vector(s) ``x`` (last axis D) at position ``pos``.

    Reading (the pages only say that positions follow depth, [INFRA-5.3]
    section 3.2): the rotate-half pairing used by Llama-family models, with
    frequency theta^(-2d/D) for pair d = (x[d], x[d + D/2]). All in float64.
    theta == 0 means no rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    D = x.shape[-1]
    half = D // 2
    d = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * d / D)
    ang = float(pos) * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# Tree-masked attention over the shared prefix plus the node's ancestors
# ---------------------------------------------------------------------------

def attention_row(q_vec, keys, values, scale):
    """softmax(keys @ q * scale) @ values, max-subtracted, float64."""
    s = keys @ q_vec * scale
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ values


def tree_attention(q, k_new, v_new, k_cache, v_cache, prefix_len, n_nodes,
                   parents, rope_theta, softmax_scale=0.0, err_in=None,
                   rows=None):
    """Verification attention for every live tree node.

    For node i of sequence b the keys are the P_b prefix keys of its KV head
    followed by the rotated keys of the nodes on the root..i path; the values
    follow the same order. This is ordinary causal attention over
    "prefix + root-to-node path", the tree mask of [INFRA-5.3] section 3.1 and
    [MEDUSA-EAGLE] ("Trees"), with position ids P_b + depth ([INFRA-5.3]
    section 3.2, [MEDUSA-EXPL] step 6).

    Readings: prefix keys in the cache are already rotated (they were rotated
    when committed); only tree q and k are rotated here, v never; the softmax
    scale defaults to 1/sqrt(D); query head h reads KV head h // (Hq/Hkv).

    Arrays: q [B,n_max,Hq,D], k_new/v_new [B,n_max,Hkv,D],
    k_cache/v_cache [B,Hkv,cap,D] (float64 views of the inputs).
    ``rows``: optional list of (b, i) pairs; only those outputs are computed.

    Returns (out [B,n_max,Hq,D] float64 with zeros where not computed or not
    live, k_cache_after, v_cache_after, err [B]). The caches after the call hold
    the rotated tree keys and raw tree values in slots [P_b, P_b + n_b); rows
    of sequences with an error are left unchanged and their outputs are zero.
    """
    B, n_max, Hq, D = q.shape
    Hkv = k_new.shape[2]
    cap = k_cache.shape[2]
    G = Hq // Hkv
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(D)
    err = np.zeros(B, dtype=np.int32) if err_in is None else np.array(err_in, dtype=np.int32)
    out = np.zeros((B, n_max, Hq, D), dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)

    want = None
    if rows is not None:
        want = {}
        for b, i in rows:
            want.setdefault(int(b), []).append(int(i))

    for b in range(B):
        n = int(n_nodes[b])
        P = int(prefix_len[b])
        if err[b] != 0 or n == 0:
            continue
        if P + n > cap:
            err[b] = ERR_CAPACITY
            continue
        par = [int(x) for x in parents[b, :n]]
        dep = tree_depth(par)
        # rotated tree keys, one per node, at position P + depth
        k_rot = np.stack([rope(k_new[b, a], P + dep[a], rope_theta) for a in range(n)])
        for a in range(n):
            kc[b, :, P + a, :] = k_rot[a]
            vc[b, :, P + a, :] = v_new[b, a]
        if want is None:
            nodes = range(n)
        else:
            nodes = [i for i in want.get(b, []) if i < n]
        for i in nodes:
            path = ancestors_or_self(par, i)
            q_rot = rope(q[b, i], P + dep[i], rope_theta)   # [Hq, D]
            for h in range(Hq):
                g = h // G
                keys = np.concatenate([k_cache[b, g, :P, :], k_rot[path, g, :]], axis=0)
                vals = np.concatenate([v_cache[b, g, :P, :], v_new[b, path, g, :]], axis=0)
                out[b, i, h] = attention_row(q_rot[h], keys, vals, scale)
    return out, kc, vc, err


# ---------------------------------------------------------------------------
# Greedy acceptance of the longest matching root path
# ---------------------------------------------------------------------------

def accept(cand_tok, tgt_argmax, parents, n_nodes, err_in=None):
    """Greedy longest-path acceptance per sequence.

    [MEDUSA-EAGLE] ("Typical acceptance", greedy case) and [DRAFTERS]: under
    greedy decoding a drafted token is kept iff it equals the target's own
    choice; [MEDUSA-EXPL] step 7 keeps the longest valid root path;
    [INFRA-5.3] section 9.2 checks left to right and stops at the first miss.

    Readings:
      * node 0 is the last verified token and is always accepted;
      * tgt_argmax[b][i] is the target's argmax computed at node i (it predicts
        the token after i), so child c is valid iff cand_tok[c] equals
        tgt_argmax[parent(c)], and c is accepted iff its parent is too;
      * "longest" is greatest depth; equal depths go to the lowest node index;
      * accept_len counts accepted drafted tokens (the root excluded); the
        bonus token is the target's argmax at the deepest accepted node, so a
        step emits accept_len + 1 tokens.

    Sequences with n_nodes == 0 or a nonzero error produce accept_len = -1 and
    all-(-1) path / tokens. Returns (accept_len [B], path [B,n_max],
    bonus [B], out_tokens [B,n_max]) as int32.
    """
    B, n_max = cand_tok.shape
    accept_len = np.full(B, -1, dtype=np.int32)
    path = np.full((B, n_max), -1, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    out_tokens = np.full((B, n_max), -1, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if n == 0 or (err_in is not None and int(err_in[b]) != 0):
            continue
        par = [int(x) for x in parents[b, :n]]
        dep = tree_depth(par)
        ok = [False] * n
        ok[0] = True
        for i in range(1, n):
            ok[i] = ok[par[i]] and int(cand_tok[b, i]) == int(tgt_argmax[b, par[i]])
        best = 0
        for i in range(n):
            if ok[i] and dep[i] > dep[best]:
                best = i
        p = ancestors_or_self(par, best)
        L = dep[best]
        accept_len[b] = L
        path[b, :L + 1] = p
        bonus[b] = int(tgt_argmax[b, best])
        toks = [int(cand_tok[b, a]) for a in p[1:]] + [bonus[b]]
        out_tokens[b, :L + 1] = toks
    return accept_len, path, bonus, out_tokens


# ---------------------------------------------------------------------------
# Typical acceptance: entropy-dependent probability floor instead of argmax
# ---------------------------------------------------------------------------

def next_token_distribution(logits_row):
    """Softmax of one row of target logits, its entropy in nats, and argmax.

    The distribution is the plain softmax of the logits (no temperature: a
    caller sampling at temperature T passes logits / T). Entropy is
    -sum p ln p over tokens with p > 0. The argmax is the lowest index among
    equal maxima. Returns (p [V] float64, H float, argmax int).
    """
    x = np.asarray(logits_row, dtype=np.float64)
    e = np.exp(x - x.max())
    p = e / e.sum()
    nz = p[p > 0.0]
    H = float(-(nz * np.log(nz)).sum())
    return p, H, int(np.argmax(x))


def typical_accept(logits, cand_tok, parents, n_nodes, epsilon, delta, err_in=None):
    """Typical acceptance over a draft tree, longest accepted path.

    [MEDUSA-EXPL] "Typical acceptance", [MEDUSA-EAGLE] "Typical acceptance",
    [INFRA-5.3] section 9.1: a drafted token x passes iff the target's
    probability of it exceeds min(epsilon, delta * exp(-H)), H being the
    entropy of the target's distribution at that point; the first token of a
    step is always the target's own greedy choice.

    Readings:
      * the target distribution at node i is the softmax of logits[b][i]; it
        predicts the token after i, so child c is judged under its parent's
        distribution (the alignment of the greedy rule);
      * H in nats; the comparison is strict;
      * a token id outside [0, V) has probability 0 and never passes;
      * the root is always accepted; a node is accepted iff its parent is
        and its own token passes; the deepest accepted node wins, equal
        depths going to the lowest index (as in greedy acceptance);
      * the bonus token is the target's greedy argmax at that deepest node.

    Returns (entropy [B,n_max] f64, p_tok [B,n_max] f64, tgt_argmax
    [B,n_max] int32, accept_len, path, bonus, out_tokens) with the accept
    outputs as in ``accept``. p_tok[b][c] is the probability of node c's
    token under its parent's distribution (1 for the root). Padding nodes and
    skipped sequences get entropy 0, p_tok 0 and argmax -1.
    """
    B, n_max, V = logits.shape
    entropy = np.zeros((B, n_max), dtype=np.float64)
    p_tok = np.zeros((B, n_max), dtype=np.float64)
    tgt_argmax = np.full((B, n_max), -1, dtype=np.int32)
    accept_len = np.full(B, -1, dtype=np.int32)
    path = np.full((B, n_max), -1, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    out_tokens = np.full((B, n_max), -1, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if n == 0 or (err_in is not None and int(err_in[b]) != 0):
            continue
        par = [int(x) for x in parents[b, :n]]
        dists = [next_token_distribution(logits[b, i]) for i in range(n)]
        for i in range(n):
            entropy[b, i] = dists[i][1]
            tgt_argmax[b, i] = dists[i][2]
        p_tok[b, 0] = 1.0
        for c in range(1, n):
            t = int(cand_tok[b, c])
            p_tok[b, c] = dists[par[c]][0][t] if 0 <= t < V else 0.0
        ok = [False] * n
        ok[0] = True
        for c in range(1, n):
            floor = min(epsilon, delta * math.exp(-entropy[b, par[c]]))
            ok[c] = ok[par[c]] and p_tok[b, c] > floor
        dep = tree_depth(par)
        best = 0
        for i in range(n):
            if ok[i] and dep[i] > dep[best]:
                best = i
        p = ancestors_or_self(par, best)
        L = dep[best]
        accept_len[b] = L
        path[b, :L + 1] = p
        bonus[b] = tgt_argmax[b, best]
        out_tokens[b, :L + 1] = [int(cand_tok[b, a]) for a in p[1:]] + [bonus[b]]
    return entropy, p_tok, tgt_argmax, accept_len, path, bonus, out_tokens


# ---------------------------------------------------------------------------
# Commit of the accepted path's KV; sibling branches are dropped
# ---------------------------------------------------------------------------

def commit(k_cache, v_cache, prefix_len, accept_len, path):
    """Keep only the accepted path's KV ([INFRA-5.3] section 3.2 and summary).

    The tree's KV sits in slots [P_b, P_b + n_b) in flattened order. The node at
    depth d of the accepted path moves to slot P_b + d (all KV heads, K and V),
    so the prefix grows by accept_len + 1 entries and the slots after it are
    free. The move is a simultaneous assignment: every source is read from the
    cache as it was before the call. A node at depth d was rotated at position
    P_b + d, which is exactly its new slot, so the move is a plain copy.
    Sequences with accept_len < 0 are left unchanged.

    Returns (k_after, v_after, prefix_len_out).
    """
    k_old = np.array(k_cache, copy=True)
    v_old = np.array(v_cache, copy=True)
    k_new = np.array(k_cache, copy=True)
    v_new = np.array(v_cache, copy=True)
    B = k_cache.shape[0]
    plen = np.array(prefix_len, dtype=np.int32, copy=True)
    for b in range(B):
        L = int(accept_len[b])
        if L < 0:
            continue
        P = int(prefix_len[b])
        for d in range(L + 1):
            src = P + int(path[b, d])
            k_new[b, :, P + d, :] = k_old[b, :, src, :]
            v_new[b, :, P + d, :] = v_old[b, :, src, :]
        plen[b] = P + L + 1
    return k_new, v_new, plen


# ---------------------------------------------------------------------------
# Chain speculative sampling: keep with probability min(1, p/q), else resample
# ---------------------------------------------------------------------------

def softmax64(logits_row):
    """Plain float64 softmax of one row of logits."""
    x = np.asarray(logits_row, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def inverse_cdf(weights, u):
    """The first index whose running sum of weights exceeds u * total: a draw
    from the distribution proportional to weights, for u uniform in [0, 1)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    t = u * c[-1]
    return int(min(np.searchsorted(c, t, side="right"), len(c) - 1))


def speculative_sample(p_logits, q_logits, draft, u_acc, u_res):
    """Chain speculative sampling of one draft ([DRAFTERS] "Why the answer does
    not change"; [MEDUSA-EAGLE] on lossless verification).

    Drafted token x_i (i < L) is kept with probability min(1, p_i(x_i) /
    q_i(x_i)), p_i the target's and q_i the draft's distribution at position
    i; checking stops at the first rejection j. The step then emits a token
    drawn from the target's distribution with the draft's subtracted,
    max(0, p_j - q_j) normalised, or, when all L are kept, from p_L.

    Readings: distributions are plain softmaxes of the logits; the draws are
    inputs (u_acc[i] for position i: keep iff u_acc[i] * q_i(x_i) < p_i(x_i),
    which is u < min(1, p/q) for u in [0, 1); u_res for the final draw, by
    inverse CDF over token ids in ascending order).

    p_logits [L+1][V], q_logits [L][V], draft [L], u_acc [L], u_res scalar.
    Returns (accepted, tokens [L+1] (-1 padded), p_tok [L], q_tok [L]).
    """
    L = len(draft)
    p_tok = np.zeros(L)
    q_tok = np.zeros(L)
    j = L
    for i in range(L):
        p = softmax64(p_logits[i])
        q = softmax64(q_logits[i])
        x = int(draft[i])
        p_tok[i], q_tok[i] = p[x], q[x]
        if not u_acc[i] * q[x] < p[x]:
            j = i
            break
    for i in range(j + 1, L):      # (not checked, reported for completeness)
        p_tok[i] = softmax64(p_logits[i])[int(draft[i])]
        q_tok[i] = softmax64(q_logits[i])[int(draft[i])]
    if j < L:
        w = np.maximum(softmax64(p_logits[j]) - softmax64(q_logits[j]), 0.0)
    else:
        w = softmax64(p_logits[L])
    tokens = np.full(L + 1, -1, dtype=np.int32)
    tokens[:j] = draft[:j]
    tokens[j] = inverse_cdf(w, u_res)
    return j, tokens, p_tok, q_tok


# ---------------------------------------------------------------------------
# EAGLE-2 dynamic draft tree: expansion by path value, rerank, flatten
# ---------------------------------------------------------------------------

def eagle2_tree(conf, cand, root_tok, n_max):
    """Builds one dynamic draft tree ([INFRA-5.3] section 5.2).

    A node's value is the product of the draft's confidences along its path
    from the root (the root, the last verified token, has value 1). The
    expansion phase grows, at each of S steps, the K highest-valued nodes of
    the newest layer, each by the M children the draft proposes for it; the
    rerank phase keeps the n_max - 1 highest-valued nodes of all created
    ones, plus the root, for verification.

    Inputs (the draft's proposals, given rather than computed):
      conf [S][K][M] float32: confidence of child c of the k-th expanded node
        (in value order) at step s; cand [S][K][M] int32: that child's token.
    Readings: values are float32 products v(parent) * c, rounded once per
    node; confidences are clamped into [0, 1] (NaN counts as 0), so values
    never grow along a path; ties in value go to the node created first
    (at a step, children in (k, c) order), in both phases; a layer with
    fewer than K nodes expands all of them; the kept nodes are flattened in
    creation order, which is depth order, so every parent precedes its
    children. With conf in [0, 1] the kept set is closed under ancestors (a
    parent is worth at least as much as its child and was created first).

    Returns (parents [n_max] int32, tokens [n_max] int32, values [n_max]
    float32, n) with n kept nodes and -1 / -1 / 0 padding.
    """
    S, K, M = conf.shape
    val = [np.float32(1.0)]
    par = [-1]
    tok = [int(root_tok)]
    layer = [0]
    for s in range(S):
        grow = sorted(layer, key=lambda i: (-val[i], i))[:K]
        new = []
        for k, p in enumerate(grow):
            for c in range(M):
                x = np.float32(conf[s, k, c])
                x = np.float32(0.0) if np.isnan(x) else min(max(x, np.float32(0.0)), np.float32(1.0))
                val.append(np.float32(val[p] * x))
                par.append(p)
                tok.append(int(cand[s, k, c]))
                new.append(len(val) - 1)
        layer = new
    kept = sorted(range(1, len(val)), key=lambda i: (-val[i], i))[:n_max - 1]
    order = [0] + sorted(kept)
    index = {old: new for new, old in enumerate(order)}
    n = len(order)
    parents = np.full(n_max, -1, dtype=np.int32)
    tokens = np.full(n_max, -1, dtype=np.int32)
    values = np.zeros(n_max, dtype=np.float32)
    for new_i, old in enumerate(order):
        parents[new_i] = -1 if old == 0 else index[par[old]]
        tokens[new_i] = tok[old]
        values[new_i] = val[old]
    return parents, tokens, values, n


# ---------------------------------------------------------------------------
# Paged KV: the cache of each sequence as a list of fixed-size pages
# ---------------------------------------------------------------------------

PAGE = 64   # slots per page


def gather_pages(k_pool, v_pool, block_table):
    """The dense per-sequence cache that a paged cache stands for.

    [INFRA-5.3] section 8 names the block table of a paged KV cache as what a
    real implementation adds: logical slot s of sequence b lives in page
    block_table[b][s // PAGE], at offset s % PAGE. Pools are slot-major here:
    k_pool and v_pool [num_pages][Hkv][PAGE][D]. Returns k, v
    [B][Hkv][max_pages * PAGE][D] (a copy).
    """
    B, max_pages = block_table.shape
    _, Hkv, page, D = k_pool.shape
    k = np.zeros((B, Hkv, max_pages * page, D), dtype=k_pool.dtype)
    v = np.zeros((B, Hkv, max_pages * page, D), dtype=v_pool.dtype)
    for b in range(B):
        for j in range(max_pages):
            pg = int(block_table[b, j])
            k[b, :, j * page:(j + 1) * page] = k_pool[pg]
            v[b, :, j * page:(j + 1) * page] = v_pool[pg]
    return k, v


def scatter_pages(k, v, block_table, k_pool, v_pool):
    """Writes a dense per-sequence cache back into (copies of) the pools: the
    inverse of gather_pages on the pages the table references. Pages that no
    sequence references keep their contents. Returns (k_pool, v_pool)."""
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    B, max_pages = block_table.shape
    page = kp.shape[2]
    for b in range(B):
        for j in range(max_pages):
            pg = int(block_table[b, j])
            kp[pg] = k[b, :, j * page:(j + 1) * page]
            vp[pg] = v[b, :, j * page:(j + 1) * page]
    return kp, vp


def verify_step(inputs: dict, rows=None) -> dict:
    """One whole verification step: tree set-up, attention, acceptance, commit.

    ``inputs`` holds float64 views of the tensors and the integer arrays (keys:
    parents, n_nodes, prefix_len, q, k_new, v_new, k_cache, v_cache, tok, tgt,
    rope_theta, softmax_scale).
    """
    anc, depth, err = build_tree(inputs["parents"], inputs["n_nodes"])
    out, kc, vc, err = tree_attention(
        inputs["q"], inputs["k_new"], inputs["v_new"], inputs["k_cache"],
        inputs["v_cache"], inputs["prefix_len"], inputs["n_nodes"],
        inputs["parents"], inputs["rope_theta"], inputs.get("softmax_scale", 0.0),
        err_in=err, rows=rows)
    acc_len, path, bonus, toks = accept(inputs["tok"], inputs["tgt"], inputs["parents"],
                                        inputs["n_nodes"], err_in=err)
    kc2, vc2, plen = commit(kc, vc, inputs["prefix_len"], acc_len, path)
    return dict(anc=anc, depth=depth, err=err, out=out, k_cache_attn=kc, v_cache_attn=vc,
                accept_len=acc_len, path=path, bonus=bonus, out_tokens=toks,
                k_cache=kc2, v_cache=vc2, prefix_len_out=plen)
