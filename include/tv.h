/*
 * tv.h -- C ABI of the draft-tree verification library (libtv.so, gfx950).
 *
 * One verification step of self-speculative decoding (Medusa / EAGLE): the
 * target model scores a whole flattened draft tree in one pass, keeps the
 * longest root path it agrees with, and keeps only that path's KV.
 *
 * Sources (web pages, cited by title and section):
 *   [MEDUSA-EAGLE] "Medusa and EAGLE: self-speculative decoding heads,
 *                  explained" (pofe.ai), "Medusa: heads, losses and trees".
 *   [MEDUSA-EXPL]  "Medusa, explained" (vibeengines.com), steps 6 and 7,
 *                  "Typical acceptance".
 *   [INFRA-5.3]    "5.3 Medusa、EAGLE 与 MTP" (infra-guide), sections 3.1,
 *                  3.2, 5.2, 8, 9.1 and 9.2.
 *   [DRAFTERS]     "Drafters: draft models, Medusa, EAGLE, MTP, DFlash,
 *                  DSpark" (robertz.co), "Why the answer does not change".
 *
 * Conventions for every call:
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     args struct of tv_tree_attention, which is host memory read during the
 *     call only. The library never allocates or frees device memory on these
 *     paths and keeps no per-call state.
 *   - Every call is asynchronous on the given HIP stream (0 = null stream)
 *     and never synchronises. The return value reports host-side argument
 *     checks and launch errors only.
 *   - Data-dependent problems are reported per sequence in a device array
 *     `err[B]` (0 = ok, TV_ERR_BAD_TREE, TV_ERR_CAPACITY, TV_ERR_BAD_PAGE).
 *     Later calls treat a sequence with err != 0 as inactive.
 *   - Trees: node 0 is the root (the last verified token), parents[b][0] ==
 *     -1 and 0 <= parents[b][i] < i for 1 <= i < n_nodes[b]; nodes
 *     n_nodes[b] .. n_max-1 are padding and ignored. n_nodes[b] == 0 marks an
 *     inactive sequence. At most TV_MAX_NODES nodes per tree.
 *   - Integer arrays are int32 unless noted; tensors are row-major in the
 *     shapes given, all of one dtype (TV_F32 or TV_BF16).
 *   - Environment: TV_ATTN_TUNE="waves=W qt=Q splits=S fused=F spin=T"
 *     (any subset) overrides the bf16 attention's launch plan (wavefronts
 *     per workgroup 2, 4 or 8, query tiles per wavefront 1 or 2, key splits
 *     1..16; fused=0 makes a separate kernel merge the key splits, fused=1
 *     merges up to eight splits in the attention kernel when its grid runs
 *     at once (automatic: up to four), fused=2 lets only the last split to
 *     arrive merge them; spin=T bounds the fused merge's wait for the other
 *     splits at T ticks of 10 ns, 0 = one look, default 20000), read once
 *     per process, for
 *     tuning sweeps; tv_tree_attention_workspace_size follows the same plan.
 *     Results do not depend on it beyond rounding order.
 */
#ifndef TV_H
#define TV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_MAX_NODES 64

typedef enum tv_status {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = 1,   /* null pointer, bad size or bad enum          */
  TV_ERR_BAD_TREE = 2,      /* per-sequence only: parents not a tree        */
  TV_ERR_CAPACITY = 3,      /* per-sequence only: prefix + tree > cache     */
  TV_ERR_UNSUPPORTED = 4,   /* valid but not implemented (e.g. head dim)    */
  TV_ERR_HIP = 5,           /* a HIP launch or runtime call failed          */
  TV_ERR_BAD_PAGE = 6,      /* per-sequence only: a block-table entry names
                               a page outside the pools                     */
  TV_ERR_SCRATCH = 7        /* tv_tree_attention_noalloc only: the shapes
                               need more scratch than its static buffer     */
} tv_status;

typedef enum tv_dtype { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Human-readable name of a status code (static string). */
const char* tv_status_string(tv_status s);

/* Library version string (static). */
const char* tv_version(void);

/*
 * tv_build_tree -- parents array -> ancestor bitmask and depth per node.
 *
 * Defines the tree mask of [INFRA-5.3] section 3.1 (a node sees the shared
 * prefix, its ancestors and itself; siblings and other branches are hidden)
 * and the depth-based position ids of section 3.2 / [MEDUSA-EXPL] step 6.
 *
 *   parents  [B][n_max]  parent index of each node (see conventions)
 *   n_nodes  [B]         live nodes per sequence, 0 <= n_nodes[b] <= n_max
 *   anc      [B][n_max]  uint64 out: bit j set iff node j is node i or an
 *                        ancestor of it (least significant bit = node 0)
 *   depth    [B][n_max]  out: edges from the root (root = 0)
 *   err      [B]         out: 0, or TV_ERR_BAD_TREE if the tree is not laid
 *                        out parents-first or n_nodes is out of range
 * Padding nodes, and every node of a bad tree, get anc = 0 and depth = 0.
 * Host checks: pointers non-null (unless B == 0), B >= 0,
 * 1 <= n_max <= TV_MAX_NODES. B == 0 is a no-op.
 */
tv_status tv_build_tree(const int32_t* parents, const int32_t* n_nodes, int32_t B,
                        int32_t n_max, uint64_t* anc, int32_t* depth, int32_t* err,
                        hipStream_t stream);

/*
 * tv_eagle2_tree -- an EAGLE-2 dynamic draft tree from the draft's proposals.
 *
 * [INFRA-5.3] section 5.2: a node's value is the product of the draft's
 * confidences along its path from the root (the root, the last verified
 * token, is worth 1); the expansion grows, at each of S steps, the K best
 * nodes of the newest layer by the M children the draft proposes for each;
 * the rerank keeps the n_max - 1 best of all created nodes, plus the root,
 * for verification. Readings fixed here: values are float32 products
 * v(parent) * c, c the confidence clamped into [0, 1] (NaN counts as 0);
 * ties in value go to the node created first (a step creates its children
 * in (k, c) order), in both phases; a layer with fewer than K nodes grows
 * all of them. The kept nodes are numbered in creation order (= depth
 * order), so the output is a parents-first tree for tv_build_tree.
 *
 *   conf     [B][S][K][M] float  confidence of child c of the k-th best node
 *                                of the newest layer at step s
 *   cand     [B][S][K][M]        that child's token
 *   root_tok [B]                 token of the root
 *   parents  [B][n_max] out      parent of each kept node (-1 for the root),
 *                                -1 padding
 *   tokens   [B][n_max] out      token of each kept node, -1 padding
 *   values   [B][n_max] float out  its path value, 0 padding
 *   n_nodes  [B] out             kept nodes, min(n_max, nodes created)
 * Host checks: pointers non-null unless B == 0, B >= 0, S, K, M >= 1,
 * 1 <= n_max <= TV_MAX_NODES; S * K * M <= TV_MAX_DRAFT_PROPOSALS, else
 * TV_ERR_UNSUPPORTED. B == 0 is a no-op.
 */
#define TV_MAX_DRAFT_PROPOSALS 512
tv_status tv_eagle2_tree(const float* conf, const int32_t* cand, const int32_t* root_tok, int32_t B,
                         int32_t S, int32_t K, int32_t M, int32_t n_max, int32_t* parents,
                         int32_t* tokens, float* values, int32_t* n_nodes, hipStream_t stream);

/*
 * tv_tree_attention -- tree-masked GQA attention of every tree node over the
 * shared-prefix KV cache plus its own ancestors, one attention layer.
 *
 * For node i of sequence b (P = prefix_len[b]) and query head h, with KV head
 * g = h / (Hq / Hkv): the keys are the P prefix keys of head g followed by the
 * keys of the nodes on the root..i path, RoPE-rotated at position P + depth;
 * the query is rotated at P + depth[i]; output = softmax(scale * q.K) V.
 * This is [INFRA-5.3] sections 3.1-3.2 and [MEDUSA-EAGLE] ("Trees"): every
 * node shares the prefix KV and sees only its ancestors.
 *
 * Cache layouts: K is slot-major, [B][Hkv][cap][D]. V is stored in blocks
 * of 64 slots, head-dim-major inside a block, [B][Hkv][cap/64][D][64], so that
 * 64 consecutive slots of one head dim are contiguous (the order in which the
 * value product consumes them); cap must be a multiple of 64.
 *
 * Side effect (the tree's temporary KV, [INFRA-5.3] section 3.2): cache slots
 * [P, P + n_nodes[b]) of every KV head receive the rotated tree keys and the
 * raw tree values in flattened node order (rounded to the cache dtype).
 * Prefix slots [0, P) are read only; they must already hold rotated keys.
 */
typedef struct tv_attn_args {
  const void* q;          /* [B][n_max][Hq][D]   tree queries, before RoPE   */
  const void* k_new;      /* [B][n_max][Hkv][D]  tree keys, before RoPE      */
  const void* v_new;      /* [B][n_max][Hkv][D]  tree values                 */
  void* k_cache;          /* [B][Hkv][cap][D]    prefix keys (rotated)       */
  void* v_cache;          /* [B][Hkv][cap/64][D][64]  prefix values, blocked:
                             slot s, dim d at ((s/64)*D + d)*64 + s%64      */
  const int32_t* prefix_len;  /* [B] P, 0 <= P                               */
  const int32_t* n_nodes;     /* [B]                                         */
  const uint64_t* anc;        /* [B][n_max] from tv_build_tree               */
  const int32_t* depth;       /* [B][n_max] from tv_build_tree               */
  int32_t* err;               /* [B] in/out: sequences with err != 0 are
                                 skipped (output rows zero); set to
                                 TV_ERR_CAPACITY when P + n_nodes > cap      */
  void* out;              /* [B][n_max][Hq][D]   attention output; rows of
                             padding nodes and skipped sequences are zero    */
  void* workspace;        /* device scratch, >= tv_tree_attention_workspace_size
                             bytes (may be NULL when that size is 0). Its
                             first 16 KiB (when the size is not 0) hold
                             synchronisation words of the split merge: zero
                             them before the first use; every call leaves
                             them zero again (the rest needs no initial
                             contents). Calls that may run at the same time
                             need separate workspaces.                      */
  size_t workspace_bytes;
  int32_t B, n_max, Hq, Hkv, D, cap;
  int32_t dtype;          /* tv_dtype                                        */
  float rope_theta;       /* RoPE base (rotate-half pairing); 0 = no RoPE    */
  float softmax_scale;    /* <= 0 selects 1/sqrt(D)                          */
} tv_attn_args;

/*
 * Workspace bytes tv_tree_attention needs for these shapes (0 if none).
 * Depends only on B, n_max, Hq, Hkv, D, cap and dtype. Returns 0 and leaves
 * nothing set for arguments tv_tree_attention would reject.
 */
size_t tv_tree_attention_workspace_size(const tv_attn_args* a);

/*
 * Host checks: a non-null; tensor pointers non-null unless B == 0;
 * 1 <= n_max <= TV_MAX_NODES; Hq % Hkv == 0; D in {64, 128} (TV_BF16 at
 * D == 128 runs the matrix-core kernels and needs a query-head group
 * Hq / Hkv of at most 4096; fp32, and bf16 at D == 64, run a tree-append
 * kernel and a second attention kernel (fp32 or bf16 matrix products,
 * streaming the cache after the append) that need no workspace), else
 * TV_ERR_UNSUPPORTED; cap >= n_max and
 * cap % 64 == 0; workspace large enough. B == 0 is a no-op.
 */
tv_status tv_tree_attention(const tv_attn_args* a, hipStream_t stream);

/*
 * tv_tree_attention_from_parents -- tv_build_tree and tv_tree_attention in
 * one launch (bf16; fp32 makes the two launches). The tree mask and depths
 * are those of infra-guide "5.3 Medusa、EAGLE 与 MTP", sections 3.1, 3.2 and
 * 8; the attention is tv_tree_attention's.
 *   a         as for tv_tree_attention, except that a->anc and a->depth are
 *             not read, and a->err is output only: it receives what
 *             tv_build_tree writes (0 or TV_ERR_BAD_TREE), then
 *             TV_ERR_CAPACITY as tv_tree_attention sets it
 *   parents   [B][n_max] int32 parent of each node (-1 for the root), as for
 *             tv_build_tree
 *   anc       [B][n_max] uint64 out: ancestors-or-self bitmasks
 *   depth     [B][n_max] int32 out: depths
 * anc, depth, err, out and the cache append are bit for bit those of
 * tv_build_tree followed by tv_tree_attention; the pair feeds tv_accept /
 * tv_accept_commit as usual.
 * Host checks: those of tv_tree_attention, and parents, anc and depth
 * non-null unless B == 0. tv_tree_attention_paged_from_parents is the
 * paged-cache form.
 */
tv_status tv_tree_attention_from_parents(const tv_attn_args* a, const int32_t* parents, uint64_t* anc,
                                         int32_t* depth, hipStream_t stream);

/*
 * tv_tree_attention_noalloc -- tv_tree_attention for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, computation, outputs and
 * host checks as tv_tree_attention, except that a->workspace and
 * a->workspace_bytes are ignored: the workspace is a static device buffer of
 * the library (48 MiB per device, zero when the library's module loads,
 * held until the process ends; its address is looked up once per device on
 * the first call with that device current). The call allocates nothing.
 * Shapes whose workspace (tv_tree_attention_workspace_size) exceeds 48 MiB
 * return TV_ERR_SCRATCH before any device work; the workloads of this
 * library need at most about 35 MB. All calls on one device share that
 * device's buffer, which keeps the last call's contents: calls that may
 * overlap on one device (other streams, other host threads) race and must
 * not be issued. Kernels and launch plan are those of tv_tree_attention, so
 * the results are the same bit for bit.
 */
tv_status tv_tree_attention_noalloc(const tv_attn_args* a, hipStream_t stream);

/*
 * Paged KV cache ([INFRA-5.3] section 8 names the block table of a paged KV
 * cache as what a real implementation adds to the dense sketch).
 *
 * The cache is a pool of pages of 64 slots (the V block size): K pages
 * [num_pages][Hkv][64][D] (slot-major within a page) and V pages
 * [num_pages][Hkv][D][64] (head-dim-major, as one block of the dense V
 * layout). Logical slot s of sequence b is slot s % 64 of page
 * block_table[b * max_pages + s / 64]. A sequence's capacity is
 * 64 * max_pages slots. Pages that only hold prefix slots (below P) are read
 * only and may be shared by several sequences; the pages holding slots
 * [P, P + n_nodes) are written (tree append, commit) and must belong to one
 * sequence. Entries past a sequence's P + n_nodes slots are never read.
 */
#define TV_MAX_PAGES_PER_SEQ 256

typedef struct tv_paged_kv {
  const int32_t* block_table;  /* [B][max_pages] page ids, device memory     */
  int32_t max_pages;           /* 1 .. TV_MAX_PAGES_PER_SEQ (attention)      */
  int32_t num_pages;           /* pages in each pool                         */
} tv_paged_kv;

/*
 * tv_tree_attention_paged -- tv_tree_attention over a paged cache.
 *
 * Same computation, arguments and side effect as tv_tree_attention, except
 * that a->k_cache and a->v_cache are the K and V page pools and a->cap must
 * equal 64 * pk->max_pages; the workspace is tv_tree_attention_workspace_size
 * of the same arguments. A sequence whose blocks [0, (P + n) / 64] name a page
 * outside [0, num_pages) gets err = TV_ERR_BAD_PAGE and zero output rows;
 * no page outside the pools is read or written.
 * Host checks as tv_tree_attention, plus pk non-null with a non-null table,
 * max_pages >= 1, num_pages >= 1, a->cap == 64 * max_pages; TV_BF16 at D == 128 only and
 * max_pages <= TV_MAX_PAGES_PER_SEQ, else TV_ERR_UNSUPPORTED.
 */
tv_status tv_tree_attention_paged(const tv_attn_args* a, const tv_paged_kv* pk,
                                  hipStream_t stream);

/*
 * tv_tree_attention_paged_from_parents -- tv_build_tree and
 * tv_tree_attention_paged in one launch: the tree mask and depths of
 * infra-guide "5.3 Medusa、EAGLE 与 MTP" (sections 3.1, 3.2, 8) built inside
 * the attention kernel over a paged cache (the page-table layout and the
 * per-request tree boundaries of that page's section 8).
 *   a, pk     as for tv_tree_attention_paged, except that a->anc and
 *             a->depth are not read, and a->err is output only: it receives
 *             TV_ERR_BAD_TREE as tv_build_tree writes it, else
 *             TV_ERR_CAPACITY, else TV_ERR_BAD_PAGE as
 *             tv_tree_attention_paged sets them, else 0
 *   parents, anc, depth  as for tv_tree_attention_from_parents
 * anc, depth, err, out and the append into the pages are bit for bit those of
 * tv_build_tree followed by tv_tree_attention_paged.
 * Host checks: those of tv_tree_attention_paged, and parents, anc and depth
 * non-null unless B == 0.
 */
tv_status tv_tree_attention_paged_from_parents(const tv_attn_args* a, const tv_paged_kv* pk, const int32_t* parents,
                                               uint64_t* anc, int32_t* depth, hipStream_t stream);

/*
 * tv_accept -- greedy longest-accepted-path selection.
 *
 * Under greedy decoding a drafted token is kept iff it equals the target's
 * own argmax ([MEDUSA-EAGLE] "Typical acceptance", [DRAFTERS]); the longest
 * fully valid root path is kept ([MEDUSA-EXPL] step 7); checking stops at the
 * first miss on a path ([INFRA-5.3] section 9.2). Readings fixed here:
 *   - tgt_argmax[b][i] is the target's argmax computed AT node i (it predicts
 *     the token after i); node c >= 1 is valid iff cand_tok[b][c] ==
 *     tgt_argmax[b][parent(c)], and accepted iff valid and its parent is
 *     accepted; the root is always accepted;
 *   - the deepest accepted node e wins; equal depths go to the lower index;
 *   - accept_len = depth(e) = accepted drafted tokens; the step emits
 *     accept_len + 1 tokens, the last being the bonus tgt_argmax[b][e].
 *
 *   cand_tok   [B][n_max]  token of each node ([0] = root token, unused)
 *   tgt_argmax [B][n_max]
 *   parents, anc, depth, n_nodes as from tv_build_tree
 *   err        [B] or NULL: sequences with err != 0 are skipped
 *   accept_len [B]         out; -1 for skipped or empty sequences
 *   path       [B][n_max]  out: nodes root..e (ascending), then -1
 *   bonus_tok  [B]         out; -1 for skipped sequences
 *   out_tokens [B][n_max]  out, may be NULL: the accept_len + 1 emitted
 *                          tokens (drafted tokens of path[1..], then bonus),
 *                          then -1
 * Host checks as tv_build_tree. B == 0 is a no-op.
 */
tv_status tv_accept(const int32_t* cand_tok, const int32_t* tgt_argmax,
                    const int32_t* parents, const uint64_t* anc, const int32_t* depth,
                    const int32_t* n_nodes, const int32_t* err, int32_t B, int32_t n_max,
                    int32_t* accept_len, int32_t* path, int32_t* bonus_tok,
                    int32_t* out_tokens, hipStream_t stream);

/*
 * tv_accept_typical -- typical acceptance, longest accepted path.
 *
 * A drafted token passes iff the target gives it probability above
 * min(epsilon, delta * exp(-H)), H being the entropy of the target's
 * distribution at that point ([MEDUSA-EXPL] "Typical acceptance",
 * [MEDUSA-EAGLE] "Typical acceptance", [INFRA-5.3] section 9.1); the first
 * token of a step is the target's own greedy choice. Readings fixed here:
 *   - logits[b][i] are the target's next-token logits AT node i; the
 *     distribution is their plain softmax (a caller sampling at temperature
 *     T passes logits / T); node c >= 1 is judged under its parent's
 *     distribution, H in nats, the comparison strict;
 *   - a node is accepted iff its parent is and its token passes; the root
 *     always is; the deepest accepted node e wins, equal depths going to the
 *     lower index; accept_len = depth(e); the bonus token is the target's
 *     argmax at e (lowest token id among equal maxima);
 *   - a token id outside [0, vocab) has probability 0 and never passes.
 *
 *   logits     [B][n_max][vocab] of dtype (TV_BF16 or TV_F32), finite, all of
 *              it readable; each live row is read once. A row's first
 *              64 KiB go out before the node count is known, so rows of
 *              padding nodes and skipped sequences may be read that far,
 *              never further, and are otherwise ignored. 16-byte aligned
 *              rows (vocab * element size a multiple of 16, aligned base)
 *              take the vector path; others work too.
 *   cand_tok, parents, anc, depth, n_nodes, err as for tv_accept
 *   epsilon, delta  the two thresholds (not NaN)
 *   entropy    [B][n_max] float out: H at node i (nats)
 *   p_tok      [B][n_max] float out: probability of node i's token under its
 *              parent's distribution; 1 for the root
 *   tgt_argmax [B][n_max] out: the target's argmax at node i
 *              (padding nodes and skipped sequences: entropy 0, p_tok 0,
 *              tgt_argmax -1; with err == NULL and a tree that is not laid
 *              out parents-first, p_tok entries are unspecified)
 *   accept_len, path, bonus_tok, out_tokens  as for tv_accept
 * Two kernels on the stream: per-node statistics, then the tree scan.
 * Host checks: pointers non-null (err and out_tokens may be NULL) unless
 * B == 0, 0 <= B <= 65535, 1 <= n_max <= TV_MAX_NODES, vocab >= 1, dtype
 * valid. B == 0 is a no-op.
 */
tv_status tv_accept_typical(const void* logits, int32_t dtype, int32_t vocab,
                            const int32_t* cand_tok, const int32_t* parents, const uint64_t* anc,
                            const int32_t* depth, const int32_t* n_nodes, const int32_t* err,
                            int32_t B, int32_t n_max, float epsilon, float delta, float* entropy,
                            float* p_tok, int32_t* tgt_argmax, int32_t* accept_len, int32_t* path,
                            int32_t* bonus_tok, int32_t* out_tokens, hipStream_t stream);

/*
 * tv_speculative_sample -- chain speculative sampling of L drafted tokens.
 *
 * [DRAFTERS] "Why the answer does not change": drafted token x_i is kept with
 * probability min(1, p_i(x_i) / q_i(x_i)), p the target's and q the draft's
 * distribution at position i; at the first rejection j the step emits a
 * token drawn from the target's distribution with the draft's subtracted,
 * max(0, p_j - q_j) normalised, or, when all L are kept, from p_L. The
 * output is then distributed as sampling from the target alone. Readings
 * fixed here: distributions are plain softmaxes of the logits (a caller
 * sampling at temperature T passes logits / T); the uniform draws are
 * inputs: token i is kept iff u_acc[i] * q_i(x_i) < p_i(x_i) (u in [0, 1)),
 * and the final token is the first id (ascending) whose running weight
 * exceeds u_res * total weight; a drafted id outside [0, vocab) has
 * probability 0 under both.
 *
 *   p_logits  [B][L + 1][vocab]  target logits at the L drafted positions and
 *                                after them; dtype TV_BF16 or TV_F32, finite
 *   q_logits  [B][L][vocab]      draft logits at the L drafted positions
 *   draft     [B][L]             drafted tokens
 *   u_acc     [B][L] float, u_res [B] float   uniform draws in [0, 1)
 *   p_tok, q_tok [B][L] float out  p_i(x_i) and q_i(x_i)
 *   accept_len [B] out           kept drafted tokens j (0 .. L)
 *   tokens    [B][L + 1] out     the j kept tokens, the drawn token, then -1
 *   workspace                    >= tv_speculative_sample_workspace_size(B, L)
 *                                bytes of device scratch (row statistics)
 * Two kernels: per-row statistics (grid (2L + 1, B)), then one workgroup per
 * sequence for the decisions and the draw. Host checks: pointers non-null
 * unless B == 0, 0 <= B <= 65535, 1 <= L <= TV_MAX_NODES, vocab >= 1, dtype
 * valid, workspace large enough. B == 0 is a no-op.
 */
size_t tv_speculative_sample_workspace_size(int32_t B, int32_t L);
tv_status tv_speculative_sample(const void* p_logits, const void* q_logits, int32_t dtype, int32_t vocab,
                                const int32_t* draft, const float* u_acc, const float* u_res, int32_t B,
                                int32_t L, float* p_tok, float* q_tok, int32_t* accept_len,
                                int32_t* tokens, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * tv_commit -- keep the accepted path's KV in place, drop the other branches.
 *
 * [INFRA-5.3] section 3.2 and summary: only the accepted path is committed.
 * For each sequence with accept_len[b] = L >= 0 and P = prefix_len_in[b]:
 * slot P + d <- slot P + path[b][d] for d = 0..L, every KV head, K and V, as
 * one simultaneous move (all sources read before any slot is written); then
 * prefix_len_out[b] = P + L + 1. Sequences with L < 0 are copied through
 * unchanged. Slots from P + L + 1 on are left as they were (free space).
 *
 *   k_cache [B][Hkv][cap][D], v_cache [B][Hkv][cap/64][D][64]  in place
 *                    (the layouts of tv_tree_attention)
 *   prefix_len_in    [B]
 *   accept_len, path as from tv_accept (path rows of length n_max)
 *   prefix_len_out   [B] out; may be the same array as prefix_len_in
 * Host checks: pointers non-null unless B == 0, Hkv >= 1, D in {64, 128},
 * 1 <= n_max <= TV_MAX_NODES, cap >= n_max, cap % 64 == 0, dtype valid. Device side,
 * a path entry outside [0, n_max), accept_len outside [0, n_max), or a move
 * that would read or write outside [P, cap) leaves that sequence unchanged
 * (prefix_len_out = prefix_len_in). Any path with entries in [0, n_max) is
 * moved as the simultaneous copy above (tv_accept's paths are strictly
 * increasing, but the copy does not rely on it).
 */
tv_status tv_commit(void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t cap,
                    int32_t D, int32_t dtype, const int32_t* prefix_len_in,
                    const int32_t* accept_len, const int32_t* path, int32_t n_max,
                    int32_t* prefix_len_out, hipStream_t stream);

/*
 * tv_accept_commit -- tv_accept followed by tv_commit, in one launch.
 *
 * The greedy selection of tv_accept ([MEDUSA-EAGLE] "Typical acceptance",
 * [MEDUSA-EXPL] step 7) and the in-place commit of the accepted path's KV of
 * tv_commit ([INFRA-5.3] section 3.2 and summary) for the dense cache, with
 * the arguments of both: the accept outputs are the same, and for each
 * sequence with accept_len = L >= 0 slot P + d <- slot P + path[d] (d = 0..L,
 * every KV head, K and V, all sources read before any slot is written),
 * prefix_len_out[b] = P + L + 1. Sequences tv_accept skips (accept_len -1),
 * or whose path would move a slot outside [P, cap), keep their cache and
 * prefix length. prefix_len_out may be the same array as prefix_len_in
 * (then one workgroup per sequence walks every KV head; otherwise one per
 * KV head and sequence). Host checks as tv_accept and tv_commit.
 * B == 0 is a no-op.
 */
tv_status tv_accept_commit(const int32_t* cand_tok, const int32_t* tgt_argmax, const int32_t* parents,
                           const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                           const int32_t* err, int32_t B, int32_t n_max, int32_t* accept_len, int32_t* path,
                           int32_t* bonus_tok, int32_t* out_tokens, void* k_cache, void* v_cache, int32_t Hkv,
                           int32_t cap, int32_t D, int32_t dtype, const int32_t* prefix_len_in,
                           int32_t* prefix_len_out, hipStream_t stream);

/*
 * tv_commit_paged -- tv_commit over a paged cache (see tv_tree_attention_paged
 * for the layout): slot P + d <- slot P + path[b][d], d = 0..L, through the
 * block table. A move touching a page outside the pools leaves that sequence
 * unchanged (prefix_len_out = prefix_len_in). Host checks as tv_commit with
 * cap = 64 * pk->max_pages, plus pk non-null with a non-null table,
 * max_pages >= 1, num_pages >= 1.
 */
tv_status tv_commit_paged(void* k_pool, void* v_pool, const tv_paged_kv* pk, int32_t B,
                          int32_t Hkv, int32_t D, int32_t dtype, const int32_t* prefix_len_in,
                          const int32_t* accept_len, const int32_t* path, int32_t n_max,
                          int32_t* prefix_len_out, hipStream_t stream);

/*
 * tv_accept_commit_paged -- tv_accept followed by tv_commit_paged, in one
 * launch: the arguments, outputs and effect of tv_accept_commit with the K
 * and V page pools and block table of tv_commit_paged instead of the dense
 * cache (cap = 64 * pk->max_pages). A move touching a page outside the pools
 * leaves that sequence's cache and prefix length unchanged, as with
 * tv_commit_paged; the accept outputs are written regardless.
 * Host checks as tv_accept_commit and tv_commit_paged, plus
 * max_pages <= TV_MAX_PAGES_PER_SEQ, else TV_ERR_UNSUPPORTED.
 */
tv_status tv_accept_commit_paged(const int32_t* cand_tok, const int32_t* tgt_argmax, const int32_t* parents,
                                 const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                                 const int32_t* err, int32_t B, int32_t n_max, int32_t* accept_len, int32_t* path,
                                 int32_t* bonus_tok, int32_t* out_tokens, void* k_pool, void* v_pool,
                                 const tv_paged_kv* pk, int32_t Hkv, int32_t D, int32_t dtype,
                                 const int32_t* prefix_len_in, int32_t* prefix_len_out, hipStream_t stream);

/*
 * tv_v_cache_layout -- converts a V cache between the row layout a model's
 * KV cache usually has and the blocked layout the calls above read.
 * Not an operation of the pages: the blocked layout is this library's (it
 * gives the attention's value-times-probability product contiguous 64-key
 * runs per head dim), and this call lets a caller that holds rows convert
 * once, when the prefix is written, instead of per step.
 *   rows:    [n][cap][D]       slot s, dim d at s*D + d
 *   blocked: [n][cap/64][D][64] slot s, dim d at ((s/64)*D + d)*64 + s%64
 * n = B*Hkv for a dense cache ([B][Hkv][...]); for page pools n =
 * num_pages*Hkv and cap = 64 (a page's V is one block).
 *   src, dst    device buffers of n*cap*D elements of dtype, 16-byte
 *               aligned, not overlapping (the conversion is out of place);
 *               the caller owns both.
 *   to_rows     0: rows -> blocked; 1: blocked -> rows.
 * One kernel on stream (a 64 x D transpose per block through LDS; each byte
 * read and written once). TV_ERR_INVALID_ARG for n < 0, cap not a positive
 * multiple of 64, a bad dtype or to_rows, null, misaligned or overlapping
 * buffers; TV_ERR_UNSUPPORTED for D other than 64 or 128 or more than
 * 2^31 - 1 blocks. n == 0 launches nothing.
 */
tv_status tv_v_cache_layout(const void* src, void* dst, int64_t n, int32_t cap, int32_t D, int32_t dtype,
                            int32_t to_rows, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H */
