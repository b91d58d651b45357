// Tree set-up, acceptance and KV commit: the integer side of a verification
// step. One 64-lane wavefront per sequence; lane i is node i.
//
// Tree mask and depth positions: infra-guide "5.3 Medusa、EAGLE 与 MTP",
// sections 3.1, 3.2 and 8. Acceptance: pofe.ai "Medusa and EAGLE ...",
// greedy case of "Typical acceptance"; vibeengines.com "Medusa, explained",
// step 7 and "Typical acceptance"; infra-guide sections 9.1 and 9.2. Commit:
// infra-guide section 3.2 and summary.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

// ---------------------------------------------------------------------------
// build_tree: ancestors-or-self bitmask and depth by pointer jumping
// (build_tree_lane), one wavefront per sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void build_tree_kernel(const int32_t* __restrict__ parents,
                                                        const int32_t* __restrict__ n_nodes,
                                                        int n_max, uint64_t* __restrict__ anc,
                                                        int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ err) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  // (the parent load does not wait for the node count: one memory round trip)
  const int p_in = i < n_max ? parents[static_cast<size_t>(b) * n_max + i] : -1;
  const int n = n_nodes[b];
  const LaneTree t = build_tree_lane(p_in, n, n_max, i);
  if (i < n_max) {
    anc[static_cast<size_t>(b) * n_max + i] = t.anc;
    depth[static_cast<size_t>(b) * n_max + i] = t.depth;
  }
  if (i == 0) err[b] = t.ok ? 0 : static_cast<int32_t>(TV_ERR_BAD_TREE);
}

// ---------------------------------------------------------------------------
// accept: the root always matches. Greedy rule: node c >= 1 matches iff its
// token equals the target's choice at its parent. Typical rule: node c >= 1
// matches iff the target's probability of its token at its parent, p_tok[c],
// exceeds min(eps, delta * exp(-H(parent))). A node is accepted iff every
// node in its ancestors-or-self mask matches, i.e. (anc & ~match_mask) == 0.
// The deepest accepted node wins (ties: lowest index); its mask, read bit by
// bit in ascending order, is the path. The bonus token is tgt at that node
// (the target's argmax there, for both rules).
// ---------------------------------------------------------------------------
// The accept's inputs of node i (lane i) and of its sequence. Every load is
// unconditional (the node index is clamped into the row; lanes past n_max
// are masked when the inputs are used), so all of them go out together,
// before the first wait, and none is moved behind a branch.
struct AcceptIn {
  uint64_t a;
  int p, tk, tg, dp, n, e;
  float pt, h;
};

template <bool TYPICAL>
__device__ __forceinline__ AcceptIn accept_load(
    const int32_t* __restrict__ cand_tok, const int32_t* __restrict__ tgt,
    const int32_t* __restrict__ parents, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ err, int n_max, const float* __restrict__ p_tok,
    const float* __restrict__ entropy, int b, int i) {
  const size_t at = static_cast<size_t>(b) * n_max + min(i, n_max - 1);
  AcceptIn in;
  in.p = parents[at];
  in.tk = cand_tok[at];
  in.tg = tgt[at];
  in.a = anc[at];
  in.dp = depth[at];
  if constexpr (TYPICAL) {
    in.pt = p_tok[at];
    in.h = entropy[at];
  } else {
    in.pt = in.h = 0.f;
  }
  in.n = n_nodes[b];
  in.e = err ? err[b] : 0;
  return in;
}

// Accept of sequence b by one wavefront (lane i = node i) from its loaded
// inputs; writes the outputs (if `write`) and returns the accepted length
// (-1: skipped) in every lane, and in `on_pos` the path position of node i
// (-1 if i is not on the path).
template <bool TYPICAL>
__device__ __forceinline__ int accept_decide(
    const AcceptIn& in, int n_max, int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
    int32_t* __restrict__ bonus, int32_t* __restrict__ out_tokens, float eps, float delta, int b, int i,
    int& on_pos, bool write = true) {
  on_pos = -1;
  const size_t row = static_cast<size_t>(b) * n_max;
  const int n = in.n;
  bool active = (in.e == 0) && (n > 0) && (n <= n_max);

  const bool live = active && (i < n);
  const int p = live ? in.p : -1;
  const int tk = live ? in.tk : 0;
  const int tg = live ? in.tg : 0;
  const uint64_t a = live ? in.a : 0ull;
  const int dp = live ? in.dp : 0;

  // every lane takes part in the shuffles (none sits behind a branch)
  const int src = (p >= 0 && p < 64) ? p : i;
  const int tg_parent = __shfl(tg, src);
  const float h_parent = TYPICAL ? __shfl(in.h, src) : 0.f;
  bool match;
  if constexpr (TYPICAL) {
    match = live && (i == 0 || in.pt > fminf(eps, delta * expf(-h_parent)));
  } else {
    match = live && (i == 0 || tk == tg_parent);
  }
  const uint64_t M = __ballot(match);
  const bool accepted = live && (a != 0ull) && ((a & ~M) == 0ull);
  int key = accepted ? ((dp << 8) | (255 - i)) : -1;
  key = wave_max_i32(key);
  if (key < 0) active = false;   // no accepted root: tree unusable

  if (!active) {
    if (write && i < n_max) {
      path[row + i] = -1;
      if (out_tokens) out_tokens[row + i] = -1;
    }
    if (write && i == 0) {
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    return -1;
  }
  const int e = 255 - (key & 255);
  const int L = key >> 8;
  const uint64_t ae = shfl_u64(a, e);
  const int bonus_tok = __shfl(tg, e);
  if (i < n_max) {
    const bool on = (ae >> i) & 1ull;
    const int pos = __popcll(ae & ((1ull << i) - 1ull));
    if (on) on_pos = pos;
  }
  if (write && i < n_max) {
    const bool on = (ae >> i) & 1ull;
    const int pos = __popcll(ae & ((1ull << i) - 1ull));
    if (on) path[row + pos] = i;
    if (i > L) path[row + i] = -1;
    if (out_tokens) {
      if (on && i != 0 && pos >= 1) out_tokens[row + pos - 1] = tk;
      if (i == L) out_tokens[row + i] = bonus_tok;
      if (i > L) out_tokens[row + i] = -1;
    }
  }
  if (write && i == 0) {
    accept_len[b] = L;
    bonus[b] = bonus_tok;
  }
  return L;
}

template <bool TYPICAL>
__global__ __launch_bounds__(64) void accept_kernel(
    const int32_t* __restrict__ cand_tok, const int32_t* __restrict__ tgt,
    const int32_t* __restrict__ parents, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ err, int n_max, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ bonus, int32_t* __restrict__ out_tokens,
    const float* __restrict__ p_tok, const float* __restrict__ entropy, float eps, float delta) {
  int on_pos;
  const AcceptIn in = accept_load<TYPICAL>(cand_tok, tgt, parents, anc, depth, n_nodes, err, n_max, p_tok, entropy,
                                           blockIdx.x, threadIdx.x);
  accept_decide<TYPICAL>(in, n_max, accept_len, path, bonus, out_tokens, eps, delta, blockIdx.x, threadIdx.x,
                         on_pos);
}

// ---------------------------------------------------------------------------
// commit: slot P+d <- slot P+path[d] for d = 0..L. A path from accept is
// strictly increasing with path[d] >= d, so a source slot may be another
// lane's destination; all sources of one KV head are staged in LDS before any
// slot is written, which makes any path with entries in [0, n_max) a plain
// simultaneous copy.
// K is [cap][D] per head; V is blocked [cap/64][D][64] per head. With a
// paged cache (bt non-null) the 64-slot block j of sequence b is page
// bt[b * max_pages + j] of pools [num_pages][Hkv][64][D] (K) and
// [num_pages][Hkv][D][64] (V). The moved slots lie in [P, P + n_max), at most
// two blocks, whose offsets are found once per head.
// Grid: (Hkv / heads_per_block, B). The block of head 0 writes prefix_len_out;
// when that array is also prefix_len_in, one block per sequence walks every
// head, so no block can read a length another block has already replaced.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void commit_kernel(
    T* __restrict__ k_cache, T* __restrict__ v_cache, int Hkv, int cap, int D,
    const int32_t* prefix_len_in, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ path, int n_max, int32_t* prefix_len_out, int heads_per_block,
    const int32_t* __restrict__ bt, int max_pages, int num_pages) {
  constexpr int kStage = TV_MAX_NODES_DEV * 128 * 4 / sizeof(T);   // elements
  __shared__ T k_stage[kStage];
  __shared__ T v_stage[kStage];
  __shared__ int s_path[TV_MAX_NODES_DEV];
  __shared__ int s_L, s_P, s_ok, s_top;
  __shared__ int s_page[2];

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  // the path goes out with the lengths (one memory round trip)
  const int src_in = tid < n_max ? path[static_cast<size_t>(b) * n_max + tid] : 0;
  if (tid == 0) {
    const int L = accept_len[b];
    const int P = prefix_len_in[b];
    const int ok = (L >= 0) && (L < n_max) && (P >= 0) && (P + L < cap);
    if (bt && ok) {
      // the table entries of the (at most two) blocks from P on
      for (int u = 0; u < 2; ++u)
        s_page[u] = bt[static_cast<size_t>(b) * max_pages + min((P >> 6) + u, max_pages - 1)];
    }
    s_L = L;
    s_P = P;
    s_ok = ok;
    s_top = L;
  }
  __syncthreads();
  const int L = s_L, P = s_P;
  if (tid <= L && tid < n_max && s_ok) {
    s_path[tid] = src_in;
    // every source must be a tree node, 0 <= path[d] < n_max (so all moved
    // slots lie in [P, P + 64): the two blocks from P >> 6), inside the cache
    if (src_in < 0 || src_in >= n_max || P + src_in >= cap) atomicAnd(&s_ok, 0);
    atomicMax(&s_top, src_in);
  }
  __syncthreads();
  if (bt && tid == 0 && s_ok) {
    // the pages the move touches (slots P .. P + max(L, largest path entry))
    // must be pages of the pools, else the sequence is left unchanged
    const int blocks = ((P + s_top) >> 6) - (P >> 6) + 1;
    for (int u = 0; u < 2; ++u) {
      const int e = s_page[u];
      if (u < blocks && (e < 0 || e >= num_pages)) s_ok = 0;
      s_page[u] = min(max(e, 0), num_pages - 1);
    }
  }
  if (bt) __syncthreads();
  const bool ok = s_ok;
  if ((heads_per_block == Hkv || blockIdx.x == 0) && tid == 0) prefix_len_out[b] = ok ? P + L + 1 : P;
  if (!ok) return;

  const int g0 = (heads_per_block == Hkv) ? 0 : blockIdx.x;
  const int total = (L + 1) * D;
  const int blk0 = P >> 6;
  for (int gg = 0; gg < heads_per_block; ++gg) {
    const int g = g0 + gg;
    // element offsets of blocks blk0 and blk0 + 1 of this head
    size_t off[2];
    if (bt) {
      off[0] = (static_cast<size_t>(s_page[0]) * Hkv + g) * 64 * D;
      off[1] = (static_cast<size_t>(s_page[1]) * Hkv + g) * 64 * D;
    } else {
      off[0] = ((static_cast<size_t>(b) * Hkv + g) * cap + static_cast<size_t>(blk0) * 64) * D;
      off[1] = off[0] + static_cast<size_t>(64) * D;
    }
    auto k_at = [&](int slot, int c) { return off[(slot >> 6) - blk0] + static_cast<size_t>(slot & 63) * D + c; };
    auto v_at = [&](int slot, int c) { return off[(slot >> 6) - blk0] + static_cast<size_t>(c) * 64 + (slot & 63); };
    for (int idx = tid; idx < total; idx += blockDim.x) {
      const int d = idx / D, c = idx % D;
      const int src = P + s_path[d];
      if (src == P + d) continue;
      k_stage[idx] = k_cache[k_at(src, c)];
      v_stage[idx] = v_cache[v_at(src, c)];
    }
    __syncthreads();
    for (int idx = tid; idx < total; idx += blockDim.x) {
      const int d = idx / D, c = idx % D;
      if (s_path[d] == d) continue;
      const int dst = P + d;
      k_cache[k_at(dst, c)] = k_stage[idx];
      v_cache[v_at(dst, c)] = v_stage[idx];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// accept + commit in one launch: grid (Hkv / heads_per_block, B), 256
// threads. Every wavefront of every workgroup of sequence b runs the accept
// of accept_kernel (a few hundred bytes of loads, repeated rather than
// waited for across a launch); the workgroup of heads 0.. writes its
// outputs. The length and path stay in LDS, and the workgroup moves the
// path's K and V of its KV heads (slot P + d <- slot P + path[d]) in batches
// whose sources fit the LDS stage: all of a batch's sources are read before
// any slot is written. When prefix_len_out is prefix_len_in, one workgroup
// per sequence walks every head (heads_per_block = Hkv), so no workgroup
// reads a length another has replaced. A skipped sequence (accept length
// -1) or a move outside [P, cap) leaves the cache and the prefix length
// unchanged.
// ---------------------------------------------------------------------------
// A 16-byte chunk held as four words: rows kept in registers between their
// load and their LDS store are copied word by word, so the compiler does not
// turn the pair into a memory-to-memory copy through a stack buffer.
struct Words4 {
  uint32_t w[4];
};
__device__ __forceinline__ Words4 words(uint4 x) { return Words4{{x.x, x.y, x.z, x.w}}; }
__device__ __forceinline__ uint4 chunk(const Words4& x) { return make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]); }

template <typename T>
__global__ __launch_bounds__(256) void accept_commit_kernel(
    const int32_t* __restrict__ cand_tok, const int32_t* __restrict__ tgt,
    const int32_t* __restrict__ parents, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ err, int n_max, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ bonus, int32_t* __restrict__ out_tokens,
    T* __restrict__ k_cache, T* __restrict__ v_cache, int Hkv, int cap, int D,
    const int32_t* prefix_len_in, int32_t* prefix_len_out, int heads_per_block,
    const int32_t* __restrict__ bt, int max_pages, int num_pages) {
  // the tree's slots [P, P + n) of one KV head: K rows [slot][D], V [D][slot]
  constexpr int kRows = TV_MAX_NODES_DEV, kMaxD = 128;
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  // V rows: head dim c, slots from P rounded down to a 16-byte chunk
  constexpr int kVSlots = kRows + EPC;
  __shared__ uint4 k_rows[kRows * kMaxD / EPC];
  // (plus one 16-byte chunk that takes the stores of lanes with no chunk)
  __shared__ __attribute__((aligned(16))) T v_rows[kMaxD * kVSlots + EPC];
  __shared__ int s_path[TV_MAX_NODES_DEV];
  __shared__ int s_L;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int g_first = blockIdx.x * heads_per_block, g_last = min(Hkv, g_first + heads_per_block);
  const int P = prefix_len_in[b];
  const int n_in = n_nodes[b];
  // tree rows that lie in the cache (any move from outside it is refused)
  const int nr = (P >= 0 && n_in > 0 && n_in <= n_max) ? max(0, min(n_in, cap - P)) : 0;
  const int kpr = D / EPC;   // 16-byte chunks per K row
  // With a paged cache (bt non-null, max_pages <= 256) lane l of pg[u] holds
  // the page of block l + 64 u (loaded with the accept's loads, needing no
  // prefix length); the tree's slots lie in the two blocks from P >> 6,
  // whose pages are picked once (uniform) and clamped into the pools for
  // addressing; whether they are pages of the pools is decided after the
  // accept, like tv_commit_paged (a move through a bad page leaves the
  // sequence unchanged).
  // (the loads are unconditional, reading the prefix length again without a
  // table, so that the compiler's wait counts stay exact)
  uint32_t pg[4];
  {
    const int32_t* row = bt ? bt + static_cast<size_t>(b) * max_pages : prefix_len_in + b;
    const int last = bt ? max_pages - 1 : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) pg[u] = static_cast<uint32_t>(row[min((tid & 63) + 64 * u, last)]);
  }
  const int blk0 = nr > 0 ? P >> 6 : 0;
  auto page_entry = [&](int blk) {
    const int bc = min(blk, max_pages - 1);
    const uint32_t reg = bc < 64 ? pg[0] : bc < 128 ? pg[1] : bc < 192 ? pg[2] : pg[3];
    return static_cast<int>(__builtin_amdgcn_readlane(reg, bc & 63));
  };
  int e0 = 0, e1 = 0;
  if (bt) {
    e0 = page_entry(blk0);
    e1 = page_entry(blk0 + 1);
  }
  const int page0 = min(max(e0, 0), max(num_pages - 1, 0)), page1 = min(max(e1, 0), max(num_pages - 1, 0));
  // element offset of the 64-slot block holding `slot` (head g); paged: of
  // the page holding it (slots of the two blocks from P >> 6 only)
  auto base = [=](int g, int slot) {
    if (bt) return (static_cast<size_t>((slot >> 6) == blk0 ? page0 : page1) * Hkv + g) * 64 * D;
    return ((static_cast<size_t>(b) * Hkv + g) * cap + static_cast<size_t>(slot >> 6) * 64) * D;
  };
  // The tree rows of head g are loaded into registers, every load of a
  // thread in flight together (fully unrolled, constant indices), then
  // written to LDS: K as 16-byte chunks of its rows, V as 16-byte chunks of
  // its head-dim rows (the tree's slots of one head dim are contiguous inside
  // a 64-slot block, and chunks never straddle blocks).
  // per thread: enough chunks for 64 rows of D = 128
  constexpr int KU = kRows * kMaxD / EPC / 256, VU = (kMaxD * (kRows / EPC + 1) + 255) / 256;
  static_assert(KU * 256 * EPC == kRows * kMaxD, "one round covers the tree's K rows");
  const int v0 = P & ~(EPC - 1);                                       // first slot of the first V chunk
  const int vchunks = nr > 0 ? ((P + nr - 1 - v0) / EPC + 1) : 0;     // V chunks per head-dim row
  const int ktotal = nr * kpr, vtotal = vchunks * D;
  const int p_safe = nr > 0 ? P : 0, v0_safe = nr > 0 ? v0 : 0;
  auto load_rows = [=](int g, Words4 (&kv)[KU], Words4 (&vv)[VU]) __attribute__((always_inline)) {
    // Every load is unconditional, so the compiler counts them exactly and the
    // accept waits only for its own: with no tree rows (nr == 0) they read
    // slot 0 of the head (p_safe = v0_safe = 0, idx = 0), which always
    // exists, and are never used.
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = min(tid + u * 256, max(ktotal - 1, 0)), r = idx / kpr, c = idx % kpr;
      const int slot = p_safe + r;
      kv[u] = words(*reinterpret_cast<const uint4*>(k_cache + base(g, slot) + static_cast<size_t>(slot & 63) * D +
                                                    EPC * c));
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      // consecutive lanes walk the chunks of one head-dim row
      const int idx = min(tid + u * 256, max(vtotal - 1, 0)), c = idx / max(vchunks, 1), k = idx % max(vchunks, 1);
      const int slot = v0_safe + EPC * k;
      vv[u] = words(*reinterpret_cast<const uint4*>(v_cache + base(g, slot) + static_cast<size_t>(c) * 64 +
                                                    (slot & 63)));
    }
  };
  // Unconditional stores as well: K chunks past the tree's rows are never
  // read, and V lanes with no chunk all write the spare chunk.
  auto put_rows = [=](const Words4 (&kv)[KU], const Words4 (&vv)[VU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KU; ++u) k_rows[tid + u * 256] = chunk(kv[u]);
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int idx = tid + u * 256, vc = max(vchunks, 1);
      const int at = idx < vtotal ? (idx / vc) * kVSlots + EPC * (idx % vc) : kMaxD * kVSlots;
      *reinterpret_cast<uint4*>(&v_rows[at]) = chunk(vv[u]);
    }
  };
  // slot P + d <- tree row path[d], d = 0 .. L, of head g (rows on their own
  // slot stay)
  auto move_rows = [&](int g, int L) __attribute__((always_inline)) {
    for (int idx = tid; idx < (L + 1) * kpr; idx += 256) {
      const int d = idx / kpr, c = idx % kpr, src = s_path[d];
      if (src == d) continue;
      const int dst = P + d;
      *reinterpret_cast<uint4*>(k_cache + base(g, dst) + static_cast<size_t>(dst & 63) * D + EPC * c) =
          k_rows[src * kpr + c];
    }
    for (int idx = tid; idx < (L + 1) * D; idx += 256) {
      const int c = idx / (L + 1), d = idx % (L + 1), src = s_path[d];
      if (src == d) continue;
      const int dst = P + d;
      v_cache[base(g, dst) + static_cast<size_t>(c) * 64 + (dst & 63)] = v_rows[c * kVSlots + (P + src - v0)];
    }
  };
  // The accept's loads go out first (every wavefront makes them: they need
  // no prefix length), then the first head's rows; every wavefront decides
  // the accept, wavefront 0 keeps the path and (workgroup of heads 0..)
  // writes the outputs.
  const AcceptIn ain = accept_load<false>(cand_tok, tgt, parents, anc, depth, n_nodes, err, n_max, nullptr, nullptr,
                                          b, tid & 63);
  Words4 kv[KU], vv[VU];
  load_rows(g_first, kv, vv);
  {
    int on_pos;
    const int L = accept_decide<false>(ain, n_max, accept_len, path, bonus, out_tokens, 0.f, 0.f, b, tid & 63,
                                       on_pos, blockIdx.x == 0 && tid < 64);
    if (tid < 64 && on_pos >= 0) s_path[on_pos] = tid;
    if (tid == 0) s_L = L;
  }
  put_rows(kv, vv);
  __syncthreads();
  // the path ascends, so its end node path[L] is the largest moved slot;
  // paged: the blocks from P >> 6 to that of slot P + path[L] must be pages
  // of the pools
  const int top = s_path[max(s_L, 0)];
  const bool pages_ok = !bt || ((e0 >= 0 && e0 < num_pages) &&
                                (((P + top) >> 6) == blk0 || (e1 >= 0 && e1 < num_pages)));
  const int L = (s_L >= 0 && P >= 0 && top < nr && pages_ok) ? s_L : -1;
  if (blockIdx.x == 0 && tid == 0) prefix_len_out[b] = L >= 0 ? P + L + 1 : P;
  if (L < 0) return;
  move_rows(g_first, L);
  for (int g = g_first + 1; g < g_last; ++g) {
    Words4 kv_g[KU], vv_g[VU];
    __syncthreads();   // (the previous head's rows are written)
    load_rows(g, kv_g, vv_g);
    put_rows(kv_g, vv_g);
    __syncthreads();
    move_rows(g, L);
  }
}

// ------------------------------------------------------------------ launches

hipError_t launch_build_tree(const int32_t* parents, const int32_t* n_nodes, int B, int n_max,
                             uint64_t* anc, int32_t* depth, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, s, parents, n_nodes, n_max, anc,
                     depth, err);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* cand_tok, const int32_t* tgt, const int32_t* parents,
                         const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                         const int32_t* err, int B, int n_max, int32_t* accept_len,
                         int32_t* path, int32_t* bonus, int32_t* out_tokens, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel<false>, dim3(B), dim3(64), 0, s, cand_tok, tgt, parents, anc,
                     depth, n_nodes, err, n_max, accept_len, path, bonus, out_tokens, nullptr,
                     nullptr, 0.f, 0.f);
  return hipGetLastError();
}

hipError_t launch_accept_typical(const int32_t* cand_tok, const int32_t* tgt_argmax,
                                 const float* p_tok, const float* entropy, float eps, float delta,
                                 const int32_t* parents, const uint64_t* anc, const int32_t* depth,
                                 const int32_t* n_nodes, const int32_t* err, int B, int n_max,
                                 int32_t* accept_len, int32_t* path, int32_t* bonus,
                                 int32_t* out_tokens, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel<true>, dim3(B), dim3(64), 0, s, cand_tok, tgt_argmax, parents,
                     anc, depth, n_nodes, err, n_max, accept_len, path, bonus, out_tokens, p_tok,
                     entropy, eps, delta);
  return hipGetLastError();
}

hipError_t launch_accept_commit(const int32_t* cand_tok, const int32_t* tgt, const int32_t* parents,
                                const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                                const int32_t* err, int B, int n_max, int32_t* accept_len, int32_t* path,
                                int32_t* bonus, int32_t* out_tokens, void* k_cache, void* v_cache, int Hkv,
                                int cap, int D, int elem_bytes, const int32_t* prefix_len_in,
                                int32_t* prefix_len_out, const tv_paged_kv* pk, hipStream_t s) {
  const int32_t* bt = pk ? pk->block_table : nullptr;
  const int max_pages = pk ? pk->max_pages : 1, num_pages = pk ? pk->num_pages : 1;
  // one workgroup per (KV head, sequence), or per sequence when the new
  // prefix lengths overwrite the old ones
  const int hpb = (prefix_len_in == prefix_len_out) ? Hkv : 1;
  const dim3 grid(Hkv / hpb, B);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(accept_commit_kernel<uint16_t>, grid, dim3(256), 0, s, cand_tok, tgt, parents, anc, depth,
                       n_nodes, err, n_max, accept_len, path, bonus, out_tokens, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), Hkv, cap, D, prefix_len_in, prefix_len_out, hpb, bt,
                       max_pages, num_pages);
  } else {
    hipLaunchKernelGGL(accept_commit_kernel<uint32_t>, grid, dim3(256), 0, s, cand_tok, tgt, parents, anc, depth,
                       n_nodes, err, n_max, accept_len, path, bonus, out_tokens, static_cast<uint32_t*>(k_cache),
                       static_cast<uint32_t*>(v_cache), Hkv, cap, D, prefix_len_in, prefix_len_out, hpb, bt,
                       max_pages, num_pages);
  }
  return hipGetLastError();
}

hipError_t launch_commit(void* k_cache, void* v_cache, int B, int Hkv, int cap, int D,
                         int elem_bytes, const int32_t* prefix_len_in, const int32_t* accept_len,
                         const int32_t* path, int n_max, int32_t* prefix_len_out,
                         const tv_paged_kv* pk, hipStream_t s) {
  const int32_t* bt = pk ? pk->block_table : nullptr;
  const int max_pages = pk ? pk->max_pages : 0, num_pages = pk ? pk->num_pages : 0;
  // One block per (kv head, sequence) unless the new prefix lengths overwrite
  // the old ones, in which case one block per sequence walks every head so
  // that no block reads a length another block has already replaced.
  const bool alias = (prefix_len_in == prefix_len_out);
  const int hpb = alias ? Hkv : 1;
  dim3 grid(alias ? 1 : Hkv, B);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(commit_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), Hkv, cap, D, prefix_len_in, accept_len,
                       path, n_max, prefix_len_out, hpb, bt, max_pages, num_pages);
  } else {
    hipLaunchKernelGGL(commit_kernel<uint32_t>, grid, dim3(256), 0, s, static_cast<uint32_t*>(k_cache),
                       static_cast<uint32_t*>(v_cache), Hkv, cap, D, prefix_len_in, accept_len,
                       path, n_max, prefix_len_out, hpb, bt, max_pages, num_pages);
  }
  return hipGetLastError();
}

}  // namespace tv
