// Issue-order model of the vector memory operations of one thread of the
// bf16 attention kernel (tv_attn_bf16.hip), from which every s_waitcnt
// vmcnt that kernel writes by hand is derived. The copies into LDS and the
// register loads it issues from inline asm are invisible to the compiler's
// own wait insertion, so these counts are the kernel's only guard on them.
//
// Vector memory operations complete in issue order (and the count of those
// in flight is a 6-bit field), so "wait until operation X has completed" is
// s_waitcnt vmcnt(n), n = the operations issued after X.
//
// Issue order, per thread:
//   start   [the sequence's page ids (paged caches)], the depths of the
//           wavefront's rows' nodes and of node `lane` (or, when the kernel
//           builds the tree itself, the parent of node `lane`, which it
//           waits for right after the next group), the query
//           copies, [the tree's keys, values and depths and the rows'
//           ancestor masks (keys and values only when it builds the tree),
//           when the split holds tree tiles], then tile 0; tiles 1 and 2 go
//           out once the queries have landed;
//   pass    before the tree fill (splits holding tree tiles) the tree tiles
//           must have landed; iteration t waits for tile t and issues tile
//           t + kAhead (if any); a redo pass starts with nothing in flight
//           and issues tiles 0 .. kAhead - 1 first.
// No other vector memory operation is issued between these (the loop
// writes nothing to global memory), which the kernel keeps.
//
// Plain constexpr functions: the kernel instantiates its waits from them,
// and a host program (tests/wait_model_check.cpp) simulates the issue order
// for every instantiation and tile layout and checks each wait against it.
#pragma once

namespace tv {
namespace waits {

constexpr int kKeys = 64;       // keys per tile
constexpr int kDim = 128;       // head dim
constexpr int kAhead = 3;       // tiles in flight
constexpr int kMaxCount = 63;   // largest count the vmcnt field holds

constexpr int threads(int waves) { return waves * 64; }
// 16-byte copies per thread of a tile's K (and as many of its V)
constexpr int tile_chunks(int waves) { return kKeys * kDim * 2 / 16 / threads(waves); }
constexpr int tile_ops(int waves) { return 2 * tile_chunks(waves); }
constexpr int page_ops(bool paged) { return paged ? 4 : 0; }
constexpr int depth_ops(int qt, bool build) { return build ? 1 : qt + 1; }
constexpr int query_ops(int waves, int qt) { return waves * 32 * qt * kDim / 8 / threads(waves); }
// tree items per thread: 16-byte key pairs (8 per node) and value chunks (16 per node)
constexpr int tree_k_items(int waves) { return 8 * 64 / threads(waves); }
constexpr int tree_v_items(int waves) { return 16 * 64 / threads(waves); }
// two loads per key pair plus its node's depth, one per value chunk, one
// ancestor mask per query tile (depths and masks are not loaded when the
// kernel builds the tree)
constexpr int tree_ops(int waves, int qt, bool build) {
  return build ? 2 * tree_k_items(waves) + tree_v_items(waves) : 3 * tree_k_items(waves) + tree_v_items(waves) + qt;
}
constexpr int start_ops(int waves, int qt, bool paged, bool build, bool tree) {
  return page_ops(paged) + depth_ops(qt, build) + query_ops(waves, qt) + (tree ? tree_ops(waves, qt, build) : 0);
}

// If the start's operations and tile 0 could overflow the counter, enough of
// the former land first (no instantiation needs it today).
constexpr bool start_guard(int waves, int qt, bool paged, bool build) {
  return start_ops(waves, qt, paged, build, true) + tile_ops(waves) > kMaxCount;
}
constexpr int vm_start_guard(int waves) { return kMaxCount - tile_ops(waves); }

// The page ids (the oldest operations) have landed, tile 0 not yet issued.
constexpr int vm_pages(int waves, int qt, bool build, bool tree) {
  return depth_ops(qt, build) + query_ops(waves, qt) + (tree ? tree_ops(waves, qt, build) : 0);
}
// (Kernel building the tree) the parents have landed, right after the
// query copies went out.
constexpr int vm_parents(int waves, int qt) { return query_ops(waves, qt); }
// The depths (or parents) have landed (after tile 0, if the split has tiles).
constexpr int vm_depths(int waves, int qt, bool build, bool tree, bool tile0) {
  return query_ops(waves, qt) + (tree ? tree_ops(waves, qt, build) : 0) + (tile0 ? tile_ops(waves) : 0);
}
// Everything of the start has landed, only tile 0 may be in flight.
constexpr int vm_queries(int waves, bool tile0) { return tile0 ? tile_ops(waves) : 0; }
// A tile has landed, `later` whole tiles having been issued after it.
constexpr int vm_tile(int waves, int later) { return later * tile_ops(waves); }

// Tiles issued after tile t at the top of iteration t of a pass.
constexpr int later_tiles(int t, int n_tiles) {
  return (kAhead - 1) < (n_tiles - 1 - t) ? (kAhead - 1) : (n_tiles - 1 - t);
}
// Tiles issued after the last tree tile when the tree fill runs: only tiles
// 0 .. kAhead - 1 are out then, the first n_masked of them the tree's.
constexpr int after_tree(int n_tiles, int n_masked) {
  return (kAhead < n_tiles ? kAhead : n_tiles) - n_masked;
}

}  // namespace waits
}  // namespace tv
