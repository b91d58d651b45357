// Host check of the bf16 attention kernel's hand-counted waits.
//
// For every kernel instantiation (wavefronts, query tiles, paged or not,
// tree built by the kernel or given),
// tile count, tree-tile count and pass (the fast pass, and the redo passes
// that re-issue the first tiles), this program replays, in order, the vector
// memory operations one thread issues and the waits it executes (the
// kernel's control flow, written out here on its own), taking each wait's
// count from the model in tv_attn_waits.h that the kernel instantiates.
// Operations complete oldest first, so a wait with count n completes all but
// the newest n. Each wait is checked to
//   cover  every operation it guards (none of them among the newest n), and
//   be exact: the guarded operations are followed by exactly n others, so the
//          wait does not hold the thread for more than it needs;
// and the number in flight never exceeds the counter's range.
//
//   wait_model_check                 all cases; prints "ok <cases> <waits>"
//   wait_model_check --legacy-tree   the tree-tile wait of an earlier kernel
//                                    (it waited as for the last tree tile at
//                                    the top of an iteration); must fail
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "tv_attn_waits.h"

namespace w = tv::waits;

namespace {

struct Op {
  std::string tag;   // "page", "depth", "query", "tree", "tile<k>"
  long seq;          // issue order
};

struct Replay {
  std::deque<Op> q;   // in flight, oldest first
  long seq = 0;
  int waits = 0;
  std::vector<std::string> errors;
  std::string where;

  void issue(const std::string& tag, int count) {
    for (int i = 0; i < count; ++i) q.push_back(Op{tag, seq++});
    if (static_cast<int>(q.size()) > w::kMaxCount)
      errors.push_back(where + ": " + std::to_string(q.size()) + " operations in flight after issuing " + tag);
  }
  void issue_tile(int k, int waves) { issue("tile" + std::to_string(k), w::tile_ops(waves)); }

  // wait with count n; `guarded` names the tags that must have completed
  void wait(int n, const std::vector<std::string>& guarded, const char* site) {
    ++waits;
    auto is_guarded = [&](const Op& o) {
      for (const auto& g : guarded)
        if (o.tag == g) return true;
      return false;
    };
    // exactness: operations issued after the newest guarded one still in flight
    long newest = -1;
    for (const Op& o : q)
      if (is_guarded(o)) newest = o.seq;
    int after = 0;
    for (const Op& o : q)
      if (o.seq > newest) ++after;
    while (static_cast<int>(q.size()) > n) q.pop_front();
    for (const Op& o : q)
      if (is_guarded(o)) {
        errors.push_back(where + ": wait " + site + " (vmcnt " + std::to_string(n) + ") leaves " + o.tag +
                         " in flight");
        return;
      }
    if (newest >= 0 && after != n)
      errors.push_back(where + ": wait " + site + " (vmcnt " + std::to_string(n) + ") is not exact: " +
                       std::to_string(after) + " operations follow what it guards");
  }
};

std::vector<std::string> tiles_tags(int from, int to) {
  std::vector<std::string> v;
  for (int k = from; k < to; ++k) v.push_back("tile" + std::to_string(k));
  return v;
}

// One pass over the split's tiles; tiles 0 .. kAhead - 1 are already issued.
void replay_pass(Replay& r, int waves, int n_tiles, int n_masked, bool legacy_tree) {
  int t = 0;
  if (n_masked > 0) {
    // the tree fill needs every tree tile
    const int later = legacy_tree ? w::later_tiles(n_masked - 1, n_tiles) : w::after_tree(n_tiles, n_masked);
    r.wait(w::vm_tile(waves, later), tiles_tags(0, n_masked), "tree tiles");
    for (; t < n_masked; ++t) {
      if (t > 0) r.wait(w::vm_tile(waves, w::later_tiles(t, n_tiles)), tiles_tags(t, t + 1), "tree tile");
      if (t + w::kAhead < n_tiles) r.issue_tile(t + w::kAhead, waves);
    }
  }
  for (; t < n_tiles; ++t) {
    r.wait(w::vm_tile(waves, w::later_tiles(t, n_tiles)), tiles_tags(t, t + 1), "tile");
    if (t + w::kAhead < n_tiles) r.issue_tile(t + w::kAhead, waves);
  }
}

void replay(Replay& r, int waves, int qt, bool paged, bool build, int n_tiles, int n_masked, bool redo,
            bool legacy_tree) {
  const bool tree = n_masked > 0;
  const bool guard = w::start_guard(waves, qt, paged, build);
  // start
  if (paged) r.issue("page", w::page_ops(true));
  r.issue("depth", w::depth_ops(qt, build));
  r.issue("query", w::query_ops(waves, qt));
  // the kernel that builds the tree waits for the parents before the rest
  if (build) r.wait(w::vm_parents(waves, qt), {"page", "depth"}, "parents");
  if (tree) r.issue("tree", w::tree_ops(waves, qt, build));
  if (guard) r.wait(w::vm_start_guard(waves), {}, "start guard");
  if (paged) r.wait(w::vm_pages(waves, qt, build, tree), {"page"}, "page ids");
  if (n_tiles > 0) r.issue_tile(0, waves);
  if (!guard)
    r.wait(w::vm_depths(waves, qt, build, tree, n_tiles > 0), {"page", "depth"}, "depths");
  else
    r.wait(w::vm_queries(waves, n_tiles > 0), {"page", "depth", "query", "tree"}, "depths (guarded start)");
  r.wait(w::vm_queries(waves, n_tiles > 0), {"page", "depth", "query", "tree"}, "queries");
  if (n_tiles > 1) r.issue_tile(1, waves);
  if (n_tiles > 2) r.issue_tile(2, waves);
  replay_pass(r, waves, n_tiles, n_masked, legacy_tree);
  if (redo) {
    // the scores-only pass and the repeated pass: each re-issues the first
    // tiles with nothing in flight (the tree rows are reloaded by ordinary
    // loads, which the compiler waits for itself)
    for (int pass = 0; pass < 2; ++pass) {
      if (!r.q.empty()) r.errors.push_back(r.where + ": operations in flight when a redo pass starts");
      for (int k = 0; k < w::kAhead && k < n_tiles; ++k) r.issue_tile(k, waves);
      replay_pass(r, waves, n_tiles, n_masked, legacy_tree);
    }
  }
  // the epilogue waits for everything
  r.wait(0, {}, "epilogue");
  if (!r.q.empty()) r.errors.push_back(r.where + ": operations left in flight");
}

}  // namespace

int main(int argc, char** argv) {
  const bool legacy_tree = argc > 1 && std::strcmp(argv[1], "--legacy-tree") == 0;
  // the kernel's instantiations: (wavefronts, query tiles per wavefront)
  const int shapes[][2] = {{2, 1}, {4, 1}, {4, 2}, {8, 1}};
  long cases = 0, waits = 0, failures = 0;
  for (const auto& sh : shapes)
    for (int paged = 0; paged < 2; ++paged)
      for (int build = 0; build < 2; ++build)
      for (int n_tiles = 0; n_tiles <= 12; ++n_tiles)
        // a tree of at most 64 nodes spans at most two 64-key tiles
        for (int n_masked = 0; n_masked <= 2 && n_masked <= n_tiles; ++n_masked)
          for (int redo = 0; redo < 2; ++redo) {
            Replay r;
            r.where = "waves=" + std::to_string(sh[0]) + " qt=" + std::to_string(sh[1]) +
                      " paged=" + std::to_string(paged) + " build=" + std::to_string(build) +
                      " n_tiles=" + std::to_string(n_tiles) +
                      " n_masked=" + std::to_string(n_masked) + " redo=" + std::to_string(redo);
            replay(r, sh[0], sh[1], paged != 0, build != 0, n_tiles, n_masked, redo != 0, legacy_tree);
            ++cases;
            waits += r.waits;
            for (size_t e = 0; e < r.errors.size(); ++e)
              if (failures + static_cast<long>(e) < 20) std::printf("FAIL %s\n", r.errors[e].c_str());
            if (!r.errors.empty()) ++failures;
          }
  if (failures) {
    std::printf("failing cases %ld of %ld\n", failures, cases);
    return 1;
  }
  std::printf("ok %ld %ld\n", cases, waits);
  return 0;
}
