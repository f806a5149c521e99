// SpecFit verification-subtree selection: the exact search over the draft
// pool's ancestor-closed subtrees for the largest predicted reward / cycle
// time, with the experts of each candidate carried as per-layer bitmaps.
//
// SpecFit page: section 3.1 (a legal subtree holds every selected node's
// ancestors and at most K nodes), 3.2 (reward = 1 + the selected nodes'
// commit probabilities, estimated from path probabilities; cycle time from
// the node count and the per-layer union of activated experts, a coverage
// function), 3.3 (maximise reward / time over legal subtrees) and appendix
// A.3 (depth-first search that reaches every legal subtree once by adding
// nodes in parent-before-descendant order, expert bitmaps carried
// incrementally).
//
// The search grows a subtree from the root. It keeps a list of candidate
// nodes (children of the root or of a chosen node, not yet decided); taking
// the candidate at position j decides against the candidates before it for
// the whole branch, and the taken node's children join the end of the list.
// Every ancestor-closed subtree is produced exactly once (its nodes are
// taken in the order they appear in the list). Each level of the recursion
// keeps the union bitmaps of its subtree, so a node costs one OR per word.
#include <algorithm>
#include <cstring>
#include <vector>

#include "smoe_internal.hpp"

// reward, time and ratio are each one IEEE double operation at a time (no
// fused multiply-add), so a caller can reproduce every ratio bit for bit
#pragma clang fp contract(off)

namespace smoe {
namespace {

constexpr int kMaxNodes = 64;     // pool size the search takes
constexpr int kMaxWords = 4;      // 256 experts per layer

struct Search {
  int n, L, W, K;
  const int32_t* parent;
  const double* prob;
  const uint64_t* bits;           // [n + 1][L][W], row 0 the root
  const uint64_t* resident;       // [L][W] or null
  const double* b;                // intercepts [K + 1]
  double beta;
  std::vector<std::vector<int>> kids;  // children of each node (index n = root)
  // best so far
  double best_ratio = -1.0;
  int best_n = 0;
  int best[kMaxNodes];
  long long evaluated = 0;
  // current subtree
  int cur[kMaxNodes];
  int cur_n = 0;
  std::vector<uint64_t> unions;   // [K + 1][L * W]: union at each depth of the recursion

  // ratio of the current subtree, its reward summed in ascending node order
  void evaluate(const uint64_t* u) {
    ++evaluated;
    int sorted[kMaxNodes];
    std::copy(cur, cur + cur_n, sorted);
    std::sort(sorted, sorted + cur_n);
    double reward = 1.0;
    for (int i = 0; i < cur_n; ++i) reward += prob[sorted[i]];
    long long F = 0;
    for (int i = 0; i < L * W; ++i) {
      const uint64_t w = resident ? (u[i] & ~resident[i]) : u[i];
      F += __builtin_popcountll(w);
    }
    const double t = b[cur_n] + beta * static_cast<double>(F);
    const double r = reward / t;
    bool better = best_ratio < 0.0 || r > best_ratio;
    if (!better && r == best_ratio) {
      if (cur_n != best_n) {
        better = cur_n < best_n;
      } else {
        int bs[kMaxNodes];
        std::copy(best, best + best_n, bs);  // (best is kept sorted)
        better = std::lexicographical_compare(sorted, sorted + cur_n, bs, bs + best_n);
      }
    }
    if (better) {
      best_ratio = r;
      best_n = cur_n;
      std::copy(sorted, sorted + cur_n, best);
    }
  }

  // cand: the undecided candidates of this branch
  void grow(const std::vector<int>& cand, int depth) {
    const uint64_t* u = unions.data() + static_cast<size_t>(depth) * L * W;
    evaluate(u);
    if (cur_n == K) return;
    uint64_t* next = unions.data() + static_cast<size_t>(depth + 1) * L * W;
    std::vector<int> rest;
    for (size_t j = 0; j < cand.size(); ++j) {
      const int v = cand[j];
      const uint64_t* bv = bits + static_cast<size_t>(v + 1) * L * W;
      for (int i = 0; i < L * W; ++i) next[i] = u[i] | bv[i];
      rest.assign(cand.begin() + j + 1, cand.end());
      rest.insert(rest.end(), kids[v].begin(), kids[v].end());
      cur[cur_n++] = v;
      grow(rest, depth + 1);
      --cur_n;
    }
  }
};

}  // namespace
}  // namespace smoe

using namespace smoe;

extern "C" smoe_status smoe_specfit_select(int n, const int32_t* parent, const double* path_prob,
                                           int L, int E, const uint64_t* expert_bits,
                                           const uint64_t* resident_bits, int K,
                                           const double* intercepts, double beta,
                                           int32_t* selected, int* n_selected, double* ratio,
                                           int64_t* n_evaluated) {
  clear_error();
  const char* who = "specfit_select";
  SMOE_REQUIRE(n >= 0 && n <= kMaxNodes && L > 0 && E > 0 && E <= 64 * kMaxWords && K >= 0,
               SMOE_EINVAL, "%s: need 0 <= n <= %d, L > 0, 0 < E <= %d, K >= 0 (n=%d L=%d E=%d "
               "K=%d)", who, kMaxNodes, 64 * kMaxWords, n, L, E, K);
  SMOE_REQUIRE((n == 0 || (parent && path_prob)) && expert_bits && intercepts && selected &&
                   n_selected,
               SMOE_EINVAL, "%s: null argument", who);
  SMOE_REQUIRE(beta >= 0.0, SMOE_EINVAL, "%s: beta must be >= 0", who);
  const int Kc = std::min(K, n);
  for (int i = 0; i <= Kc; ++i)
    SMOE_REQUIRE(intercepts[i] > 0.0 && intercepts[i] < 1e300, SMOE_EINVAL,
                 "%s: intercept %d must be finite and > 0", who, i);
  Search s;
  s.n = n;
  s.L = L;
  s.W = (E + 63) / 64;
  s.K = Kc;
  s.parent = parent;
  s.prob = path_prob;
  s.bits = expert_bits;
  s.resident = resident_bits;
  s.b = intercepts;
  s.beta = beta;
  s.kids.assign(n + 1, {});
  for (int v = 0; v < n; ++v) {
    // parents come before their children, so the pool is a tree
    SMOE_REQUIRE(parent[v] >= -1 && parent[v] < v, SMOE_EINVAL,
                 "%s: node %d has parent %d (parents must precede their children; -1 = root)",
                 who, v, parent[v]);
    s.kids[parent[v] < 0 ? n : parent[v]].push_back(v);
  }
  s.unions.assign(static_cast<size_t>(Kc + 2) * L * s.W, 0);
  std::memcpy(s.unions.data(), expert_bits, sizeof(uint64_t) * L * s.W);  // the root's experts
  s.grow(s.kids[n], 0);
  for (int i = 0; i < s.best_n; ++i) selected[i] = s.best[i];
  *n_selected = s.best_n;
  if (ratio) *ratio = s.best_ratio;
  if (n_evaluated) *n_evaluated = s.evaluated;
  return SMOE_OK;
}
