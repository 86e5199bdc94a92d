// The register form of a whole call: deriving each element's expression from
// the schedule (host only).
#include "regs.hpp"

#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <utility>

namespace hbmc {
namespace {

constexpr size_t kMaxIntervals = 4096;

// Expression nodes: ids below P are the ranks' inputs, larger ids are
// op(a, b), stored with a <= b (the element ops commute bit for bit) and
// shared by structure, so two expressions are equal exactly when their ids
// are.
struct Exprs {
  int P;
  std::vector<std::pair<int, int>> node;
  std::unordered_map<uint64_t, int> ids;
  explicit Exprs(int p) : P(p) {}
  int op(int a, int b) {
    if (a > b) std::swap(a, b);
    const uint64_t key = (uint64_t(uint32_t(a)) << 32) | uint32_t(b);
    auto it = ids.find(key);
    if (it != ids.end()) return it->second;
    const int id = P + static_cast<int>(node.size());
    node.emplace_back(a, b);
    ids.emplace(key, id);
    return id;
  }
  bool leaf(int x) const { return x < P; }
  const std::pair<int, int>& kids(int x) const { return node[x - P]; }
};

// The value an item leaves in its destinations (send-then-combine: the
// sources as they were before the step).
int item_value(Exprs& X, const Step& st, const Item& it, const int* val) {
  if (st.mode == kCopy) return val[it.rank[0]];
  if (st.mode == kFold) {
    int acc = val[it.rank[0]];
    for (int q = 1; q < it.nsrc; ++q) acc = X.op(acc, val[it.rank[q]]);
    return acc;
  }
  // op(received, left fold of the other sources)
  int acc = val[it.rank[1]];
  for (int q = 2; q < it.nsrc; ++q) acc = X.op(acc, val[it.rank[q]]);
  return X.op(val[it.rank[0]], acc);
}

void depths(const Exprs& X, int x, int d, int* dmin, int* dmax) {
  if (X.leaf(x)) {
    *dmin = std::min(*dmin, d);
    *dmax = std::max(*dmax, d);
    return;
  }
  depths(X, X.kids(x).first, d + 1, dmin, dmax);
  depths(X, X.kids(x).second, d + 1, dmin, dmax);
}

void units_at(const Exprs& X, int x, int d, int k, std::vector<int>* out) {
  if (d == k) {
    out->push_back(x);
    return;
  }
  units_at(X, X.kids(x).first, d + 1, k, out);
  units_at(X, X.kids(x).second, d + 1, k, out);
}

// Tree form of expression e: leaves (a, b) with b = 0xff for a single rank;
// false when e is not a complete tree of such leaves.
bool as_tree(Exprs& X, int e, std::vector<std::pair<int, int>>* leaves) {
  if (X.leaf(e)) return false;
  int dmin = 1 << 30, dmax = -1;
  depths(X, e, 0, &dmin, &dmax);
  if (dmax - dmin > 1 || dmin > 4) return false;
  std::vector<int> u;
  units_at(X, e, 0, dmin, &u);
  if (u.size() != (size_t(1) << dmin)) return false;
  leaves->clear();
  std::vector<int> level;
  for (int x : u) {
    if (X.leaf(x)) {
      leaves->emplace_back(x, 0xff);
      level.push_back(x);
      continue;
    }
    const auto& k = X.kids(x);
    if (!X.leaf(k.first) || !X.leaf(k.second)) return false;
    leaves->emplace_back(k.first, k.second);
    level.push_back(X.op(k.first, k.second));
  }
  // rebuild pairwise, (0,1), (2,3), ... level by level: must give e back
  while (level.size() > 1) {
    std::vector<int> next;
    for (size_t i = 0; i + 1 < level.size(); i += 2) next.push_back(X.op(level[i], level[i + 1]));
    level.swap(next);
  }
  return level[0] == e;
}

// Fold form of e: the left fold over `seq`; false when e is not one.
bool as_fold(Exprs& X, int e, std::vector<int>* seq) {
  std::vector<int> rev;
  int x = e;
  while (x >= 0 && !X.leaf(x)) {
    const auto k = X.kids(x);
    if (X.leaf(k.first) && X.leaf(k.second)) {
      rev.push_back(k.second);
      rev.push_back(k.first);
      x = -1;
    } else if (X.leaf(k.second)) {
      rev.push_back(k.second);
      x = k.first;
    } else if (X.leaf(k.first)) {
      rev.push_back(k.first);
      x = k.second;
    } else {
      return false;
    }
  }
  if (x >= 0) return false;  // a bare input: no operation at all
  seq->assign(rev.rbegin(), rev.rend());
  if (seq->size() > size_t(kRegMaxLeaves)) return false;
  int acc = (*seq)[0];
  for (size_t i = 1; i < seq->size(); ++i) acc = X.op(acc, (*seq)[i]);
  return acc == e;
}

}  // namespace

void derive_regs(const Schedule& s, int P, uint64_t count, RegPlan* out) {
  *out = RegPlan();
  if (P < 2 || P > 2 * kRegMaxLeaves || count == 0) return;
  // intervals that the same items cover
  std::vector<uint64_t> cut{0, count};
  for (const Step& st : s.steps)
    for (const Item& it : st.items) {
      cut.push_back(it.begin);
      cut.push_back(it.begin + it.count);
    }
  std::sort(cut.begin(), cut.end());
  cut.erase(std::unique(cut.begin(), cut.end()), cut.end());
  if (cut.back() != count || cut.size() - 1 > kMaxIntervals) return;
  const size_t nint = cut.size() - 1;
  Exprs X(P);
  std::vector<int> val(nint * P);
  for (size_t t = 0; t < nint; ++t)
    for (int r = 0; r < P; ++r) val[t * P + r] = r;
  for (const Step& st : s.steps)
    for (const Item& it : st.items) {
      const size_t t0 = std::lower_bound(cut.begin(), cut.end(), it.begin) - cut.begin();
      const size_t t1 = std::lower_bound(cut.begin(), cut.end(), it.begin + it.count) - cut.begin();
      for (size_t t = t0; t < t1; ++t) {
        int* v = &val[t * P];
        const int x = item_value(X, st, it, v);
        for (int q = it.nsrc; q < it.nsrc + it.ndst; ++q) v[it.rank[q]] = x;
      }
    }
  std::vector<RegRegion> regs;
  auto push = [&](uint64_t end, const RegRegion& r) {
    if (!regs.empty() && std::memcmp(regs.back().a, r.a, sizeof(r.a)) == 0 &&
        std::memcmp(regs.back().b, r.b, sizeof(r.b)) == 0 && std::memcmp(regs.back().lvl, r.lvl, sizeof(r.lvl)) == 0) {
      regs.back().end = end;
      return;
    }
    regs.push_back(r);
    regs.back().end = end;
  };
  std::vector<std::pair<int, int>> leaves;
  std::vector<int> seq;
  auto finish = [&](RegForm form, uint32_t n, uint32_t loads, uint32_t stores) {
    if (regs.size() > size_t(form == kRegTree ? kRegMaxTreeRegions : kRegMaxFoldRegions)) return;
    out->ok = true;
    out->form = form;
    out->n = n;
    out->loads = loads;
    out->stores = stores;
    out->regions = regs;
  };
  bool same = true;
  std::vector<int> expr(nint);
  for (size_t t = 0; t < nint; ++t) {
    expr[t] = val[t * P];
    for (int r = 1; r < P; ++r) same = same && val[t * P + r] == expr[t];
  }
  if (!same) {
    if (P > kRegMaxLeaves) return;
    // prefixes of one fold: the first rank holding a fold over all P ranks
    // names the sequence; rank seq[0] keeps its input and rank seq[i] holds
    // the fold over seq[0..i]
    auto prefix = [&]() {
      for (size_t t = 0; t < nint; ++t) {
        const int* v = &val[t * P];
        bool found = false;
        for (int r = 0; r < P && !found; ++r) found = as_fold(X, v[r], &seq) && seq.size() == size_t(P);
        if (!found) return false;
        // the first two operands of a fold commute: the one that keeps its input goes first
        if (v[seq[0]] != seq[0]) std::swap(seq[0], seq[1]);
        if (v[seq[0]] != seq[0]) return false;
        int pre = seq[0];
        for (int i = 1; i < P; ++i) {
          pre = X.op(pre, seq[i]);
          if (v[seq[i]] != pre) return false;
        }
        RegRegion r;
        std::memset(&r, 0xff, sizeof(r));
        for (int i = 0; i < P; ++i) r.a[i] = static_cast<uint8_t>(seq[i]);
        push(cut[t + 1], r);
      }
      return true;
    };
    // nodes of one complete tree of single ranks over all P ranks: every rank
    // keeps its input or holds a node above its own leaf (how many ranks
    // receive a node may differ between intervals: `stores` is the most)
    uint32_t stores = 0;
    auto nodes = [&]() {
      if (P & (P - 1)) return false;
      int k = 0;
      while ((1 << k) < P) ++k;
      for (size_t t = 0; t < nint; ++t) {
        const int* v = &val[t * P];
        bool found = false;
        for (int r = 0; r < P && !found; ++r) {
          if (!as_tree(X, v[r], &leaves) || leaves.size() != size_t(P)) continue;
          found = true;
          for (const auto& lf : leaves) found = found && lf.second == 0xff;
        }
        if (!found) return false;
        // node ids level by level, as the kernel pairs them
        std::vector<std::vector<int>> lv(k + 1);
        for (const auto& lf : leaves) lv[0].push_back(lf.first);
        for (int l = 1; l <= k; ++l)
          for (size_t j = 0; j + 1 < lv[l - 1].size(); j += 2) lv[l].push_back(X.op(lv[l - 1][j], lv[l - 1][j + 1]));
        RegRegion r;
        std::memset(&r, 0xff, sizeof(r));
        uint32_t n_st = 0;
        for (int i = 0; i < P; ++i) {
          const int rank = lv[0][i];
          r.a[i] = static_cast<uint8_t>(rank);
          int got = -1;
          if (v[rank] == rank) got = 0;
          for (int l = 1; l <= k && got < 0; ++l)
            if (lv[l][i >> l] == v[rank]) got = l;
          if (got < 0) return false;
          r.lvl[i] = static_cast<uint8_t>(got);
          n_st += got > 0;
        }
        stores = std::max(stores, n_st);
        push(cut[t + 1], r);
      }
      return true;
    };
    if (prefix()) {
      finish(kRegPrefix, static_cast<uint32_t>(P), static_cast<uint32_t>(P), static_cast<uint32_t>(P - 1));
      return;
    }
    regs.clear();
    if (nodes()) finish(kRegNodes, static_cast<uint32_t>(P), static_cast<uint32_t>(P), stores);
    return;
  }
  bool copy = true;
  for (size_t t = 0; t < nint; ++t) copy = copy && X.leaf(expr[t]);
  if (copy) {
    // every rank ends with rank expr[t]'s input
    if (P > kRegMaxLeaves) return;
    for (size_t t = 0; t < nint; ++t) {
      RegRegion r;
      std::memset(&r, 0xff, sizeof(r));
      r.a[0] = static_cast<uint8_t>(expr[t]);
      for (int q = 0, i = 1; q < P; ++q)
        if (q != expr[t]) r.a[i++] = static_cast<uint8_t>(q);
      push(cut[t + 1], r);
    }
    finish(kRegCopy, static_cast<uint32_t>(P), 1, static_cast<uint32_t>(P - 1));
    return;
  }
  bool tree = true;
  uint32_t n = 0;
  for (size_t t = 0; t < nint && tree; ++t) {
    if (!as_tree(X, expr[t], &leaves) || (n && leaves.size() != n)) tree = false;
    n = static_cast<uint32_t>(leaves.size());
    if (!tree) break;
    RegRegion r;
    std::memset(&r, 0xff, sizeof(r));
    for (size_t v = 0; v < leaves.size(); ++v) {
      r.a[v] = static_cast<uint8_t>(leaves[v].first);
      r.b[v] = static_cast<uint8_t>(leaves[v].second);
    }
    push(cut[t + 1], r);
  }
  RegForm form = kRegTree;
  if (!tree) {
    regs.clear();
    n = 0;
    form = kRegFold;
    for (size_t t = 0; t < nint; ++t) {
      if (!as_fold(X, expr[t], &seq) || (n && seq.size() != n)) return;
      n = static_cast<uint32_t>(seq.size());
      RegRegion r;
      std::memset(&r, 0xff, sizeof(r));
      for (size_t i = 0; i < seq.size(); ++i) r.a[i] = static_cast<uint8_t>(seq[i]);
      push(cut[t + 1], r);
    }
  }
  // every rank exactly once among each region's operands: they are also the
  // destinations the result is stored to
  for (const RegRegion& r : regs) {
    std::vector<int> seen(P, 0);
    for (uint32_t v = 0; v < n; ++v) {
      if (r.a[v] >= P || seen[r.a[v]]++) return;
      if (r.b[v] != 0xff && (r.b[v] >= P || seen[r.b[v]]++)) return;
    }
    for (int q = 0; q < P; ++q)
      if (!seen[q]) return;
  }
  finish(form, n, static_cast<uint32_t>(P), static_cast<uint32_t>(P));
}

}  // namespace hbmc
