// Schedule builder (host).  Each collective becomes a list of steps; a step is
// a set of work items that one fused kernel launch executes for all ranks at
// once, so every step here is written from the receiving rank's side.
//
// Ring ([RING-RHD] "Ring AllReduce带宽最优的环形流水线"; [TOPO]
// "AllReduce算法实现"): P-1 reduce-scatter steps in which rank r combines the
// partial of segment (r-t-2) mod P received from rank r-1 with its own
// (ending with segment r reduced on rank r), then P-1 all-gather steps in
// which rank r copies segment (r-1-t) mod P from rank r-1.
//
// Recursive halving-doubling ([RHD] "算法描述", Table 1): with
// r = P - 2^floor(log2 P), ranks 2i+1 (i < r) are first merged into 2i;
// virtual rank v (real rank 2v for v < r, v + r otherwise) halves its window
// with partner v xor 2^j at step j (keeping the lower half when bit j of v is
// 0), then doubles it back in reverse; ranks 2i+1 finally receive a copy.
// Stand-alone reduce-scatter / all-gather for P = 2^k are order-preserving:
// distances P/2 .. 1 (rank v keeps the aligned block containing segment v),
// then 1 .. P/2 for the all-gather.
//
// Stand-alone RHD reduce-scatter / all-gather for P not a power of two
// ([RHD] Table 1): Reduce (two-share pairs merge), a non-uniform halving over
// the 2^k virtual ranks, Scatter (and the mirror image for all-gather).  The
// P shares lie in order along the virtual ranks; virtual rank v carries two
// shares when the k-bit reversal of v is below r, which bounds the exchange
// of halving step i by ceil(P / 2^i) shares.  RHD Reduce / Broadcast with a
// root: in part1 the rank of each pair with the root's parity takes part in
// the 2^k block; Reduce = merge + order-preserving reduce-scatter over the
// 2^k-way split + gather to the root; Broadcast = distance halving from the
// root, then one copy to each part1 partner.
//
// Flat, tree and hierarchical AllReduce ([TOPO] "AllReduce算法实现"; [PIPE]
// "与其它分级算法的关系"): Flat folds all P vectors at rank 0 in rank order and
// copies the result to every rank (one read, P-1 writes); the tree reduces a
// heap-ordered K-ary tree level by level (each parent folds itself and its
// children in rank order) and copies back down; the hierarchical AllReduce is
// an intra-server full-mesh reduce-scatter of block m onto (s,m), a ring
// AllReduce of block m over the servers, and an intra-server copy of block m
// from (s,m) to its peers.
//
// Pipeline ([PIPE] "AllGather 算子的 Pipeline 时序编排", "Rank0 视角的传输任务编排",
// Table 1): rank g = s*M + m; each loop (slice of at most loop_bytes) is split
// into P blocks.  Reduce-scatter: one intra-server step in which (s,m) folds
// its server's M contributions to block ((s-1)M+m), then S-1 steps in which
// (s,m) combines the partial received from (s-1,m) with its server's fold of
// block ((s-t-2)M+m).  All-gather: S-1 steps in which (s,m) sends block
// ((s-t)M+m) both to (s+1,m) and to its M-1 server peers (one read, M
// writes), then one intra-server pass of block ((s+1)M+m).
#include "plan.hpp"

#include <algorithm>

namespace hbmc {
namespace {

// Ceiling split of n elements into `parts` contiguous parts.
struct Split {
  uint64_t n, parts, q;
  Split(uint64_t n_, uint64_t parts_) : n(n_), parts(parts_), q(parts_ ? (n_ + parts_ - 1) / parts_ : 0) {}
  uint64_t at(uint64_t k) const { return std::min(k * q, n); }
};

inline int wrap(long a, long m) {
  long r = a % m;
  return static_cast<int>(r < 0 ? r + m : r);
}

inline int log2_floor(int p) {
  int k = 0;
  while ((2 << k) <= p) ++k;
  return k;
}

class Builder {
 public:
  explicit Builder(Schedule* s) : sched_(s) {}

  Step& open(Mode mode) {
    sched_->steps.emplace_back();
    Step& st = sched_->steps.back();
    st.mode = mode;
    return st;
  }

  // Append an item [base + b, base + e) with the given sources / destinations.
  static void add(Step& st, uint64_t b, uint64_t e, std::initializer_list<int> src,
                  std::initializer_list<int> dst) {
    std::vector<int> s(src), d(dst);
    add(st, b, e, s, d);
  }
  static void add(Step& st, uint64_t b, uint64_t e, const std::vector<int>& src,
                  const std::vector<int>& dst) {
    if (e <= b || dst.empty()) return;
    Item it;
    it.begin = b;
    it.count = e - b;
    it.nsrc = static_cast<int32_t>(src.size());
    it.ndst = static_cast<int32_t>(dst.size());
    int k = 0;
    for (int r : src) it.rank[k++] = static_cast<uint8_t>(r);
    for (int r : dst) it.rank[k++] = static_cast<uint8_t>(r);
    st.items.push_back(it);
  }

 private:
  Schedule* sched_;
};

// ---------------------------------------------------------------- ring
void ring(const Topology& t, Coll coll, uint64_t L, Builder& B) {
  const int P = t.P;
  Split seg(L, P);
  if (coll != kAllGather) {
    for (int step = 0; step < P - 1; ++step) {
      Step& st = B.open(kRecvFold);
      for (int r = 0; r < P; ++r) {
        int c = wrap(r - step - 2, P);
        Builder::add(st, seg.at(c), seg.at(c + 1), {wrap(r - 1, P), r}, {r});
      }
    }
  }
  if (coll != kReduceScatter) {
    for (int step = 0; step < P - 1; ++step) {
      Step& st = B.open(kCopy);
      for (int r = 0; r < P; ++r) {
        int c = wrap(r - 1 - step, P);
        Builder::add(st, seg.at(c), seg.at(c + 1), {wrap(r - 1, P)}, {r});
      }
    }
  }
}

// ---------------------------------------------------------------- RHD
// First segment of virtual rank v's window after halving steps 0..j.
inline int hd_window_start(int v, int j, int pp) {
  int start = 0;
  for (int i = 0; i <= j; ++i)
    if ((v >> i) & 1) start += pp >> (i + 1);
  return start;
}

void rhd_allreduce(const Topology& t, uint64_t L, Builder& B) {
  const int P = t.P, k = log2_floor(P), pp = 1 << k, extra = P - pp;
  auto real = [extra](int v) { return v < extra ? 2 * v : v + extra; };
  Split seg(L, pp);
  if (extra > 0) {  // merge part1
    Step& st = B.open(kRecvFold);
    for (int i = 0; i < extra; ++i) Builder::add(st, 0, L, {2 * i + 1, 2 * i}, {2 * i});
  }
  for (int j = 0; j < k; ++j) {  // halving
    Step& st = B.open(kRecvFold);
    const int len = pp >> (j + 1);
    for (int v = 0; v < pp; ++v) {
      int a = hd_window_start(v, j, pp);
      Builder::add(st, seg.at(a), seg.at(a + len), {real(v ^ (1 << j)), real(v)}, {real(v)});
    }
  }
  for (int j = k - 1; j >= 0; --j) {  // doubling
    Step& st = B.open(kCopy);
    const int len = pp >> (j + 1);
    for (int v = 0; v < pp; ++v) {
      int u = v ^ (1 << j);
      int a = hd_window_start(u, j, pp);
      Builder::add(st, seg.at(a), seg.at(a + len), {real(u)}, {real(v)});
    }
  }
  if (extra > 0) {  // restore part1
    Step& st = B.open(kCopy);
    for (int i = 0; i < extra; ++i) Builder::add(st, 0, L, {2 * i}, {2 * i + 1});
  }
}

void rhd_ordered(const Topology& t, Coll coll, uint64_t L, Builder& B) {
  const int P = t.P;
  Split seg(L, P);
  if (coll == kReduceScatter) {
    for (int d = P / 2; d >= 1; d /= 2) {
      Step& st = B.open(kRecvFold);
      for (int v = 0; v < P; ++v) {
        int a = v & ~(d - 1);
        Builder::add(st, seg.at(a), seg.at(a + d), {v ^ d, v}, {v});
      }
    }
  } else {
    for (int d = 1; d < P; d *= 2) {
      Step& st = B.open(kCopy);
      for (int v = 0; v < P; ++v) {
        int a = (v ^ d) & ~(d - 1);
        Builder::add(st, seg.at(a), seg.at(a + d), {v ^ d}, {v});
      }
    }
  }
}

// ---------------------------------------------------------------- RHD, P not 2^k
struct ShareMap {
  int k, pp, r;
  std::vector<int> first;  // first share of virtual rank v, first[pp] == P
  std::vector<bool> two;   // virtual rank v carries two shares
};

ShareMap share_map(int P) {
  ShareMap m;
  m.k = log2_floor(P);
  m.pp = 1 << m.k;
  m.r = P - m.pp;
  m.first.assign(m.pp + 1, 0);
  m.two.assign(m.pp, false);
  for (int v = 0; v < m.pp; ++v) {
    int rev = 0;
    for (int b = 0; b < m.k; ++b) rev |= ((v >> b) & 1) << (m.k - 1 - b);
    m.two[v] = rev < m.r;
    m.first[v + 1] = m.first[v] + (m.two[v] ? 2 : 1);
  }
  return m;
}

void rhd_unordered_np2(const Topology& t, Coll coll, uint64_t L, Builder& B) {
  const ShareMap m = share_map(t.P);
  Split seg(L, t.P);
  auto span = [&](int v0, int v1, uint64_t* lo, uint64_t* hi) {  // shares of virtual ranks [v0, v1)
    *lo = seg.at(m.first[v0]);
    *hi = seg.at(m.first[v1]);
  };
  uint64_t lo, hi;
  if (coll == kReduceScatter) {
    Step& merge = B.open(kRecvFold);
    for (int v = 0; v < m.pp; ++v)
      if (m.two[v]) Builder::add(merge, 0, L, {m.first[v] + 1, m.first[v]}, {m.first[v]});
    for (int d = m.pp / 2; d >= 1; d /= 2) {
      Step& st = B.open(kRecvFold);
      for (int v = 0; v < m.pp; ++v) {
        const int a = v & ~(d - 1);  // the aligned block of d virtual ranks that holds v
        span(a, a + d, &lo, &hi);
        Builder::add(st, lo, hi, {m.first[v ^ d], m.first[v]}, {m.first[v]});
      }
    }
    Step& scatter = B.open(kCopy);
    for (int v = 0; v < m.pp; ++v)
      if (m.two[v]) {
        const int g = m.first[v] + 1;
        Builder::add(scatter, seg.at(g), seg.at(g + 1), {m.first[v]}, {g});
      }
  } else {
    Step& gather = B.open(kCopy);
    for (int v = 0; v < m.pp; ++v)
      if (m.two[v]) {
        const int g = m.first[v] + 1;
        Builder::add(gather, seg.at(g), seg.at(g + 1), {g}, {m.first[v]});
      }
    for (int d = 1; d < m.pp; d *= 2) {
      Step& st = B.open(kCopy);
      for (int v = 0; v < m.pp; ++v) {
        const int a = (v ^ d) & ~(d - 1);  // the partner's collected block
        span(a, a + d, &lo, &hi);
        Builder::add(st, lo, hi, {m.first[v ^ d]}, {m.first[v]});
      }
    }
    Step& spread = B.open(kCopy);
    for (int v = 0; v < m.pp; ++v)
      if (m.two[v]) Builder::add(spread, 0, L, {m.first[v]}, {m.first[v] + 1});
  }
}

// ---------------------------------------------------------------- RHD rooted
void rhd_rooted(const Topology& t, Coll coll, uint64_t L, int root, Builder& B) {
  const int k = log2_floor(t.P), pp = 1 << k, r = t.P - pp;
  const int par = (root < 2 * r) ? (root & 1) : 0;  // part1 side that joins the block
  auto real = [&](int v) { return v < r ? 2 * v + par : v + r; };
  auto mate = [&](int i) { return 2 * i + 1 - par; };
  const int vroot = root < 2 * r ? root / 2 : root - r;
  Split seg(L, pp);
  if (coll == kReduce) {
    if (r > 0) {
      Step& merge = B.open(kRecvFold);
      for (int i = 0; i < r; ++i) Builder::add(merge, 0, L, {mate(i), real(i)}, {real(i)});
    }
    for (int d = pp / 2; d >= 1; d /= 2) {
      Step& st = B.open(kRecvFold);
      for (int v = 0; v < pp; ++v) {
        const int a = v & ~(d - 1);
        Builder::add(st, seg.at(a), seg.at(a + d), {real(v ^ d), real(v)}, {real(v)});
      }
    }
    for (int d = 1; d < pp; d *= 2) {
      Step& st = B.open(kCopy);
      for (int v = 0; v < pp; ++v) {
        const int rel = v ^ vroot;
        if ((rel & d) == 0 || (rel & (d - 1)) != 0) continue;  // lowest set bit of rel must be d
        const int a = v & ~(d - 1);
        Builder::add(st, seg.at(a), seg.at(a + d), {real(v)}, {real(v ^ d)});
      }
    }
  } else {
    for (int d = pp / 2; d >= 1; d /= 2) {
      Step& st = B.open(kCopy);
      for (int v = 0; v < pp; ++v)
        if (((v ^ vroot) % (2 * d)) == 0) Builder::add(st, 0, L, {real(v)}, {real(v ^ d)});
    }
    if (r > 0) {
      Step& st = B.open(kCopy);
      for (int i = 0; i < r; ++i) Builder::add(st, 0, L, {real(i)}, {mate(i)});
    }
  }
}

// ---------------------------------------------------------------- pipeline
void pipeline(const Topology& t, Coll coll, uint64_t L, uint32_t esize, Builder& B,
              Schedule* sched) {
  const int S = t.S, M = t.M, P = t.P;
  const uint64_t lb = t.loop_bytes ? t.loop_bytes : (uint64_t(32) << 20);
  const uint64_t C = std::max<uint64_t>(1, lb / esize);
  const int rs_steps = (coll != kAllGather) ? S : 0;
  const int ag_steps = (coll != kReduceScatter) ? S : 0;
  std::vector<size_t> idx;
  for (int i = 0; i < rs_steps; ++i) {
    B.open(i == 0 ? kFold : kRecvFold);
    idx.push_back(sched->steps.size() - 1);
  }
  for (int i = 0; i < ag_steps; ++i) {
    B.open(kCopy);
    idx.push_back(sched->steps.size() - 1);
  }
  auto g = [M](int s, int m) { return s * M + m; };
  for (uint64_t base = 0; base < L; base += C) {
    const uint64_t n = std::min(C, L - base);
    Split blk(n, P);
    auto range = [&](int b, uint64_t* lo, uint64_t* hi) {
      *lo = base + blk.at(b);
      *hi = base + blk.at(b + 1);
    };
    uint64_t lo, hi;
    int si = 0;
    if (rs_steps) {
      Step& st = sched->steps[idx[si++]];
      for (int s = 0; s < S; ++s)
        for (int m = 0; m < M; ++m) {
          if (M == 1) continue;  // a fold of one block onto itself is no work
          std::vector<int> src;
          for (int l = 0; l < M; ++l) src.push_back(g(s, l));
          range(wrap(s - 1, S) * M + m, &lo, &hi);
          Builder::add(st, lo, hi, src, {g(s, m)});
        }
      for (int step = 0; step < S - 1; ++step) {
        Step& rst = sched->steps[idx[si++]];
        for (int s = 0; s < S; ++s)
          for (int m = 0; m < M; ++m) {
            std::vector<int> src{g(wrap(s - 1, S), m)};
            for (int l = 0; l < M; ++l) src.push_back(g(s, l));
            range(wrap(s - step - 2, S) * M + m, &lo, &hi);
            Builder::add(rst, lo, hi, src, {g(s, m)});
          }
      }
    }
    if (ag_steps) {
      for (int step = 0; step < S - 1; ++step) {
        Step& st = sched->steps[idx[si++]];
        for (int s = 0; s < S; ++s)
          for (int m = 0; m < M; ++m) {
            std::vector<int> dst{g(wrap(s + 1, S), m)};
            for (int l = 0; l < M; ++l)
              if (l != m) dst.push_back(g(s, l));
            range(wrap(s - step, S) * M + m, &lo, &hi);
            Builder::add(st, lo, hi, {g(s, m)}, dst);
          }
      }
      Step& st = sched->steps[idx[si++]];
      for (int s = 0; s < S; ++s)
        for (int m = 0; m < M; ++m) {
          std::vector<int> dst;
          for (int l = 0; l < M; ++l)
            if (l != m) dst.push_back(g(s, l));
          range(wrap(s + 1, S) * M + m, &lo, &hi);
          Builder::add(st, lo, hi, {g(s, m)}, dst);
        }
    }
  }
}

// ---------------------------------------------------------------- flat / tree / hier
void flat(const Topology& t, uint64_t L, Builder& B) {
  std::vector<int> all, rest;
  for (int r = 0; r < t.P; ++r) {
    all.push_back(r);
    if (r) rest.push_back(r);
  }
  Step& red = B.open(kFold);
  Builder::add(red, 0, L, all, {0});
  Step& out = B.open(kCopy);
  Builder::add(out, 0, L, {0}, rest);
}

void tree(const Topology& t, uint64_t L, Builder& B) {
  const int P = t.P, K = t.K;
  std::vector<int> level(P, 0);
  for (int i = 1; i < P; ++i) level[i] = level[(i - 1) / K] + 1;
  const int height = level[P - 1];
  auto children = [&](int p) {
    std::vector<int> c;
    for (int q = K * p + 1; q <= K * p + K && q < P; ++q) c.push_back(q);
    return c;
  };
  for (int lvl = height - 1; lvl >= 0; --lvl) {
    Step& st = B.open(kFold);
    for (int p = 0; p < P; ++p) {
      if (level[p] != lvl) continue;
      std::vector<int> src{p}, c = children(p);
      if (c.empty()) continue;
      src.insert(src.end(), c.begin(), c.end());
      Builder::add(st, 0, L, src, {p});
    }
  }
  for (int lvl = 0; lvl < height; ++lvl) {
    Step& st = B.open(kCopy);
    for (int p = 0; p < P; ++p)
      if (level[p] == lvl) Builder::add(st, 0, L, {p}, children(p));
  }
}

void hier(const Topology& t, uint64_t L, Builder& B) {
  const int S = t.S, M = t.M;
  auto g = [M](int s, int m) { return s * M + m; };
  Split blk(L, M);
  Step& rs = B.open(kFold);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      if (M == 1) continue;  // a fold of one block onto itself is no work
      std::vector<int> src;
      for (int l = 0; l < M; ++l) src.push_back(g(s, l));
      Builder::add(rs, blk.at(m), blk.at(m + 1), src, {g(s, m)});
    }
  for (int phase = 0; phase < 2; ++phase)
    for (int step = 0; step < S - 1; ++step) {
      Step& st = B.open(phase == 0 ? kRecvFold : kCopy);
      for (int m = 0; m < M; ++m) {
        const uint64_t b0 = blk.at(m);
        Split sub(blk.at(m + 1) - b0, S);
        for (int s = 0; s < S; ++s) {  // receiver (s, m)
          const int c = phase == 0 ? wrap(s - step - 2, S) : wrap(s - 1 - step, S);
          const int from = g(wrap(s - 1, S), m);
          if (phase == 0)
            Builder::add(st, b0 + sub.at(c), b0 + sub.at(c + 1), {from, g(s, m)}, {g(s, m)});
          else
            Builder::add(st, b0 + sub.at(c), b0 + sub.at(c + 1), {from}, {g(s, m)});
        }
      }
    }
  Step& ag = B.open(kCopy);
  for (int s = 0; s < S; ++s)
    for (int m = 0; m < M; ++m) {
      std::vector<int> peers;
      for (int l = 0; l < M; ++l)
        if (l != m) peers.push_back(g(s, l));
      Builder::add(ag, blk.at(m), blk.at(m + 1), {g(s, m)}, peers);
    }
}

// ---------------------------------------------------------------- checks
// No two items of a step may touch overlapping ranges of one rank where
// either writes; within an item a destination may only be read on its own
// range (the in-place local operand).
bool step_is_race_free(const Step& st) {
  struct Touch {
    int rank;
    uint64_t b, e;
    size_t item;
    bool write;
  };
  std::vector<Touch> v;
  for (size_t i = 0; i < st.items.size(); ++i) {
    const Item& it = st.items[i];
    for (int k = 0; k < it.nsrc + it.ndst; ++k)
      v.push_back({it.rank[k], it.begin, it.begin + it.count, i, k >= it.nsrc});
    for (int a = it.nsrc; a < it.nsrc + it.ndst; ++a)
      for (int b = a + 1; b < it.nsrc + it.ndst; ++b)
        if (it.rank[a] == it.rank[b]) return false;  // one destination twice
  }
  std::sort(v.begin(), v.end(), [](const Touch& x, const Touch& y) {
    return x.rank != y.rank ? x.rank < y.rank : x.b < y.b;
  });
  for (size_t i = 0; i < v.size(); ++i)
    for (size_t j = i + 1; j < v.size() && v[j].rank == v[i].rank && v[j].b < v[i].e; ++j)
      if (v[i].item != v[j].item && (v[i].write || v[j].write)) return false;
  return true;
}

}  // namespace

BuildStatus build_schedule(const Topology& topo, Coll coll, uint64_t count, uint32_t esize, int root,
                           Schedule* out) {
  *out = Schedule{};
  if (topo.P < 1 || topo.P > kMaxRanks || esize == 0) return kBadArg;
  if (coll < kAllReduce || coll > kBroadcast) return kBadArg;
  if ((topo.algo == kPipeline || topo.algo == kHier) &&
      (topo.S < 1 || topo.M < 1 || topo.S * topo.M != topo.P))
    return kBadArg;
  if (topo.algo == kTree && (topo.K < 2 || topo.K > kMaxRanks)) return kBadArg;
  const bool rooted = coll == kReduce || coll == kBroadcast;
  if ((topo.algo == kFlat || topo.algo == kTree || topo.algo == kHier) && coll != kAllReduce)
    return kUnsupported;
  if (rooted && (root < 0 || root >= topo.P)) return kBadArg;
  if (rooted && topo.algo != kRhd) return kUnsupported;
  const bool pow2 = (topo.P & (topo.P - 1)) == 0;
  if (topo.P == 1) return kBuilt;

  Builder B(out);
  switch (topo.algo) {
    case kRing: ring(topo, coll, count, B); break;
    case kRhd:
      if (coll == kAllReduce)
        rhd_allreduce(topo, count, B);
      else if (rooted)
        rhd_rooted(topo, coll, count, root, B);
      else if (pow2)
        rhd_ordered(topo, coll, count, B);
      else
        rhd_unordered_np2(topo, coll, count, B);
      break;
    case kPipeline: pipeline(topo, coll, count, esize, B, out); break;
    case kFlat: flat(topo, count, B); break;
    case kTree: tree(topo, count, B); break;
    case kHier: hier(topo, count, B); break;
    default: return kBadArg;
  }

  std::vector<uint64_t> recv(topo.P, 0);
  for (Step& st : out->steps) {
    bool first = true, mixed = false;
    for (const Item& it : st.items) {
      if (first) {
        st.nsrc = it.nsrc;
        st.ndst = it.ndst;
        first = false;
      } else if (it.nsrc != st.nsrc || it.ndst != st.ndst) {
        mixed = true;  // items of different shapes: the kernel reads each item's counts
      }
      st.hbm_bytes += uint64_t(it.nsrc + it.ndst) * it.count * esize;
      st.max_count = std::max(st.max_count, it.count);
      for (int d = it.nsrc; d < it.nsrc + it.ndst; ++d) {
        int others = 0;
        for (int s = 0; s < it.nsrc; ++s) others += it.rank[s] != it.rank[d];
        recv[it.rank[d]] += uint64_t(others) * it.count * esize;
      }
    }
    if (mixed) st.nsrc = st.ndst = 0;
    if (!step_is_race_free(st)) return kBadArg;
    out->hbm_bytes += st.hbm_bytes;
  }
  out->max_recv_bytes = *std::max_element(recv.begin(), recv.end());
  return kBuilt;
}

}  // namespace hbmc
