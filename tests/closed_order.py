"""Closed-order evaluators: the reduction order each schedule implies, per element.

Written from the orders the schedules produce (not by replaying steps), using
the library element ops of ``refops``.  ``op(recv, local)`` is how a step
combines a received partial with a local block.

  ring AllReduce, element in segment c of the P-way ceiling split:
      ((X_{c+1} op X_{c+2}) op ...) op X_c        (indices mod P)
  RHD AllReduce, k = floor(log2 P), p' = 2^k, r = P - p':
      leaves X'_v = X_{2v+1} op X_{2v} for v < r, else X_{v+r};
      balanced binary tree over v in natural order (pairs (2w, 2w+1) first)
  RHD order-preserving reduce-scatter, P = 2^k:
      tree pairing v with v + P/2 first, then v + P/4, ...
  RHD stand-alone reduce-scatter, P not a power of two (shares in order
  along 2^k virtual ranks, two-share ranks where the k-bit reversal of v
  is below r): leaves X'_v = X_{s+1} op X_s for a two-share rank with
  first share s, else X_s; tree pairing v with v + 2^k/2 first, ...
  RHD Reduce to a root: part1 pairs (2i, 2i+1) keep on the root's
  parity side: X'_v = X_partner op X_keeper; the same halving tree.
  Flat AllReduce: left fold in rank order X_0 op X_1 op ... op X_{P-1}.
  K-ary tree AllReduce (heap order): value(p) = fold of X_p, value(c_1),
  ..., value(c_K) over its children in rank order; the root's value.
  hierarchical AllReduce (S x M): element in block m (M-way split), and in
  sub-segment c of that block's S-way split: I_sigma = fold over l of
  X_(sigma,l); result ((I_{c+1} op I_{c+2}) op ...) op I_c.
  pipeline (S servers x M ranks), block (s, m) of each loop:
      I_sigma = ((X_(sigma,0) op X_(sigma,1)) op ...) op X_(sigma,M-1)
      result  = ((I_{s+1} op I_{s+2}) op ...) op I_s
"""
from __future__ import annotations

import numpy as np

from refops import STORAGE, combine, seg_bounds


def ring_allreduce(dtype, op, xs):
    P = len(xs)
    L = xs[0].size
    out = np.empty(L, STORAGE[dtype])
    for c in range(P):
        b, e = seg_bounds(L, P, c)
        if b == e:
            continue
        acc = xs[(c + 1) % P][b:e].copy()
        for i in range(2, P + 1):
            acc = combine(dtype, op, acc, xs[(c + i) % P][b:e])
        out[b:e] = acc
    return out


def _tree(dtype, op, leaves):
    while len(leaves) > 1:
        leaves = [combine(dtype, op, leaves[2 * w + 1], leaves[2 * w]) for w in range(len(leaves) // 2)]
    return leaves[0]


def rhd_allreduce(dtype, op, xs):
    P = len(xs)
    k = P.bit_length() - 1
    pp = 1 << k
    r = P - pp
    leaves = []
    for v in range(pp):
        if v < r:
            leaves.append(combine(dtype, op, xs[2 * v + 1], xs[2 * v]))
        else:
            leaves.append(xs[v + r].copy())
    return _tree(dtype, op, leaves)


def rhd_reduce_scatter_value(dtype, op, xs):
    P = len(xs)
    vals = [x.copy() for x in xs]
    d = P // 2
    while d >= 1:
        vals = [combine(dtype, op, vals[w + d], vals[w]) for w in range(d)]
        d //= 2
    return vals[0]


def _bitrev(v, k):
    return int(format(v, f"0{k}b")[::-1], 2) if k else 0


def np2_share_layout(P):
    """(k, first share of each virtual rank + end, two-share flags)."""
    k = P.bit_length() - 1
    pp = 1 << k
    r = P - pp
    two = [_bitrev(v, k) < r for v in range(pp)]
    first, s = [], 0
    for v in range(pp):
        first.append(s)
        s += 2 if two[v] else 1
    return k, first + [s], two


def _halving_tree(dtype, op, leaves):
    vals = [x.copy() for x in leaves]
    d = len(vals) // 2
    while d >= 1:
        vals = [combine(dtype, op, vals[w + d], vals[w]) for w in range(d)]
        d //= 2
    return vals[0]


def rhd_reduce_scatter_np2_value(dtype, op, xs):
    P = len(xs)
    k, first, two = np2_share_layout(P)
    leaves = [combine(dtype, op, xs[first[v] + 1], xs[first[v]]) if two[v] else xs[first[v]].copy()
              for v in range(1 << k)]
    return _halving_tree(dtype, op, leaves)


def rhd_reduce_value(dtype, op, xs, root):
    P = len(xs)
    k = P.bit_length() - 1
    pp = 1 << k
    r = P - pp
    odd = 1 if (root < 2 * r and root % 2) else 0
    leaves = []
    for v in range(pp):
        if v < r:
            keeper, partner = 2 * v + odd, 2 * v + 1 - odd
            leaves.append(combine(dtype, op, xs[partner], xs[keeper]))
        else:
            leaves.append(xs[v + r].copy())
    return _halving_tree(dtype, op, leaves)


def pipeline_allreduce(dtype, op, xs, S, M, loop_elems):
    P = S * M
    L = xs[0].size
    out = np.empty(L, STORAGE[dtype])
    for lb in range(0, L, loop_elems):
        n = min(loop_elems, L - lb)
        for s in range(S):
            for m in range(M):
                b, e = seg_bounds(n, P, s * M + m)
                b, e = b + lb, e + lb
                if b == e:
                    continue

                def intra(sigma):
                    acc = xs[sigma * M][b:e].copy()
                    for l in range(1, M):
                        acc = combine(dtype, op, acc, xs[sigma * M + l][b:e])
                    return acc

                acc = intra((s + 1) % S)
                for i in range(2, S + 1):
                    acc = combine(dtype, op, acc, intra((s + i) % S))
                out[b:e] = acc
    return out


def left_fold(dtype, op, xs):
    acc = xs[0].copy()
    for x in xs[1:]:
        acc = combine(dtype, op, acc, x)
    return acc


def tree_allreduce(dtype, op, xs, K):
    P = len(xs)

    def value(p):
        acc = xs[p].copy()
        for c in range(K * p + 1, min(K * p + K, P - 1) + 1):
            acc = combine(dtype, op, acc, value(c))
        return acc

    return value(0)


def hier_allreduce(dtype, op, xs, S, M):
    L = xs[0].size
    out = np.empty(L, STORAGE[dtype])
    for m in range(M):
        b0, e0 = seg_bounds(L, M, m)
        n = e0 - b0
        for c in range(S):
            b, e = seg_bounds(n, S, c)
            b, e = b + b0, e + b0
            if b == e:
                continue

            def intra(sigma):
                acc = xs[sigma * M][b:e].copy()
                for l in range(1, M):
                    acc = combine(dtype, op, acc, xs[sigma * M + l][b:e])
                return acc

            acc = intra((c + 1) % S)
            for i in range(2, S + 1):
                acc = combine(dtype, op, acc, intra((c + i) % S))
            out[b:e] = acc
    return out
