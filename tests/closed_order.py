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
