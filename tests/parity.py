"""Helpers for comparing the HIP path with the oracle (test-only).

Acceptance rule for sampled ids: an id must match exactly where the decision
is clear -- for greedy, the oracle's top-1 margin over the (masked, fp32)
logits exceeds 1e-2; for top-p, the uniform is more than 1e-4 from every
kept-CDF boundary and the nucleus edge is more than 1e-4 from top_p.  Where
it is not clear either id is accepted, and that sequence is not compared
further (its later frames follow different histories).
"""
from __future__ import annotations

import sys

import numpy as np

GREEDY_MARGIN = 1e-2
TOPP_MARGIN = 1e-4
REL_L2 = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def decision_margin(z, greedy, temperature=1.0, top_p=1.0, u=None):
    """How far the oracle's sampling decision on logits z (-inf = masked) is
    from flipping.  Greedy: the top-1 logit gap.  Top-p: the smallest of the
    distance from u (and from top_p) to the cumulative boundaries around it,
    and the scaled-logit gap between the chosen token and its neighbours in
    the sort order.  A logit perturbation of at most dz moves each of these
    by about 2 dz / T."""
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    if greedy or u is None:
        s = np.sort(z[np.isfinite(z)])[::-1]
        return float(s[0] - s[1]) if len(s) > 1 else np.inf
    ok = np.isfinite(z)
    zz = np.where(ok, z / temperature, -np.inf)
    p = np.exp(zz - zz[ok].max())
    p /= p.sum()
    ids = np.nonzero(p > 0)[0]
    order = ids[np.lexsort((ids, -p[ids]))]
    cum = np.cumsum(p[order])
    hit = np.nonzero(cum >= top_p)[0]
    n_keep = int(hit[0]) + 1 if len(hit) else len(order)
    edge = [abs(cum[n_keep - 1] - top_p)]
    if n_keep > 1:
        edge.append(abs(cum[n_keep - 2] - top_p))
    ck = np.cumsum(p[order[:n_keep]]) / cum[n_keep - 1]
    # the draw also flips when the chosen token trades places with a
    # neighbour in the (p desc, id asc) order, i.e. when their scaled logits
    # are within the perturbation of each other, wherever u sits
    j = min(int(np.searchsorted(ck, float(u), side="right")), n_keep - 1)
    gaps = []
    if j + 1 < len(order):
        gaps.append(zz[order[j]] - zz[order[j + 1]])
    if j > 0:
        gaps.append(zz[order[j - 1]] - zz[order[j]])
    return float(min(min(edge), np.min(np.abs(ck - float(u))), *gaps))


def margin_ok(margin, greedy):
    return margin > (GREEDY_MARGIN if greedy else TOPP_MARGIN)
