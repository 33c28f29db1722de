"""Local same-ID token merging (LITM) of a history, in plain Python / numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "TM20K：老师读全文，学生读缩写" (notes page on TM20K), section 4.2.1 (LITM: tokens that carry
the same key ID, the product ID, are summed into one token, but only when their positions are at
most a threshold T apart: a local merge, not a deduplication of the whole sequence), section 4.1
(the merge is rule-based preprocessing done before the embedding sum pooling, and it moves only
IDs and grouping metadata), section 3.2 (observation one: same-ID tokens close in position get
nearly equal attention) and section 5.4 (T = 3 is the knee of the threshold ablation).

Readings where the page is silent (shared with the HIP path by definition):

* R1 (chaining).  Positions are scanned in order.  Token p joins the group of the nearest earlier
  token q of the same user with the same ID if p - q <= T; otherwise it starts a group of its own.
  So a group is a maximal run of same-ID occurrences whose consecutive gaps are all <= T.
* R2 (merged token).  The merged token is the sum of its members' embedding rows (the page's sum
  pooling applied to the member tokens); it sits at the position of the group's first member, so
  the merged history keeps the order of first occurrences.
* R3 (scope).  Only tokens of the same user merge.  T = 0 merges nothing.
* R4 (precision).  The oracle sums in float64; the device path sums bf16 rows in fp32 in member
  order and rounds once (RNE) to the storage type.
"""
from __future__ import annotations

import numpy as np


def group_roots(item_id, hist_off, T: int):
    """R1: root[p] = first position of the group token p belongs to (global row index)."""
    item_id = np.asarray(item_id, np.int64)
    hist_off = np.asarray(hist_off, np.int64)
    root = np.arange(len(item_id), dtype=np.int64)
    for u in range(len(hist_off) - 1):
        a, b = int(hist_off[u]), int(hist_off[u + 1])
        for p in range(a, b):
            for q in range(p - 1, max(a, p - T) - 1, -1):   # nearest earlier first
                if item_id[q] == item_id[p]:
                    root[p] = root[q]
                    break
    return root


def plan(item_id, hist_off, T: int):
    """Groups of every user, in order of first occurrence.

    Returns (merged_off, group_off, members): the merged history of user u is groups
    merged_off[u] .. merged_off[u+1]-1; group g has source rows members[group_off[g]:group_off[g+1]]
    in position order."""
    hist_off = np.asarray(hist_off, np.int64)
    root = group_roots(item_id, hist_off, T)
    merged_off = np.zeros(len(hist_off), np.int64)
    group_off = [0]
    members = []
    for u in range(len(hist_off) - 1):
        a, b = int(hist_off[u]), int(hist_off[u + 1])
        groups = {}
        for p in range(a, b):
            groups.setdefault(int(root[p]), []).append(p)
        for r in sorted(groups):
            members.extend(groups[r])
            group_off.append(len(members))
        merged_off[u + 1] = merged_off[u] + len(groups)
    return merged_off, np.asarray(group_off, np.int64), np.asarray(members, np.int64)


def merge(X, group_off, members):
    """R2: merged rows, each the float64 sum of its members' rows."""
    X = np.asarray(X, np.float64)
    group_off = np.asarray(group_off, np.int64)
    out = np.zeros((len(group_off) - 1, X.shape[1]), np.float64)
    for g in range(len(group_off) - 1):
        for m in members[group_off[g]:group_off[g + 1]]:
            out[g] += X[m]
    return out
