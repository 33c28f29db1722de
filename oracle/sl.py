"""Stochastic-length (SL) training batches for STCA, in plain Python / numpy integers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [notes] "Make It Long, Keep It Fast: End-to-End 10k-Sequence Modeling at Billion Scale
on Douyin", the length-extrapolation part: stochastic length sampling (eqs. (15)-(17)), the
element selection strategy, and the two-step batch-level load balancing; the same steps are
discussed in the STCA review page, section 2.6.

Steps, in the pages' order:

1. Draw a normalised length s ~ Beta(alpha, beta) per sequence, with beta fixed by the mean
   constraint (eq. (17)) so that E[L_train] = L_avg; map it to L_raw = L_min + s (L_max - L_min)
   (eq. (16)) and align it to a multiple of 8.  Sequence sparsity SS = L_avg / L_max (eq. (15)).
2. Element selection: keep the most recent L_train interactions of the user's history (the
   temporal suffix), the history itself being truncated to L_infer first.
3. Load balancing, step 1 (global length allocation): randomly truncate sequences so that the
   batch holds exactly B * L_avg tokens.
4. Load balancing, step 2 (sequence compression): lay the selected sequences end to end and
   view them as B rows of L_avg tokens; a long sequence's surplus tokens continue in the next
   row, filling the space short sequences leave, so there is no padding; an index tensor of
   segment boundaries says which tokens belong to which sequence.

Readings where the pages are silent (shared with the HIP path by definition):

* R1. Alignment to 8 rounds L_raw to the nearest multiple of 8 (halves up), then clamps it to
  [8 ceil(L_min / 8), 8 floor(L_max / 8)].
* R2. A user whose (L_infer-truncated) history is shorter than its sampled length keeps all of
  it: L = min(L_train, available).
* R3. The random draws (s per sequence; the order in which sequences are truncated) are inputs.
* R4. Global allocation only truncates: when the sampled total exceeds the budget B * L_avg,
  sequences are visited in the given random order and each is shortened by as much of the
  remaining excess as it can give without going below 8 ceil(L_min / 8), so the total equals
  the budget exactly (the pages ask for exactly B * L_avg tokens; a cut need not be a multiple of
  8, since lengths capped by a short history are not).  A total at or under the budget is left
  as is.
* R5. Compression concatenates sequences in user order; the boundary index is the prefix sum of
  lengths (hist_off), and row r of the compressed view covers tokens [r L_avg, (r+1) L_avg).
"""
from __future__ import annotations

import numpy as np


def beta_param(alpha: float, L_min: float, L_max: float, L_avg: float) -> float:
    """eq. (17): the Beta shape beta that puts the mean of L_min + s (L_max - L_min) at L_avg."""
    if not L_min < L_avg < L_max:
        raise ValueError("need L_min < L_avg < L_max")
    return alpha * (L_max - L_avg) / (L_avg - L_min)


def sequence_sparsity(L_avg: float, L_max: float) -> float:
    """eq. (15): SS = E[L_train] / L_max = L_avg / L_max."""
    return L_avg / L_max


def align8(L_raw, L_min: int, L_max: int):
    """R1: nearest multiple of 8 (halves up), clamped into the aligned [L_min, L_max]."""
    lo, hi = 8 * -(-L_min // 8), 8 * (L_max // 8)
    L = 8 * np.floor(np.asarray(L_raw, np.float64) / 8.0 + 0.5).astype(np.int64)
    return np.clip(L, lo, hi)


def train_lengths(s, L_min: int, L_max: int):
    """eq. (16) then R1: per-sequence training lengths from the normalised draws s."""
    s = np.asarray(s, np.float64)
    return align8(L_min + s * (L_max - L_min), L_min, L_max)


def available(full_len, L_infer: int):
    """History rows a user can offer: its full history truncated to the most recent L_infer."""
    return np.minimum(np.asarray(full_len, np.int64), L_infer)


def allocate(L, budget: int, order, L_min: int):
    """Load balancing step 1 (R4): truncate sequences, in the given order, until sum == budget."""
    L = np.array(L, np.int64)
    floor = 8 * -(-L_min // 8)
    excess = int(L.sum()) - int(budget)
    for u in order:
        if excess <= 0:
            break
        cut = min(excess, max(int(L[u]) - floor, 0))
        L[u] -= cut
        excess -= cut
    return L


def suffix_rows(full_off, L):
    """Element selection: for each user the source rows of its last L[u] history rows (R2 has
    already capped L[u] at what the user has).  Returns the gather index, in user order."""
    full_off = np.asarray(full_off, np.int64)
    idx = [np.arange(full_off[u + 1] - L[u], full_off[u + 1], dtype=np.int64) for u in range(len(L))]
    return np.concatenate(idx) if idx else np.zeros(0, np.int64)


def plan(full_len, s, order, L_min: int, L_max: int, L_avg: int, L_infer: int):
    """Steps 1-3: lengths (eq. (16), R1, R2), then the global budget (R4).  Returns
    (lengths, hist_off) of the compressed batch."""
    B = len(full_len)
    L = np.minimum(train_lengths(s, L_min, L_max), available(full_len, L_infer))
    L = allocate(L, B * L_avg, order, L_min)
    off = np.zeros(B + 1, np.int64)
    np.cumsum(L, out=off[1:])
    return L, off


def pack(X_full, full_off, L):
    """Step 4: the selected suffix rows end to end (no padding) and the gather index."""
    idx = suffix_rows(full_off, L)
    return np.asarray(X_full)[idx], idx


def rows_view(hist_off, L_avg: int):
    """R5: for each row r of the compressed B x L_avg view, the users whose segments intersect
    it, as (first user, last user) inclusive."""
    hist_off = np.asarray(hist_off, np.int64)
    total = int(hist_off[-1])
    n_rows = -(-total // L_avg)
    out = []
    for r in range(n_rows):
        a, b = r * L_avg, min((r + 1) * L_avg, total)
        first = int(np.searchsorted(hist_off, a, side="right")) - 1
        last = int(np.searchsorted(hist_off, b, side="left")) - 1
        out.append((first, last))
    return out
