"""Seeded draws for histories, targets and weights (no STCA arithmetic here)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import Config

# Stream identifiers inside the per-workload SeedSequence.
_LAYOUT, _HISTORY, _TARGETS, _WEIGHTS, _PREDICT, _SL = 0, 1, 2, 3, 4, 5


def _rng(cfg: Config, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=tuple(key)))


# ----------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even from float32)
# ----------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 bit pattern (ties to even), as uint16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value."""
    return bits_to_f32(bf16_bits(a))


def _store(cfg: Config, a: np.ndarray) -> np.ndarray:
    """Values as the workload stores them: float32, rounded to bf16 for bf16 workloads."""
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if cfg.dtype == "bf16" else a


# ----------------------------------------------------------------------------
# batch layout
# ----------------------------------------------------------------------------
def batch_layout(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Per-user history lengths L_u and target counts m_u (int64 arrays)."""
    rng = _rng(cfg, _LAYOUT)
    n = cfg.n_users
    kind = cfg.length[0]
    if kind == "fixed":
        L = np.full(n, int(cfg.length[1]), dtype=np.int64)
    elif kind == "lognormal":
        _, median, mean, lo, hi = cfg.length
        sigma = np.sqrt(2.0 * np.log(mean / median))   # unclipped mean = median * exp(sigma^2/2)
        L = np.exp(rng.normal(np.log(median), sigma, size=n))
        L = np.clip(np.rint(L), lo, hi).astype(np.int64)
    else:
        raise ValueError(f"unknown length law {kind!r}")
    tkind = cfg.targets[0]
    if tkind == "fixed":
        m = np.full(n, int(cfg.targets[1]), dtype=np.int64)
    elif tkind == "1+poisson":
        m = 1 + rng.poisson(cfg.targets[1], size=n).astype(np.int64)
    else:
        raise ValueError(f"unknown target law {tkind!r}")
    return L, m


def offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum with a leading 0: the ragged-segment index tensor."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    np.cumsum(np.asarray(counts, dtype=np.int64), out=off[1:])
    return off


# ----------------------------------------------------------------------------
# histories and targets
# ----------------------------------------------------------------------------
def _duplicate_sources(rng: np.random.Generator, L: int, p: float, window: int) -> np.ndarray:
    """Index map for same-ID repeats.

    Walking p = 1 .. L-1 in order, token p becomes (with probability ``p``) a
    bitwise copy of the token k positions earlier, k ~ U{1..window} clipped so
    the source index stays >= 0.  Because a copy may itself be a copy, the map
    is resolved to the original source of every position.
    """
    dup = rng.random(L) < p
    k = rng.integers(1, window + 1, size=L)
    pos = np.arange(L, dtype=np.int64)
    src = np.where(dup, np.maximum(pos - k, 0), pos)
    src[0] = 0
    while True:
        nxt = src[src]
        if np.array_equal(nxt, src):
            return src
        src = nxt


def user_history_ids(cfg: Config, u: int, L_u: int) -> tuple[np.ndarray, np.ndarray]:
    """History embeddings X of user ``u`` (L_u x d, float32, bf16-valued if bf16) and the item
    ID of every position: a repeat carries the ID of the token it copies (its resolved source
    position), any other token a fresh one (its own position).  IDs are user-local."""
    rng = _rng(cfg, _HISTORY, int(u))
    X = rng.standard_normal((int(L_u), cfg.d), dtype=np.float32)
    src = np.arange(int(L_u), dtype=np.int64)
    if cfg.dup_prob > 0.0:
        src = _duplicate_sources(rng, int(L_u), cfg.dup_prob, cfg.dup_window)
        X = X[src]
    return _store(cfg, X), src


def user_history(cfg: Config, u: int, L_u: int) -> np.ndarray:
    """History embeddings X of user ``u`` (L_u x d, float32, bf16-valued if bf16)."""
    return user_history_ids(cfg, u, L_u)[0]


def targets(cfg: Config, T: int) -> np.ndarray:
    """Target embeddings x_t for all T targets of the batch, in user order."""
    rng = _rng(cfg, _TARGETS)
    return _store(cfg, rng.standard_normal((int(T), cfg.d), dtype=np.float32))


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
@dataclass
class Weights:
    """Per-layer parameters, layer index i = 0 .. M-1 (the pages' layer i+1).

    Matrices are row-major float32 (bf16-valued for bf16 workloads) with the
    shapes the STCA pages give: ``Wu, Wv`` d x rd, ``Wo`` rd x d, ``WQ, WK,
    WV, WO`` d x d (head j = columns j*d_h .. (j+1)*d_h), ``WC[i]`` (i+1)d x d
    for i >= 1 (``WC[0]`` is None), LayerNorm ``gamma, beta`` of length d.
    ``qWu/qWv/qWo`` are the query-side SwiGLU FFN weights; by default they are
    the same arrays as the history-side ones of the same layer.
    """
    Wu: list = field(default_factory=list)
    Wv: list = field(default_factory=list)
    Wo: list = field(default_factory=list)
    gamma: list = field(default_factory=list)
    beta: list = field(default_factory=list)
    qWu: list = field(default_factory=list)
    qWv: list = field(default_factory=list)
    qWo: list = field(default_factory=list)
    qgamma: list = field(default_factory=list)
    qbeta: list = field(default_factory=list)
    WQ: list = field(default_factory=list)
    WK: list = field(default_factory=list)
    WV: list = field(default_factory=list)
    WO: list = field(default_factory=list)
    WC: list = field(default_factory=list)


def make_weights(cfg: Config, random_ln: bool = False, separate_query_ffn: bool = False) -> Weights:
    """Draw all weights, layer-major, in the order Wu, Wv, Wo, [gamma, beta],
    [query Wu, Wv, Wo, gamma, beta], WQ, WK, WV, WO, WC (layers >= 1)."""
    rng = _rng(cfg, _WEIGHTS)
    d, rd = cfg.d, cfg.r * cfg.d

    def mat(rows, cols):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(1.0 / np.sqrt(rows))
        return _store(cfg, w)

    def ln_params():
        if random_ln:
            g = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
            b = (0.5 * rng.standard_normal(d)).astype(np.float32)
            return g, b
        return np.ones(d, np.float32), np.zeros(d, np.float32)

    W = Weights()
    for i in range(cfg.M):
        W.Wu.append(mat(d, rd))
        W.Wv.append(mat(d, rd))
        W.Wo.append(mat(rd, d))
        g, b = ln_params()
        W.gamma.append(g)
        W.beta.append(b)
        if separate_query_ffn:
            W.qWu.append(mat(d, rd))
            W.qWv.append(mat(d, rd))
            W.qWo.append(mat(rd, d))
            g, b = ln_params()
            W.qgamma.append(g)
            W.qbeta.append(b)
        else:
            W.qWu.append(W.Wu[i])
            W.qWv.append(W.Wv[i])
            W.qWo.append(W.Wo[i])
            W.qgamma.append(W.gamma[i])
            W.qbeta.append(W.beta[i])
        W.WQ.append(mat(d, d))
        W.WK.append(mat(d, d))
        W.WV.append(mat(d, d))
        W.WO.append(mat(d, d))
        W.WC.append(mat((i + 1) * d, d) if i >= 1 else None)
    return W


@dataclass
class PredictWeights:
    """Parameters of the prediction token (eq. (9) of the STCA notes page): ``WZ``
    (M+1)d x d, row blocks in the order [o^(1); ...; o^(M); x_t], and the SwiGLU FFN
    ``Wu, Wv`` d x rd, ``Wo`` rd x d.  Same storage conventions as ``Weights``."""
    WZ: np.ndarray
    Wu: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray


def make_predict_weights(cfg: Config) -> PredictWeights:
    """Draw the prediction-token weights from a stream of their own (the other draws are
    unchanged), in the order WZ, Wu, Wv, Wo, each N(0, 1/fan_in)."""
    rng = _rng(cfg, _PREDICT)
    d, rd = cfg.d, cfg.r * cfg.d

    def mat(rows, cols):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(1.0 / np.sqrt(rows))
        return _store(cfg, w)

    WZ = mat((cfg.M + 1) * d, d)
    return PredictWeights(WZ, mat(d, rd), mat(d, rd), mat(rd, d))


def make_sl_draws(cfg: Config, n: int, alpha: float, beta: float):
    """The random draws of stochastic-length batching for n sequences, from a stream of their
    own: s ~ Beta(alpha, beta) per sequence (float64), then a random order of the sequences
    (int32) for the truncation pass.  The shape parameters are the caller's."""
    rng = _rng(cfg, _SL)
    s = rng.beta(alpha, beta, size=n)
    order = rng.permutation(n).astype(np.int32)
    return s, order


# ----------------------------------------------------------------------------
# whole batches
# ----------------------------------------------------------------------------
@dataclass
class Inputs:
    """A ragged request-level batch.

    ``users`` are the workload's user indices held here (all of them, or a
    sample).  ``X`` stacks their histories (sum L_u x d) and ``xt`` their
    targets (sum m_u x d).  For bf16 workloads ``X``/``xt`` are uint16 bit
    patterns (``as_f32`` converts); for fp32 workloads they are float32.
    """
    cfg: Config
    users: np.ndarray
    L: np.ndarray
    m: np.ndarray
    hist_off: np.ndarray
    tgt_off: np.ndarray
    X: np.ndarray
    xt: np.ndarray
    item_id: np.ndarray | None = None   # int64 per history row (make_inputs(with_ids=True))

    @property
    def n_users(self) -> int:
        return len(self.users)

    @property
    def total_L(self) -> int:
        return int(self.hist_off[-1])

    @property
    def total_T(self) -> int:
        return int(self.tgt_off[-1])

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        return bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)

    def user_X(self, k: int) -> np.ndarray:
        """History of the k-th held user as float32."""
        return self.as_f32(self.X[self.hist_off[k]:self.hist_off[k + 1]])

    def user_xt(self, k: int) -> np.ndarray:
        return self.as_f32(self.xt[self.tgt_off[k]:self.tgt_off[k + 1]])


def make_inputs(cfg: Config, users=None, threads: int | None = None, with_ids: bool = False) -> Inputs:
    """Histories and targets for ``users`` (default: every user of the workload).

    A user's draws do not depend on which other users are generated, so a
    sample of users reproduces exactly the rows of the full batch.  With ``with_ids`` the
    result also carries ``item_id`` (int64 per history row, globally unique per source token:
    hist_off[k] + the user-local ID of ``user_history_ids``).
    """
    L_all, m_all = batch_layout(cfg)
    users = np.arange(cfg.n_users) if users is None else np.asarray(sorted(set(int(u) for u in users)))
    L = L_all[users]
    m = m_all[users]
    hoff = offsets(L)
    toff = offsets(m)

    bf16 = cfg.dtype == "bf16"
    X = np.empty((int(hoff[-1]), cfg.d), dtype=np.uint16 if bf16 else np.float32)
    ids = np.empty(int(hoff[-1]), dtype=np.int64) if with_ids else None

    def fill(k):
        Xu, src = user_history_ids(cfg, int(users[k]), int(L[k]))
        X[hoff[k]:hoff[k + 1]] = bf16_bits(Xu) if bf16 else Xu
        if ids is not None:
            ids[hoff[k]:hoff[k + 1]] = hoff[k] + src

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if len(users) > 1 and threads > 1 and X.nbytes > (64 << 20):
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(len(users))))
    else:
        for k in range(len(users)):
            fill(k)

    all_xt = targets(cfg, int(m_all.sum()))
    all_toff = offsets(m_all)
    rows = np.concatenate([np.arange(all_toff[u], all_toff[u + 1]) for u in users]) if len(users) else \
        np.zeros(0, np.int64)
    xt = all_xt[rows.astype(np.int64)]
    xt = bf16_bits(xt) if bf16 else xt
    return Inputs(cfg, users, L, m, hoff, toff, X, xt, ids)
