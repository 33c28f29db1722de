"""STCA forward in float64 numpy: a plain transcription of the method.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (web pages on the STCA paper, WWW'26, arXiv 2511.06077):

* [notes]  "Make It Long, Keep It Fast: End-to-End 10k-Sequence Modeling at
  Billion Scale on Douyin" -- reading notes, section 2.1 (eqs. (1)-(9)) and
  "computational optimisation: reordered matmul" (eqs. (12)-(13)), section 2.2
  (request level batching, eq. (14)).
* [review] "字节跳动-STCA：抖音 10k 长序列端到端建模的架构、系统与外推三件套" --
  review, sections 2.2-2.4 (matrix shapes of the SwiGLU FFN and of the
  attention projections, the identity shortcut of x_t, the associativity
  argument behind the reorder).

Readings taken where the pages are garbled, ambiguous or silent:

* SwiGLU FFN: [notes] eq. (1) prints W_o both as the gate and as the output
  matrix with shape d x rd, which cannot type-check.  [review] section 2.2
  gives three matrices, W_u, W_v (d x rd) and W_o (rd x d), with the SiLU gate
  on the x W_v branch.  We follow [review].  No biases ([review] 2.2 says they
  are omitted).
* LayerNorm: affine (gamma, beta), biased variance, eps = 1e-5.
* Eq. (2) encodes the raw history X for every layer i (no chaining, no
  residual).  Eqs. (3) and (7) reuse the symbol SwiGLUFFN^(i), read as the
  same weights as the history FFN of layer i (callers may pass others).
* Eq. (7) applies no LayerNorm (``query_ln=False``); ``query_ln=True`` gives the
  reading in which the fusion block ends with a LayerNorm.
* Eq. (7) concatenates the raw target embedding x_t (an identity shortcut).
* Eq. (13) writes X; eqs. (4)/(12) make clear the encoded history X~^(i) is
  meant.  The score scale is 1/sqrt(d_h) in both forms.
* Heads: head j uses columns j*d_h .. (j+1)*d_h-1 of W_Q, W_K, W_V (d x d);
  eq. (6) concatenates heads in order.
* A user must have L_u >= 1 (softmax over no tokens is undefined); a user
  with no targets contributes no output rows.
* Eq. (9) (prediction token): the SwiGLUFFN there carries no layer index; it is
  read as an FFN instance of its own, applied without a LayerNorm (none is
  printed), after the projection by W_Z ((M+1)d x d, row blocks in the order of
  the concatenation [o^(1) || ... || o^(M) || x_t]).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# eq. (1): SwiGLU FFN      [notes] 2.1 eq. (1), shapes from [review] 2.2
# ----------------------------------------------------------------------------
def silu(g):
    """SiLU / Swish gate g * sigmoid(g) = g / (1 + e^-g)."""
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(x, Wu, Wv, Wo):
    """SwiGLUFFN(x) = ((x W_u) * SiLU(x W_v)) W_o, applied row-wise, no biases."""
    x = _f64(x)
    return ((x @ _f64(Wu)) * silu(x @ _f64(Wv))) @ _f64(Wo)


def layer_norm(y, gamma, beta, eps=EPS):
    """Row-wise LayerNorm with biased variance: (y - mean) / sqrt(var + eps) * gamma + beta."""
    y = _f64(y)
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    return (y - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


# ----------------------------------------------------------------------------
# eqs. (2), (3): per-layer history encoding and query initialisation
# ----------------------------------------------------------------------------
def encode(X, Wu, Wv, Wo, gamma, beta, eps=EPS):
    """X~^(i) = LN(SwiGLUFFN^(i)(X)), one row per history token ([notes] eq. (2))."""
    return layer_norm(swiglu_ffn(X, Wu, Wv, Wo), gamma, beta, eps)


def init_query(xt, Wu, Wv, Wo, gamma, beta, eps=EPS):
    """q^(1) = LN(SwiGLUFFN^(1)(x_t)), one row per target ([notes] eq. (3))."""
    return encode(xt, Wu, Wv, Wo, gamma, beta, eps)


# ----------------------------------------------------------------------------
# eqs. (4)-(6): multi-head single-query cross attention, standard form (12)
# ----------------------------------------------------------------------------
def _softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attend_standard(q, Xt, WQ, WK, WV, WO, h):
    """Eqs. (4)-(6) as printed: per head j, alpha = softmax((q W_Q,j)(X~ W_K,j)^T / sqrt(d_h)),
    o_j = alpha (X~ W_V,j); o = [o_1 || ... || o_h] W_O.

    ``q`` is m x d (one query per target, all sharing the history ``Xt``, L x d).
    Returns (o: m x d, alpha: m x h x L).
    """
    q, Xt = _f64(q), _f64(Xt)
    WQ, WK, WV, WO = map(_f64, (WQ, WK, WV, WO))
    d = Xt.shape[1]
    dh = d // h
    m, L = q.shape[0], Xt.shape[0]
    heads = np.empty((m, d))
    alpha = np.empty((m, h, L))
    for j in range(h):
        cols = slice(j * dh, (j + 1) * dh)
        Q = q @ WQ[:, cols]                 # m x d_h
        K = Xt @ WK[:, cols]                # L x d_h
        V = Xt @ WV[:, cols]                # L x d_h
        a = _softmax_rows(Q @ K.T / np.sqrt(dh))
        alpha[:, j, :] = a
        heads[:, cols] = a @ V
    return heads @ WO, alpha


# ----------------------------------------------------------------------------
# eq. (13): the reordered single-query form used by the hot path
# ----------------------------------------------------------------------------
def attend_reordered(q, Xt, WQ, WK, WV, WO, h):
    """Eq. (13) per head j: u_j = (q W_Q,j) W_K,j^T (1 x d), alpha_j = softmax(u_j X~^T / sqrt(d_h)),
    o_j = (alpha_j X~) W_V,j; then eq. (6) o = [o_1 || ... || o_h] W_O.

    Returns (o: m x d, alpha: m x h x L, abar: m x h x d) where abar_j = alpha_j X~
    is the attention-weighted history the reorder forms before projecting.
    """
    q, Xt = _f64(q), _f64(Xt)
    WQ, WK, WV, WO = map(_f64, (WQ, WK, WV, WO))
    d = Xt.shape[1]
    dh = d // h
    m, L = q.shape[0], Xt.shape[0]
    heads = np.empty((m, d))
    alpha = np.empty((m, h, L))
    abar = np.empty((m, h, d))
    for j in range(h):
        cols = slice(j * dh, (j + 1) * dh)
        u = (q @ WQ[:, cols]) @ WK[:, cols].T          # m x d
        a = _softmax_rows(u @ Xt.T / np.sqrt(dh))       # m x L
        alpha[:, j, :] = a
        abar[:, j, :] = a @ Xt                          # m x d
        heads[:, cols] = abar[:, j, :] @ WV[:, cols]    # m x d_h
    return heads @ WO, alpha, abar


# ----------------------------------------------------------------------------
# eq. (7): target-conditioned query fusion
# ----------------------------------------------------------------------------
def update_query(o_prev, xt, WC, Wu, Wv, Wo, gamma=None, beta=None, query_ln=False, eps=EPS):
    """q^(i+1) = SwiGLUFFN^(i+1)([o^(1) || ... || o^(i) || x_t] W_C^(i+1))  ([notes] eq. (7)).

    ``o_prev`` is the list [o^(1), ..., o^(i)] of m x d arrays; ``WC`` is (i+1)d x d with
    row blocks in the same order as the concatenation.  With ``query_ln`` a LayerNorm
    follows the FFN.
    """
    c = np.concatenate([_f64(o) for o in o_prev] + [_f64(xt)], axis=1) @ _f64(WC)
    y = swiglu_ffn(c, Wu, Wv, Wo)
    return layer_norm(y, gamma, beta, eps) if query_ln else y


def prediction_token(Z, xt, WZ, Wu, Wv, Wo):
    """z = SwiGLUFFN([o^(1) || ... || o^(M) || x_t] W_Z)  ([notes] eq. (9)).

    ``Z`` is m x M x d (eq. (8) per target: the rows o^(1..M)); ``xt`` is m x d;
    ``WZ`` is (M+1)d x d.  Returns m x d.
    """
    Z, xt = _f64(Z), _f64(xt)
    m, M, d = Z.shape
    blocks = [Z[:, i, :] for i in range(M)] + [xt]
    return swiglu_ffn(np.concatenate(blocks, axis=1) @ _f64(WZ), Wu, Wv, Wo)


# ----------------------------------------------------------------------------
# eqs. (2)-(8) for one user micro-batch, and for a ragged batch of users
# ----------------------------------------------------------------------------
def forward_user(X, xt, W, h, M=None, query_ln=False, eps=EPS, trace=None):
    """Z_H for every target of one user: an m x M x d array (eq. (8) stacks o^(1..M)).

    One encoded history per layer serves all m targets of the user (request level
    batching, [notes] 2.2).  ``W`` is a ``stca_inputs.Weights``.  If ``trace`` is a
    dict, per-layer intermediates (Xt, q, o, alpha, abar) are stored in it.
    """
    M = len(W.Wu) if M is None else M
    X, xt = _f64(X), _f64(xt)
    if X.shape[0] < 1:
        raise ValueError("a user needs at least one history token")
    m, d = xt.shape[0], X.shape[1]
    Z = np.zeros((m, M, d))
    if m == 0:
        return Z
    q = init_query(xt, W.qWu[0], W.qWv[0], W.qWo[0], W.qgamma[0], W.qbeta[0], eps)
    outs = []
    for i in range(M):
        Xt = encode(X, W.Wu[i], W.Wv[i], W.Wo[i], W.gamma[i], W.beta[i], eps)
        o, alpha, abar = attend_reordered(q, Xt, W.WQ[i], W.WK[i], W.WV[i], W.WO[i], h)
        if trace is not None:
            trace.setdefault("Xt", []).append(Xt)
            trace.setdefault("q", []).append(q)
            trace.setdefault("o", []).append(o)
            trace.setdefault("alpha", []).append(alpha)
            trace.setdefault("abar", []).append(abar)
        outs.append(o)
        Z[:, i, :] = o
        if i + 1 < M:
            q = update_query(outs, xt, W.WC[i + 1], W.qWu[i + 1], W.qWv[i + 1], W.qWo[i + 1],
                             W.qgamma[i + 1], W.qbeta[i + 1], query_ln, eps)
    return Z


def forward_batch(inp, W, query_ln=False, eps=EPS, users=None):
    """Z for a ragged batch (``stca_inputs.Inputs``): total_T x M x d, targets in batch order.

    Users are independent (each query attends only to its own user's segment), so the
    batch result is the per-user results stacked.  ``users`` limits the work to some
    held users (indices into the batch); their rows are returned stacked in that order.
    """
    cfg = inp.cfg
    ks = range(inp.n_users) if users is None else users
    parts = [forward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, cfg.M, query_ln, eps) for k in ks]
    if not parts:
        return np.zeros((0, cfg.M, cfg.d))
    return np.concatenate(parts, axis=0)
