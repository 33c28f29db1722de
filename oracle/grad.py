"""Gradients of the STCA forward (eqs. (2)-(8)) in float64 numpy: the chain rule written out.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Given an upstream gradient dZ of the forward's output Z (targets x M x d), this returns the
gradients of L = sum(dZ * Z) with respect to the history X, the target embeddings x_t and every
weight of the forward (the training step the pages feed with the RLB loss of eq. (14),
"Make It Long, Keep It Fast", notes page, section 2.2; the loss itself needs RankMixer and
labels and is not part of this).  The forward follows ``oracle.stca`` exactly (same readings);
each backward step below names the forward equation it differentiates.

Weights: gradients are returned per weight slot.  The history FFN of layer i and the query
FFN of layer i are separate slots even when (by the default reading) they hold the same
arrays; a caller sharing them adds the two.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .stca import EPS, _f64


def _sig(g):
    return 1.0 / (1.0 + np.exp(-g))


# ---- eq. (1) and LayerNorm with saved intermediates ------------------------------------------
def _ffn_fwd(x, Wu, Wv, Wo):
    A, G = x @ Wu, x @ Wv
    H = A * G * _sig(G)
    return H @ Wo, (x, A, G, H)


def _ffn_bwd(dY, cache, Wu, Wv, Wo):
    """Backward of ((x W_u) * SiLU(x W_v)) W_o: (dx, dWu, dWv, dWo)."""
    x, A, G, H = cache
    dWo = H.T @ dY
    dH = dY @ Wo.T
    s = _sig(G)
    dA = dH * G * s
    dG = dH * A * s * (1.0 + G * (1.0 - s))      # d/dg [g sigma(g)] = sigma (1 + g (1 - sigma))
    return dA @ Wu.T + dG @ Wv.T, x.T @ dA, x.T @ dG, dWo


def _ln_fwd(y, gamma, beta, eps):
    mu = y.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(((y - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xh = (y - mu) * rstd
    return xh * gamma + beta, (xh, rstd)


def _ln_bwd(dout, cache, gamma):
    """Backward of (y - mean) / sqrt(var + eps) * gamma + beta: (dy, dgamma, dbeta)."""
    xh, rstd = cache
    dxh = dout * gamma
    dy = rstd * (dxh - dxh.mean(axis=-1, keepdims=True) - xh * (dxh * xh).mean(axis=-1, keepdims=True))
    return dy, (dout * xh).sum(0), dout.sum(0)


@dataclass
class Grads:
    """Gradients of one batch; list index = layer i (the pages' layer i+1)."""
    dX: np.ndarray = None
    dxt: np.ndarray = None
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
    WC: list = field(default_factory=list)   # WC[0] is None

    @staticmethod
    def zeros(W, M):
        g = Grads()
        for i in range(M):
            for name in ("Wu", "Wv", "Wo", "gamma", "beta", "qWu", "qWv", "qWo", "qgamma", "qbeta",
                         "WQ", "WK", "WV", "WO"):
                getattr(g, name).append(np.zeros_like(_f64(getattr(W, name)[i])))
            g.WC.append(None if i == 0 else np.zeros_like(_f64(W.WC[i])))
        return g


def backward_user(X, xt, W, h, dZ, M=None, query_ln=False, eps=EPS, grads=None):
    """Gradients for one user (X: L x d, xt: m x d, dZ: m x M x d).  Weight gradients are added
    into ``grads`` (created if None); returns (grads, dX, dxt)."""
    M = len(W.Wu) if M is None else M
    X, xt, dZ = _f64(X), _f64(xt), _f64(dZ)
    m, d = xt.shape[0], X.shape[1]
    dh = d // h
    sc = 1.0 / np.sqrt(dh)
    g = Grads.zeros(W, M) if grads is None else grads
    dX = np.zeros_like(X)
    dxt = np.zeros_like(xt)
    if m == 0:
        return g, dX, dxt
    w = lambda name, i: _f64(getattr(W, name)[i])  # noqa: E731

    # ---- forward with saved intermediates -----------------------------------------------------
    y, c_ffn = _ffn_fwd(xt, w("qWu", 0), w("qWv", 0), w("qWo", 0))             # eq. (3)
    q, c_ln = _ln_fwd(y, w("qgamma", 0), w("qbeta", 0), eps)
    qcache = [(c_ffn, c_ln, None)]
    qs, layers, outs = [q], [], []
    for i in range(M):
        Yi, ecache = _ffn_fwd(X, w("Wu", i), w("Wv", i), w("Wo", i))             # eq. (2)
        Xt, lcache = _ln_fwd(Yi, w("gamma", i), w("beta", i), eps)
        heads = np.empty((m, d))
        att = []
        for j in range(h):                                                          # eq. (13)
            cols = slice(j * dh, (j + 1) * dh)
            P = q @ w("WQ", i)[:, cols]
            u = P @ w("WK", i)[:, cols].T
            s = u @ Xt.T * sc
            a = np.exp(s - s.max(axis=1, keepdims=True))
            a /= a.sum(axis=1, keepdims=True)
            abar = a @ Xt
            heads[:, cols] = abar @ w("WV", i)[:, cols]
            att.append((P, u, a, abar))
        o = heads @ w("WO", i)                                                      # eq. (6)
        outs.append(o)
        layers.append((ecache, lcache, Xt, heads, att))
        if i + 1 < M:                                                               # eq. (7)
            cat = np.concatenate(outs + [xt], axis=1)
            c = cat @ w("WC", i + 1)
            y, c_ffn = _ffn_fwd(c, w("qWu", i + 1), w("qWv", i + 1), w("qWo", i + 1))
            c_ln = None
            if query_ln:
                y, c_ln = _ln_fwd(y, w("qgamma", i + 1), w("qbeta", i + 1), eps)
            q = y
            qs.append(q)
            qcache.append((c_ffn, c_ln, cat))

    # ---- backward, last layer first ------------------------------------------------------------
    do = [dZ[:, i, :].copy() for i in range(M)]                                     # eq. (8)
    dq = [np.zeros((m, d)) for _ in range(M)]
    for i in range(M - 1, -1, -1):
        if i + 1 < M:                                         # q^(i+2) = f(concat(o^(1..i+1), x_t) W_C)
            c_ffn, c_ln, cat = qcache[i + 1]
            dy = dq[i + 1]
            if query_ln:
                dy, dga, dbe = _ln_bwd(dy, c_ln, w("qgamma", i + 1))
                g.qgamma[i + 1] += dga
                g.qbeta[i + 1] += dbe
            dc, dWu, dWv, dWo = _ffn_bwd(dy, c_ffn, w("qWu", i + 1), w("qWv", i + 1), w("qWo", i + 1))
            g.qWu[i + 1] += dWu
            g.qWv[i + 1] += dWv
            g.qWo[i + 1] += dWo
            g.WC[i + 1] += cat.T @ dc
            dcat = dc @ w("WC", i + 1).T
            for k in range(i + 1):
                do[k] += dcat[:, k * d:(k + 1) * d]
            dxt += dcat[:, (i + 1) * d:]
        ecache, lcache, Xt, heads, att = layers[i]
        g.WO[i] += heads.T @ do[i]                                                  # eq. (6)
        dheads = do[i] @ w("WO", i).T
        dXt = np.zeros_like(Xt)
        for j in range(h):                                                          # eq. (13)
            cols = slice(j * dh, (j + 1) * dh)
            P, u, a, abar = att[j]
            g.WV[i][:, cols] += abar.T @ dheads[:, cols]
            dabar = dheads[:, cols] @ w("WV", i)[:, cols].T
            da = dabar @ Xt.T
            ds = a * (da - (a * da).sum(axis=1, keepdims=True))                     # softmax
            dXt += a.T @ dabar + (ds.T @ u) * sc
            du = (ds @ Xt) * sc
            dP = du @ w("WK", i)[:, cols]
            g.WK[i][:, cols] += du.T @ P
            g.WQ[i][:, cols] += qs[i].T @ dP
            dq[i] += dP @ w("WQ", i)[:, cols].T
        dY, dga, dbe = _ln_bwd(dXt, lcache, w("gamma", i))                        # eq. (2)
        g.gamma[i] += dga
        g.beta[i] += dbe
        dXi, dWu, dWv, dWo = _ffn_bwd(dY, ecache, w("Wu", i), w("Wv", i), w("Wo", i))
        g.Wu[i] += dWu
        g.Wv[i] += dWv
        g.Wo[i] += dWo
        dX += dXi
    c_ffn, c_ln, _ = qcache[0]                                                      # eq. (3)
    dy, dga, dbe = _ln_bwd(dq[0], c_ln, w("qgamma", 0))
    g.qgamma[0] += dga
    g.qbeta[0] += dbe
    dx0, dWu, dWv, dWo = _ffn_bwd(dy, c_ffn, w("qWu", 0), w("qWv", 0), w("qWo", 0))
    g.qWu[0] += dWu
    g.qWv[0] += dWv
    g.qWo[0] += dWo
    dxt += dx0
    return g, dX, dxt


def backward_batch(inp, W, dZ, query_ln=False, eps=EPS):
    """Gradients for a ragged batch (``stca_inputs.Inputs``): weight gradients summed over users,
    dX (total_L x d) and dxt (total_T x d) in batch order.  dZ: total_T x M x d."""
    cfg = inp.cfg
    g = Grads.zeros(W, cfg.M)
    dX = np.zeros((inp.total_L, cfg.d))
    dxt = np.zeros((inp.total_T, cfg.d))
    for k in range(inp.n_users):
        a, b = inp.tgt_off[k], inp.tgt_off[k + 1]
        _, dXk, dxtk = backward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, dZ[a:b], cfg.M, query_ln, eps, g)
        dX[inp.hist_off[k]:inp.hist_off[k + 1]] = dXk
        dxt[a:b] = dxtk
    g.dX, g.dxt = dX, dxt
    return g
