"""Pure-Python scalar loops for the STCA forward, tiny sizes only.

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.stca`` (no numpy,
no shared helpers) so that a dropped term, a wrong sign, a swapped index or a
transposed operand in either version shows up as a disagreement.  It follows
the standard attention form of eqs. (4)-(6) ([notes] "Make It Long, Keep It
Fast ...", section 2.1), not the reorder of eq. (13), so agreement also checks
the reorder.  Same readings as ``oracle.stca``.
"""
from __future__ import annotations

import math


def _mat(a):
    return [[float(v) for v in row] for row in a]


def _vec(a):
    return [float(v) for v in a]


def ffn_row(x, Wu, Wv, Wo):
    """One row of ((x W_u) * SiLU(x W_v)) W_o."""
    d = len(x)
    rd = len(Wu[0])
    hid = []
    for c in range(rd):
        a = 0.0
        g = 0.0
        for k in range(d):
            a += x[k] * Wu[k][c]
            g += x[k] * Wv[k][c]
        hid.append(a * (g / (1.0 + math.exp(-g))))
    out = []
    for c in range(len(Wo[0])):
        s = 0.0
        for k in range(rd):
            s += hid[k] * Wo[k][c]
        out.append(s)
    return out


def ln_row(y, gamma, beta, eps):
    n = len(y)
    mu = sum(y) / n
    var = sum((v - mu) * (v - mu) for v in y) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(y[k] - mu) * inv * gamma[k] + beta[k] for k in range(n)]


def attend_one(q, Xt, WQ, WK, WV, WO, h):
    """Eqs. (4)-(6) for one query vector q against the encoded history Xt (list of rows)."""
    d = len(q)
    dh = d // h
    L = len(Xt)
    concat = []
    for j in range(h):
        c0 = j * dh
        Qj = [sum(q[k] * WQ[k][c0 + c] for k in range(d)) for c in range(dh)]
        Kj = [[sum(Xt[p][k] * WK[k][c0 + c] for k in range(d)) for c in range(dh)] for p in range(L)]
        Vj = [[sum(Xt[p][k] * WV[k][c0 + c] for k in range(d)) for c in range(dh)] for p in range(L)]
        scores = [sum(Qj[c] * Kj[p][c] for c in range(dh)) / math.sqrt(dh) for p in range(L)]
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        tot = sum(w)
        alpha = [v / tot for v in w]
        for c in range(dh):
            concat.append(sum(alpha[p] * Vj[p][c] for p in range(L)))
    return [sum(concat[k] * WO[k][c] for k in range(d)) for c in range(d)]


def forward_user(X, xt, W, h, M=None, query_ln=False, eps=1e-5):
    """Z (m x M x d, nested lists) for one user; W is a ``stca_inputs.Weights``."""
    M = len(W.Wu) if M is None else M
    X = _mat(X)
    xts = _mat(xt)
    layers = []
    for i in range(M):
        layers.append(dict(
            Wu=_mat(W.Wu[i]), Wv=_mat(W.Wv[i]), Wo=_mat(W.Wo[i]), g=_vec(W.gamma[i]), b=_vec(W.beta[i]),
            qWu=_mat(W.qWu[i]), qWv=_mat(W.qWv[i]), qWo=_mat(W.qWo[i]),
            qg=_vec(W.qgamma[i]), qb=_vec(W.qbeta[i]),
            WQ=_mat(W.WQ[i]), WK=_mat(W.WK[i]), WV=_mat(W.WV[i]), WO=_mat(W.WO[i]),
            WC=_mat(W.WC[i]) if W.WC[i] is not None else None))
    encoded = []
    for i in range(M):
        P = layers[i]
        encoded.append([ln_row(ffn_row(x, P["Wu"], P["Wv"], P["Wo"]), P["g"], P["b"], eps) for x in X])
    Z = []
    for x_t in xts:
        P0 = layers[0]
        q = ln_row(ffn_row(x_t, P0["qWu"], P0["qWv"], P0["qWo"]), P0["qg"], P0["qb"], eps)
        outs = []
        for i in range(M):
            P = layers[i]
            o = attend_one(q, encoded[i], P["WQ"], P["WK"], P["WV"], P["WO"], h)
            outs.append(o)
            if i + 1 < M:
                Pn = layers[i + 1]
                cat = [v for oo in outs for v in oo] + list(x_t)
                d = len(x_t)
                c = [sum(cat[k] * Pn["WC"][k][col] for k in range(len(cat))) for col in range(d)]
                q = ffn_row(c, Pn["qWu"], Pn["qWv"], Pn["qWo"])
                if query_ln:
                    q = ln_row(q, Pn["qg"], Pn["qb"], eps)
        Z.append(outs)
    return Z


def prediction_token(Z, xt, WZ, Wu, Wv, Wo):
    """Eq. (9) per target: z = SwiGLUFFN([o^(1) || ... || o^(M) || x_t] W_Z), nested lists.

    ``Z`` is m x M x d (nested lists or an array), ``xt`` m x d, ``WZ`` (M+1)d x d."""
    WZ, Wu, Wv, Wo = _mat(WZ), _mat(Wu), _mat(Wv), _mat(Wo)
    out = []
    for t, x_t in enumerate(_mat(xt)):
        cat = [float(v) for o in Z[t] for v in o] + x_t
        d = len(x_t)
        c = [sum(cat[k] * WZ[k][col] for k in range(len(cat))) for col in range(d)]
        out.append(ffn_row(c, Wu, Wv, Wo))
    return out
