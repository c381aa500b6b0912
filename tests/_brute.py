"""Brute-force evaluation of the MoE layer on tiny inputs (test helper).

Independent of oracle/: it evaluates EVERY expert on EVERY token with dense
matrix products, finds each token's selection by exhaustive search over all
k-subsets of experts, applies capacity from per-expert token lists, and sums
the gate-masked dense outputs. Rounding to bf16 is done exactly with Python
fractions. Only for T*E small enough to enumerate.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np


def bf16_exact(v: float) -> float:
    """Round-half-even of a float64 to 8 significant bits, via exact fractions."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)
    q = round(Fraction(m) * 256)          # Python rounds Fractions half to even
    return math.ldexp(q, e - 8)


_bf16_vec = np.vectorize(bf16_exact, otypes=[np.float64])


def _rho(bf16):
    return _bf16_vec if bf16 else (lambda a: a)


def select_bruteforce(key: np.ndarray, k: int):
    """Per token, the k-subset with the largest key sum; among equal sums the
    lexicographically smallest id set. Returned as a sorted id tuple."""
    T, E = key.shape
    out = []
    for t in range(T):
        best, best_sum = None, -math.inf
        for sub in itertools.combinations(range(E), k):
            s = float(sum(key[t, list(sub)]))
            if s > best_sum:
                best, best_sum = sub, s
        out.append(best)
    return out


def layer_bruteforce(x, w, *, E, k, S, F, d, score="softmax", renorm=True,
                     capacity=0, bf16=False, rank=0, aux_coef=0.01):
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    rho = _rho(bf16)
    l = np.einsum("tc,ce->te", x, np.asarray(w["w_router"], np.float64))
    if w.get("logit_bias") is not None:
        l = l + np.asarray(w["logit_bias"], np.float64)
    if score == "softmax":
        key = l
        full = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)
    else:
        sg = 1.0 / (1.0 + np.exp(-l))
        key = sg + (0.0 if w.get("select_bias") is None else np.asarray(w["select_bias"], np.float64))
        full = sg / sg.sum(axis=1, keepdims=True)
    sel = select_bruteforce(key, k)

    # dense gate matrix, zero off the selection
    G = np.zeros((T, E))
    for t in range(T):
        ids = list(sel[t])
        if score == "softmax":
            if renorm:
                ex = np.exp(l[t, ids])
                G[t, ids] = ex / ex.sum()
            else:
                G[t, ids] = full[t, ids]
        else:
            G[t, ids] = sg[t, ids] / sg[t, ids].sum()

    # capacity from per-expert token lists (token order)
    keepmask = np.ones((T, E), bool)
    counts = np.zeros(E, np.int64)
    for e in range(E):
        toks = [t for t in range(T) if e in sel[t]]
        counts[e] = len(toks)
        if capacity > 0:
            for t in toks[capacity:]:
                keepmask[t, e] = False
    Gk = np.where(keepmask, G, 0.0)

    # every expert on every token
    def dense_expert(wg, wu, wd):
        a = x @ wg
        b = x @ wu
        h = rho(a / (1.0 + np.exp(-a)) * b)
        return h @ wd

    def lr(v, u, s, vm):
        return rho((v @ u) * s) @ vm.T

    y = np.zeros((T, d))
    for e in range(E):
        if rank == 0:
            o = dense_expert(np.asarray(w["w_gate"][e], np.float64),
                             np.asarray(w["w_up"][e], np.float64),
                             np.asarray(w["w_down"][e], np.float64))
        else:
            f = {n: np.asarray(w[n][e], np.float64) for n in (
                "u_gate", "s_gate", "v_gate", "u_up", "s_up", "v_up",
                "u_down", "s_down", "v_down")}
            a = lr(x, f["u_gate"], f["s_gate"], f["v_gate"])
            b = lr(x, f["u_up"], f["s_up"], f["v_up"])
            h = rho(a / (1.0 + np.exp(-a)) * b)
            o = lr(h, f["u_down"], f["s_down"], f["v_down"])
        y += Gk[:, e:e + 1] * o
    for s in range(S):
        y += dense_expert(np.asarray(w["sh_gate"][s], np.float64),
                          np.asarray(w["sh_up"][s], np.float64),
                          np.asarray(w["sh_down"][s], np.float64))
    f = counts / float(T * k)
    P = full.mean(axis=0)
    aux_raw = E * float((f * P).sum())
    return dict(y=y, sel=sel, G=G, keep=keepmask, counts=counts, f=f, P=P,
                aux_raw=aux_raw, aux=aux_coef * aux_raw)
