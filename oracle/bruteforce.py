"""Scalar-loop multi-head attention in 50-digit arithmetic, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

Shares no code with ``mha_oracle``: every product is an explicit loop over
mpmath numbers, the allowed set is decided per (i, j) from the rule itself,
and the softmax is the textbook ratio exp(s_ij) / sum_k exp(s_ik) over the
allowed keys, with no shift (50 digits and small inputs leave no overflow).
It follows the same pages as ``mha_oracle``:
* page "Multi-head attention and self-attention", Definition (per-head
  projections, concatenation in head order, W^O);
* page "Self-Attention & Multi-Head", the five steps (project, score, scale,
  normalise each row, aggregate the values);
* page "From Attention to Self-Attention" review, causal and padding masks;
* page "Multi-Head Attention" review: softmax(Q K^T / sqrt(d_k) + M) (an
  additive score bias M, here any real matrix whose -inf entries forbid
  keys) and the bias convention (X W + b when biases are used).
"""

from __future__ import annotations

import mpmath

DPS = 50


def _mp(x):
    return mpmath.mpf(float(x))


def _allowed(i, j, b, causal, key_len, allowed):
    ok = True
    if causal and j > i:
        ok = False
    if key_len is not None and j >= int(key_len[b]):
        ok = False
    if allowed is not None:
        Gb = allowed[0] if len(allowed) == 1 else allowed[b]
        if not bool(Gb[i][j]):
            ok = False
    return ok


def mha_bruteforce(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, scale,
                   causal=False, key_len=None, allowed=None, add=None, biases=None):
    """Returns (Y, Z) as nested lists of mpmath numbers.

    Q [B][n_q][d_q], K [B][n_k][d_k], V [B][n_k][d_v] (any nested sequences);
    combined weights as in the definition: head r of W_Q uses columns
    r*d_h .. r*d_h + d_h - 1, and W_O is [h*d_vh][d_o].  ``add``: optional
    [B or 1][n_q][n_k] additive score bias (-inf forbids the key);
    ``biases``: optional dict with any of b_Q, b_K, b_V, b_O (vectors).
    """
    bs = biases or {}

    def bias(name, idx):
        vec = bs.get(name)
        return mpmath.mpf(0) if vec is None else _mp(vec[idx])
    with mpmath.workdps(DPS):
        B = len(Q)
        n_q = len(Q[0])
        n_k = len(K[0])
        d_q, d_k, d_v = len(Q[0][0]), len(K[0][0]), len(V[0][0])
        d_o = len(W_O[0])
        c = _mp(scale)
        Y = []
        Z = []
        for b in range(B):
            Zb = [[mpmath.mpf(0)] * (h * d_vh) for _ in range(n_q)]
            for r in range(h):
                # head projections, one scalar product at a time
                q = [[sum(_mp(Q[b][i][a]) * _mp(W_Q[a][r * d_h + e]) for a in range(d_q))
                      + bias("b_Q", r * d_h + e) for e in range(d_h)] for i in range(n_q)]
                k = [[sum(_mp(K[b][j][a]) * _mp(W_K[a][r * d_h + e]) for a in range(d_k))
                      + bias("b_K", r * d_h + e) for e in range(d_h)] for j in range(n_k)]
                v = [[sum(_mp(V[b][j][a]) * _mp(W_V[a][r * d_vh + e]) for a in range(d_v))
                      + bias("b_V", r * d_vh + e) for e in range(d_vh)] for j in range(n_k)]
                Mb = None if add is None else (add[0] if len(add) == 1 else add[b])
                for i in range(n_q):
                    keys = [j for j in range(n_k)
                            if _allowed(i, j, b, causal, key_len, allowed)
                            and (Mb is None or float(Mb[i][j]) != float("-inf"))]
                    if not keys:
                        raise ValueError(f"row {i} of item {b} has no allowed key")
                    s = {j: c * sum(q[i][e] * k[j][e] for e in range(d_h))
                         + (0 if Mb is None else _mp(Mb[i][j])) for j in keys}
                    den = sum(mpmath.exp(s[j]) for j in keys)
                    for e in range(d_vh):
                        Zb[i][r * d_vh + e] = sum(mpmath.exp(s[j]) / den * v[j][e]
                                                  for j in keys)
            Yb = [[sum(Zb[i][f] * _mp(W_O[f][o]) for f in range(h * d_vh)) + bias("b_O", o)
                   for o in range(d_o)] for i in range(n_q)]
            Y.append(Yb)
            Z.append(Zb)
        return Y, Z


def to_float(nested):
    """Nested mpmath lists -> nested Python floats."""
    if isinstance(nested, list):
        return [to_float(x) for x in nested]
    return float(nested)
