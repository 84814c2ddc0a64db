"""Dense float64 reference for multi-head attention (forward only).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.

What it computes, and from which passage
----------------------------------------
* Page "Multi-head attention and self-attention", Definition: general dims
  h, d_q, d_k, d_v, d_h, d_vh, d_o, n_q, n_k; head i is scaled dot-product
  attention of (Q W_i^Q, K W_i^K, V W_i^V) under one chosen mask shared by
  every head; the heads are concatenated along the feature axis and
  multiplied by W^O.  Self-attention is Q = K = V = X.
* Page "Multi-Head Attention" review (llmprimer), "The Complete Multi-Head
  Operation": A = softmax over the last axis of (Q K^T / sqrt(d_k) + M),
  Z^(r) = A^(r) V^(r), Z = Concat, Y = Z W_O; batch-major shapes.
  "Separate and Combined Projections": combined weights hold the heads side
  by side; (B,T,h d_k) -> (B,T,h,d_k) -> (B,h,T,d_k).
* Page "From Attention to Self-Attention" review, "The Complete Layer" and
  "Distinctions to Keep": the mask acts before the softmax; a causal mask
  removes later positions, a padding mask removes artificial key positions,
  and the two may be combined.
* Page "Stable summary of an attention key block", Definition: allowed key
  sets are nonempty; the row maximum is the stabilising shift.

* The same review page, "Parameter and Work Conventions" and "Audit Order":
  projection biases are a convention to be stated; without them the layer
  is the products above.  With them (here: optional vectors b_Q [h*d_h],
  b_K [h*d_h], b_V [h*d_vh], b_O [d_o]) each product X W becomes X W + b,
  the bias broadcast over rows, head r's block in entries r*d .. r*d+d-1.

Readings of points the pages leave open:
* masks are allowed sets (additive M in {0, -inf}); combined rules AND;
* an additive score bias M may also be a general real matrix [B or 1, n_q,
  n_k], added to the scaled scores c q.k (the review page's
  softmax(Q K^T / sqrt(d_k) + M): M is not multiplied by the scale); its
  -inf entries are forbidden keys, +inf and NaN are invalid;
* key padding masks keys only, never whole query rows;
* causal requires n_q == n_k and allows j <= i (0-based);
* a row whose allowed set is empty violates the definition: EmptyRowError;
* the scale c is an explicit argument (1/sqrt(d_h) is the caller's default).

Nothing here is blocked, fused or reordered: every (batch, head) score
matrix is materialised whole, and the softmax uses the exact row maximum.
"""

from __future__ import annotations

import numpy as np


class EmptyRowError(ValueError):
    """A query row has no allowed key (the definition requires one)."""


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_set(B, n_q, n_k, causal=False, key_len=None, allowed=None):
    """Boolean allowed[b, i, j]: may query i of item b use key j.

    Page "From Attention to Self-Attention" review, "Distinctions to Keep"
    (causal and padding masks, combinable); page "Multi-head attention and
    self-attention", Definition (one mask applied to every head, so there is
    no head axis).  ``allowed`` is an optional explicit boolean mask of shape
    [B or 1, n_q, n_k] for the general "any chosen mask" case.
    """
    A = np.ones((B, n_q, n_k), dtype=bool)
    if causal:
        if n_q != n_k:
            raise ValueError("a causal mask needs n_q == n_k")
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        A &= (j <= i)[None]
    if key_len is not None:
        key_len = np.asarray(key_len)
        j = np.arange(n_k)[None, None, :]
        A &= j < key_len[:, None, None]
    if allowed is not None:
        G = np.asarray(allowed, dtype=bool)
        A &= np.broadcast_to(G, (B, n_q, n_k))
    return A


def project_separate(X, W, h, d, bias=None):
    """Per-head products X W^(r) (+ b^(r)), r = 0..h-1, stacked as [B, h, n, d].

    Page "Multi-head attention and self-attention", Definition: each head
    has its own projection matrix.  The combined matrix W [d_in, h*d] holds
    head r in columns r*d .. r*d+d-1 (review page, "Separate and Combined
    Projections"); here each head's block is sliced out and multiplied
    on its own.  An optional bias [h*d] is sliced the same way and added to
    every row of the head's product.
    """
    X = _f64(X)
    W = _f64(W)
    B, n, _ = X.shape
    out = np.empty((B, h, n, d))
    for r in range(h):
        Wr = W[:, r * d:(r + 1) * d]
        for b in range(B):
            out[b, r] = X[b] @ Wr
            if bias is not None:
                out[b, r] += _f64(bias)[r * d:(r + 1) * d]
    return out


def project_combined(X, W, h, d, bias=None):
    """One wide product (+ bias [h*d]), then reshape and transpose to [B, h, n, d].

    Review page "Multi-Head Attention", "Separate and Combined Projections":
    (B, T, h d) -> (B, T, h, d) -> (B, h, T, d).
    """
    X = _f64(X)
    W = _f64(W)
    B, n, _ = X.shape
    wide = X @ W                       # (B, n, h*d)
    if bias is not None:
        wide = wide + _f64(bias)[None, None, :]
    split = wide.reshape(B, n, h, d)   # reshape splits the feature axis
    return split.transpose(0, 2, 1, 3).copy()  # transpose swaps head and position


def masked_softmax_rows(S, allow):
    """Stable softmax of each row of S over its allowed entries.

    S: [n_q, n_k] float64 scores; allow: [n_q, n_k] bool.
    Returns (A, m, l): weights, row maxima over allowed entries, and
    l = sum over allowed j of exp(S_ij - m_i).  Forbidden weights are
    assigned 0.0 directly (never computed from -inf), so they are exact
    zeros.  This is the one-block summary of page "Stable summary of an
    attention key block" followed by dividing by its second coordinate.
    """
    if not np.all(allow.any(axis=1)):
        bad = int(np.flatnonzero(~allow.any(axis=1))[0])
        raise EmptyRowError(f"query row {bad} has no allowed key")
    Smask = np.where(allow, S, -np.inf)
    m = Smask.max(axis=1)
    E = np.zeros_like(S)
    E[allow] = np.exp((S - m[:, None])[allow])
    l = E.sum(axis=1)
    A = E / l[:, None]
    return A, m, l


def _additive(add, B, n_q, n_k):
    """The additive score bias as [B, n_q, n_k] float64 (None: all zeros)."""
    if add is None:
        return None
    M = np.broadcast_to(_f64(add), (B, n_q, n_k))
    if np.isnan(M).any() or np.isposinf(M).any():
        raise ValueError("an additive score bias must be finite or -inf")
    return M


def attn_core_ref(Qh, Kh, Vh, scale, allow, keep_A=False, add=None):
    """Attention on projected heads; output in concatenated layout.

    Qh [B,h,n_q,d_h], Kh [B,h,n_k,d_h], Vh [B,h,n_k,d_vh];
    allow [B,n_q,n_k] (one mask for every head); add: optional additive
    score bias M [B or 1, n_q, n_k] (one for every head), added to the
    scaled scores; its -inf entries are forbidden keys.
    Returns dict with Z [B, n_q, h*d_vh] (head r in columns r*d_vh..),
    m, l [B, h, n_q] (natural-log units), and A [B,h,n_q,n_k] if keep_A.
    """
    Qh, Kh, Vh = _f64(Qh), _f64(Kh), _f64(Vh)
    B, h, n_q, _ = Qh.shape
    n_k = Kh.shape[2]
    d_vh = Vh.shape[3]
    Z = np.empty((B, n_q, h * d_vh))
    m = np.empty((B, h, n_q))
    l = np.empty((B, h, n_q))
    A_all = np.empty((B, h, n_q, n_k)) if keep_A else None
    M = _additive(add, B, n_q, n_k)
    for b in range(B):
        allow_b = np.asarray(allow[b], dtype=bool)
        if M is not None:
            allow_b = allow_b & (M[b] > -np.inf)
        for r in range(h):
            S = scale * (Qh[b, r] @ Kh[b, r].T)          # scores, materialised
            if M is not None:
                S = S + np.where(allow_b, M[b], 0.0)      # + M on the allowed entries
            A, m[b, r], l[b, r] = masked_softmax_rows(S, allow_b)
            Z[b, :, r * d_vh:(r + 1) * d_vh] = A @ Vh[b, r]   # concat in head order
            if keep_A:
                A_all[b, r] = A
    out = {"Z": Z, "m": m, "l": l}
    if keep_A:
        out["A"] = A_all
    return out


def mha_ref(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, scale, allow,
            projection="combined", keep_A=False, add=None, biases=None):
    """Full multi-head attention forward in float64.

    Q [B,n_q,d_q], K [B,n_k,d_k], V [B,n_k,d_v]; W_Q [d_q,h*d_h],
    W_K [d_k,h*d_h], W_V [d_v,h*d_vh], W_O [h*d_vh,d_o].  ``biases``: None
    (no biases) or a dict with any of b_Q [h*d_h], b_K [h*d_h], b_V [h*d_vh],
    b_O [d_o].  ``add``: optional additive score bias M [B or 1, n_q, n_k].
    ``projection`` picks one of two independent projection code paths.
    Returns dict with Y [B,n_q,d_o], Z, m, l (and A if keep_A).
    """
    bs = biases or {}
    proj = {"combined": project_combined, "separate": project_separate}[projection]
    Qh = proj(Q, W_Q, h, d_h, bs.get("b_Q"))
    Kh = proj(K, W_K, h, d_h, bs.get("b_K"))
    Vh = proj(V, W_V, h, d_vh, bs.get("b_V"))
    out = attn_core_ref(Qh, Kh, Vh, scale, allow, keep_A=keep_A, add=add)
    out["Y"] = out["Z"] @ _f64(W_O)                 # output projection
    if bs.get("b_O") is not None:
        out["Y"] = out["Y"] + _f64(bs["b_O"])[None, None, :]
    return out


def mha_ref_rows(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, scale, allow, b, rows,
                 add=None, biases=None):
    """The same computation restricted to query rows ``rows`` of item ``b``.

    Keys and values of item b are projected in full; only the selected
    query rows are projected and attended.  Used to check large problems
    at sampled positions.  Returns (Y_rows [len(rows), d_o],
    Z_rows [len(rows), h*d_vh], m_rows [h, len(rows)], l_rows [h, len(rows)]).
    """
    rows = np.asarray(rows)
    bs = biases or {}
    Qb = _f64(Q[b])[rows][None]                        # (1, R, d_q)
    Kb = _f64(K[b])[None]
    Vb = _f64(V[b])[None]
    Qh = project_combined(Qb, W_Q, h, d_h, bs.get("b_Q"))
    Kh = project_combined(Kb, W_K, h, d_h, bs.get("b_K"))
    Vh = project_combined(Vb, W_V, h, d_vh, bs.get("b_V"))
    sub_allow = np.asarray(allow[b])[rows][None]
    sub_add = None
    if add is not None:
        A = _f64(add)
        sub_add = (A[0] if A.shape[0] == 1 else A[b])[rows][None]
    out = attn_core_ref(Qh, Kh, Vh, scale, sub_allow, add=sub_add)
    Y = out["Z"][0] @ _f64(W_O)
    if bs.get("b_O") is not None:
        Y = Y + _f64(bs["b_O"])[None, :]
    return Y, out["Z"][0], out["m"][0], out["l"][0]


def attn_core_grad_ref(Qh, Kh, Vh, scale, allow, dZ, add=None):
    """Gradients of the attention core for an upstream gradient dZ.

    Same arguments as ``attn_core_ref`` plus dZ [B, n_q, h*d_vh] (the
    gradient of a scalar loss with respect to the concatenated output Z).
    Returns dict with dQh, dKh, dVh (shapes of Qh, Kh, Vh), and with an
    additive bias also dM (the shape of ``add``: [B or 1, n_q, n_k]).

    Derivation (calculus on the definitions the forward follows; the pages
    give no backward pass): for one head, with scores S = c Q K^T (+ M) and
    A = masked row softmax of S, Z_r = A V:
      dV = A^T dZ_r                          (Z_r is linear in V);
      dA = dZ_r V^T;
      dS_ij = A_ij (dA_ij - sum_k A_ik dA_ik)   (softmax Jacobian per row;
                                                forbidden entries have
                                                A_ij = 0, so dS_ij = 0);
      dQ = c dS K,  dK = c dS^T Q.
    The row term sum_k A_ik dA_ik equals sum_e dZ_ie Z_ie.
    M enters every head's scores with coefficient 1 (S = c Q K^T + M), so
    dM is dS summed over the heads, and over the batch items when one M
    serves them all; a forbidden entry (masked, or M = -inf) gets 0.
    """
    Qh, Kh, Vh = _f64(Qh), _f64(Kh), _f64(Vh)
    dZ = _f64(dZ)
    B, h, n_q, _ = Qh.shape
    n_k = Kh.shape[2]
    d_vh = Vh.shape[3]
    out = attn_core_ref(Qh, Kh, Vh, scale, allow, keep_A=True, add=add)
    A_all = out["A"]
    dQ = np.zeros_like(Qh)
    dK = np.zeros_like(Kh)
    dV = np.zeros_like(Vh)
    dM = None if add is None else np.zeros((B, n_q, n_k))
    for b in range(B):
        for r in range(h):
            A = A_all[b, r]                                   # [n_q, n_k]
            dZr = dZ[b, :, r * d_vh:(r + 1) * d_vh]           # [n_q, d_vh]
            dV[b, r] = A.T @ dZr
            dA = dZr @ Vh[b, r].T
            rowdot = np.sum(A * dA, axis=1, keepdims=True)
            dS = A * (dA - rowdot)
            dQ[b, r] = scale * (dS @ Kh[b, r])
            dK[b, r] = scale * (dS.T @ Qh[b, r])
            if dM is not None:
                dM[b] += dS
    res = {"dQh": dQ, "dKh": dK, "dVh": dV}
    if dM is not None:
        res["dM"] = dM if np.shape(add)[0] == B else dM.sum(axis=0, keepdims=True)
    return res


def mha_grad_ref(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, scale, allow, dY, add=None,
                 biases=None):
    """Gradients of the full layer for an upstream gradient dY [B, n_q, d_o].

    Returns dict with dQ, dK, dV (input gradients; for self-attention the
    gradient with respect to X is their sum), dM (with an additive bias, as
    in attn_core_grad_ref), dW_Q, dW_K, dW_V, dW_O,
    db_Q, db_K, db_V, db_O (the bias gradients, whether or not the forward
    used biases: a bias enters additively, so its gradient does not depend
    on its value) and dQ_cat, dK_cat, dV_cat (the heads' gradients side by
    side, [B, n, h*d]).  Calculus on the forward this module computes:
      Y = Z W_O (+ b_O):       dZ = dY W_O^T,  dW_O = sum_b Z_b^T dY_b,  db_O = sum dY;
      core:                    dQh, dKh, dVh from attn_core_grad_ref;
      Qh = split(Q W_Q + b_Q): dQ_flat = merge(dQh) [B, n_q, h*d_h],
                               dW_Q = sum_b Q_b^T dQ_flat_b, db_Q = sum dQ_flat,
                               dQ = dQ_flat W_Q^T;  likewise for K and V.
    """
    bs = biases or {}
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    W_Q, W_K, W_V, W_O = _f64(W_Q), _f64(W_K), _f64(W_V), _f64(W_O)
    dY = _f64(dY)
    Qh = project_combined(Q, W_Q, h, d_h, bs.get("b_Q"))
    Kh = project_combined(K, W_K, h, d_h, bs.get("b_K"))
    Vh = project_combined(V, W_V, h, d_vh, bs.get("b_V"))
    Z = attn_core_ref(Qh, Kh, Vh, scale, allow, add=add)["Z"]
    dZ = dY @ W_O.T
    out = {"dW_O": np.einsum("bnf,bno->fo", Z, dY), "db_O": dY.sum(axis=(0, 1))}
    g = attn_core_grad_ref(Qh, Kh, Vh, scale, allow, dZ, add=add)
    for name, X, W, gh in (("Q", Q, W_Q, g["dQh"]), ("K", K, W_K, g["dKh"]),
                           ("V", V, W_V, g["dVh"])):
        B, hh, n, d = gh.shape
        flat = gh.transpose(0, 2, 1, 3).reshape(B, n, hh * d)   # merge the heads back
        out["dW_" + name] = np.einsum("bni,bnj->ij", X, flat)
        out["db_" + name] = flat.sum(axis=(0, 1))
        out["d" + name + "_cat"] = flat
        out["d" + name] = flat @ W.T
    if "dM" in g:
        out["dM"] = g["dM"]
    return out
