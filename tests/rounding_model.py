"""A float64 model of the roundings the library's fp16 path makes.

Test infrastructure only: it shares no code with the HIP kernels (it is
written from what the kernels are documented to round, not from their
source) and it is not the oracle (the oracle, oracle/, is the plain
definition with no rounding at all).  Its purpose is to say how far from
the oracle an implementation that rounds exactly these intermediates must
land, so that every fp16 tolerance bar in the GPU tests is set from an
emulated error instead of from the run that passed.

What is modelled (bf16 inputs and weights, fp16 intermediates):
* projections: bf16 products accumulated exactly (fp32 accumulation of 1024
  or 2048 bf16 products loses nothing the fp16 store keeps), rounded to fp16
  (round to nearest even): Qh, Kh, Vh;
* attention core on fp16 heads (the deferred-shift form, page "Stable
  summary of an attention key block", Definition: per-row summaries merged
  block by block):
  - the query multiplied by c log2(e) in fp32 and rounded to fp16 once, so
    scores come out in base-2 units;
  - per row, a reference shift mu set from the exact maximum of the first
    64-key block; each later block's weights 2^(s - mu) rounded to fp16; when
    a block's weights sum to more than 2^8 (or overflow) mu moves up to the
    block's exact maximum and the running (l, z) are rescaled by 2^(mu_old -
    mu_new) (the page's merge rule applied at the new shift);
  - l sums the rounded weights, z the rounded weights times fp16 values (fp32
    accumulation: modelled exactly); Z = z / l rounded to the output type;
* output projection: the fp16 concatenation times W_O (bf16, exact in fp16),
  accumulated exactly, fp32 output.
The exact-shift form (the general and masked paths, the key-split form, and
bf16 heads) is modelled too: the query is not rounded again, scores are
c log2(e) q.k in fp32, each block's weights are 2^(s - m) at the running
exact maximum m, rounded to the heads' type (fp16, or bf16 with 2^-9), and
(l, z) are rescaled whenever m moves.
The kernels' own trigger for moving mu is a lane's partial sum of 32 of a
block's weights; the model uses the whole block's sum.  Either keeps every
weight in [0, 2^8]; which blocks move mu can differ, which changes the
rounding error only at the level of the error itself.
"""

from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634


def rnd16(x):
    """Round to the nearest fp16 (ties to even), returned as float64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def rnd32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def rnd_bf16(x):
    """Round to the nearest bf16 (ties to even, through fp32), as float64."""
    x32 = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ident(x):
    return np.asarray(x, np.float64)


def attn_core_f16_model(Qh, Kh, Vh, scale, allow, out_dtype="f16", block=64, tau=8.0,
                        exact=False, add=None):
    """Z [B, n_q, h*d_vh] of the fp16 attention core under the modelled roundings.

    Qh, Kh, Vh: head tensors holding fp16 values; allow [B, n_q, n_k].  A row
    with no allowed key in the first block (a boolean mask) keeps mu = -inf
    until its first block with an allowed key, which then takes the redo
    path (mu = that block's exact maximum), as the masked kernel does.
    `add`: an optional additive score bias M [B or 1, n_q, n_k] (natural-log
    units, -inf forbids a key), added in fp32 to the base-2 score as
    M log2(e) (modelled exactly).
    exact=True turns every rounding off (then the model is the plain
    definition in another order of operations, used to pin the model's
    bookkeeping against the oracle).
    """
    r16 = _ident if exact else rnd16
    rout = _ident if (exact or out_dtype == "f32") else rnd16
    Qh, Kh, Vh = (np.asarray(t, np.float64) for t in (Qh, Kh, Vh))
    B, h, n_q, _ = Qh.shape
    n_k, d_vh = Kh.shape[2], Vh.shape[3]
    if exact:
        sl = scale * LOG2E
    else:
        sl = float(np.float32(scale) * np.float32(LOG2E))
    Z = np.empty((B, n_q, h * d_vh))
    nblk = (n_k + block - 1) // block
    M = None if add is None else np.broadcast_to(np.asarray(add, np.float64), (B, n_q, n_k))
    for b in range(B):
        A = np.asarray(allow[b], bool)
        if M is not None:
            A = A & (M[b] > -np.inf)
        for r in range(h):
            if exact:
                q = Qh[b, r] * sl
            else:
                q = rnd16((Qh[b, r].astype(np.float32) * np.float32(sl)).astype(np.float64))
            S = q @ Kh[b, r].T                          # base-2 units
            if M is not None:
                S = S + np.where(A, M[b], 0.0) * LOG2E
            S = np.where(A, S, -np.inf)
            mu = S[:, :block].max(axis=1)           # -inf: no allowed key yet
            l = np.zeros(n_q)
            z = np.zeros((n_q, d_vh))
            for k in range(nblk):
                Sb = S[:, k * block:(k + 1) * block]
                Vb = Vh[b, r, k * block:(k + 1) * block]
                mu_use = np.where(np.isfinite(mu), mu, 0.0)
                with np.errstate(over="ignore", invalid="ignore"):
                    p = r16(np.exp2(Sb - mu_use[:, None]))
                p = np.where(np.isfinite(Sb), p, 0.0)
                # a row without a shift yet redoes its first block with an
                # allowed key (the kernel's +inf scores send it there)
                unset = ~np.isfinite(mu) & np.isfinite(Sb).any(axis=1)
                redo = ~(p.sum(axis=1) <= 2.0 ** tau) | unset
                if k == 0:
                    redo[:] = False
                if redo.any():
                    mx = Sb[redo].max(axis=1)
                    mu_new = np.maximum(mu[redo], mx)
                    with np.errstate(invalid="ignore"):
                        a = np.where(np.isfinite(mu_new), np.exp2(mu[redo] - mu_new), 1.0)
                    l[redo] *= a
                    z[redo] *= a[:, None]
                    mu[redo] = mu_new
                    mu_r = np.where(np.isfinite(mu_new), mu_new, 0.0)
                    with np.errstate(over="ignore", invalid="ignore"):
                        p[redo] = np.where(np.isfinite(Sb[redo]),
                                           r16(np.exp2(Sb[redo] - mu_r[:, None])), 0.0)
                l += p.sum(axis=1)
                z += p @ Vb
            Z[b, :, r * d_vh:(r + 1) * d_vh] = rout(z / l[:, None])
    return Z


def attn_core_exact_shift_model(Qh, Kh, Vh, scale, allow, elem="f16", out_dtype="f32",
                                block=64, exact=False, add=None, stats=False):
    """Z of the exact-shift form: weights 2^(c log2(e) s + M log2(e) - m), m
    the running exact maximum, rounded to `elem` ("f16", "bf16", or "f32":
    no rounding); `add`: an optional additive score bias M [B or 1, n_q, n_k]
    in natural-log units (-inf forbids a key); exact=True turns every
    rounding off.  stats=True also returns the rows' final (m, l): m in
    base-2 units, l the sum of the rounded weights at that shift."""
    rw = _ident if (exact or elem == "f32") else (rnd16 if elem == "f16" else rnd_bf16)
    rout = _ident if exact else {"f32": rnd32, "f16": rnd16, "bf16": rnd_bf16}[out_dtype]
    Qh, Kh, Vh = (np.asarray(t, np.float64) for t in (Qh, Kh, Vh))
    B, h, n_q, _ = Qh.shape
    n_k, d_vh = Kh.shape[2], Vh.shape[3]
    sl = abs(scale) * LOG2E if exact else float(np.float32(abs(scale)) * np.float32(LOG2E))
    sg = -1.0 if scale < 0 else 1.0
    Z = np.empty((B, n_q, h * d_vh))
    m_out = np.empty((B, h, n_q))
    l_out = np.empty((B, h, n_q))
    nblk = (n_k + block - 1) // block
    M = None if add is None else np.broadcast_to(np.asarray(add, np.float64), (B, n_q, n_k))
    for b in range(B):
        A = np.asarray(allow[b], bool)
        if M is not None:
            A = A & (M[b] > -np.inf)
        for r in range(h):
            S = sl * (sg * Qh[b, r] @ Kh[b, r].T)
            if M is not None:
                S = S + np.where(A, M[b], 0.0) * LOG2E
            S = np.where(A, S, -np.inf)
            m = np.full(n_q, -np.inf)
            l = np.zeros(n_q)
            z = np.zeros((n_q, d_vh))
            for k in range(nblk):
                Sb = S[:, k * block:(k + 1) * block]
                m_new = np.maximum(m, Sb.max(axis=1))
                use = np.where(np.isfinite(m_new), m_new, 0.0)
                with np.errstate(invalid="ignore"):
                    a = np.where(np.isfinite(m), np.exp2(m - use), 0.0)
                l *= a
                z *= a[:, None]
                p = np.where(np.isfinite(Sb), rw(np.exp2(Sb - use[:, None])), 0.0)
                l += p.sum(axis=1)
                z += p @ Vh[b, r, k * block:(k + 1) * block]
                m = m_new
            with np.errstate(invalid="ignore", divide="ignore"):
                Z[b, :, r * d_vh:(r + 1) * d_vh] = rout(z / l[:, None])
            m_out[b, r], l_out[b, r] = m, l
    if stats:
        return Z, m_out, l_out
    return Z


def core_bar(Qh, Kh, Vh, scale, allow, ref_Z, elem="f16", out_dtype="f32", floor=2e-4,
             add=None):
    """Twice the larger error (against the oracle's ref_Z) of the forms the
    library may run for these heads: the exact-shift form, and for fp16
    heads also the deferred shift; never below `floor`."""
    errs = [rel_err(attn_core_exact_shift_model(Qh, Kh, Vh, scale, allow, elem, out_dtype,
                                                add=add), ref_Z)]
    if elem == "f16" and scale > 0:
        errs.append(rel_err(attn_core_f16_model(Qh, Kh, Vh, scale, allow, out_dtype, add=add),
                            ref_Z))
    return max(2.0 * max(errs), floor)


def attn_core_grad_model(Qh, Kh, Vh, scale, allow, dZ, Z, elem="f16", grad_dtype="f32",
                         add=None, exact=False, stats=None):
    """Gradients (dQh, dKh, dVh, and dM with `add`) of the attention core under
    the backward kernels' roundings: with A the weights recomputed from the
    row statistics (fp32, modelled exactly; `stats` = (m in base-2 units, l)
    from the forward, else the exact softmax), the matrix-core kernels round
    dZ, A (the dV product's operand) and dS = A o (dA - D) once to the heads'
    type `elem` ("f32": no rounding); every sum is fp32 (modelled exactly);
    the gradients are stored in `grad_dtype` (the type of Z and dZ).  D_i =
    sum_e dZ_ie Z_ie uses the rounded dZ and the stored Z.  dM (fp32, shape of
    `add`) sums the unrounded dS over heads (and items for a shared bias), as
    the bias-gradient kernel does.  exact=True turns every rounding off."""
    re = _ident if (exact or elem == "f32") else (rnd16 if elem == "f16" else rnd_bf16)
    rg = _ident if exact else {"f32": rnd32, "f16": rnd16, "bf16": rnd_bf16}[grad_dtype]
    Qh, Kh, Vh = (np.asarray(t, np.float64) for t in (Qh, Kh, Vh))
    dZ = re(np.asarray(dZ, np.float64))
    Z = np.asarray(Z, np.float64)
    B, h, n_q, _ = Qh.shape
    n_k, d_vh = Kh.shape[2], Vh.shape[3]
    M = None if add is None else np.broadcast_to(np.asarray(add, np.float64), (B, n_q, n_k))
    dQ, dK, dV = np.zeros_like(Qh), np.zeros_like(Kh), np.zeros_like(Vh)
    dM = None if M is None else np.zeros((B, n_q, n_k))
    for b in range(B):
        A_ok = np.asarray(allow[b], bool)
        if M is not None:
            A_ok = A_ok & (M[b] > -np.inf)
        for r in range(h):
            S = scale * (Qh[b, r] @ Kh[b, r].T)
            if M is not None:
                S = S + np.where(A_ok, M[b], 0.0)
            S = np.where(A_ok, S, -np.inf)
            if stats is None:
                mx = S.max(axis=1, keepdims=True)
                mx = np.where(np.isfinite(mx), mx, 0.0)
                E = np.where(A_ok, np.exp(S - mx), 0.0)
                den = E.sum(axis=1, keepdims=True)
                A = np.divide(E, den, out=np.zeros_like(E), where=den > 0)
            else:
                m2, l = stats[0][b, r][:, None], stats[1][b, r][:, None]
                with np.errstate(divide="ignore", invalid="ignore"):
                    L2 = np.where((l > 0) & np.isfinite(m2), m2 + np.log2(l), np.inf)
                    A = np.where(A_ok, np.exp2(S * LOG2E - L2), 0.0)
            dZr = dZ[b, :, r * d_vh:(r + 1) * d_vh]
            D = np.sum(dZr * Z[b, :, r * d_vh:(r + 1) * d_vh], axis=1, keepdims=True)
            dA = dZr @ Vh[b, r].T
            dS32 = A * (dA - D)
            dS = re(dS32)
            dV[b, r] = re(A).T @ dZr
            dQ[b, r] = scale * (dS @ Kh[b, r])
            dK[b, r] = scale * (dS.T @ Qh[b, r])
            if dM is not None:
                dM[b] += dS32
    out = {"dQh": rg(dQ), "dKh": rg(dK), "dVh": rg(dV)}
    if dM is not None:
        out["dM"] = dM if np.shape(add)[0] == B else dM.sum(axis=0, keepdims=True)
    return out


def grad_err(out, ref):
    """(||out - ref|| / ||ref||, max|out - ref| / max|ref|), the metrics of
    the gradient bars."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    d = out - ref
    return (float(np.linalg.norm(d) / np.linalg.norm(ref)),
            float(np.abs(d).max() / np.abs(ref).max()))


def heads_f16(X, W, h, d):
    """A projection of bf16 X by bf16 W, accumulated exactly and rounded to
    fp16, in the head-major layout [B, h, n, d]."""
    X = np.asarray(X, np.float64)
    W = np.asarray(W, np.float64)
    B, n, _ = X.shape
    P = rnd16(X @ W)
    return P.reshape(B, n, h, d).transpose(0, 2, 1, 3).copy()


def mha_forward_f16_model(Q, K, V, W_Q, W_K, W_V, W_O, h, d_h, d_vh, scale, allow):
    """Y [B, n_q, d_o] (fp32) of mha_forward with bf16 inputs and fp16
    intermediates under the modelled roundings."""
    Qh = heads_f16(Q, W_Q, h, d_h)
    Kh = heads_f16(K, W_K, h, d_h)
    Vh = heads_f16(V, W_V, h, d_vh)
    Zc = attn_core_f16_model(Qh, Kh, Vh, scale, allow, out_dtype="f16")
    return rnd32(Zc @ rnd16(np.asarray(W_O, np.float64)))


def rel_err(out, ref):
    """max |out - ref| / RMS(ref), the metric of the tolerance bars."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(out - ref)) / np.sqrt(np.mean(ref * ref)))
