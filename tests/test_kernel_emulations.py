"""CPU emulations of the HIP kernels' orders of work, against the oracle.

Test infrastructure, float64, no GPU and no code shared with the kernels:
each emulation restates what a kernel is documented to do (which keys a
lane group visits, in which order summaries merge, what is rounded where)
and checks it against the oracle.

* Decode kernel (attn_decode_kernel) and the merge of key partitions
  (split_merge_kernel): each partition of 64-key multiples is walked by four
  waves of 64 / G lane groups, a group taking 4 keys per step at stride
  4 * 64 / G; each group keeps an exact-shift running summary (page "Stable
  summary of an attention key block", Definition: the merge of summaries),
  the groups of a wave merge by an xor butterfly, waves 1..3 merge into
  wave 0, and the partitions merge (skipping empty ones) before z / l.  In
  float64 this must give the oracle's result to rounding, and every allowed
  key must be visited exactly once.
* Backward: the rounding model of the gradient kernels
  (rounding_model.attn_core_grad_model) on the backward test cases, which
  sets the gradient bars of the GPU tests.
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from bars import BWD_TOL  # noqa: E402
from bwd_cases import BWD_CASES, additive_bias, bwd_case_inputs  # noqa: E402
from rounding_model import (  # noqa: E402
    attn_core_exact_shift_model, attn_core_grad_model, grad_err, rnd16, rnd32, rnd_bf16)

from oracle import allowed_set, attn_core_grad_ref, attn_core_ref  # noqa: E402
from transformer_head_self_amd.inputs import make_heads  # noqa: E402

LOG2E = 1.4426950408889634
LN2 = math.log(2.0)


# ---------------------------------------------------------------------------
# decode kernel
# ---------------------------------------------------------------------------

def _merge(a, b):
    """The page's merge of two base-2 summaries (m, l, z); the empty state
    (m = -inf) is the identity."""
    (m1, l1, z1), (m2, l2, z2) = a, b
    mn = max(m1, m2)
    if mn == -math.inf:
        return a
    c1 = 2.0 ** (m1 - mn) if m1 != -math.inf else 0.0
    c2 = 2.0 ** (m2 - mn) if m2 != -math.inf else 0.0
    return (mn, l1 * c1 + l2 * c2, z1 * c1 + z2 * c2)


def decode_partition(q2, K, V, kbeg, kend, ok, G, visits):
    """Summary (m, l, z) of keys [kbeg, kend) for one query row, in the
    decode kernel's order.  q2: the query scaled by c log2(e); ok(key) -> bias
    in base 2 (0.0) or None (forbidden); visits counts each key's use."""
    kpw, U = 64 // G, 4
    stride = 4 * kpw
    d_vh = V.shape[1]
    waves = []
    for wave in range(4):
        groups = []
        for grp in range(kpw):
            m, l, z = -math.inf, 0.0, np.zeros(d_vh)
            for k0 in range(kbeg + wave * kpw + grp, kend, U * stride):
                s = []
                for u in range(U):
                    key = k0 + u * stride
                    bias = ok(key) if key < kend else None
                    if key < kend:
                        visits[key] += 1
                    s.append(-math.inf if bias is None else float(q2 @ K[key]) + bias)
                mn = max(m, max(s))
                if mn == -math.inf:
                    continue
                a = 2.0 ** (m - mn) if m != -math.inf else 0.0
                m, l, z = mn, l * a, z * a
                for u in range(U):
                    if s[u] != -math.inf:
                        w = 2.0 ** (s[u] - mn)
                        l += w
                        z = z + w * V[k0 + u * stride]
            groups.append((m, l, z))
        st = 1
        while st < kpw:           # lanes exchange with the group st away
            groups = [_merge(groups[g], groups[g ^ st]) for g in range(kpw)]
            st *= 2
        waves.append(groups[0])
    out = waves[0]
    for w in range(1, 4):
        out = _merge(out, waves[w])
    return out


def decode_emulation(Qh, Kh, Vh, scale, n_q, split_keys, key_len=None, causal=False,
                     allowed=None, add=None):
    """Z [B, n_q, h*d_vh], row m (natural units) and l through partitions of
    `split_keys` keys merged as the merge kernel does."""
    B, h, _, d_h = Qh.shape
    n_k, d_vh = Kh.shape[2], Vh.shape[3]
    G = 4 if max(d_h, d_vh) <= 32 else 8 if max(d_h, d_vh) <= 64 else 16
    splits = -(-n_k // split_keys)
    Z = np.empty((B, n_q, h * d_vh))
    rm = np.empty((B, h, n_q))
    rl = np.empty((B, h, n_q))
    for b in range(B):
        kvalid = n_k if key_len is None else min(n_k, int(key_len[b]))
        for r in range(h):
            for i in range(n_q):
                q2 = Qh[b, r, i] * (scale * LOG2E)
                visits = np.zeros(n_k, np.int64)

                def ok(key):
                    if causal and key > i:
                        return None
                    if allowed is not None and not allowed[b, i, key]:
                        return None
                    if add is not None:
                        a = float(add[b if add.shape[0] > 1 else 0, i, key])
                        return None if a == -math.inf else a * LOG2E
                    return 0.0

                parts = []
                for sp in range(splits):
                    kbeg = sp * split_keys
                    kend = min(kvalid, kbeg + split_keys)
                    if causal:
                        kend = min(kend, n_q)
                    parts.append(decode_partition(q2, Kh[b, r], Vh[b, r], kbeg, kend, ok, G,
                                                  visits))
                # every key of the valid range once, nothing beyond it
                top = min(kvalid, n_q) if causal else kvalid
                assert np.all(visits[:top] == 1) and np.all(visits[top:] == 0)
                m = max(p[0] for p in parts)
                l, z = 0.0, np.zeros(d_vh)
                if m != -math.inf:
                    for pm, pl, pz in parts:
                        if pm == -math.inf:
                            continue
                        w = 2.0 ** (pm - m)
                        l += pl * w
                        z = z + pz * w
                with np.errstate(invalid="ignore", divide="ignore"):
                    Z[b, i, r * d_vh:(r + 1) * d_vh] = z / l
                rm[b, r, i] = m * LN2
                rl[b, r, i] = l
    return Z, rm, rl


DECODE_CASES = [
    # B, h, n_q, n_k, d_h, d_vh, split_keys, key_len, causal, mask
    (2, 3, 1, 1000, 64, 64, 256, None, False, None),
    (2, 2, 2, 700, 32, 32, 64, (700, 131), False, None),
    (1, 2, 3, 513, 128, 128, 192, None, False, "bool"),
    (2, 2, 4, 300, 64, 96, 128, (300, 5), False, "add"),
    (1, 2, 3, 3, 128, 64, 64, None, True, None),
    (1, 1, 1, 77, 40, 24, 64, None, False, None),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_emulation_matches_oracle(case):
    B, h, n_q, n_k, d_h, d_vh, split_keys, kl, causal, mask = case
    Qh, Kh, Vh = (x.astype(np.float64) for x in
                  make_heads(B, h, n_q, n_k, d_h, d_vh, "f32", seed=70 + n_k))
    rng = np.random.default_rng(71 + n_k)
    key_len = None if kl is None else np.array(kl[:B], np.int32)
    G = add = None
    if mask == "bool":
        G = rng.random((B, n_q, n_k)) < 0.3
        G[:, :, 5] = True
    elif mask == "add":
        add = additive_bias(rng, B, n_q, n_k).astype(np.float64)
    c = 1.0 / math.sqrt(d_h)
    Z, rm, rl = decode_emulation(Qh, Kh, Vh, c, n_q, split_keys, key_len, causal, G, add)
    allow = allowed_set(B, n_q, n_k, causal=causal, key_len=key_len, allowed=G)
    ref = attn_core_ref(Qh, Kh, Vh, c, allow, add=add)
    rms = math.sqrt(float(np.mean(ref["Z"] ** 2)))
    assert np.max(np.abs(Z - ref["Z"])) / rms < 1e-13
    assert np.allclose(rm, ref["m"], rtol=0, atol=1e-12)
    assert np.allclose(rl, ref["l"], rtol=1e-13, atol=0)


def test_decode_emulation_catches_a_skipped_key():
    """The coverage check is live: a partition plan that drops the last key
    of each partition trips it."""
    Qh, Kh, Vh = (x.astype(np.float64) for x in make_heads(1, 1, 1, 200, 32, 32, "f32", 72))
    q2 = Qh[0, 0, 0]
    visits = np.zeros(200, np.int64)
    for kbeg in range(0, 200, 64):
        decode_partition(q2, Kh[0, 0], Vh[0, 0], kbeg, min(200, kbeg + 64) - 1,
                         lambda k: 0.0, 4, visits)
    assert not np.all(visits == 1)


# ---------------------------------------------------------------------------
# backward rounding model -> gradient bars
# ---------------------------------------------------------------------------

_R = {"f16": rnd16, "bf16": rnd_bf16, "f32": rnd32}


def _bwd_model_errors(case):
    dt, zdt, B, h, n_q, n_k, d_h, d_vh, causal, kl, use_bool, use_add = case
    Qh, Kh, Vh, dZ, key_len, G, M, c = bwd_case_inputs(case)
    host = [_R[dt](x) for x in (Qh, Kh, Vh)]
    dZh = _R[zdt](dZ)
    allow = allowed_set(B, n_q, n_k, causal=causal, key_len=key_len, allowed=G)
    Z = np.nan_to_num(attn_core_exact_shift_model(*host, c, allow, elem=dt, out_dtype=zdt,
                                                  add=M))
    ref = attn_core_grad_ref(*host, c, allow, dZh, add=M)
    mod = attn_core_grad_model(*host, c, allow, dZh, Z, elem=dt, grad_dtype=zdt, add=M)
    return [grad_err(mod[k], ref[k]) for k in ("dQh", "dKh", "dVh")]


def test_backward_model_exact_is_the_oracle():
    """With every rounding taken out the model's bookkeeping is the oracle's
    gradient (a transposed operand or a dropped row term would show)."""
    case = BWD_CASES[6]                    # causal with an additive bias
    Qh, Kh, Vh, dZ, key_len, G, M, c = bwd_case_inputs(case)
    B, n_q, n_k = Qh.shape[0], Qh.shape[2], Kh.shape[2]
    allow = allowed_set(B, n_q, n_k, causal=True, key_len=key_len, allowed=G)
    Z = attn_core_ref(Qh, Kh, Vh, c, allow, add=M)["Z"]
    ref = attn_core_grad_ref(Qh, Kh, Vh, c, allow, dZ, add=M)
    mod = attn_core_grad_model(Qh, Kh, Vh, c, allow, dZ, Z, add=M, exact=True)
    for k in ("dQh", "dKh", "dVh"):
        assert grad_err(mod[k], ref[k])[0] < 1e-12, k


def test_backward_bars_come_from_the_model():
    worst = {"bf16": [0.0, 0.0], "f16": [0.0, 0.0]}
    for case in BWD_CASES:
        for fro, mx in _bwd_model_errors(case):
            w = worst[case[0]]
            w[0], w[1] = max(w[0], fro), max(w[1], mx)
    for dt, (fro, mx) in worst.items():
        bar_fro, bar_mx = BWD_TOL[dt]
        assert 1.5 <= bar_fro / fro <= 3.5, (dt, fro, bar_fro)
        assert 1.5 <= bar_mx / mx <= 3.5, (dt, mx, bar_mx)
    # the two element types differ by their unit roundoffs (2^-9 vs 2^-11)
    assert 5 < worst["bf16"][0] / worst["f16"][0] < 12
