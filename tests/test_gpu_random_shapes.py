"""Seeded random shapes through the attention core forward and backward
against the float64 oracle.

The shapes are drawn once from a fixed seed (ragged n_q and n_k, head widths
32 to 128, causal and key-padding masks, fp16 and bf16 heads, with and without
row statistics, Z / dZ in the heads' type or fp32), so every launch path of
the core kernels (direct-load fast paths, the general path, the decode-shaped
and the register-staged backward) meets shapes no hand-written case picked.
Bars: the forward's max |err| / RMS under twice the error of a float64
model of the heads' type's roundings (tests/rounding_model.py), the
backward's normwise and max-normalised errors as in test_gpu_parity.
"""

import math

import numpy as np
import pytest
import torch

import transformer_head_self_amd as mha
from oracle import allowed_set, attn_core_grad_ref, attn_core_ref
from rounding_model import core_bar
from test_gpu_parity import BWD_TOL, DEV, TOL, _bwd_run, _grad_err, _rel_err, _say
from transformer_head_self_amd.inputs import make_heads

pytestmark = pytest.mark.gpu


def _draw(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ("f16", "bf16")[i % 2]
        d_h = int(rng.choice([32, 64, 128]))
        d_vh = int(rng.choice([32, 64, 96, 128]))
        if i % 3 == 0:
            d_h = d_vh = 64
        B, h = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        n_q, n_k = int(rng.integers(1, 500)), int(rng.integers(1, 500))
        if i % 2 == 0:
            n_q = (n_q // 4 + 1) * 4        # whole 4-row chunks (direct-load backward)
        causal = bool(rng.integers(0, 2))
        if causal:
            n_k = n_q
        kl = tuple(int(v) for v in rng.integers(1, n_k + 1, size=B)) if rng.integers(0, 2) else None
        flag = bool(rng.integers(0, 2))
        cases.append((dt, B, h, n_q, n_k, d_h, d_vh, causal, kl, flag))
    return cases


FWD_CASES = _draw(1234, 16)
BWD_CASES = _draw(4321, 12)


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_forward_core(case):
    dt, B, h, n_q, n_k, d_h, d_vh, causal, kl, stats = case
    _say(f"[random forward] {case}")
    Qh, Kh, Vh = make_heads(B, h, n_q, n_k, d_h, d_vh, "f32" if dt == "f16" else dt,
                            seed=500 + n_q + n_k)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    dev = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(tdt) for a in (Qh, Kh, Vh)]
    host = [t.float().cpu().numpy().astype(np.float64) for t in dev]
    c = 1.0 / math.sqrt(d_h)
    key_len = None if kl is None else np.array(kl, dtype=np.int32)
    rm = torch.empty((B, h, n_q), device=DEV) if stats else None
    rl = torch.empty((B, h, n_q), device=DEV) if stats else None
    Z = mha.attn_core(*dev, scale=c, causal=causal,
                      key_len=None if key_len is None else torch.from_numpy(key_len).to(DEV),
                      out_dtype=torch.float32, row_m=rm, row_l=rl)
    torch.cuda.synchronize()
    allow = allowed_set(B, n_q, n_k, causal=causal, key_len=key_len)
    ref = attn_core_ref(*host, c, allow)
    err = _rel_err(Z.cpu().numpy(), ref["Z"])
    # twice the error of a float64 model of the heads' type's roundings
    # (tests/rounding_model.py); bf16 heads also within the 2e-2 bar
    bar = core_bar(*host, c, allow, ref["Z"], elem=dt)
    if dt == "bf16":
        bar = min(bar, TOL["bf16"])
    _say(f"  Z err {err:.3e} (bar {bar:.2e})")
    assert err <= bar
    if stats:
        np.testing.assert_allclose(rm.cpu().numpy(), ref["m"], rtol=1e-3, atol=1e-3)
        np.testing.assert_allclose(rl.cpu().numpy(), ref["l"], rtol=1e-2)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_backward_core(case):
    dt, B, h, n_q, n_k, d_h, d_vh, causal, kl, z_in_heads_type = case
    zdt = dt if z_in_heads_type else "f32"
    _say(f"[random backward] {case} z={zdt}")
    Qh, Kh, Vh = make_heads(B, h, n_q, n_k, d_h, d_vh, "f32", seed=700 + n_q + n_k)
    dZ = np.random.default_rng(701 + n_k).standard_normal((B, n_q, h * d_vh)).astype(np.float32)
    c = 1.0 / math.sqrt(d_h)
    key_len = None if kl is None else np.array(kl, dtype=np.int32)
    grads, host, dZh = _bwd_run(dt, zdt, Qh, Kh, Vh, dZ, c, causal, key_len)
    ref = attn_core_grad_ref(*host, c, allowed_set(B, n_q, n_k, causal=causal, key_len=key_len),
                             dZh)
    scale = float(np.abs(ref["dVh"]).max())
    for name, got in zip(("dQh", "dKh", "dVh"), grads):
        r = np.asarray(ref[name], np.float64)
        if float(np.abs(r).max()) <= 1e-9 * scale:
            # every row has a single allowed key: its weights do not depend on
            # Q or K, so dQ = dK = 0 up to the rounding of dA - D
            assert float(np.abs(np.asarray(got, np.float64)).max()) <= 1e-3 * scale, name
            continue
        fro, mx = _grad_err(got, r)
        _say(f"  {name} normwise {fro:.3e} max {mx:.3e}")
        assert fro <= BWD_TOL[dt][0] and mx <= BWD_TOL[dt][1], name


def _draw_masked(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ("f16", "bf16")[i % 2]
        kind = ("bool", "additive")[(i // 2) % 2]
        d_h = d_vh = int(rng.choice([32, 64, 128]))
        if i % 4 == 3:
            d_vh = int(rng.choice([32, 64, 96, 128]))
        B, h = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        mult = 16 if i % 3 != 2 else 4          # mask tile through LDS, or 4-byte loads
        n_q = int(rng.integers(1, 400))
        n_k = int(rng.integers(1, 400 // mult + 1)) * mult
        causal = bool(rng.integers(0, 2))
        if causal:
            n_q = n_k
        kl = tuple(int(v) for v in rng.integers(1, n_k + 1, size=B)) if rng.integers(0, 2) else None
        shared = bool(rng.integers(0, 2))
        density = float(rng.choice([0.1, 0.5, 0.9]))
        cases.append((dt, kind, B, h, n_q, n_k, d_h, d_vh, causal, kl, shared, density))
    return cases


MASK_CASES = _draw_masked(999, 14)


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_masked_core(case):
    """Random boolean masks and additive biases ([B or 1, n_q, n_k]) on top of
    random causal / padding rules; every row keeps one allowed key."""
    dt, kind, B, h, n_q, n_k, d_h, d_vh, causal, kl, shared, density = case
    _say(f"[random masked] {case}")
    Qh, Kh, Vh = make_heads(B, h, n_q, n_k, d_h, d_vh, "f32" if dt == "f16" else dt,
                            seed=900 + n_q + n_k)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    dev = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(tdt) for a in (Qh, Kh, Vh)]
    host = [t.float().cpu().numpy().astype(np.float64) for t in dev]
    rng = np.random.default_rng(901 + n_k)
    key_len = None if kl is None else np.array(kl, dtype=np.int32)
    Bm = 1 if shared else B
    ok = rng.random((Bm, n_q, n_k)) < density
    for bm in range(Bm):
        L = n_k if key_len is None else int(key_len.min() if shared else key_len[bm])
        for i in range(n_q):
            top = min(i if causal else n_k - 1, L - 1)
            ok[bm, i, int(rng.integers(0, top + 1))] = True
    G = M = None
    if kind == "bool":
        G = ok
    else:
        M = np.where(ok, rng.normal(size=ok.shape) * 2.0, -np.inf).astype(np.float32)
    c = 1.0 / math.sqrt(d_h)
    Z = mha.attn_core(*dev, scale=c, causal=causal,
                      key_len=None if key_len is None else torch.from_numpy(key_len).to(DEV),
                      allowed=None if G is None else torch.from_numpy(G).to(DEV),
                      add=None if M is None else torch.from_numpy(M).to(DEV),
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    allow = allowed_set(B, n_q, n_k, causal=causal, key_len=key_len, allowed=G)
    ref = attn_core_ref(*host, c, allow, add=M)
    err = _rel_err(Z.cpu().numpy(), ref["Z"])
    bar = core_bar(*host, c, allow, ref["Z"], elem=dt, add=M)
    if dt == "bf16":
        bar = min(bar, TOL["bf16"])
    _say(f"  Z err {err:.3e} (bar {bar:.2e})")
    assert err <= bar
