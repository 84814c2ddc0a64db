"""Seeded synthetic inputs for the multi-head attention forward workloads.

This module only draws numbers: it holds none of the attention arithmetic,
and both the HIP path's callers and the CPU oracle's callers take their
inputs from here.

Every value is drawn in float64 from ``numpy.random.default_rng(seed)`` in a
fixed order (inputs, then W_Q, W_K, W_V, W_O, then per-item key lengths) and
rounded once to the workload's element type:
* "f32": numpy's round-to-nearest-even float64 -> float32 cast;
* "bf16": the float32 value rounded to bfloat16 with round-to-nearest-even
  on its bit pattern; the result is returned as float32 holding a value that
  bfloat16 represents exactly, so converting it to bfloat16 (device side) or
  to float64 (oracle side) is lossless.

Inputs are N(0, 1); each weight matrix is N(0, 1/fan_in) with fan_in its row
count.  Key lengths for padding masks are integers drawn uniformly from an
inclusive range.
"""

from __future__ import annotations

import dataclasses

import numpy as np


def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _cast(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return round_to_bf16(x32)
    raise ValueError(dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Dimensions and mask of one multi-head attention problem.

    Names follow the general definition: n_q queries of width d_q, n_k keys of
    width d_k and values of width d_v, h heads of query/key width d_h and
    value width d_vh, output width d_o.
    """
    name: str
    kind: str           # "self" (Q = K = V = X) or "cross"
    dtype: str          # "f32" or "bf16" element type of inputs and weights
    B: int
    n_q: int
    n_k: int
    d_q: int
    d_k: int
    d_v: int
    h: int
    d_h: int
    d_vh: int
    d_o: int
    causal: bool = False
    pad_range: tuple | None = None   # inclusive (lo, hi) for key lengths
    seed: int = 0

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.d_h))

    def core_flops(self, key_len=None):
        """2*B*h*n_q*n_k*(d_h+d_vh), halved for causal (nominal count)."""
        f = 2.0 * self.B * self.h * self.n_q * self.n_k * (self.d_h + self.d_vh)
        return f / 2 if self.causal else f

    def core_flops_effective(self, key_len):
        """Same count with each item's key count replaced by its valid length."""
        if key_len is None:
            return self.core_flops()
        f = 2.0 * self.h * self.n_q * float(np.sum(key_len)) * (self.d_h + self.d_vh)
        return f / 2 if self.causal else f

    def proj_flops(self):
        q = 2.0 * self.B * self.n_q * self.d_q * self.h * self.d_h
        k = 2.0 * self.B * self.n_k * self.d_k * self.h * self.d_h
        v = 2.0 * self.B * self.n_k * self.d_v * self.h * self.d_vh
        o = 2.0 * self.B * self.n_q * self.h * self.d_vh * self.d_o
        return q + k + v + o


def _self(name, dtype, B, T, d_model, h, d, causal, pad_range, seed):
    return Workload(name=name, kind="self", dtype=dtype, B=B, n_q=T, n_k=T,
                    d_q=d_model, d_k=d_model, d_v=d_model, h=h, d_h=d, d_vh=d,
                    d_o=d_model, causal=causal, pad_range=pad_range, seed=seed)


WORKLOADS = {
    w.name: w for w in [
        _self("self-f32-B2-T64-dm64-h4-dh16-causal", "f32", 2, 64, 64, 4, 16,
              True, None, 1),
        _self("self-f32-B8-T512-dm512-h8-dh64-keypad", "f32", 8, 512, 512, 8, 64,
              False, (128, 512), 2),
        _self("self-bf16-B4-T4096-dm1024-h16-dh64-causal", "bf16", 4, 4096, 1024, 16, 64,
              True, None, 3),
        _self("self-bf16-B1-T16384-dm2048-h16-dh128-causal", "bf16", 1, 16384, 2048, 16, 128,
              True, None, 4),
        Workload(name="cross-bf16-B16-nq512-nk2048-h12-dh64-dvh96-keypad", kind="cross",
                 dtype="bf16", B=16, n_q=512, n_k=2048, d_q=768, d_k=512, d_v=640,
                 h=12, d_h=64, d_vh=96, d_o=768, causal=False, pad_range=(256, 2048),
                 seed=5),
    ]
}

# The headline workload: bf16, T=4096, h=16, d_h=64, causal.
HEADLINE = "self-bf16-B4-T4096-dm1024-h16-dh64-causal"


def make_inputs(w: Workload, seed=None, with_weights=True):
    """Draw the inputs of workload ``w``.  Returns a dict of numpy arrays.

    Keys: Q, K, V (the same array object for self-attention), W_Q, W_K, W_V,
    W_O, key_len (int32 [B] or None).  Floating arrays are float32 holding
    values exact in ``w.dtype``.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.kind == "self":
        X = _cast(rng.standard_normal((w.B, w.n_q, w.d_q)), w.dtype)
        Q = K = V = X
    else:
        Q = _cast(rng.standard_normal((w.B, w.n_q, w.d_q)), w.dtype)
        K = _cast(rng.standard_normal((w.B, w.n_k, w.d_k)), w.dtype)
        V = _cast(rng.standard_normal((w.B, w.n_k, w.d_v)), w.dtype)
    out = {"Q": Q, "K": K, "V": V}
    if with_weights:
        def W(rows, cols):
            return _cast(rng.standard_normal((rows, cols)) / np.sqrt(rows), w.dtype)
        out["W_Q"] = W(w.d_q, w.h * w.d_h)
        out["W_K"] = W(w.d_k, w.h * w.d_h)
        out["W_V"] = W(w.d_v, w.h * w.d_vh)
        out["W_O"] = W(w.h * w.d_vh, w.d_o)
    if w.pad_range is not None:
        lo, hi = w.pad_range
        out["key_len"] = rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)
    else:
        out["key_len"] = None
    return out


def make_heads(B, h, n_q, n_k, d_h, d_vh, dtype, seed, scale_q=1.0):
    """Already-projected heads Qh [B,h,n_q,d_h], Kh [B,h,n_k,d_h], Vh [B,h,n_k,d_vh]."""
    rng = np.random.default_rng(seed)
    Qh = _cast(rng.standard_normal((B, h, n_q, d_h)) * scale_q, dtype)
    Kh = _cast(rng.standard_normal((B, h, n_k, d_h)), dtype)
    Vh = _cast(rng.standard_normal((B, h, n_k, d_vh)), dtype)
    return Qh, Kh, Vh


def custom_workload(name="custom", kind="self", dtype="f32", B=1, n_q=8, n_k=8,
                    d_q=8, d_k=8, d_v=8, h=1, d_h=8, d_vh=8, d_o=8, causal=False,
                    pad_range=None, seed=0):
    return Workload(name=name, kind=kind, dtype=dtype, B=B, n_q=n_q, n_k=n_k,
                    d_q=d_q, d_k=d_k, d_v=d_v, h=h, d_h=d_h, d_vh=d_vh, d_o=d_o,
                    causal=causal, pad_range=pad_range, seed=seed)
