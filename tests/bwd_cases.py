"""Cases of the attention-core backward tests and their seeded inputs.

Shared by the GPU parity test (tests/test_gpu_parity.py) and the CPU test
that sets the gradient bars from the backward's rounding model
(tests/test_kernel_emulations.py); only draws numbers.
"""

from __future__ import annotations

import math

import numpy as np

from transformer_head_self_amd.inputs import make_heads

BWD_CASES = [
    # dtype, grad dtype, B, h, n_q, n_k, d_h, d_vh, causal, key_len, bool, additive
    ("bf16", "f32", 2, 3, 100, 333, 64, 64, False, None, False, False),
    ("f16", "f32", 2, 2, 200, 200, 64, 64, True, None, False, False),
    ("bf16", "bf16", 2, 2, 130, 257, 64, 96, False, (257, 100), False, False),
    ("f16", "f32", 1, 2, 300, 300, 128, 128, True, (300,), False, False),
    ("f16", "f16", 3, 2, 65, 65, 40, 24, True, (65, 10, 1), False, False),
    ("bf16", "f32", 2, 2, 96, 160, 32, 32, False, None, True, False),
    ("f16", "f32", 2, 2, 150, 150, 64, 64, True, None, False, True),
    ("f16", "f32", 2, 2, 1, 700, 64, 64, False, (700, 300), False, False),
    # dZ in the heads' type, n_q a multiple of 4: the direct-load dK/dV kernel
    # (ragged query and key tiles, causal, padding, both widths, 4 rows)
    ("f16", "f16", 2, 3, 100, 333, 64, 64, False, None, False, False),
    ("bf16", "bf16", 2, 2, 200, 200, 64, 64, True, (200, 77), False, False),
    ("f16", "f16", 1, 2, 300, 300, 128, 128, True, (300,), False, False),
    ("f16", "f16", 2, 2, 4, 700, 64, 64, False, (700, 300), False, False),
    ("bf16", "bf16", 2, 2, 132, 90, 128, 128, False, (90, 45), False, False),
]


def additive_bias(rng, Bm, n_q, n_k, frac_forbidden=0.1):
    """An additive score bias M [Bm, n_q, n_k]: N(0, 4) entries, a fraction
    set to -inf (forbidden), key 0 always finite."""
    M = rng.normal(size=(Bm, n_q, n_k)) * 2.0
    M[rng.random(M.shape) < frac_forbidden] = -np.inf
    M[:, :, 0] = rng.normal(size=(Bm, n_q))  # key 0 stays allowed in every row
    return M.astype(np.float32)


def bwd_case_inputs(case):
    """(Qh, Kh, Vh, dZ) as float32 draws (rounded to the case's types where
    they are used), key_len, the boolean mask G, the additive bias M and c."""
    dt, zdt, B, h, n_q, n_k, d_h, d_vh, causal, kl, use_bool, use_add = case
    Qh, Kh, Vh = make_heads(B, h, n_q, n_k, d_h, d_vh, "f32", seed=60 + n_q + n_k)
    rng = np.random.default_rng(61 + n_k)
    dZ = rng.standard_normal((B, n_q, h * d_vh)).astype(np.float32)
    key_len = None if kl is None else np.array(kl[:B], dtype=np.int32)
    G = None
    if use_bool:
        G = rng.random((B, n_q, n_k)) < 0.5
        G[:, :, 0] = True
    M = additive_bias(rng, B, n_q, n_k) if use_add else None
    return Qh, Kh, Vh, dZ, key_len, G, M, 1.0 / math.sqrt(d_h)
