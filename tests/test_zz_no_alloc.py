"""GPU test of attn_core_split_noalloc, the key-split attention entry point
that allocates nothing (its partitions' summaries live in a static scratch
array the library holds on each GPU).  It is compared, through the C ABI,
with attn_core_split on the same inputs and the same partition count: the
two run the same kernels, so every output must agree bit for bit.  Two calls
in a row, the second on a smaller problem (the scratch still holds the first
call's summaries), and the oracle as a third opinion on each.
"""

import ctypes
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import transformer_head_self_amd as mha  # noqa: E402
from transformer_head_self_amd.inputs import make_heads  # noqa: E402
from oracle import allowed_set, attn_core_ref  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rel_err(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(out - ref))) / math.sqrt(float(np.mean(ref * ref)))


def _case(B, h, n_q, n_k, d_h, d_vh, splits, key_len, seed):
    """One call of each entry point on the same fp16 heads; returns both
    outputs, the row statistics and the oracle's Z."""
    _say(f"[noalloc] B={B} h={h} n_q={n_q} n_k={n_k} d_h={d_h} d_vh={d_vh} splits={splits}")
    Qh, Kh, Vh = make_heads(B, h, n_q, n_k, d_h, d_vh, "f32", seed=seed)
    dev = [torch.from_numpy(a).to(DEV).half() for a in (Qh, Kh, Vh)]
    host = [t.float().cpu().numpy().astype(np.float64) for t in dev]
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device=DEV)
    c = 1.0 / math.sqrt(d_h)
    outs = []
    for fn in (mha.attn_core_split_noalloc, mha.attn_core_split):
        Z = torch.full((B, n_q, h * d_vh), float("nan"), dtype=torch.float32, device=DEV)
        rm = torch.full((B, h, n_q), float("nan"), device=DEV)
        rl = torch.full_like(rm, float("nan"))
        fn(*dev, splits=splits, scale=c, key_len=kl, Z=Z, row_m=rm, row_l=rl)
        torch.cuda.synchronize()
        outs.append((Z.cpu().numpy(), rm.cpu().numpy(), rl.cpu().numpy()))
    ref = attn_core_ref(*host, c, allowed_set(B, n_q, n_k, key_len=None if key_len is None
                                                else np.array(key_len, np.int32)))["Z"]
    return outs, ref


def _check(outs, ref):
    (Za, ma, la), (Zb, mb, lb) = outs
    np.testing.assert_array_equal(Za, Zb)
    np.testing.assert_array_equal(ma, mb)
    np.testing.assert_array_equal(la, lb)
    err = _rel_err(Za, ref)
    _say(f"  identical to attn_core_split; Z err vs oracle {err:.3e}")
    assert err <= 1e-2   # fp16 heads and weights, fp32 accumulation


def test_noalloc_matches_split_twice_then_smaller():
    # first call: a decode step (one query row) against 8192 ragged keys
    outs, ref = _case(8, 16, 1, 8192, 64, 64, 0, [8192, 5000, 1, 64, 8000, 4097, 100, 7777], 60)
    _check(outs, ref)
    # second call, smaller, on the same scratch: the matrix-core split form
    outs, ref = _case(2, 3, 150, 700, 64, 32, 3, [700, 333], 61)
    _check(outs, ref)
    # third call, smaller still: the decode kernel with four query rows
    outs, ref = _case(1, 2, 4, 300, 32, 64, 2, None, 62)
    _check(outs, ref)


def test_noalloc_rejects_requests_beyond_its_scratch():
    """A plan whose summaries exceed MHA_STATIC_SCRATCH_BYTES is refused on
    the host with MHA_ERR_SCRATCH (nothing launched, Z untouched)."""
    B, h, n_q, n_k, d = 4, 16, 512, 65536, 128
    dims = mha.MhaDims(B=B, h=h, n_q=n_q, n_k=n_k, d_q=1, d_k=1, d_v=1, d_h=d, d_vh=d, d_o=1,
                       scale=0.1, in_dtype=mha.MHA_F16, out_dtype=mha.MHA_F32,
                       work_dtype=mha.MHA_F16)
    assert mha.attn_split_workspace_bytes(dims, 64) > mha.MHA_STATIC_SCRATCH_BYTES
    q = torch.zeros(16, dtype=torch.float16, device=DEV)   # never read
    Z = torch.full((4,), 7.0, device=DEV)
    L = mha.lib()
    st = L.attn_core_split_noalloc(ctypes.byref(dims), None, q.data_ptr(), q.data_ptr(),
                                   q.data_ptr(), Z.data_ptr(), None, None, 64, None)
    assert st == mha.MHA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(Z == 7.0)
