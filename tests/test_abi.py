"""CPU tests of the C ABI: the library loads, exports what include/mha.h
declares, lays out its structs as the binding does, and rejects every
host-checkable violation before touching the GPU (no kernel is launched in
these tests: each call fails validation first).
"""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import transformer_head_self_amd as mha
from transformer_head_self_amd import MhaDims, MhaMask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")

FAKE = 0x10000  # a non-null, 256-byte aligned address; never dereferenced here


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("mha_forward", "attn_core", "mha_workspace_bytes", "mha_status_string",
              "mha_max_head_dim"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = mha.lib()
    for name in _declared_functions():
        assert hasattr(L, name), f"libmha.so does not export {name}"
    out = subprocess.run(["nm", "-D", "--defined-only", mha.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported


def test_struct_layout_matches_header():
    """Compile a tiny C program against the header and compare with ctypes."""
    prog = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "mha.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(mha_dims),
             offsetof(mha_dims, scale), offsetof(mha_dims, out_dtype),
             offsetof(mha_dims, work_dtype), sizeof(mha_mask), offsetof(mha_mask, key_len),
             offsetof(mha_mask, allowed_batch_stride), offsetof(mha_mask, add),
             offsetof(mha_mask, add_batch_stride), sizeof(mha_bias), offsetof(mha_bias, b_O));
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert vals == [ctypes.sizeof(MhaDims), MhaDims.scale.offset, MhaDims.out_dtype.offset,
                    MhaDims.work_dtype.offset, ctypes.sizeof(MhaMask), MhaMask.key_len.offset,
                    MhaMask.allowed_batch_stride.offset, MhaMask.add.offset,
                    MhaMask.add_batch_stride.offset, ctypes.sizeof(mha.MhaBias),
                    mha.MhaBias.b_O.offset]


def _dims(**kw):
    base = dict(B=2, h=4, n_q=64, n_k=64, d_q=64, d_k=64, d_v=64, d_h=16, d_vh=16, d_o=64,
                scale=0.25, in_dtype=mha.MHA_F32, out_dtype=mha.MHA_F32, work_dtype=mha.MHA_F32)
    base.update(kw)
    return MhaDims(**base)


def _fwd(d, m=None, ptrs=None, ws_bytes=1 << 30, ws=FAKE, bias=None):
    L = mha.lib()
    p = [FAKE] * 8 if ptrs is None else ptrs
    mp = ctypes.byref(m) if m is not None else None
    bp = ctypes.byref(bias) if bias is not None else None
    return L.mha_forward(ctypes.byref(d) if d is not None else None, mp, *p[:7], bp, p[7], None,
                         None, ws, ws_bytes, None)


def _core(d, m=None, ptrs=None):
    L = mha.lib()
    p = [FAKE] * 4 if ptrs is None else ptrs
    mp = ctypes.byref(m) if m is not None else None
    return L.attn_core(ctypes.byref(d) if d is not None else None, mp, *p, None, None, None)


def test_status_strings():
    for code in range(0, -10, -1):
        s = mha.mha_status_string(code)
        assert s.startswith("MHA_")
    assert "unknown" in mha.mha_status_string(-99)


@pytest.mark.parametrize("field", ["B", "h", "n_q", "n_k", "d_q", "d_k", "d_v", "d_h", "d_vh",
                                   "d_o"])
def test_nonpositive_dims_rejected(field):
    d = _dims(**{field: 0})
    assert _fwd(d) == -2
    if field in ("B", "h", "n_q", "n_k", "d_h", "d_vh"):
        assert _core(_dims(**{field: -3})) == -2


def test_overflowing_dims_rejected():
    assert _fwd(_dims(B=1 << 16, n_q=1 << 16, n_k=1 << 16)) == -2


def test_null_dims_and_pointers():
    assert _fwd(None) == -1
    assert _core(None) == -1
    for i in range(8):
        p = [FAKE] * 8
        p[i] = None
        assert _fwd(_dims(), ptrs=p) == -1
    for i in range(4):
        p = [FAKE] * 4
        p[i] = None
        assert _core(_dims(), ptrs=p) == -1


def test_bad_dtype_and_scale():
    assert _fwd(_dims(in_dtype=7)) == -3
    assert _core(_dims(out_dtype=-1)) == -3
    # (in, work) pairs: fp32 inputs need fp32 intermediates; 2-byte inputs 2-byte ones
    assert _fwd(_dims(in_dtype=mha.MHA_F32, work_dtype=mha.MHA_F16)) == -3
    assert _fwd(_dims(in_dtype=mha.MHA_BF16, work_dtype=mha.MHA_F32)) == -3
    assert _fwd(_dims(in_dtype=mha.MHA_F16, work_dtype=mha.MHA_BF16)) == -3
    # attn_core ignores work_dtype
    assert _core(_dims(work_dtype=9, scale=float("nan"))) == -9
    assert _fwd(_dims(scale=float("inf"))) == -9
    assert _core(_dims(scale=float("nan"))) == -9


def test_head_width_above_instantiated_maximum():
    top = mha.lib().mha_max_head_dim()
    assert top >= 128
    assert _fwd(_dims(d_h=top + 1)) == -7
    assert _core(_dims(d_vh=top + 8)) == -7


def test_mask_descriptor_errors():
    m = MhaMask(flags=8)
    assert _fwd(_dims(), m) == -4
    m = MhaMask(flags=mha.MHA_MASK_CAUSAL)
    assert _fwd(_dims(n_k=65), m) == -4         # causal needs n_q == n_k
    assert _core(_dims(n_q=10, n_k=11), m) == -4
    m = MhaMask(flags=mha.MHA_MASK_KEY_PADDING)  # no key_len
    assert _fwd(_dims(), m) == -4
    m = MhaMask(flags=mha.MHA_MASK_BOOL)         # no allowed
    assert _core(_dims(), m) == -4
    m = MhaMask(flags=mha.MHA_MASK_BOOL, allowed=FAKE, allowed_batch_stride=5)
    assert _core(_dims(), m) == -4               # stride shorter than one mask plane
    m = MhaMask(flags=mha.MHA_MASK_KEY_PADDING, key_len=FAKE + 2)
    assert _core(_dims(), m) == -5               # int32 array misaligned
    m = MhaMask(flags=mha.MHA_MASK_ADDITIVE)     # no additive bias
    assert _core(_dims(), m) == -4
    m = MhaMask(flags=mha.MHA_MASK_ADDITIVE, add=FAKE, add_batch_stride=64 * 64 - 1)
    assert _fwd(_dims(), m) == -4                # stride shorter than one plane
    m = MhaMask(flags=mha.MHA_MASK_ADDITIVE, add=FAKE + 2)
    assert _core(_dims(), m) == -5               # fp32 array misaligned
    m = MhaMask(flags=mha.MHA_MASK_ADDITIVE | 16, add=FAKE)
    assert _core(_dims(), m) == -4               # unknown flag bit


def test_misaligned_pointers():
    p = [FAKE] * 8
    p[0] = FAKE + 2                              # fp32 needs 4-byte alignment
    assert _fwd(_dims(), ptrs=p) == -5
    p = [FAKE] * 8
    p[0] = FAKE + 2                              # bf16 accepts 2-byte alignment ...
    p[7] = FAKE + 2                              # ... but Y (fp32 out) does not
    assert _fwd(_dims(in_dtype=mha.MHA_BF16, work_dtype=mha.MHA_F16), ptrs=p) == -5
    q = [FAKE] * 4
    q[3] = FAKE + 1
    assert _core(_dims(), ptrs=q) == -5


def test_projection_bias_alignment():
    ok = mha.MhaBias(b_Q=FAKE, b_K=FAKE, b_V=FAKE, b_O=FAKE)
    # every check passes except the missing workspace: the biases were accepted
    assert _fwd(_dims(), bias=ok, ws=None) == -6
    for f in ("b_Q", "b_K", "b_V", "b_O"):
        b = mha.MhaBias(b_Q=FAKE, b_K=FAKE, b_V=FAKE, b_O=FAKE)
        setattr(b, f, FAKE + 2)                  # fp32 bias must be 4-byte aligned
        assert _fwd(_dims(), bias=b) == -5
    b = mha.MhaBias(b_O=FAKE + 2)                # bf16 biases need 2-byte alignment only
    assert _fwd(_dims(in_dtype=mha.MHA_BF16, work_dtype=mha.MHA_F16), bias=b, ws=None) == -6


def test_workspace_checks():
    d = _dims()
    need = mha.mha_workspace_bytes(d)
    assert need > 0
    assert _fwd(d, ws_bytes=need - 1) == -6
    assert _fwd(d, ws=None) == -6
    assert _fwd(d, ws=FAKE + 16, ws_bytes=need) == -5   # workspace must be 256-byte aligned


def test_workspace_bytes_formula_and_monotonicity():
    def r256(x):
        return (x + 255) // 256 * 256
    for dt, wt, es in ((mha.MHA_F32, mha.MHA_F32, 4), (mha.MHA_BF16, mha.MHA_F16, 2),
                       (mha.MHA_BF16, mha.MHA_BF16, 2), (mha.MHA_F16, mha.MHA_F16, 2)):
        d = _dims(B=3, h=5, n_q=37, n_k=101, d_h=24, d_vh=40, in_dtype=dt, work_dtype=wt)
        expect = (r256(3 * 5 * 37 * 24 * es) + r256(3 * 5 * 101 * 24 * es) +
                  r256(3 * 5 * 101 * 40 * es) + r256(3 * 37 * 5 * 40 * es))
        assert mha.mha_workspace_bytes(d) == expect
    base = mha.mha_workspace_bytes(_dims())
    for f in ("B", "h", "n_q", "n_k", "d_h", "d_vh"):
        bigger = _dims(**{f: getattr(_dims(), f) * 2})
        assert mha.mha_workspace_bytes(bigger) > base
    assert mha.mha_workspace_bytes(_dims(B=0)) == 0


# ---- key-split form -------------------------------------------------------

def _split(d, m=None, ptrs=None, splits=0, ws=FAKE, ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else [FAKE] * 4
    return mha.lib().attn_core_split(
        ctypes.byref(d) if d is not None else None, ctypes.byref(m) if m is not None else None,
        p[0], p[1], p[2], p[3], None, None, splits, ws, ws_bytes, None)


def _split_layout(d, splits):
    """Partitions and workspace bytes the header specifies for explicit splits."""
    P = -(-d.n_k // splits)
    P = -(-P // 64) * 64
    S = -(-d.n_k // P)
    rows = d.B * d.h * d.n_q

    def r256(x):
        return (x + 255) // 256 * 256
    return S, 2 * r256(S * rows * 4) + r256(S * rows * d.d_vh * 4)


def test_split_workspace_bytes_explicit():
    for B, h, n_q, n_k, d_vh, splits in ((1, 16, 1, 4096, 64, 8), (2, 3, 5, 1000, 40, 7),
                                         (1, 1, 1, 65, 8, 100), (3, 2, 9, 64, 64, 1),
                                         (1, 2, 3, 130, 128, 2)):
        d = _dims(B=B, h=h, n_q=n_q, n_k=n_k, d_vh=d_vh)
        S, need = _split_layout(d, splits)
        assert 1 <= S <= splits
        assert mha.attn_split_workspace_bytes(d, splits) == need
    # 65 keys asked in 100 partitions: whole 64-key blocks, so two partitions
    assert _split_layout(_dims(n_k=65), 100)[0] == 2


def test_split_workspace_bytes_auto_is_one_of_the_explicit_layouts():
    for B, h, n_q, n_k in ((1, 16, 1, 8192), (4, 16, 4096, 4096), (1, 1, 1, 100), (8, 8, 2, 300)):
        d = _dims(B=B, h=h, n_q=n_q, n_k=n_k)
        auto = mha.attn_split_workspace_bytes(d, 0)
        options = {_split_layout(d, s)[1] for s in range(1, -(-n_k // 64) + 1)}
        assert auto in options
    # many query tiles already fill the chip: no split
    d = _dims(B=4, h=16, n_q=4096, n_k=4096)
    assert mha.attn_split_workspace_bytes(d, 0) == _split_layout(d, 1)[1]
    # one query row against 8192 keys: many partitions of >= 256 keys
    d = _dims(B=1, h=16, n_q=1, n_k=8192)
    assert mha.attn_split_workspace_bytes(d, 0) == _split_layout(d, 32)[1]


def test_split_argument_errors():
    d = _dims()
    need = mha.attn_split_workspace_bytes(d, 4)
    assert need > 0
    assert mha.attn_split_workspace_bytes(d, -1) == 0
    assert mha.attn_split_workspace_bytes(None, 1) == 0
    assert _split(d, splits=-1) == -2
    assert _split(None) == -1
    for i in range(4):
        p = [FAKE] * 4
        p[i] = None
        assert _split(d, ptrs=p) == -1
    assert _split(d, splits=4, ws_bytes=need - 1) == -6
    assert _split(d, splits=4, ws=None) == -6
    assert _split(d, splits=4, ws=FAKE + 64, ws_bytes=need) == -5
    assert _split(_dims(d_vh=mha.lib().mha_max_head_dim() + 1)) == -7
    assert _split(_dims(scale=float("inf"))) == -9
    assert _split(_dims(n_q=3, n_k=4), MhaMask(flags=mha.MHA_MASK_CAUSAL)) == -4
    # partition rows beyond 32-bit indexing
    big = _dims(B=1, h=1, n_q=1 << 16, n_k=1 << 22)
    assert mha.attn_split_workspace_bytes(big, 1 << 16) == 0
    assert _split(big, splits=1 << 16) == -2


# ---- backward of the attention core -----------------------------------------

def _bwd(d, m=None, ptrs=None, ws=FAKE, ws_bytes=1 << 30):
    p = [FAKE] * 10 if ptrs is None else ptrs
    return mha.lib().attn_core_backward(
        ctypes.byref(d) if d is not None else None, ctypes.byref(m) if m is not None else None,
        *p, ws, ws_bytes, None)


def test_backward_workspace_and_errors():
    d = _dims(in_dtype=mha.MHA_BF16, out_dtype=mha.MHA_BF16, B=3, h=5, n_q=37)
    need = mha.attn_backward_workspace_bytes(d)
    assert need == 2 * ((3 * 5 * 37 * 4 + 255) // 256 * 256)
    assert mha.attn_backward_workspace_bytes(None) == 0
    assert _bwd(None) == -1
    assert _bwd(_dims(), ws=None) == -6              # fp32 heads pass the type checks
    for i in range(10):
        p = [FAKE] * 10
        p[i] = None
        assert _bwd(d, ptrs=p) == -1                 # row_m and row_l are required
    p = [FAKE] * 10
    p[4] = FAKE + 1                                  # dZ misaligned for bf16
    assert _bwd(d, ptrs=p) == -5
    assert _bwd(d, ws_bytes=need - 1) == -6
    assert _bwd(d, ws=None) == -6
    assert _bwd(d, ws=FAKE + 128, ws_bytes=need) == -5
    assert _bwd(d, MhaMask(flags=mha.MHA_MASK_CAUSAL)) == -4   # n_q != n_k
    assert _bwd(_dims(in_dtype=mha.MHA_F16, out_dtype=mha.MHA_F32, d_h=200)) == -7


def _bias_bwd(d, m, ptrs=None, dM=FAKE, ws=FAKE, ws_bytes=1 << 30):
    p = [FAKE] * 7 if ptrs is None else ptrs
    return mha.lib().attn_bias_backward(
        ctypes.byref(d) if d is not None else None, ctypes.byref(m) if m is not None else None,
        *p, dM, ws, ws_bytes, None)


def test_bias_backward_errors():
    d = _dims(in_dtype=mha.MHA_BF16, out_dtype=mha.MHA_BF16, B=3, h=5, n_q=37)
    add = MhaMask(flags=mha.MHA_MASK_ADDITIVE, add=FAKE, add_batch_stride=0)
    assert _bias_bwd(None, add) == -1
    assert _bias_bwd(d, None) == -4                  # the additive bias is required
    assert _bias_bwd(d, MhaMask(flags=0)) == -4
    for i in range(7):
        p = [FAKE] * 7
        p[i] = None
        assert _bias_bwd(d, add, ptrs=p) == -1
    assert _bias_bwd(d, add, dM=None) == -1
    assert _bias_bwd(d, add, dM=FAKE + 2) == -5      # fp32 output
    assert _bias_bwd(d, add, ws=None) == -6
    assert _bias_bwd(d, MhaMask(flags=mha.MHA_MASK_ADDITIVE, add=FAKE, add_batch_stride=5)) == -4
    assert _bias_bwd(_dims(), add, ws=None) == -6    # fp32 heads too


def test_layer_backward_workspace_and_errors():
    d = _dims(in_dtype=mha.MHA_BF16, work_dtype=mha.MHA_F16, out_dtype=mha.MHA_F32)
    need = mha.mha_backward_workspace_bytes(d)
    assert need > 0
    assert mha.mha_backward_workspace_bytes(_dims(B=0)) == 0
    L = mha.lib()
    fwd = mha.mha_workspace_bytes(d)

    def call(dd, ptrs=None, fws=FAKE, fwb=fwd, ws=FAKE, wsb=need):
        p = [FAKE] * 10 if ptrs is None else ptrs
        return L.mha_backward(ctypes.byref(dd) if dd is not None else None, None, *p, fws, fwb,
                              *([FAKE] * 7), None, ws, wsb, None)
    assert call(None) == -1
    assert call(_dims(), wsb=0) == -6                  # fp32 intermediates pass the type checks
    for i in range(10):
        p = [FAKE] * 10
        p[i] = None
        assert call(d, ptrs=p) == -1
    assert call(d, fws=None) == -1
    assert call(d, fwb=fwd - 1) == -6
    assert call(d, wsb=need - 1) == -6
    assert call(d, ws=FAKE + 16) == -5
