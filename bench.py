"""Benchmark: multi-head attention forward on one MI355X.

One "step" is one full forward pass (Q/K/V projections, fused masked
attention with running summaries, concatenation, W^O projection) over one
batch of the headline workload: self-attention, bf16 inputs with fp32
accumulation, B=4, T=4096, d_model=1024, h=16, d_h=d_vh=64, causal mask.
Inputs are seeded synthetic draws already resident in HBM when timing starts.

Printed JSON line (rank 0):
* value: whole-forward TFLOP/s, counting 2*B*h*n_q*n_k*(d_h+d_vh) (halved
  for causal) for the attention core plus 2*M*N*K for each projection GEMM;
* roofline: the attention-core kernel (dominant kernel) timed with HIP
  events around its own launches on the stream it runs on, against the
  bf16 dense matrix-core peak;
* cpu_baseline: the float64 CPU oracle on a bounded sample (one batch item)
  of the same workload, in the same unit; that leg also compares the timed
  output's rows of that item with the oracle's (``parity``);
* ms_median / ms_min: per-step times from events around every timed step;
* settled: the same forward timed again after about 0.2 s of back-to-back
  steps, then the attention kernel alone (the GPU clock rises over the
  first milliseconds of sustained load; ``value`` and ``roofline`` keep the
  requested warm-up and steps).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MHA fwd TFLOP/s and % bf16 MFMA peak (T=4096, h=16, d_k=64, causal)"
# sources that define the attention kernel; a traffic measurement is only
# reported while their hash matches the one recorded with it
ATTN_SOURCES = ["transformer_head_self_amd/csrc/attn.hpp", "transformer_head_self_amd/csrc/attn_pipe.hpp",
                "transformer_head_self_amd/csrc/attn_pipe3.hpp",
                "transformer_head_self_amd/csrc/attn_launch.hpp", "transformer_head_self_amd/csrc/common.hpp",
                "transformer_head_self_amd/csrc/internal.hpp", "transformer_head_self_amd/csrc/lds_dma.hpp"]


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense matrix-core peaks
HBM_PEAK_GBS = 8000.0
# Exponential (v_exp_f32) peak: 256 CUs x 4 SIMDs x 8 results per cycle (a
# wave64 exponential occupies its SIMD for 8 cycles: SQ_ACTIVE_INST_VALU of the
# attention kernel accounts for 32 exponentials per block at 8 cycles and the
# other VALU instructions at 4) x 2.4 GHz.
EXP_PEAK_T_PER_S = 256 * 4 * 8 * 2.4e9 / 1e12


def core_kernel_name(w):
    """The attention kernel the library's launcher picks for this workload's
    forward (fp16 heads for bf16 inputs, no row statistics requested)."""
    if w.dtype != "bf16":
        return "attn_fwd_kernel (attention core)"
    dh = next(d for d in (32, 64, 128) if w.d_h <= d)
    dv = next(d for d in (32, 64, 96, 128) if w.d_vh <= d)
    fast = dh == w.d_h and dv == w.d_vh
    if fast and dh in (64, 128) and dv in (64, 128) and 128 in (dh, dv):
        return "attn_pipe_kernel, eight waves (attention core)"
    if fast and (dv >= 96 or dh >= 128):
        return "attn_pipe_kernel (attention core)"
    if fast and dh == 64 and dv == 64 and not w.causal:
        return "attn_fwd3_kernel (attention core)"
    return "attn_fwd_kernel (attention core)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The default warm-up (about 0.1 s of GPU work at the headline size) lets
    # the GPU clock settle under sustained load: with 5 warm-up steps the
    # timed steps ran ~16 % slower than in steady state (measured).
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "forward", "core"], default="all",
                    help="profiling aid: time only the whole forward or only the attention core")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="profiling aid: run a plain device-to-device copy of this many bytes "
                         "(three times) and exit; calibrates the HBM byte counters")
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the hash of the attention kernel sources and exit")
    ap.add_argument("--decode", action="store_true",
                    help="time the key-split attention core on a decode step instead "
                         "(one query row per item and head against 32768 cached keys)")
    ap.add_argument("--backward", action="store_true",
                    help="time the attention-core backward pass on the headline shape instead")
    ap.add_argument("--mask", choices=["bool", "additive"], default=None,
                    help="time the attention core on the headline shape with the causal rule "
                         "also given as a boolean mask [B, T, T] or an additive bias (0 / -inf) "
                         "instead, next to the causal flag alone")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters (optional)")
    return ap.parse_args()


def workspace_views(ws, w, torch, work):
    """Qh, Kh, Vh inside the forward's workspace (layout documented in mha.h)."""
    es = work.itemsize
    dt = work

    def r256(x):
        return (x + 255) // 256 * 256
    sizes = [w.B * w.h * w.n_q * w.d_h, w.B * w.h * w.n_k * w.d_h, w.B * w.h * w.n_k * w.d_vh]
    shapes = [(w.B, w.h, w.n_q, w.d_h), (w.B, w.h, w.n_k, w.d_h), (w.B, w.h, w.n_k, w.d_vh)]
    out, off = [], 0
    for n, shp in zip(sizes, shapes):
        out.append(ws[off:off + n * es].view(dt).view(shp))
        off += r256(n * es)
    return out


def cpu_baseline(w, x, Y_gpu):
    """Time the float64 oracle on one batch item of the workload, and compare
    the timed forward's output rows of that item with it."""
    import numpy as np
    from oracle import allowed_set, mha_ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    sub = {k: x[k][:1].astype(np.float64) for k in ("Q", "K", "V")}
    kl = None if x["key_len"] is None else x["key_len"][:1]
    Ws = {k: x[k].astype(np.float64) for k in ("W_Q", "W_K", "W_V", "W_O")}
    allow = allowed_set(1, w.n_q, w.n_k, causal=w.causal, key_len=kl)
    t0 = time.perf_counter()
    ref = mha_ref(sub["Q"], sub["K"], sub["V"], Ws["W_Q"], Ws["W_K"], Ws["W_V"], Ws["W_O"], w.h,
                  w.d_h, w.d_vh, w.scale, allow)["Y"][0]
    dt = time.perf_counter() - t0
    flops = (w.core_flops_effective(kl) + w.proj_flops()) / w.B
    y = np.asarray(Y_gpu[0], dtype=np.float64)
    err = float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref * ref)))
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": int(blas_threads),
            "kind": "oracle", "seconds": dt,
            "sample": f"1 of {w.B} batch items of {w.name}: dense float64 oracle (full score "
                      f"matrix per head, no causal skipping), FLOPs counted as for the GPU"}
    parity = {"metric": "max|Y - Y_oracle| / RMS(Y_oracle)", "value": err,
              "bar": 1e-4 if w.dtype == "f32" else 2e-2,
              "rows": f"all {w.n_q} query rows of batch item 0 of the timed output"}
    return base, parity


def timed_steps(fn, steps, stream, torch):
    """Run fn `steps` times between events on `stream`: the total time of the
    region and each step's time (ms)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps, per


DECODE = dict(B=8, h=16, n_k=32768, d=64)


def decode_bench(args, torch):
    """Decode step: Qh [B,h,1,d] against a key/value cache Kh, Vh [B,h,n_k,d]
    (fp16, the projections' output type), no mask.  Bound by HBM: the cache
    is read once.  The unsplit kernel (one workgroup per item and head) is
    timed beside the split form for comparison."""
    import numpy as np
    import transformer_head_self_amd as mha
    from transformer_head_self_amd.inputs import make_heads
    B, h, n_k, d = DECODE["B"], DECODE["h"], DECODE["n_k"], DECODE["d"]
    dev = torch.device("cuda:0")
    Qh, Kh, Vh = (torch.from_numpy(a).to(dev).to(torch.float16)
                  for a in make_heads(B, h, 1, n_k, d, d, "f32", seed=50))
    Z = torch.empty((B, 1, h * d), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    dims = mha.MhaDims(B=B, h=h, n_q=1, n_k=n_k, d_q=1, d_k=1, d_v=1, d_h=d, d_vh=d, d_o=1,
                       scale=1 / math.sqrt(d), in_dtype=2, out_dtype=2, work_dtype=2)
    ws = torch.empty(mha.attn_split_workspace_bytes(dims, 0), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_split = timed(lambda: mha.attn_core_split(Qh, Kh, Vh, splits=0, out_dtype=torch.float16,
                                                 Z=Z, workspace=ws, stream=stream))
    ms_plain = timed(lambda: mha.attn_core(Qh, Kh, Vh, out_dtype=torch.float16, Z=Z,
                                           stream=stream))
    # algorithmic bytes: the cache once, the query rows, the output rows
    nbytes = B * h * n_k * 2 * d * 2 + 2 * B * h * d * 2
    gbs = nbytes / (ms_split * 1e-3) / 1e9
    print(json.dumps({
        "metric": "split-KV decode attention, HBM GB/s", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_split, 5), "higher_is_better": True, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"decode-f16-B{B}-h{h}-nq1-nk{n_k}-d{d}",
                   "splits": "auto", "workspace_bytes": int(ws.numel())},
        "roofline": {"bound": "hbm", "kernel": "attn_decode_kernel + split_merge_kernel",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": nbytes},
        "unsplit_ms": round(ms_plain, 5),
        "unsplit_gbs": round(nbytes / (ms_plain * 1e-3) / 1e9, 1),
    }), flush=True)


def mask_bench(args, torch):
    """Attention core at the headline shape (fp16 heads): causal flag alone,
    then the causal flag with the same rule as a boolean mask or an additive
    bias, which sends every key block through the mask step."""
    import transformer_head_self_amd as mha
    from transformer_head_self_amd.inputs import HEADLINE, WORKLOADS
    w = WORKLOADS[HEADLINE]
    B, h, T, d = w.B, w.h, w.n_q, w.d_h
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(11)
    Qh, Kh, Vh = (torch.randn(B, h, T, d, generator=gen).to(dev).half() for _ in range(3))
    Z = torch.empty((B, T, h * d), dtype=torch.float16, device=dev)
    tri = torch.tril(torch.ones(T, T, dtype=torch.bool, device=dev))
    G = tri.expand(B, T, T).contiguous() if args.mask == "bool" else None
    A = (torch.zeros(B, T, T, device=dev).masked_fill(~tri, float("-inf"))
         if args.mask == "additive" else None)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_flag = timed(lambda: mha.attn_core(Qh, Kh, Vh, scale=w.scale, causal=True,
                                          out_dtype=torch.float16, Z=Z, stream=stream))
    ms_mask = timed(lambda: mha.attn_core(Qh, Kh, Vh, scale=w.scale, causal=True, allowed=G,
                                          add=A, out_dtype=torch.float16, Z=Z, stream=stream))
    flops = 2.0 * B * h * T * T * (2 * d) * 0.5
    print(json.dumps({
        "metric": f"attention core with a {args.mask} mask, causal rule, TFLOP/s",
        "value": round(flops / (ms_mask * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "ms_masked": round(ms_mask, 5), "ms_causal_flag_only": round(ms_flag, 5),
        "steps": args.steps, "warmup": args.warmup, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{HEADLINE} heads, attn_core, {args.mask} mask [B, T, T]",
                   "B": B, "h": h, "n_q": T, "n_k": T, "d_h": d, "d_vh": d},
    }), flush=True)


def backward_bench(args, torch):
    import numpy as np
    """Attention-core backward on the headline shape (B=4, T=4096, h=16,
    d=64, causal), fp16 heads and fp16 Z/dZ/gradients (the forward's
    intermediate type).  FLOPs counted as 2.5 x the forward's (five products
    of n_q x n_k x d instead of two: the recomputed scores, dZ V^T, A^T dZ,
    dS K and dS^T Q), halved for causal."""
    import transformer_head_self_amd as mha
    from transformer_head_self_amd.inputs import make_heads
    B, h, T, d = 4, 16, 4096, 64
    dev = torch.device("cuda:0")
    Qh, Kh, Vh = (torch.from_numpy(a).to(dev).to(torch.float16)
                  for a in make_heads(B, h, T, T, d, d, "f32", seed=70))
    gen = torch.Generator(device="cpu").manual_seed(71)
    dZ = torch.randn(B, T, h * d, generator=gen).to(dev).half()
    Z = torch.empty((B, T, h * d), dtype=torch.float16, device=dev)
    rm = torch.empty((B, h, T), device=dev)
    rl = torch.empty_like(rm)
    stream = torch.cuda.current_stream()
    scale = 1 / math.sqrt(d)
    dims = mha.MhaDims(B=B, h=h, n_q=T, n_k=T, d_q=1, d_k=1, d_v=1, d_h=d, d_vh=d, d_o=1,
                       scale=scale, in_dtype=2, out_dtype=2, work_dtype=2)
    ws = torch.empty(mha.attn_backward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(Qh), torch.empty_like(Kh), torch.empty_like(Vh)]

    def fwd():
        mha.attn_core(Qh, Kh, Vh, scale=scale, causal=True, out_dtype=torch.float16, Z=Z,
                      row_m=rm, row_l=rl, stream=stream)

    def bwd():
        mha.attn_core_backward(Qh, Kh, Vh, Z, dZ, rm, rl, scale=scale, causal=True,
                               dQh=grads[0], dKh=grads[1], dVh=grads[2], workspace=ws,
                               stream=stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_fwd = timed(fwd)
    ms_bwd = timed(bwd)

    # the whole layer's backward on the headline workload (bf16 inputs and
    # weights, fp16 intermediates, fp32 dY and gradients)
    from transformer_head_self_amd.inputs import HEADLINE, WORKLOADS, make_inputs
    w = WORKLOADS[HEADLINE]
    x = make_inputs(w)
    put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    X = put(x["Q"])
    Wt = {k: put(x[k]) for k in ("W_Q", "W_K", "W_V", "W_O")}
    ldims = mha.MhaDims(B=w.B, h=w.h, n_q=w.n_q, n_k=w.n_k, d_q=w.d_q, d_k=w.d_k, d_v=w.d_v,
                        d_h=w.d_h, d_vh=w.d_vh, d_o=w.d_o, scale=w.scale, in_dtype=1,
                        out_dtype=0, work_dtype=2)
    fws = torch.empty(mha.mha_workspace_bytes(ldims), dtype=torch.uint8, device=dev)
    bws = torch.empty(mha.mha_backward_workspace_bytes(ldims), dtype=torch.uint8, device=dev)
    lrm = torch.empty((w.B, w.h, w.n_q), device=dev)
    lrl = torch.empty_like(lrm)
    dY = torch.randn(w.B, w.n_q, w.d_o, generator=gen).to(dev)
    mha.mha_forward(X, X, X, Wt["W_Q"], Wt["W_K"], Wt["W_V"], Wt["W_O"], w.h, w.d_h, w.d_vh,
                    scale=w.scale, causal=True, row_m=lrm, row_l=lrl, workspace=fws,
                    stream=stream)

    def layer_bwd():
        mha.mha_backward(X, X, X, Wt["W_Q"], Wt["W_K"], Wt["W_V"], Wt["W_O"], w.h, w.d_h,
                         w.d_vh, dY, lrm, lrl, fws, scale=w.scale, causal=True, workspace=bws,
                         stream=stream)

    ms_layer = timed(layer_bwd)
    layer_flops = 2.5 * w.core_flops_effective(None) + 2.0 * w.proj_flops()  # 2 products per GEMM
    fwd_flops = 2.0 * B * h * T * T * (d + d) / 2
    bwd_flops = 2.5 * fwd_flops
    peak = PEAK_TFLOPS["bf16"]
    tf = bwd_flops / (ms_bwd * 1e-3) / 1e12
    print(json.dumps({
        "metric": "attention-core backward TFLOP/s (T=4096, h=16, d=64, causal)",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_bwd, 5), "higher_is_better": True,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "attn-backward-f16-B4-T4096-h16-d64-causal",
                   "flops_per_step": bwd_flops},
        "roofline": {"bound": "mfma", "kernel": "attn_bwd_kv_dma_kernel + attn_bwd_q_dma_kernel",
                     "achieved": round(tf, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tf / peak, 4)},
        "forward_ms": round(ms_fwd, 5),
        "layer_backward": {"workload": HEADLINE, "ms": round(ms_layer, 5),
                           "tflops": round(layer_flops / (ms_layer * 1e-3) / 1e12, 3),
                           "flops": layer_flops},
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding plan is design-only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.print_source_hash:
        print(attn_source_hash())
        return
    if args.copy_bytes:
        n = args.copy_bytes // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}), flush=True)
        return

    if args.decode:
        decode_bench(args, torch)
        return
    if args.backward:
        backward_bench(args, torch)
        return
    if args.mask:
        mask_bench(args, torch)
        return

    import transformer_head_self_amd as mha
    from transformer_head_self_amd.inputs import HEADLINE, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload or HEADLINE]
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(tdt)

    Q = put(x["Q"])
    K, V = (Q, Q) if w.kind == "self" else (put(x["K"]), put(x["V"]))
    W = {k: put(x[k]) for k in ("W_Q", "W_K", "W_V", "W_O")}
    kl = None if x["key_len"] is None else torch.from_numpy(x["key_len"]).to(dev)
    Y = torch.empty((w.B, w.n_q, w.d_o), dtype=torch.float32, device=dev)
    dims = mha.MhaDims(B=w.B, h=w.h, n_q=w.n_q, n_k=w.n_k, d_q=w.d_q, d_k=w.d_k, d_v=w.d_v,
                       d_h=w.d_h, d_vh=w.d_vh, d_o=w.d_o, scale=w.scale,
                       in_dtype=1 if w.dtype == "bf16" else 0, out_dtype=0)
    work = mha.default_work_dtype(tdt)
    dims.work_dtype = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[work]
    ws = torch.empty(mha.mha_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        mha.mha_forward(Q, K, V, W["W_Q"], W["W_K"], W["W_V"], W["W_O"], w.h, w.d_h, w.d_vh,
                        scale=w.scale, causal=w.causal, key_len=kl, Y=Y, workspace=ws,
                        stream=stream)

    # ---- whole forward --------------------------------------------------------
    steps_fwd = args.steps if args.only != "core" else 1
    for _ in range(args.warmup if args.only != "core" else 1):
        step()
    ms_step, per_step = timed_steps(step, steps_fwd, stream, torch)
    Y_timed = Y.float().cpu().numpy()
    if args.only == "forward":
        print(json.dumps({"ms_per_step": ms_step}), flush=True)
        return

    # ---- the dominant kernel alone: attention core on the projected heads ----
    # (the same launch configuration mha_forward uses: fp16 heads, fp16 Z)
    Qh, Kh, Vh = workspace_views(ws, w, torch, work)
    Z = torch.empty((w.B, w.n_q, w.h * w.d_vh), dtype=work, device=dev)

    def core():
        mha.attn_core(Qh, Kh, Vh, scale=w.scale, causal=w.causal, key_len=kl, out_dtype=work,
                      Z=Z, stream=stream)

    for _ in range(args.warmup):
        core()
    ms_core, per_core = timed_steps(core, args.steps, stream, torch)

    # ---- the forward again after about 0.2 s of sustained load -------------------
    settled = None
    if args.only == "all":
        t_end = time.perf_counter() + 0.2
        n_settle = 0
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
            n_settle += 20
        ms_settled, per_settled = timed_steps(step, args.steps, stream, torch)
        # the attention kernel alone right after, still under sustained load
        ms_core_settled, per_core_settled = timed_steps(core, args.steps, stream, torch)
        settled = {"settle_steps": n_settle, "ms_per_step": round(ms_settled, 5),
                   "ms_median": round(per_settled[len(per_settled) // 2], 5),
                   "attn_core_ms": round(ms_core_settled, 5),
                   "attn_core_ms_median": round(per_core_settled[len(per_core_settled) // 2], 5)}

    core_flops = w.core_flops_effective(x["key_len"])
    total_flops = core_flops + w.proj_flops()
    value = total_flops / (ms_step * 1e-3) / 1e12
    core_tflops = core_flops / (ms_core * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    exps = core_flops / (2.0 * (w.d_h + w.d_vh))   # allowed scores

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            entry = tj.get(w.name, {}).get("attn_core")
            if entry is not None and entry.get("source_hash") == attn_source_hash():
                traffic = entry.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    nominal = w.core_flops() + w.proj_flops()
    if settled is not None:
        settled["value"] = round(total_flops / (settled["ms_per_step"] * 1e-3) / 1e12, 3)
        settled["attn_core_frac_of_peak"] = round(
            core_flops / (settled["attn_core_ms"] * 1e-3) / 1e12 / peak, 4)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_median": round(per_step[len(per_step) // 2], 5),
        "ms_min": round(per_step[0], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f16" if w.dtype == "bf16" else "f32",
        "precision": ("bf16 inputs and weights; bf16 MFMA for the Q/K/V projections; fp16 "
                      "projected heads, softmax weights and concatenation; fp32 accumulation "
                      "and fp32 output") if w.dtype == "bf16" else "fp32 throughout",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "n_q": w.n_q, "n_k": w.n_k, "d_q": w.d_q,
                   "h": w.h, "d_h": w.d_h, "d_vh": w.d_vh, "d_o": w.d_o,
                   "mask": "causal" if w.causal else ("key_padding" if w.pad_range else "none"),
                   "parallelism": "single-gpu"},
        # value counts the effective work (padded keys excluded); nominal counts
        # every key of n_k (the two differ for key-padding workloads)
        "flops_per_step": {"effective": total_flops, "nominal": nominal},
        "e2e_frac_of_peak": round(value / peak, 4),
        "attn_core": {"ms": round(ms_core, 5), "ms_median": round(per_core[len(per_core) // 2], 5),
                      "ms_min": round(per_core[0], 5), "tflops": round(core_tflops, 3),
                      "frac_of_peak": round(core_tflops / peak, 4),
                      "gflop": round(core_flops / 1e9, 3),
                      "gflop_nominal": round(w.core_flops() / 1e9, 3)},
        "roofline": {"bound": "mfma", "kernel": core_kernel_name(w),
                     "achieved": round(core_tflops, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(core_tflops / peak, 4), "traffic": traffic},
        # the softmax's second ceiling: one exponential per allowed score
        # (counted as the metric counts scores)
        "exp_co_roof": {"exps_per_launch": int(exps),
                        "achieved": round(exps / (ms_core * 1e-3) / 1e12, 3),
                        "peak": round(EXP_PEAK_T_PER_S, 2), "unit": "T exp/s",
                        "frac": round(exps / (ms_core * 1e-3) / 1e12 / EXP_PEAK_T_PER_S, 4)},
    }
    if settled is not None:
        out["settled"] = settled
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(w, x, Y_timed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
