"""Benchmark: absorbed-MLA decode on one MI355X.

A step is one pass of the whole hot path over one batch: the split-KV
scheduler (mla_get_decode_metadata) followed by the decode call
(mla_decode_fwd / mla_sparse_decode_fwd: partial-attention kernel + LSE
combine), with every input resident in HBM.  The default workload is the
DeepSeek-V3 decode shape b=64, s_q=1, h_q=128, seqlen=4096 (64-token pages
shuffled over a 4096-page pool, bf16 N(0,1) inputs).

``--workload`` selects another timed shape:
  config1 .. config5     the five parity workloads (tiny dense; the headline;
                         variable-length causal s_q=2; top-k 2048 sparse;
                         656-byte FP8 cache), each with the roofline that
                         bounds it (HBM for 1, 2, 4; MFMA for 3, 5);
  fp8_sparse_topk2048 / fp8_sparse_topk32768 / v41_sparse_topk2048 /
  fp4_sparse_topk2048    the pages' sparse decode shape (b=128, s_q=2,
                         h_q=128) over the 656-, 528- and 288-byte records;
  sparse_prefill         top-k 2048 sparse prefill of 4096 query rows over a
                         32768-row bf16 cache.

Timing.  Untimed warm-up steps run for at least ``--warmup`` steps and at
least 100 ms (the GPU clock ramps up over the first 10-20 ms of sustained
work), then exactly ``--steps`` steps are timed with HIP events on the stream
the kernels run on, one event per step boundary: ``us_per_step`` is the mean
over the timed region, ``us_p10/p50/p90`` the per-step percentiles.
``--cold`` writes a 512 MiB scratch buffer (larger than the 256 MiB MALL)
before every timed step and times the steps alone.

The roofline is that of the dominant kernel, the partial-attention kernel,
launched alone through the measurement hook in the configuration the step
launches it (same split partial format), timed with HIP events on the same
stream.  ``achievable`` holds measured peaks on this GPU (a device copy's
GB/s and a large bf16 matmul's TFLOP/s) as second denominators.
``cpu_baseline`` is the fp64 oracle timed on this host on a bounded sample.

Prints one JSON line.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096)
METRIC = "MLA decode TFLOPS + HBM GB/s, µs/step at b=64,h_q=128,seqlen=4096 (1 GPU)"
# sources of the partial-attention kernel a workload runs: the 64-head dense
# kernel for a bf16 cache without top-k, the 128-head kernel otherwise
KERNEL_SOURCES = {
    "decode64": ("mla_decode_amd/csrc/decode64.hip", "mla_decode_amd/csrc/common.h",
                 "mla_decode_amd/csrc/wave_sched.h"),
    "decode": ("mla_decode_amd/csrc/decode.hip", "mla_decode_amd/csrc/common.h",
               "mla_decode_amd/csrc/wave_sched.h"),
}
DECODE64_WORKLOADS = ("dense_b64_s4096", "config1", "config2", "config3", "config4", "sparse_prefill")
WARMUP_MIN_S = 0.1

# workload -> (counter summary file, roofline bound)
COUNTER_FILES = {
    "dense_b64_s4096": "decode64_kernel_dense_b64_h128_s4096_counters.json",
    "config2": "decode64_kernel_dense_b64_h128_s4096_counters.json",
    "config3": "decode64_kernel_config3_b128_s2_causal_varlen_counters.json",
    "config4": "decode64_kernel_sparse_config4_b64_topk2048_counters.json",
    "config5": "decode_kernel_fp8_config5_b32_s16384_counters.json",
    "fp8_sparse_topk2048": "decode_kernel_fp8_sparse_b128_s2_h128_topk2048_counters.json",
    "fp8_sparse_topk32768": "decode_kernel_fp8_sparse_b128_s2_h128_topk32768_counters.json",
    "v41_sparse_topk2048": "decode_kernel_fp8_528_sparse_b128_s2_h128_topk2048_counters.json",
    "fp4_sparse_topk2048": "decode_kernel_fp4_sparse_b128_s2_h128_topk2048_counters.json",
    "sparse_prefill": "decode64_kernel_sparse_prefill_s4096_kv32768_topk2048_counters.json",
}
BOUND = {"config1": "hbm", "config2": "hbm", "dense_b64_s4096": "hbm", "config3": "mfma", "config4": "hbm",
         "config5": "mfma"}


def kernel_source_hash(workload):
    """Hash of the source files of the partial-attention kernel ``workload`` runs."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES["decode64" if workload in DECODE64_WORKLOADS else "decode"]:
        p = os.path.join(ROOT, f)
        if os.path.exists(p):
            with open(p, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the partial-attention kernel from the committed
    rocprofv3 counter runs, or None when they are missing or were taken on
    other kernel source."""
    name = COUNTER_FILES.get(workload)
    if name is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != kernel_source_hash(workload):
        return None
    return c.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- host facts

def host_facts():
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return ncpu, model


def blas_threads():
    import threadpoolctl
    return max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
               or [1])


# ----------------------------------------------------------------------------- CPU oracle baselines

def _bits16(t):
    import numpy as np
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def cpu_single_thread_config1():
    """Milliseconds for the fp64 oracle on the whole tiny workload, one BLAS thread."""
    import threadpoolctl
    from oracle import attention as A
    from workloads import make_config
    w = make_config(1)
    q, kv = _bits16(w.q), _bits16(w.kv).reshape(-1, 576)
    bt, sl = w.block_table.numpy(), w.cache_seqlens.numpy()
    with threadpoolctl.threadpool_limits(1):
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 0.5:
            A.decode(q, kv, w.softmax_scale, block_table=bt, cache_seqlens=sl, causal=w.causal)
            reps += 1
        return (time.perf_counter() - t0) / reps * 1e3


def cpu_baseline(w, budget_s=10.0):
    """The fp64 oracle on a bounded sample of the same workload: query tokens
    in order, each over the KV rows it sees, until about ``budget_s`` of CPU
    work; the value is the oracle's algorithmic TFLOP/s on that sample."""
    import numpy as np
    import torch
    from oracle import attention as A
    ncpu, model = host_facts()
    threads = blas_threads()
    q = _bits16(w.q)
    rec = int(w.kv.shape[-1])
    kv_rows = w.kv.view(-1, rec)
    nrows = kv_rows.shape[0]
    d_qk = int(w.q.shape[-1])
    done, flops, dt = 0, 0.0, 0.0
    total = w.batch * w.s_q
    bt = None if w.topk else w.block_table.cpu().numpy()
    sl = None if w.topk else w.cache_seqlens.cpu().numpy()
    idx = w.indices.cpu().numpy() if w.topk else None
    for b in range(w.batch):
        for i in range(w.s_q):
            if w.topk:
                rows = idx[b, i][(idx[b, i] >= 0) & (idx[b, i] < nrows)].astype(np.int64)
            else:
                vis = int(sl[b]) if not w.causal else min(max(int(sl[b]) - w.s_q + 1 + i, 0), int(sl[b]))
                t = np.arange(vis)
                rows = (bt[b][t // 64].astype(np.int64) * 64 + t % 64)
            got = kv_rows[torch.from_numpy(rows).to(w.kv.device)].cpu()        # gathered on the GPU
            kv = got.numpy() if w.kv_format != "bf16" else got.view(torch.int16).numpy().view(np.uint16)
            t0 = time.perf_counter()
            A.decode_partial(q, kv, w.softmax_scale, np.arange(len(rows)), b, i, kv_format=w.kv_format)
            dt += time.perf_counter() - t0
            flops += 2.0 * w.h_q * (d_qk + 512) * len(rows)
            done += 1
            if dt >= budget_s:
                break
        if dt >= budget_s:
            break
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {total} query tokens in order (all {w.h_q} heads x every KV row each sees), "
                      f"fp64 numpy, {dt:.1f} s of oracle time",
            "nproc": ncpu, "cpu_model": model, "blas_threads": int(threads)}


# ----------------------------------------------------------------------------- GPU timing helpers

def _warmup(fn, count, min_s=WARMUP_MIN_S):
    """Untimed steps: at least ``count`` and at least ``min_s`` seconds of
    work; returns (steps run, seconds)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < (count or 0) or time.perf_counter() - t0 < min_s:
        for _ in range(5):
            fn()
        n += 5
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def _timed(fn, steps, stream, before=None):
    """Exactly ``steps`` calls, one HIP event per step boundary on ``stream``.
    ``before`` (untimed) runs ahead of each step; with it every step gets its
    own start event.  Returns (mean ms over the region, per-step ms list)."""
    import torch
    torch.cuda.synchronize()
    if before is None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for k in range(steps):
            fn()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        return ev[0].elapsed_time(ev[-1]) / steps, per
    per = []
    for _ in range(steps):
        before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    return sum(per) / steps, per


def _pct(xs, p):
    s = sorted(xs)
    if not s:
        return None
    k = (len(s) - 1) * p / 100.0
    lo, hi = int(k), min(int(k) + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def achievable_peaks(dev):
    """Measured peaks on this GPU: device-to-device copy of 1 GiB (bytes read
    + written per second) and a 8192^3 bf16 matmul (TFLOP/s)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        dst.copy_(src)
    ms, _ = _timed(lambda: dst.copy_(src), 10, stream)
    copy_gbs = 2 * n / (ms * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    ms, _ = _timed(lambda: a @ b, 10, stream)
    mm = 2.0 * m ** 3 / (ms * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy_gbs, 1), "bf16_matmul_tflops": round(mm, 1),
            "how": "torch copy_ of 1 GiB (read + write bytes / time); torch bf16 matmul 8192^3 (hipBLASLt)"}


# ----------------------------------------------------------------------------- workloads

def load_workload(name, dev):
    from workloads import make_config, make_fp8_sparse, make_v41_sparse, make_fp4_sparse
    if name == "dense_b64_s4096":
        return make_config(2, device=dev)
    if name.startswith("config"):
        return make_config(int(name[6:]), device=dev)
    if name.startswith("v41"):
        return make_v41_sparse(128, 2, 128, pool_tokens_per_seq=32768, topk=2048, seed=4000, device=dev,
                               name="v41_sparse_b128_s2_topk2048")
    if name.startswith("fp4"):
        return make_fp4_sparse(128, 2, 128, pool_tokens_per_seq=32768, topk=2048, seed=4100, device=dev,
                               name="fp4_sparse_b128_s2_topk2048")
    return make_fp8_sparse(int(name.split("topk")[1]), device=dev)


STEP_DENSE = ("mla_decode_step: schedule computed in the partial-attention kernel (batch * s_q <= 256, else "
              "the scheduler kernel first), partial attention, combine")
STEP_SPARSE = ("mla_decode_step: schedule computed in the partial-attention kernel (batch * s_q <= 256, else the "
               "scheduler kernel first), partial attention, combine where an item is split")


def describe(name, w):
    """(metric, config dict, roofline bound) of a decode workload."""
    v41 = w.kv_format in ("fp8_528", "fp4_288")
    base = {"batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "d_qk": 512 if v41 else 576, "d_v": 512,
            "block_size": 64, "kv_format": w.kv_format if w.kv_format != "fp8" else "fp8_656"}
    if name in ("dense_b64_s4096", "config2"):
        cfg = {"workload": "dense absorbed-MLA decode b=64 s_q=1 h_q=128 seqlen=4096 (64-token pages, "
                           "4096-page shuffled pool, bf16 q/kv N(0,1))", "seqlen": 4096, **base,
               "step": STEP_DENSE}
        return METRIC, cfg, "hbm"
    if name == "config1":
        cfg = {"workload": "tiny dense decode b=2 s_q=1 h_q=16 seqlens {200,256}, 8-page pool, fp32 out",
               **base, "step": STEP_DENSE}
        return "MLA decode µs/step, tiny dense b=2,h_q=16,seqlens={200,256} (1 GPU)", cfg, "hbm"
    if name == "config3":
        cfg = {"workload": "variable-length speculative decode b=128 s_q=2 causal h_q=128, seqlens uniform in "
                           "[1, 8192], shuffled 64-token pages, bf16 N(0,1)", "causal": True, **base,
               "step": STEP_DENSE}
        return "MLA decode TFLOPS, µs/step at b=128,s_q=2 causal,h_q=128,seqlen~U[1,8192] (1 GPU)", cfg, "mfma"
    if name == "config4":
        cfg = {"workload": "DSA top-k sparse decode b=64 s_q=1 h_q=128, top-k 2048 of a 32768-token pool per "
                           "request, 5% of slots -1, bf16 N(0,1)", "topk": w.topk, **base,
               "step": STEP_SPARSE}
        return "MLA sparse decode TFLOPS, µs/step at b=64,h_q=128,topk=2048 (1 GPU)", cfg, "hbm"
    if name == "config5":
        cfg = {"workload": "FP8 latent-cache decode b=32 s_q=1 h_q=128 seqlen=16384, 656-byte records (512 "
                           "e4m3 + 4 fp32 scales + 64 bf16 RoPE), q bf16 N(0,1)", "seqlen": 16384, **base,
               "step": STEP_SPARSE}
        return "MLA FP8-cache decode TFLOPS, µs/step at b=32,h_q=128,seqlen=16384 (1 GPU)", cfg, "mfma"
    topk = w.topk
    rec = {"fp8_528": "528-byte records of the 512-wide head (e8m0 scales per 32 values)",
           "fp4_288": "288-byte FP4 records of the 512-wide head (e2m1 pairs, e4m3 scales per 16 values)"}.get(
               w.kv_format, "656-byte records")
    tag = {"fp8_528": ",528B records,d_qk=512", "fp4_288": ",288B FP4 records,d_qk=512"}.get(w.kv_format, "")
    kind = "FP4" if w.kv_format == "fp4_288" else "FP8"
    cfg = {"workload": f"{kind} sparse absorbed-MLA decode b=128 s_q=2 h_q=128 top-k {topk} ({rec}, "
                       f"{max(32768, 2 * topk)} cached tokens per request, every slot valid, N(0,1) sources)",
           "topk": topk, **base, "step": STEP_SPARSE}
    return f"MLA sparse {kind} decode TFLOPS, µs/step at b=128,s_q=2,h_q=128,topk={topk}{tag} (1 GPU)", cfg, "mfma"


def kernel_name(w):
    """The partial-attention kernel a workload runs (the library's dispatch rule)."""
    fused = w.batch * w.s_q <= 256
    if w.kv_format == "bf16" and (not w.topk or (w.num_blocks * 64 + 2) * 1152 < 1 << 32):
        return (f"decode64_kernel<{'true' if fused else 'false'}, {'true' if w.topk else 'false'}> "
                f"(bf16 cache, {'top-k rows' if w.topk else 'dense pages'}, 64 heads per workgroup"
                + (", schedule computed in the kernel)" if fused else ")"))
    fmt = {"bf16": 0, "fp8": 1, "fp8_528": 2, "fp4_288": 3}[w.kv_format]
    # the third argument selects the dense instantiation that computes its own schedule
    dense_fused = "true" if not w.topk and fused else "false"
    return (f"decode_kernel<{'true' if w.topk else 'false'}, {fmt}, {dense_fused}> (128 heads per workgroup"
            + (", schedule computed in the kernel)" if fused else ")"))


def bench_decode(args):
    import torch
    import mla_decode_amd as mla
    from workloads import flops_and_bytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = load_workload(args.workload, dev)
    metric, cfg, bound = describe(args.workload, w)
    acct = flops_and_bytes(w)
    dec = mla.Decoder.for_workload(w, dev, rescale_threshold=args.rescale_threshold)
    stream = torch.cuda.current_stream(dev)
    seqlens = None if w.topk else w.cache_seqlens

    def step():
        dec.step(w.q, w.kv, w.block_table, seqlens, w.indices, stream)

    scratch = None
    before = None
    if args.cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def before():
            scratch.fill_(7)

    nwarm, warm_s = _warmup(step, args.warmup)
    ms_step, per_step = _timed(step, args.steps, stream, before)

    # the step recorded once into a HIP graph, replayed with one host launch per
    # step; the first replay must reproduce the eager step bit for bit
    ref_out, ref_lse = dec.out.clone(), dec.lse.clone()
    graph = dec.capture(w.q, w.kv, w.block_table, seqlens, w.indices)
    dec.out.fill_(3.0)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(dec.out.view(torch.int16 if dec.out.dtype == torch.bfloat16 else torch.int32),
                       ref_out.view(torch.int16 if ref_out.dtype == torch.bfloat16 else torch.int32)) \
        and torch.equal(dec.lse, ref_lse), "graph replay differs from the eager step"
    _warmup(graph.replay, 10, 0.02)
    # eager and graph steps in alternating blocks, so both see the same clock
    # (the chip slows as it heats, and a block timed later would look slower)
    blk = max(args.steps // 4, 5)
    eager_blocks, graph_blocks = [], []
    for _ in range(4):
        eager_blocks.append(_timed(step, blk, stream, before)[0])
        graph_blocks.append(_timed(graph.replay, blk, stream, before)[0])
    ms_graph = sum(graph_blocks) / len(graph_blocks)
    ms_eager_inter = sum(eager_blocks) / len(eager_blocks)

    ms_decode, _ = _timed(lambda: dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream),
                          args.steps, stream, before)
    # the dominant kernel alone, in the launch configuration of the step
    ms_kernel, per_kernel = _timed(
        lambda: dec.decode_partial(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream, production=True,
                                   fused=True),
        args.steps, stream, before)

    flops, nbytes, kbytes = acct["flops"], acct["bytes"], acct["partial_bytes"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    kern_gbs = kbytes / (ms_kernel * 1e-3) / 1e9
    kern_tflops = flops / (ms_kernel * 1e-3) / 1e12
    hbm = {"achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": kbytes}
    mfma = {"achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops}
    main, other = (hbm, mfma) if bound == "hbm" else (mfma, hbm)
    roofline = {"bound": bound, "kernel": kernel_name(w) + ", launched as the step launches it",
                **{k: main[k] for k in ("achieved", "peak", "unit", "frac")},
                "traffic": measured_traffic(args.workload), "us_per_launch": round(ms_kernel * 1e3, 2),
                "us_per_launch_p50": round(_pct(per_kernel, 50) * 1e3, 2)}
    roofline.update({k: v for k, v in main.items() if k.startswith("algorithmic")})
    line = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "us_p10": round(_pct(per_step, 10) * 1e3, 2),
        "us_p50": round(_pct(per_step, 50) * 1e3, 2),
        "us_p90": round(_pct(per_step, 90) * 1e3, 2),
        "graph_us_per_step": round(ms_graph * 1e3, 2),
        "graph_vs_eager": {"graph_us": round(ms_graph * 1e3, 2), "eager_us": round(ms_eager_inter * 1e3, 2),
                           "how": f"4 alternating blocks of {blk} eager and {blk} graph-replayed steps"},
        "hbm_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "cold": bool(args.cold),
        "config": cfg,
        "roofline": roofline,
        "roofline_other": {"bound": "mfma" if bound == "hbm" else "hbm", **other},
        "decode_call_us": round(ms_decode * 1e3, 2),
    }
    if args.rescale_threshold:
        line["rescale_threshold"] = args.rescale_threshold
    del graph
    if scratch is not None:
        del scratch
    if not args.no_peaks:
        pk = achievable_peaks(dev)
        pk["frac_hbm"] = round(kern_gbs / pk["copy_gbs"], 4)
        pk["frac_mfma"] = round(kern_tflops / pk["bf16_matmul_tflops"], 4)
        line["achievable"] = pk
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w)
        cb["single_thread_config1_ms"] = round(cpu_single_thread_config1(), 3)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


PREFILL_SHAPE = (4096, 32768, 128, 2048)   # s_q, s_kv, h_q, topk


def prefill_workload(dev):
    """The prefill workload and its problem: 4096 query rows, the last of a 32768-row bf16 cache, top-k 2048,
    128 heads."""
    import mla_decode_amd as mla
    from workloads import make_sparse_prefill
    s_q, s_kv, h_q, topk = PREFILL_SHAPE
    w = make_sparse_prefill(s_q, s_kv, h_q, topk, seed=3000, device=dev)
    return w, mla.make_problem(1, s_q, h_q, s_kv // 64, topk=topk, softmax_scale=w.softmax_scale)


def bench_prefill(args):
    """Top-k sparse prefill: 4096 query rows, the last of a 32768-row bf16 cache, top-k 2048, 128 heads."""
    import types
    import torch
    import mla_decode_amd as mla
    dev = torch.device("cuda:0")
    s_q, s_kv, h_q, topk = PREFILL_SHAPE
    w, p = prefill_workload(dev)
    dec = mla.Decoder(p, dev)
    stream = torch.cuda.current_stream(dev)
    valid = int(((w.indices >= 0) & (w.indices < s_kv)).sum())
    flops = 2.0 * h_q * (576 + 512) * valid
    nbytes = float(s_q * h_q * 1152 + s_kv * 1152 + s_q * h_q * (1024 + 4) + w.indices.numel() * 4)

    def step():
        dec.metadata(None, stream)
        mla.sparse_prefill_fwd(p, s_kv, w.q, w.kv, w.indices, dec.meta, dec.workspace, dec.out, dec.lse, stream)

    nwarm, warm_s = _warmup(step, args.warmup)
    ms_step, per_step = _timed(step, args.steps, stream)
    ms_kernel, _ = _timed(lambda: dec.decode_partial(w.q, w.kv, None, None, w.indices, stream, production=True),
                          args.steps, stream)
    kern_tflops = flops / (ms_kernel * 1e-3) / 1e12
    line = {
        "metric": "MLA sparse prefill TFLOPS, µs/step at s_q=4096,s_kv=32768,h_q=128,topk=2048 (1 GPU)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": nwarm, "warmup_s": round(warm_s, 3), "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2), "us_p10": round(_pct(per_step, 10) * 1e3, 2),
        "us_p50": round(_pct(per_step, 50) * 1e3, 2), "us_p90": round(_pct(per_step, 90) * 1e3, 2),
        "hbm_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "top-k sparse prefill: 4096 query rows at the end of a 32768-row flat bf16 cache, "
                               "top-k 2048 of each row's visible rows, 128 heads, N(0,1) inputs",
                   "s_q": s_q, "s_kv": s_kv, "h_q": h_q, "topk": topk, "d_qk": 576, "d_v": 512,
                   "step": "metadata + sparse prefill (partial + combine when needed)"},
        "roofline": {"bound": "mfma",
                     "kernel": kernel_name(types.SimpleNamespace(kv_format="bf16", topk=topk, batch=1, s_q=s_q,
                                                                 num_blocks=p.num_blocks)),
                     "algorithmic_bytes_per_launch": nbytes,
                     "achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic("sparse_prefill"),
                     "algorithmic_flops": flops, "us_per_launch": round(ms_kernel * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        view = types.SimpleNamespace(batch=1, s_q=s_q, h_q=h_q, topk=topk, kv=w.kv, kv_format="bf16", causal=False,
                                     q=w.q[None], indices=w.indices[:, 0, :][None], softmax_scale=w.softmax_scale)
        line["cpu_baseline"] = cpu_baseline(view)
    print(json.dumps(line), flush=True)


WORKLOADS = ["dense_b64_s4096", "config1", "config2", "config3", "config4", "config5", "fp8_sparse_topk2048",
             "fp8_sparse_topk32768", "sparse_prefill", "v41_sparse_topk2048", "fp4_sparse_topk2048"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10,
                    help="minimum untimed steps; warm-up also lasts at least 100 ms of work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / matmul peaks")
    ap.add_argument("--cold", action="store_true", help="write 512 MiB of scratch before every timed step")
    ap.add_argument("--rescale-threshold", type=float, default=0.0,
                    help="lazy rescale: raise a row's running max only past this many log2 units (0: the exact max)")
    ap.add_argument("--workload", default="dense_b64_s4096", choices=WORKLOADS,
                    help="dense_b64_s4096 (= config2) is the headline line; see the module docstring")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--kernel-only", type=int, default=0, metavar="N",
                    help="profiling mode: build the workload, run the scheduler once, then launch only the "
                         "partial-attention kernel N times in the step's own partial format (for counter runs "
                         "whose dispatches are all production launches)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode path has no multi-GPU code); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return
    if args.kernel_only:
        return kernel_only(args)
    if args.workload == "sparse_prefill":
        return bench_prefill(args)
    return bench_decode(args)


def kernel_only(args):
    """The partial-attention kernel alone, ``--kernel-only`` times after the
    warm-up, in the launch configuration the decode step uses."""
    import torch
    import mla_decode_amd as mla
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.workload == "sparse_prefill":
        w, p = prefill_workload(dev)
        dec = mla.Decoder(p, dev)
        dec.metadata(None, stream)

        def k():
            dec.decode_partial(w.q, w.kv, None, None, w.indices, stream, production=True)
    else:
        w = load_workload(args.workload, dev)
        dec = mla.Decoder.for_workload(w, dev)
        dec.metadata(None if w.topk else w.cache_seqlens, stream)

        def k():
            dec.decode_partial(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream, production=True,
                               fused=True)

    nwarm, _ = _warmup(k, args.warmup)
    ms, per = _timed(k, args.kernel_only, stream)
    print(json.dumps({"workload": args.workload, "launches": args.kernel_only, "warmup_launches": nwarm,
                      "us_per_launch": round(ms * 1e3, 2), "us_p50": round(_pct(per, 50) * 1e3, 2)}), flush=True)


if __name__ == "__main__":
    main()
