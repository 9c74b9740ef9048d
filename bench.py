"""Benchmark: absorbed-MLA decode on one MI355X.

A step is one pass of the whole hot path over one batch: the split-KV
scheduler (mla_get_decode_metadata) followed by the decode call
(mla_decode_fwd: partial-attention kernel + LSE combine), on the DeepSeek-V3
decode shape b=64, s_q=1, h_q=128, seqlen=4096 (64-token pages shuffled over
a 4096-page pool, bf16 N(0,1) inputs, inputs resident in HBM).

``--workload fp8_sparse_topk2048`` / ``fp8_sparse_topk32768`` time instead
the FP8 sparse decode shape the pages quote for their H800 kernel (b=128,
s_q=2, h_q=128, top-k 2048 or 32768 over 656-byte records,
mla_sparse_decode_fwd); ``--workload sparse_prefill`` times the top-k sparse
prefill (mla_sparse_prefill_fwd) of 4096 query rows at the end of a
32768-row bf16 cache, top-k 2048, 128 heads.  Those lines' roofline is the
MFMA one.

The same step recorded once into a HIP graph is timed as well
(``graph_us_per_step``, after a bit-for-bit check of its first replay against
the eager step); on this path the eager launches are as fast or faster, so
``value`` is the eager step.

Prints one JSON line.  ``value`` is TFLOP/s of algorithmic work (FLOPs =
2 h_q (576 + 512) per visible query-token/KV-token pair) per step; the line
also carries HBM GB/s and microseconds per step, the roofline of the decode
call (HBM-bound at this shape), and the fp64 CPU oracle timed on the host.
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
KERNEL_SOURCES = ("mla_decode_amd/csrc/decode.hip", "mla_decode_amd/csrc/common.h")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_kernel_dense_b64_h128_s4096_counters.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None when they are missing or were taken on other kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline_sparse(w):
    """The fp64 oracle on a bounded sample of a top-k workload: query tokens in
    order, each over its gathered rows, until about 10 s of CPU work."""
    import numpy as np
    import threadpoolctl
    import torch
    from oracle import attention as A
    q = w.q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    kv_rows = w.kv.view(-1, w.kv.shape[-1])
    nrows = kv_rows.shape[0]
    idx = w.indices.cpu().numpy()
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    done, flops, dt = 0, 0.0, 0.0
    for b in range(w.batch):
        for i in range(w.s_q):
            rows = idx[b, i][(idx[b, i] >= 0) & (idx[b, i] < nrows)]
            got = kv_rows[torch.from_numpy(rows.astype(np.int64)).to(w.kv.device)].cpu()   # gathered on the GPU
            kv = got.numpy() if w.kv_format != "bf16" else got.view(torch.int16).numpy().view(np.uint16)
            t0 = time.perf_counter()
            A.decode_partial(q, kv, w.softmax_scale, np.arange(len(rows)), b, i, kv_format=w.kv_format)
            dt += time.perf_counter() - t0
            flops += 2.0 * w.h_q * (int(w.q.shape[-1]) + 512) * len(rows)
            done += 1
            if dt >= 10.0:
                break
        if dt >= 10.0:
            break
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.batch * w.s_q} query tokens (all {w.h_q} heads x top-k {w.topk} rows each), "
                      f"fp64 numpy, {dt:.1f} s in total"}


def cpu_baseline(w, flops):
    """The fp64 oracle on the same workload, on this host's cores."""
    import numpy as np
    import threadpoolctl
    import torch
    from oracle import attention as A
    q = w.q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    kv = w.kv.cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1, 576)
    bt = w.block_table.cpu().numpy()
    sl = w.cache_seqlens.cpu().numpy()
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    # whole steps, repeated until about 10 s of CPU work have been timed
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 10.0 and reps < 64):
        t0 = time.perf_counter()
        A.decode(q, kv, w.softmax_scale, block_table=bt, cache_seqlens=sl, causal=w.causal)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": flops * reps / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full steps (all {w.batch} requests x {w.h_q} heads x 4096 tokens each), "
                      f"fp64 numpy, {dt:.1f} s in total"}


def _warmup(fn, count, stream, budget_s=0.06):
    """Run ``count`` untimed steps, or (count None) steps until ``budget_s`` of
    work has run, at least 10; returns the number run."""
    import time
    import torch
    if count is not None:
        for _ in range(count):
            fn()
        torch.cuda.synchronize()
        return count
    n, t0 = 0, time.perf_counter()
    while n < 10 or time.perf_counter() - t0 < budget_s:
        for _ in range(5):
            fn()
        n += 5
        torch.cuda.synchronize()
    return n


def _timed(fn, steps, stream):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill(args):
    """Top-k sparse prefill: 4096 query rows, the last of a 32768-row bf16 cache, top-k 2048, 128 heads."""
    import types
    import torch
    import mla_decode_amd as mla
    from workloads import make_sparse_prefill
    dev = torch.device("cuda:0")
    s_q, s_kv, h_q, topk = 4096, 32768, 128, 2048
    w = make_sparse_prefill(s_q, s_kv, h_q, topk, seed=3000, device=dev)
    p = mla.make_problem(1, s_q, h_q, s_kv // 64, topk=topk, softmax_scale=w.softmax_scale)
    dec = mla.Decoder(p, dev)
    stream = torch.cuda.current_stream(dev)
    valid = int(((w.indices >= 0) & (w.indices < s_kv)).sum())
    flops = 2.0 * h_q * (576 + 512) * valid
    nbytes = float(s_q * h_q * 1152 + s_kv * 1152 + s_q * h_q * (1024 + 4) + w.indices.numel() * 4)

    def step():
        dec.metadata(None, stream)
        mla.sparse_prefill_fwd(p, s_kv, w.q, w.kv, w.indices, dec.meta, dec.workspace, dec.out, dec.lse, stream)

    args.warmup = _warmup(step, args.warmup, stream)
    ms_step = _timed(step, args.steps, stream)
    ms_kernel = _timed(lambda: dec.decode_partial(w.q, w.kv, None, None, w.indices, stream), args.steps, stream)
    kern_tflops = flops / (ms_kernel * 1e-3) / 1e12
    line = {
        "metric": "MLA sparse prefill TFLOPS, µs/step at s_q=4096,s_kv=32768,h_q=128,topk=2048 (1 GPU)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "hbm_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "top-k sparse prefill: 4096 query rows at the end of a 32768-row flat bf16 cache, "
                               "top-k 2048 of each row's visible rows, 128 heads, N(0,1) inputs",
                   "s_q": s_q, "s_kv": s_kv, "h_q": h_q, "topk": topk, "d_qk": 576, "d_v": 512,
                   "step": "metadata + sparse prefill (partial + combine when needed)"},
        "roofline": {"bound": "mfma", "kernel": "decode_kernel<sparse, bf16 cache> (partial attention)",
                     "achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops": flops, "us_per_launch": round(ms_kernel * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        view = types.SimpleNamespace(batch=1, s_q=s_q, h_q=h_q, topk=topk, kv=w.kv, kv_format="bf16",
                                     q=w.q[None], indices=w.indices[:, 0, :][None], softmax_scale=w.softmax_scale)
        line["cpu_baseline"] = cpu_baseline_sparse(view)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Default: untimed steps until about 60 ms of work has run (at least 10).
    # The GPU clock ramps up over the first ~10-20 ms of sustained work, so the
    # timed steps then see the steady state a serving loop runs at; a fixed
    # count would either stop inside the ramp (short steps) or heat the chip
    # for seconds first (long steps).
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="dense_b64_s4096",
                    choices=["dense_b64_s4096", "fp8_sparse_topk2048", "fp8_sparse_topk32768", "sparse_prefill",
                             "v41_sparse_topk2048", "fp4_sparse_topk2048"],
                    help="dense_b64_s4096 is the headline line; the others time the pages' sparse decode shape "
                         "(b=128, s_q=2, top-k 2048 or 32768) over the 656-, 528- and 288-byte record caches, "
                         "and top-k sparse prefill")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
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
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode path has no multi-GPU code); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_decode_amd as mla
    from workloads import make_config, make_fp8_sparse, make_v41_sparse, make_fp4_sparse, flops_and_bytes

    if args.workload == "sparse_prefill":
        return bench_prefill(args)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    headline = args.workload == "dense_b64_s4096"
    if headline:
        w = make_config(2, device=dev)
    elif args.workload.startswith("v41"):
        w = make_v41_sparse(128, 2, 128, pool_tokens_per_seq=32768, topk=2048, seed=4000, device=dev,
                            name="v41_sparse_b128_s2_topk2048")
    elif args.workload.startswith("fp4"):
        w = make_fp4_sparse(128, 2, 128, pool_tokens_per_seq=32768, topk=2048, seed=4100, device=dev,
                            name="fp4_sparse_b128_s2_topk2048")
    else:
        w = make_fp8_sparse(int(args.workload.split("topk")[1]), device=dev)
    acct = flops_and_bytes(w)
    dec = mla.Decoder.for_workload(w, dev)
    stream = torch.cuda.current_stream(dev)
    seqlens = None if w.topk else w.cache_seqlens

    def step():
        dec.metadata(seqlens, stream)
        dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream)

    args.warmup = _warmup(step, args.warmup, stream)
    # timed region: exactly K whole steps
    ms_step = _timed(step, args.steps, stream)

    # The step recorded once into a HIP graph (scheduler, decode kernel,
    # combine) and replayed with one host launch per step; the first replay
    # must reproduce the eager step bit for bit.
    ref_out, ref_lse = dec.out.clone(), dec.lse.clone()
    graph = dec.capture(w.q, w.kv, w.block_table, seqlens, w.indices)
    dec.out.fill_(3.0)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(dec.out.view(torch.int16), ref_out.view(torch.int16)) and torch.equal(dec.lse, ref_lse), \
        "graph replay differs from the eager step"
    for _ in range(args.warmup):
        graph.replay()
    ms_graph = _timed(graph.replay, args.steps, stream)

    # decode call alone (partial-attention kernel + combine), same stream, same inputs
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k0.record(stream)
    for _ in range(args.steps):
        dec.decode(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream)
    k1.record(stream)
    torch.cuda.synchronize()
    ms_decode = k0.elapsed_time(k1) / args.steps

    # the dominant kernel alone: the partial-attention kernel (decode_kernel),
    # launched through the test hook on the same stream
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record(stream)
    for _ in range(args.steps):
        dec.decode_partial(w.q, w.kv, w.block_table, w.cache_seqlens, w.indices, stream)
    p1.record(stream)
    torch.cuda.synchronize()
    ms_kernel = p0.elapsed_time(p1) / args.steps

    # scheduler alone
    m0 = torch.cuda.Event(enable_timing=True)
    m1 = torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for _ in range(args.steps):
        dec.metadata(seqlens, stream)
    m1.record(stream)
    torch.cuda.synchronize()
    ms_meta = m0.elapsed_time(m1) / args.steps

    flops, nbytes, kbytes = acct["flops"], acct["bytes"], acct["partial_bytes"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    kern_gbs = kbytes / (ms_kernel * 1e-3) / 1e9
    kern_tflops = flops / (ms_kernel * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "graph_us_per_step": round(ms_graph * 1e3, 2),
        "hbm_gbs": round(gbs, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense absorbed-MLA decode b=64 s_q=1 h_q=128 seqlen=4096 (64-token pages, "
                               "4096-page shuffled pool, bf16 q/kv N(0,1))",
                   "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "seqlen": 4096, "d_qk": 576, "d_v": 512,
                   "block_size": 64, "kv_format": "bf16",
                   "step": "metadata + decode (partial + combine)"},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<dense, bf16 cache> (partial attention)",
                     "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": kbytes, "us_per_launch": round(ms_kernel * 1e3, 2)},
        "roofline_mfma": {"achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops},
        "decode_call_us": round(ms_decode * 1e3, 2),
        "metadata_us": round(ms_meta * 1e3, 2),
    }
    if not headline:
        topk = w.topk
        v41 = w.kv_format in ("fp8_528", "fp4_288")
        rec = {"fp8_528": "528-byte records of the 512-wide head (e8m0 scales per 32 values)",
               "fp4_288": "288-byte FP4 records of the 512-wide head (e2m1 pairs, e4m3 scales per 16 values)"}.get(
                   w.kv_format, "656-byte records")
        tag = {"fp8_528": ",528B records,d_qk=512", "fp4_288": ",288B FP4 records,d_qk=512"}.get(w.kv_format, "")
        kind = "FP4" if w.kv_format == "fp4_288" else "FP8"
        line["metric"] = f"MLA sparse {kind} decode TFLOPS, µs/step at b=128,s_q=2,h_q=128,topk={topk}{tag} (1 GPU)"
        line["config"] = {"workload": f"{kind} sparse absorbed-MLA decode b=128 s_q=2 h_q=128 top-k {topk} "
                                      f"({rec}, {max(32768, 2 * topk)} cached tokens per request, "
                                      "every slot valid, N(0,1) sources)",
                          "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "topk": topk,
                          "d_qk": 512 if v41 else 576, "d_v": 512,
                          "block_size": 64, "kv_format": w.kv_format if v41 else "fp8_656",
                          "step": "metadata + sparse decode (partial + combine)"}
        line["roofline"] = {"bound": "mfma", "kernel": f"decode_kernel<sparse, {kind.lower()} cache> (partial attention)",
                            "achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "algorithmic_flops": flops, "us_per_launch": round(ms_kernel * 1e3, 2)}
        line["roofline_hbm"] = {"achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": kbytes}
        del line["roofline_mfma"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, flops) if headline else cpu_baseline_sparse(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
