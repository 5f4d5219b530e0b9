#!/usr/bin/env python3
"""Benchmark of the block-selection hot path on one MI355X.

One step = one pass of the whole path over one batch: the block scorer
(qsa_block_scores) and then the block top-k (qsa_block_topk) on the scores it
wrote - exactly what qsa_select enqueues - on the prompt-call workload:
256 queries, 32 indexer heads, 128-wide keys, 131,072 blocks of 4 cells,
a 2,048-cell selection. Inputs are seeded synthetic tensors (synth.c5) that
are resident in HBM before the timed region starts.

Prints ONE JSON line. Per-kernel times come from HIP events recorded on the
stream the kernels run on (torch's current stream), around each entry point.
The GPU raises its clock over the first ten or so calls of sustained matrix
work, so the default warm-up is 20 steps (about 40 ms).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "qsa_select µs/call (score+top-k) decode nq=3 & prompt nq=256; % HBM/MFMA peak"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense FP32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
ROTATION_BYTES = 512 << 20      # score lines touched per rotation cycle: 2x the 256 MB last-level cache
SCORER_SOURCES = [os.path.join(ROOT, "sparse_attention_block_scores_amd", "csrc", f)
                  for f in ("scores_kernel.hip", "scores_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scores_kernel_c5_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode / top-k-only figures")
    ap.add_argument("--only-attention", action="store_true",
                    help="time only the attention over the selected cells (for profiling runs)")
    ap.add_argument("--only-topk", action="store_true",
                    help="time only the top-k-only figures (for profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (to scale profiler byte counters)")
    return ap.parse_args()


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def event_pairs_mean_us(pairs) -> float:
    return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) * 1000.0


def measured_traffic(per_launch_flops_unit):
    """HBM bytes per scorer launch from committed profiler counters, or None
    when they are missing or were taken on another version of the kernel."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_digest(SCORER_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def timed_loop(torch, steps, body):
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        body(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)  # ms


def cpu_baseline(wl, q, k, w, budget_s=12.0):
    """The oracle as it is, on the first queries of the same workload, until
    about budget_s seconds of CPU work; scaled to microseconds per call."""
    import numpy as np

    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    done, elapsed, batch = 0, 0.0, 8
    while done < wl.nq and elapsed < budget_s:
        n = min(batch, wl.nq - done)
        t = time.perf_counter()
        s = oracle.block_scores(q[done:done + n], k, w[done:done + n])
        oracle.topk_sort(s.astype(np.float32), wl.n_blocks, wl.block_size, wl.width)
        elapsed += time.perf_counter() - t
        done += n
    return {
        "value": round(elapsed / done * wl.nq * 1e6, 1),
        "unit": "us/call",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {done} of {wl.nq} queries of the same workload (FP64 scores over all "
                  f"{wl.n_blocks} blocks, then the full-sort top-k), {elapsed:.1f} s, scaled x{wl.nq / done:.2f}",
    }


def graph_us(torch, dev, fn, n):
    """Mean GPU time of fn(i) for i < n, captured once in a HIP graph and
    replayed, so host-side call overhead does not enter small latencies."""
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n * 1000.0


def secondary(torch, qsa, synth, dev, reps=50):
    """Decode-call latency at each context, top-k-only prompt figures, the
    BF16 scorer and the attention over the selected cells.
    Every figure is the mean over a HIP graph of back-to-back calls on
    torch's current stream (the library is capture-safe: no allocation, no
    host synchronisation, no memset nodes)."""
    out = {}

    def time_us(fn, n=reps):
        return graph_us(torch, dev, lambda i: fn(i), n)

    cur = torch.cuda.current_stream

    wl = synth.c1()
    q, k, w = [torch.from_numpy(x).to(dev) for x in wl.tensors()]
    ws = qsa.workspace(qsa.topk_workspace_bytes(wl.nq, wl.n_blocks, 4, wl.width, "decode"), dev)
    s = torch.empty((wl.nq, wl.n_blocks), device=dev)
    ids = torch.empty((wl.nq, wl.width), dtype=torch.int32, device=dev)
    cnt = torch.empty((wl.nq,), dtype=torch.int32, device=dev)
    out["decode_nq3_select_us"] = round(time_us(lambda i: qsa.select(q, k, w, 4, wl.width, "decode", scores=s,
                                                                      ids=ids, counts=cnt, ws=ws,
                                                                      stream=cur())), 2)
    # The same 3 queries x 8 heads over the decode contexts of the top-k
    # figures (scores and top-k, one call).
    by_cells = {}
    for nb in synth.C2_BLOCKS:
        wlc = synth.SelectWorkload(f"C1@{nb}", nq=3, heads=8, n_blocks=nb, block_size=4, width=2048,
                                   call="decode")
        qc, kc, wc = [torch.from_numpy(x).to(dev) for x in wlc.tensors()]
        wsc = qsa.workspace(qsa.topk_workspace_bytes(3, nb, 4, 2048, "decode"), dev)
        sc = torch.empty((3, nb), device=dev)
        idc = torch.empty((3, 2048), dtype=torch.int32, device=dev)
        cc = torch.empty((3,), dtype=torch.int32, device=dev)
        by_cells[str(nb * 4)] = round(time_us(lambda i: qsa.select(qc, kc, wc, 4, 2048, "decode", scores=sc, ids=idc,
                                                                   counts=cc, ws=wsc, stream=cur())), 2)
        del qc, kc, wc, wsc, sc
    out["decode_nq3_select_us_by_cells"] = by_cells
    wl3 = synth.c3()
    q3, k3, w3 = [torch.from_numpy(x).to(dev) for x in wl3.tensors()]
    ws3 = qsa.workspace(qsa.topk_workspace_bytes(wl3.nq, wl3.n_blocks, 4, wl3.width, "decode"), dev)
    s3 = torch.empty((wl3.nq, wl3.n_blocks), device=dev)
    ids3 = torch.empty((wl3.nq, wl3.width), dtype=torch.int32, device=dev)
    cnt3 = torch.empty((wl3.nq,), dtype=torch.int32, device=dev)
    out["decode_nq16_select_us"] = round(time_us(lambda i: qsa.select(q3, k3, w3, 4, wl3.width, "decode",
                                                                       scores=s3, ids=ids3, counts=cnt3,
                                                                       ws=ws3, stream=cur())), 2)
    out.update(topk_figures(torch, qsa, synth, dev, time_us, s3))

    # The BF16-input scorer (qsa_block_scores_bf16) on the prompt-call and
    # 16-query decode shapes; torch's float -> bfloat16 conversion rounds to
    # nearest even, as the parity tests do.
    bf = {}
    for wlb in (synth.c5(), synth.c3()):
        qh, kh, wh = wlb.tensors()
        qb = torch.from_numpy(qh).to(dev).to(torch.bfloat16)
        kb = torch.from_numpy(kh).to(dev).to(torch.bfloat16)
        wb = torch.from_numpy(wh).to(dev)
        sb = torch.empty((wlb.nq, wlb.n_blocks), device=dev)
        us = time_us(lambda i: qsa.block_scores_bf16(qb, kb, wb, scores=sb, stream=cur()), n=20)
        tf = wlb.flops() / (us * 1e-6) / 1e12
        bf[wlb.name] = {"us": round(us, 2), "TFLOPs": round(tf, 1), "bf16_peak_frac": round(tf / PEAK_BF16_MFMA_TFLOPS, 4)}
        del qb, kb, wb, sb
    out["bf16_scorer"] = bf
    out["vendor_gemm"] = vendor_gemm(torch, synth, dev)

    out["selection_attention"] = attention_figures(torch, qsa, synth, dev, time_us)
    return out


def vendor_gemm(torch, synth, dev, reps=10):
    """The vendor GEMM (torch.matmul, hipBLASLt) on this GPU, as a yardstick
    for the scorer's fraction of the matrix peaks: 8192^3 in FP32 and BF16,
    and the scorer's own contraction on the prompt-call shape (32 heads x 256
    queries = 8,192 rows of K = 128 against 131,072 keys, FP32) as a plain
    GEMM that writes every head's dot products (4 GiB) and applies no relu,
    weights or head sum. Event-timed means over `reps` calls after 3 warm-up
    calls."""
    def mean_us(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / reps

    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    n = 8192
    for name, dt, peak in (("fp32", torch.float32, PEAK_FP32_MFMA_TFLOPS), ("bf16", torch.bfloat16, PEAK_BF16_MFMA_TFLOPS)):
        a = torch.randn((n, n), device=dev, generator=g).to(dt)
        b = torch.randn((n, n), device=dev, generator=g).to(dt)
        us = mean_us(lambda: torch.matmul(a, b))
        tf = 2.0 * n ** 3 / (us * 1e-6) / 1e12
        out[f"{name}_8192cube"] = {"us": round(us, 1), "TFLOPs": round(tf, 1), "peak_frac": round(tf / peak, 4)}
        del a, b
    wl = synth.c5()
    qh, kh, _ = wl.tensors()
    q2 = torch.from_numpy(qh).to(dev).reshape(wl.nq * wl.heads, wl.head_dim)
    kt = torch.from_numpy(kh).to(dev)
    c = torch.empty((wl.nq * wl.heads, wl.n_blocks), device=dev)
    us = mean_us(lambda: torch.matmul(q2, kt.t(), out=c))
    tf = wl.flops() / (us * 1e-6) / 1e12
    out["fp32_scorer_contraction_unfused"] = {"us": round(us, 1), "TFLOPs": round(tf, 1),
                                              "peak_frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4)}
    del q2, kt, c
    return out


def topk_figures(torch, qsa, synth, dev, time_us, c3_scores=None):
    """Top-k-only figures: decode contexts (3 queries) as dispatched, with the
    chunked split and with the filtered split forced; the 16-query decode
    top-k on the scorer's C3 scores; prompt calls (256 queries) at each
    context and key variant over rotated score buffers, and with every query
    flagged (the exact pass that follows a failed sampled bound)."""
    cur = torch.cuda.current_stream
    out = {}
    dec, dec_split, dec_filter = {}, {}, {}
    split = qsa.make_options(topk_path=qsa.PATH_SPLIT)
    filt = qsa.make_options(topk_path=qsa.PATH_FILTER)
    for nb in synth.C2_BLOCKS:
        t = synth.c2(nb)
        sc = torch.from_numpy(t.scores()).to(dev)
        idd = torch.empty((t.nq, t.width), dtype=torch.int32, device=dev)
        cd = torch.empty((t.nq,), dtype=torch.int32, device=dev)
        for table, opt in ((dec, None), (dec_split, split), (dec_filter, filt)):
            wsd = qsa.workspace(qsa.topk_workspace_bytes(t.nq, nb, 4, t.width, "decode", opt), dev)
            table[str(nb * 4)] = round(time_us(lambda i: qsa.block_topk(sc, nb, 4, t.width, "decode", ids=idd,
                                                                        counts=cd, ws=wsd, options=opt,
                                                                        stream=cur())), 2)
    out["decode_nq3_topk_us_by_cells"] = dec                # the dispatch's choice
    out["decode_nq3_topk_split_us_by_cells"] = dec_split    # the exact chunked split, forced
    out["decode_nq3_topk_filter_us_by_cells"] = dec_filter  # the two-launch filtered split, forced
    if c3_scores is not None:
        wl3 = synth.c3()
        ids3 = torch.empty((wl3.nq, wl3.width), dtype=torch.int32, device=dev)
        cnt3 = torch.empty((wl3.nq,), dtype=torch.int32, device=dev)
        ws3 = qsa.workspace(qsa.topk_workspace_bytes(wl3.nq, wl3.n_blocks, 4, wl3.width, "decode"), dev)
        out["decode_nq16_topk_us"] = round(time_us(lambda i: qsa.block_topk(c3_scores, wl3.n_blocks, 4, wl3.width,
                                                                          "decode", ids=ids3, counts=cnt3, ws=ws3,
                                                                          stream=cur())), 2)
    prm = {}
    for nb in synth.C4_BLOCKS:
        entry = {}
        for variant in ("continuous", "q64", "equal"):
            t = synth.c4(nb, variant)
            host = t.scores()
            # Distinct score buffers, cycled, so that the score lines one cycle
            # touches (nq x n_blocks x 4 bytes per buffer, rows ld apart) add
            # up to at least 512 MiB: twice the 256 MB last-level cache, so
            # every call reads its scores from HBM.
            touched = t.nq * nb * 4
            nbuf = -(-ROTATION_BYTES // touched)
            bufs = [torch.from_numpy(host).to(dev) for _ in range(nbuf)]
            wsp = qsa.workspace(qsa.topk_workspace_bytes(t.nq, nb, 4, t.width, "prompt"), dev)
            idp = torch.empty((t.nq, t.width), dtype=torch.int32, device=dev)
            cp = torch.empty((t.nq,), dtype=torch.int32, device=dev)
            us = time_us(lambda i: qsa.block_topk(bufs[i % nbuf], nb, 4, t.width, "prompt", ids=idp, counts=cp,
                                                  ws=wsp, stream=cur()), n=max(40, 2 * nbuf))
            gbs = touched / us / 1e3
            if variant == "continuous":
                warm = time_us(lambda i: qsa.block_topk(bufs[0], nb, 4, t.width, "prompt", ids=idp, counts=cp,
                                                        ws=wsp, stream=cur()), n=40)
                # Every query flagged (as if its sampled bound had failed): the
                # exact rule with one more read of the row.
                flag = qsa.make_options(topk_path=qsa.PATH_ONEREAD, force_fallback=1)
                flagged = time_us(lambda i: qsa.block_topk(bufs[i % nbuf], nb, 4, t.width, "prompt", ids=idp,
                                                           counts=cp, ws=wsp, options=flag, stream=cur()),
                                  n=max(40, 2 * nbuf))
                entry.update({"us": round(us, 2), "scores_GBps": round(gbs, 1),
                              "hbm_frac": round(gbs / PEAK_HBM_GBS, 3), "rotated_buffers": nbuf,
                              "rotated_MiB": round(nbuf * touched / 2 ** 20), "warm_us": round(warm, 2),
                              "flagged_us": round(flagged, 2)})
            else:  # 64-level keys; all-equal keys (detected during the stream)
                entry[variant + "_us"] = round(us, 2)
            del bufs
        prm[str(nb * 4)] = entry
    out["prompt_nq256_topk_by_cells"] = prm
    return out


def attention_figures(torch, qsa, synth, dev, time_us):
    """Attention over the selected cells (qsa_selection_attention), decode
    and prompt shapes; bytes are the gathered key and value rows. The prompt
    shape is also timed over three rotated key/value copies (768 MiB), so that
    its reads come from HBM rather than the 256 MB last-level cache."""
    import numpy as np

    cur = torch.cuda.current_stream
    att = {}
    for wla in (synth.a3(), synth.a5()):
        qh, kh, vh = wla.tensors()
        sel = wla.selection()

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        qa, ids_a = bf16(qh), torch.from_numpy(sel).to(dev)
        copies = 3 if wla.nq >= 256 else 1
        ks = [bf16(kh) for _ in range(copies)]
        vs = [bf16(vh) for _ in range(copies)]
        oa = torch.empty((wla.nq, wla.heads, 128), device=dev)
        la = torch.empty((wla.nq, wla.heads), device=dev)
        need = qsa.attention_workspace_bytes(wla.nq, wla.heads, wla.kv_heads, wla.width)
        wsa = qsa.workspace(need, dev) if need else None
        gathered = wla.gathered_bytes(sel)

        def call(i, rot):
            j = i % len(ks) if rot else 0
            qsa.selection_attention(qa, ks[j], vs[j], ids_a, scale=wla.scale(), out=oa, lse=la, ws=wsa,
                                    stream=cur())

        us = time_us(lambda i: call(i, False), n=30)
        entry = {"us": round(us, 2), "gathered_MiB": round(gathered / 2 ** 20, 1),
                 "gathered_GBps": round(gathered / us / 1e3, 1),
                 "hbm_frac": round(gathered / us / 1e3 / PEAK_HBM_GBS, 3)}
        if copies > 1:
            us_r = time_us(lambda i: call(i, True), n=30)
            entry.update({"rotated_us": round(us_r, 2), "rotated_GBps": round(gathered / us_r / 1e3, 1),
                          "rotated_hbm_frac": round(gathered / us_r / 1e3 / PEAK_HBM_GBS, 3)})
        att[wla.name] = entry
        del ks, vs, qa, ids_a, oa, la, wsa

    # A6: the shared-block path (pairs of neighbouring queries over their
    # merged lists) against the plain one on the same lists, both over three
    # rotated key/value copies; "unique" bytes are the rows of each pair's
    # distinct cells, the gather the shared path needs.
    wl6 = synth.a6()
    qh, kh, vh = wl6.tensors()
    sel = wl6.selection()

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    q6, ids6 = bf16(qh), torch.from_numpy(sel).to(dev)
    ks = [bf16(kh) for _ in range(3)]
    vs = [bf16(vh) for _ in range(3)]
    o6 = torch.empty((wl6.nq, wl6.heads, 128), device=dev)
    l6 = torch.empty((wl6.nq, wl6.heads), device=dev)
    row_bytes = wl6.kv_heads * wl6.head_dim * 2 * 2
    unique = 0
    for p in range(0, wl6.nq, 2):
        rows = sel[p:p + 2]
        unique += np.unique(rows[(rows >= 0) & (rows < wl6.n_cells)]).size
    entry = {"listed_MiB": round(wl6.gathered_bytes(sel) / 2 ** 20, 1),
             "unique_MiB": round(unique * row_bytes / 2 ** 20, 1)}
    for shared in (False, True):
        need = qsa.attention_workspace_bytes(wl6.nq, wl6.heads, wl6.kv_heads, wl6.width, shared=shared)
        ws6 = qsa.workspace(need, dev) if need else None
        us = time_us(lambda i: qsa.selection_attention(q6, ks[i % 3], vs[i % 3], ids6, scale=wl6.scale(), out=o6,
                                                       lse=l6, ws=ws6, stream=cur(), shared=shared), n=30)
        entry["shared_rotated_us" if shared else "plain_rotated_us"] = round(us, 2)
    entry["shared_unique_GBps"] = round(unique * row_bytes / entry["shared_rotated_us"] / 1e3, 1)
    entry["shared_hbm_frac"] = round(entry["shared_unique_GBps"] / PEAK_HBM_GBS, 3)
    att["A6"] = entry
    del ks, vs, q6, ids6, o6, l6
    return att


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: it measures the single-GPU hot path "
              "(use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_block_scores_amd as qsa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only_attention:
        att = attention_figures(torch, qsa, synth, dev, lambda fn, n: graph_us(torch, dev, fn, n))
        print(json.dumps({"selection_attention": att}), flush=True)
        return
    if args.only_topk:
        tk = topk_figures(torch, qsa, synth, dev, lambda fn, n=50: graph_us(torch, dev, fn, n))
        print(json.dumps(tk), flush=True)
        return
    wl = synth.c5()
    q_h, k_h, w_h = wl.tensors()
    q, k, w = (torch.from_numpy(x).to(dev) for x in (q_h, k_h, w_h))
    scores = torch.empty((wl.nq, wl.n_blocks), dtype=torch.float32, device=dev)
    ids = torch.empty((wl.nq, wl.width), dtype=torch.int32, device=dev)
    counts = torch.empty((wl.nq,), dtype=torch.int32, device=dev)
    ws = qsa.workspace(qsa.topk_workspace_bytes(wl.nq, wl.n_blocks, wl.block_size, wl.width, wl.call), dev)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(i, record=True):
        if record:
            ev[i][0].record()
        qsa.block_scores(q, k, w, scores=scores)
        if record:
            ev[i][1].record()
        qsa.block_topk(scores, wl.n_blocks, wl.block_size, wl.width, wl.call, ids=ids, counts=counts, ws=ws)
        if record:
            ev[i][2].record()

    for _ in range(args.warmup):
        step(0, record=False)
    torch.cuda.synchronize()
    total_ms = timed_loop(torch, args.steps, step)
    ms_per_step = total_ms / args.steps
    scorer_us = event_pairs_mean_us([(e[0], e[1]) for e in ev])
    topk_us = event_pairs_mean_us([(e[1], e[2]) for e in ev])

    # The same work through the single qsa_select entry point.
    for _ in range(2):
        qsa.select(q, k, w, wl.block_size, wl.width, wl.call, scores=scores, ids=ids, counts=counts, ws=ws)
    sel_ms = timed_loop(torch, args.steps, lambda i: qsa.select(q, k, w, wl.block_size, wl.width, wl.call,
                                                                scores=scores, ids=ids, counts=counts, ws=ws))
    select_us = sel_ms / args.steps * 1000.0

    tflops = wl.flops() / (scorer_us * 1e-6) / 1e12
    traffic = measured_traffic(None)
    line = {
        "metric": METRIC,
        "value": round(ms_per_step * 1000.0, 1),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prompt-call select: 256 queries x 32 indexer heads x K=128 against "
                               "131,072 blocks of 4 cells, width 2,048 cells",
                   "nq": wl.nq, "heads": wl.heads, "head_dim": wl.head_dim, "n_blocks": wl.n_blocks,
                   "block_size": wl.block_size, "width": wl.width, "call": wl.call},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": traffic, "kernel": "scores_kernel (FP32 MFMA scorer)",
                     "flops_per_launch": wl.flops(), "kernel_us": round(scorer_us, 2)},
        "topk_us": round(topk_us, 2),
        "qsa_select_single_call_us": round(select_us, 1),
    }
    if not args.no_secondary:
        line["secondary"] = secondary(torch, qsa, synth, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, q_h, k_h, w_h)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
