#!/usr/bin/env python3
"""Throughput of the block-quantized weight x activation product on one
MI355X, printed as one JSON line.

A step is one pass of the product over one batch of synthetic input (seeded,
block_quant_weight_amd.synth).  The weights of successive steps rotate over
enough byte-identical copies (>= 512 MB in total) that neither the 256 MB
MALL nor the L2 can serve them: every step reads its weights from HBM.  The
timed steps run as one captured HIP graph (launch overhead out of the way),
after the graph has been replayed for at least --warm-seconds (so that the
GPU clock has left its idle state), bracketed by device synchronisation and
HIP events on the launching stream.

Default (no --workload): the five configurations in one process, one JSON
line whose headline is the shared-classifier LM head at batch 1 (the largest
single-GPU workload) and whose "configs" object holds every workload's rate,
step time, roofline and oracle baseline:
  q8_gemv_512         Q8_0 GEMV 512x512, f32 scales, batch 1
  q4_gemv_4096        Q4_0 GEMV 4096x4096, f16 scales, batch 1
  decode_layer        mixed Q4_0/Q8_0 decode layer (wq|wk|wv and w1|w3 grouped)
  gemm_q4_14336x4096  prefill GEMM, Q4_0 f16 scales x bf16 [512x4096]
  gemm_q8_4096x14336  prefill GEMM, Q8_0 f32 scales x bf16 [512x14336]
  lm_head_b1/_b64     Q8_0 248320x1024 f16 scales as the LM head, batch 1 / 64
  embed_64            dequantized gather of 64 rows of the same table
Each GEMV workload also carries the read ceiling at its largest launch's byte
count (a plain 16-byte-load read of that many bytes, qmv_read_probe).

Other workloads (--workload): decode_layer_gated (w1|w3 as one gated launch,
SiLU(w1 x) * (w3 x), whose output is w2's input), decode_layer_7 (one launch
per matrix), writer_q4_14336x4096 (float32 weights to a Q4_0 f16-scale image
by the round rule), writer_q4_search_14336x4096 (the least-squares search,
bound by float32 arithmetic), gemm_q8act_q4_14336x4096 and
gemm_q8act_q8_4096x14336 (the prefill shapes on the int8 path), read_stream
(the read ceiling over a range of sizes), mfma_rate (the prefill product's
matrix-core instruction back to back, on constant and on random operands),
and copy (a plain device copy, used to calibrate HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_0/Q8_0 GEMV effective GB/s (% HBM peak); prefill GEMM TFLOP/s (% MFMA)"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16/f16 MFMA, published (2.4 GHz)
INT8_PEAK_TOPS = 5033.2       # MI355X dense int8 MFMA, published (2.4 GHz)
# plain float32 vector operations (multiply, add, round, clamp, each one
# operation): the published 157.3 TFLOP/s counts a fused multiply-add as two,
# and an unfused operation takes the same issue slot, so 157.3 / 2 per second
F32_OPS_PEAK_T = 157.3 / 2
# float32 operations per 32-weight block of the Q4_0 least-squares search:
# 13 candidates x (32 x 13 per element + 2 divisions) + 4 x 32 (the largest
# element, the weights x^2 and x^3)
SEARCH_OPS_PER_BLOCK = 13 * (32 * 13 + 2) + 4 * 32
Q8, Q4 = 1, 2
ROTATE_BYTES = 512 << 20

LAYER = [("wq", 4, 4096, 4096), ("wk", 4, 1024, 4096), ("wv", 8, 1024, 4096),
         ("wo", 16, 4096, 4096), ("w1", 32, 11008, 4096), ("w3", 32, 11008, 4096),
         ("w2", 64, 4096, 11008)]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload(name):
    """(description, kind, config id, [(matrix id, wtype, scale_f16, rows, cols)], batch)."""
    from block_quant_weight_amd import qmv as Q
    if name == "q4_gemv_4096":
        return ("Q4_0 GEMV 4096x4096, f16 scales, batch 1", "gemv", 2,
                [(0, Q4, 1, 4096, 4096)], 1)
    if name == "q8_gemv_512":
        return ("Q8_0 GEMV 512x512, f32 scales, batch 1", "gemv", 1,
                [(0, Q8, 0, 512, 512)], 1)
    if name in ("decode_layer", "decode_layer_7", "decode_layer_gated"):
        mats = []
        for m, (_, cls, r, c) in enumerate(LAYER):
            mats.append((m, Q.qmv_class_wtype(Q4, 8 | 64, cls, 0), 1, r, c))
        how = {"decode_layer": "4 launches: wq|wk|wv and w1|w3 grouped on their shared inputs",
               "decode_layer_gated": "4 launches: wq|wk|wv grouped, w1|w3 as one gated "
                                     "launch h = SiLU(w1 x) * (w3 x), w2 on h",
               "decode_layer_7": "7 launches, one per matrix"}[name]
        return ("mixed decode layer (q8_mask 8|64: wv, w2 Q8_0; others Q4_0), "
                f"dim 4096, kv 1024, ffn 11008, f16 scales, batch 1, {how}", "gemv", 3, mats, 1)
    if name == "gemm_q4_14336x4096":
        return ("prefill GEMM Q4_0 14336x4096 f16 scales x bf16 [512x4096]", "gemm", 4,
                [(0, Q4, 1, 14336, 4096)], 512)
    if name == "gemm_q8_4096x14336":
        return ("prefill GEMM Q8_0 4096x14336 f32 scales x bf16 [512x14336]", "gemm", 4,
                [(1, Q8, 0, 4096, 14336)], 512)
    if name == "gemm_q8act_q4_14336x4096":
        return ("prefill on quantized activations: float32 [512x4096] -> Q8_0, then Q4_0 "
                "14336x4096 f16 scales on the int8 matrix cores", "gemm_q8", 4,
                [(0, Q4, 1, 14336, 4096)], 512)
    if name == "gemm_q8act_q8_4096x14336":
        return ("prefill on quantized activations: float32 [512x14336] -> Q8_0, then Q8_0 "
                "4096x14336 f32 scales on the int8 matrix cores", "gemm_q8", 4,
                [(1, Q8, 0, 4096, 14336)], 512)
    if name == "writer_q4_14336x4096":
        return ("weight writer: float32 14336x4096 -> Q4_0 f16 scales (round rule)", "writer", 4,
                [(0, Q4, 1, 14336, 4096)], 1)
    if name == "writer_q4_search_14336x4096":
        return ("weight writer: float32 14336x4096 -> Q4_0 f16 scales (least-squares search)",
                "writer", 4, [(0, Q4, 1, 14336, 4096)], 1)
    if name in ("lm_head_b1", "lm_head_b64"):
        b = 1 if name.endswith("b1") else 64
        return (f"shared-classifier LM head Q8_0 248320x1024 f16 scales, f32 hidden, "
                f"batch {b}", "gemv", 5, [(0, Q8, 1, 248320, 1024)], b)
    if name == "embed_64":
        return ("embedding gather of 64 ids from Q8_0 248320x1024 f16 scales", "embed", 5,
                [(0, Q8, 1, 248320, 1024)], 64)
    if name == "copy":
        return ("plain device copy of 256 MiB (counter calibration)", "copy", 0, [], 0)
    if name == "read_stream":
        return ("read ceiling: qmv_read_probe over a range of sizes", "read", 0, [], 0)
    if name == "mfma_rate":
        return ("matrix-core rate: qmv_mfma_probe, v_mfma_f32_32x32x16_f16 back to back", "mfma", 0, [], 0)
    raise SystemExit(f"unknown workload {name}")


# launches of the fused decode layer: indexes into LAYER (shared activations)
LAYER_GROUPS = [(0, 1, 2), (3,), (4, 5), (6,)]
# the gated pair (w1, w3) and the matrix that takes its output (w2)
GATED_PAIR, GATED_NEXT = (4, 5), 6

# The kernel that the library's dispatch runs for each workload's largest
# launch (the roofline's kernel), and the source file it is built from.
DOMINANT_KERNEL = {
    "q4_gemv_4096": ("gemv_oneshot_kernel", "gemv.hip"),
    "q8_gemv_512": ("gemv_oneshot_kernel", "gemv.hip"),
    "decode_layer": ("gemv_stream_kernel (w1|w3)", "gemv.hip"),
    "decode_layer_gated": ("gemv_stream_kernel, gated (w1|w3)", "gemv.hip"),
    "decode_layer_7": ("gemv_oneshot_kernel (w2)", "gemv.hip"),
    "lm_head_b1": ("gemv_oneshot_kernel_occ6", "gemv.hip"),
    "lm_head_b64": ("gemv_mfma_kernel (f16 operands)", "gemv_mfma.hip"),
    "gemm_q4_14336x4096": ("qmv_gemm call: stage_x_kernel + gemm_f16_kernel", "gemm.hip"),
    "gemm_q8_4096x14336": ("qmv_gemm call: stage_x_kernel + gemm_f16_kernel + "
                           "splitk_reduce_kernel", "gemm.hip"),
    "gemm_q8act_q4_14336x4096": ("gemm_q8act_kernel", "gemm_i8.hip"),
    "gemm_q8act_q8_4096x14336": ("gemm_q8act_kernel + splitk_reduce_kernel", "gemm_i8.hip"),
    "embed_64": ("embed_kernel", "misc.hip"),
    "writer_q4_14336x4096": ("quantize_q4_round_kernel", "writer.hip"),
    "writer_q4_search_14336x4096": ("quantize_q4_search_kernel", "writer.hip"),
}


def launch_groups(name, mats):
    """Lists of matrix positions that share one launch and one x."""
    if name in ("decode_layer", "decode_layer_gated"):
        return [list(g) for g in LAYER_GROUPS]
    return [[i] for i in range(len(mats))]


def matrix_bytes(wt, sf, r, c):
    q = r * c if wt == Q8 else r * c // 2
    return q + (r * c // 32) * (2 if sf else 4)


def step_work(kind, mats, batch, groups=None, gated=False):
    """Algorithmic bytes and flops of one step (an activation vector shared
    by a launch group is counted once; with gated, the group of two writes
    one output vector, act(y1) * y3)."""
    byts = flops = 0
    if kind == "gemv" and groups is not None:
        for g in groups:
            byts += 4 * mats[g[0]][4] * batch
            if gated and len(g) == 2:
                byts -= 4 * mats[g[1]][3] * batch
        for _, wt, sf, r, c in mats:
            byts += matrix_bytes(wt, sf, r, c) + 4 * r * batch
            flops += 2 * r * c * batch
        return byts, flops
    for _, wt, sf, r, c in mats:
        w = matrix_bytes(wt, sf, r, c)
        if kind == "gemv":
            byts += w + 4 * c * batch + 4 * r * batch
            flops += 2 * r * c * batch
        elif kind == "gemm":
            byts += w + 2 * c * batch + 4 * r * batch
            flops += 2 * r * c * batch
        elif kind == "gemm_q8":
            byts += w + 4 * c * batch + 4 * r * batch
            flops += 2 * r * c * batch
        elif kind == "writer":
            byts += 4 * r * c + w          # float32 weights in, the image out
        elif kind == "embed":
            byts += batch * (matrix_bytes(wt, sf, 1, c)) + 4 * batch + 4 * batch * c
    return byts, flops


def make_image(config, m, wt, sf, r, c):
    from block_quant_weight_amd import qmv as Q
    from block_quant_weight_amd import synth
    gq = synth.rng(config, m, synth.STREAM_QUANTS)
    gd = synth.rng(config, m, synth.STREAM_SCALES)
    q = synth.q8_quants(gq, r, c) if wt == Q8 else synth.q4_quants(gq, r, c)
    d = synth.scales(gd, r * c // 32, bool(sf))
    sp = Q.qmv_span(wt, sf, r, c)
    img = np.zeros(sp["min_span"], dtype=np.uint8)
    img[:sp["q_bytes"]] = q.view(np.uint8)
    img[sp["d_offset"]:] = d.view(np.uint8)
    return img


def writer_weights(config, m, r, c):
    """float32 weights for the writer workload: N(0,1) values drawn from the
    matrix's seeded activation stream."""
    from block_quant_weight_amd import synth
    g = synth.rng(config, m, synth.STREAM_ACT)
    return synth.act_f32(g, r, c)


def kernel_source_hash(src):
    """sha256[:16] of a kernel source file under block_quant_weight_amd/csrc."""
    with open(os.path.join(ROOT, "block_quant_weight_amd", "csrc", src), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_from_profiles(name, src):
    """HBM bytes per launch of the roofline's kernel from the committed
    counter summary, if it was taken on the kernel source as it stands."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            t = json.load(fh)
        if t.get("kernel_source_sha256_16") != kernel_source_hash(src):
            return None
        return t.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(kind, config, mats, batch, budget_s):
    """The oracle, as it stands, on this host's cores over a bounded sample."""
    import oracle as O
    from block_quant_weight_amd import synth
    threads = max(1, min(16, os.cpu_count() or 1))
    m, wt, sf, r, c = mats[0]
    img = make_image(config, m, wt, sf, r, c)
    if kind == "embed":
        ids = synth.token_ids(synth.rng(config, 0, synth.STREAM_IDS), batch, 3, r - 1)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < budget_s and reps < 100000:
            O.dequant_rows(img, wt, sf, r, c, ids.astype(np.int64))
            reps += 1
        el = time.perf_counter() - t0
        b, _ = step_work(kind, mats[:1], batch)
        return {"value": reps * b / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{reps} gathers of {batch} rows, single thread"}
    if kind in ("writer", "writer_search"):
        w = writer_weights(config, m, r, c)
        n_rows = 64 if kind == "writer" else 8
        reps = 0
        t0 = time.perf_counter()
        while True:
            lo = (reps * n_rows) % (r - n_rows)
            if kind == "writer":
                O.quantize_weights(wt, sf, n_rows, c, w[lo:lo + n_rows])
            else:
                O.quantize_q4_search(sf, n_rows, c, w[lo:lo + n_rows])
            reps += 1
            el = time.perf_counter() - t0
            if el >= 0.5 * budget_s or reps >= 10000:
                break
        byts = reps * n_rows * c * 4 + reps * n_rows * matrix_bytes(wt, sf, 1, c)
        return {"value": byts / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{reps} x {n_rows} rows of {r} (single thread, {el:.1f} s)"}
    if kind == "gemm_q8":
        x = synth.act_f32(synth.rng(config, m, synth.STREAM_ACT), batch, c)
        xq = np.zeros((batch, c), dtype=np.int8)
        dx = np.zeros((batch, c // 32), dtype=np.float32)
        for t in range(batch):
            xq[t], dx[t] = O.quantize_q8(x[t])
        probe = np.arange(min(r, 4), dtype=np.int64)
        t0 = time.perf_counter()
        O.gemm_q8act(img, wt, sf, r, c, xq, dx, sel=probe, threads=1)
        per_row = max((time.perf_counter() - t0) / probe.size, 1e-7)
        n_rows = int(min(r, max(threads, 0.5 * budget_s * threads / per_row)))
        sel = np.linspace(0, r - 1, n_rows).astype(np.int64)
        t0 = time.perf_counter()
        O.gemm_q8act(img, wt, sf, r, c, xq, dx, sel=sel, threads=threads)
        el = time.perf_counter() - t0
        ops = 2 * n_rows * c * batch
        return {"value": ops / el / 1e12, "unit": "TOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{n_rows} of {r} rows x {batch} tokens (int32 block sums, f64 "
                          f"combine, {threads} threads, {el:.1f} s)"}
    if kind == "gemm":
        x = synth.act_bf16(synth.rng(config, m, synth.STREAM_ACT), batch, c)
    else:
        x = synth.act_f32(synth.rng(config, m, synth.STREAM_ACT), batch, c)
    # rows per sample sized for about budget_s of work
    probe = np.arange(min(r, 16), dtype=np.int64)
    t0 = time.perf_counter()
    O.product(img, wt, sf, r, c, x, sel=probe, threads=1)
    per_row = max((time.perf_counter() - t0) / probe.size, 1e-7)
    n_rows = int(min(r, max(threads, budget_s * threads / per_row)))
    sel = np.linspace(0, r - 1, n_rows).astype(np.int64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.product(img, wt, sf, r, c, x, sel=sel, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 0.5 * budget_s or reps >= 1000:
            break
    frac = reps * n_rows / r
    if kind == "gemm":
        flops = 2 * reps * n_rows * c * batch
        return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle",
                "sample": f"{reps} x {n_rows} of {r} rows x {batch} tokens "
                          f"(f64, {threads} threads, {el:.1f} s)"}
    byts, _ = step_work(kind, [mats[0]], batch)
    return {"value": byts * frac / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {n_rows} of {r} rows of matrix 0, batch {batch} "
                      f"(f64, {threads} threads, {el:.1f} s)"}


def measure(name, args, stream, cpu_budget):
    """Times one workload; returns its JSON record (the printed line's fields)."""
    import torch
    from block_quant_weight_amd import qmv as Q
    from block_quant_weight_amd import synth

    desc, kind, config, mats, batch = workload(name)

    if kind == "copy":
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        return {"workload": "copy", "bytes_read": n, "bytes_written": n,
                "ms_per_copy": ms, "GB/s": 2 * n / ms / 1e6}

    if kind == "writer":
        return run_writer(args, name, desc, config, mats, stream, cpu_budget)
    if kind == "read":
        return read_stream(args, stream)
    if kind == "mfma":
        return mfma_rate(args, stream)

    groups = launch_groups(name, mats)
    gated = name == "decode_layer_gated"
    step_bytes, step_flops = step_work(kind, mats, batch, groups if kind == "gemv" else None,
                                       gated)
    set_bytes = sum(matrix_bytes(wt, sf, r, c) for _, wt, sf, r, c in mats)
    ncopies = max(2, -(-ROTATE_BYTES // set_bytes))
    if kind == "embed":
        ncopies = 1   # a gather touches 64 rows; rows are drawn afresh per step
    steps = args.steps if args.steps is not None else (200 if kind in ("gemm", "gemm_q8") else 1000)
    warmup = args.warmup if args.warmup is not None else 20
    log(f"workload {name}: {desc}; {ncopies} weight copies; "
        f"{steps} steps after {warmup} warm-up")

    imgs = {m: make_image(config, m, wt, sf, r, c) for (m, wt, sf, r, c) in mats}
    handles = []
    for _ in range(ncopies):
        hs = []
        for (m, wt, sf, r, c) in mats:
            h = Q.qmv_create(wt, sf, r, c)
            Q.qmv_upload(h, imgs[m], stream=stream)
            hs.append(h)
        handles.append(hs)
    del imgs
    log("weights uploaded")

    xs, ys = [], []
    shared = kind == "gemv" and len(groups) < len(mats)
    for pos, (m, wt, sf, r, c) in enumerate(mats):
        # a launch group's matrices share one activation vector (the group's
        # own seed stream); otherwise each matrix has its own
        gi = [i for i, gr in enumerate(groups) if pos in gr][0] if kind == "gemv" else 0
        g = synth.rng(config, 20 + gi if shared else m, synth.STREAM_ACT)
        if kind == "gemm":
            xb = synth.act_bf16(g, batch, c)
            xs.append(torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16))
        elif kind in ("gemv", "gemm_q8"):
            xs.append(torch.from_numpy(synth.act_f32(g, batch, c)).cuda())
        ys.append(torch.empty((batch, r), dtype=torch.float32, device="cuda"))
    # the int8 path's quantized activations (written by each step)
    xqs = [torch.empty((batch, c), dtype=torch.int8, device="cuda") for (_, _, _, _, c) in mats] \
        if kind == "gemm_q8" else []
    dxs = [torch.empty((batch, c // 32), dtype=torch.float32, device="cuda")
           for (_, _, _, _, c) in mats] if kind == "gemm_q8" else []
    id_sets = []
    if kind == "embed":
        r = mats[0][3]
        for k in range(64):
            ids = synth.token_ids(synth.rng(config, k, synth.STREAM_IDS), batch, 3, r - 1)
            id_sets.append(torch.from_numpy(ids).cuda())
        out = torch.empty((batch, mats[0][4]), dtype=torch.float32, device="cuda")

    def run_group(hs, gr):
        if gated and tuple(gr) == GATED_PAIR:
            Q.qmv_gemv_gated(hs[gr[0]], hs[gr[1]], xs[gr[0]], ys[gr[0]], act=Q.ACT_SILU)
        elif gated and gr[0] == GATED_NEXT:
            Q.qmv_gemv(hs[gr[0]], ys[GATED_PAIR[0]], ys[gr[0]])
        elif len(gr) == 1:
            Q.qmv_gemv(hs[gr[0]], xs[gr[0]], ys[gr[0]])
        else:
            Q.qmv_gemv_group([hs[j] for j in gr], xs[gr[0]], [ys[j] for j in gr])

    def step(i):
        hs = handles[i % ncopies]
        if kind == "gemv":
            for gr in groups:
                run_group(hs, gr)
            return
        for j, h in enumerate(hs):
            if kind == "gemv":
                Q.qmv_gemv(h, xs[j], ys[j])
            elif kind == "gemm":
                Q.qmv_gemm(h, xs[j], ys[j])
            elif kind == "gemm_q8":
                Q.qmv_quantize_q8(xs[j], xqs[j], dxs[j])
                Q.qmv_gemm_q8(h, xqs[j], dxs[j], ys[j])
            else:
                Q.qmv_embed_rows(h, id_sets[i % len(id_sets)], out)

    use_graph = not args.no_graph
    ms_step = timed_steps(step, steps, warmup, stream, use_graph, args.warm_seconds)
    log(f"timed {steps} steps: {ms_step * steps:.3f} ms")

    launches_per_step = len(groups) if kind == "gemv" else len(mats)
    if kind == "gemm":
        value, unit = step_flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        bound, peak, runit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
        dtype = "bf16"
    elif kind == "gemm_q8":
        value, unit = step_flops / (ms_step * 1e-3) / 1e12, "TOP/s"
        bound, peak, runit = "mfma", INT8_PEAK_TOPS, "TOP/s (int8)"
        dtype = "i8"
        launches_per_step = 2 * len(mats)
    else:
        value, unit = step_bytes / (ms_step * 1e-3) / 1e9, "GB/s"
        bound, peak, runit = "hbm", HBM_PEAK_GBS, "GB/s"
        dtype = "f32"
    # The roofline's kernel is the step's largest launch.  With one launch per
    # step it is the step; otherwise that launch alone is timed again the same
    # way (rotated copies, one captured graph, events on the launch stream).
    if kind == "gemv" and len(groups) > 1:
        # every launch of the step alone, each over its own >= 512 MB of
        # copies (the step's copies plus extra uploads of its matrices)
        per_launch = []
        for gr in groups:
            g_bytes, _ = step_work(kind, [mats[j] for j in gr], batch, [list(range(len(gr)))],
                                   gated)
            g_set = sum(matrix_bytes(*mats[j][1:]) for j in gr)
            g_copies = max(ncopies, -(-ROTATE_BYTES // g_set))
            g_handles = [{j: handles[k][j] for j in gr} for k in range(ncopies)]
            extra = []
            for _ in range(g_copies - ncopies):
                hs = {}
                for j in gr:
                    m, wt, sf, r, c = mats[j]
                    h = Q.qmv_create(wt, sf, r, c)
                    Q.qmv_upload(h, make_image(config, m, wt, sf, r, c), stream=stream)
                    hs[j] = h
                    extra.append(h)
                g_handles.append(hs)

            def launch(i, gr=gr, g_handles=g_handles, g_copies=g_copies):
                run_group(g_handles[i % g_copies], gr)
            g_ms = timed_steps(launch, steps, warmup, stream, use_graph, args.warm_seconds)
            for h in extra:
                Q.qmv_destroy(h)
            log(f"launch {[LAYER[j][0] for j in gr]} alone, {g_copies} copies: "
                f"{g_ms * 1e3:.3f} us")
            per_launch.append({"matrices": [LAYER[j][0] for j in gr] if name.startswith("decode")
                               else gr, "algorithmic_bytes_per_launch": g_bytes,
                               "us_per_launch": round(g_ms * 1e3, 3),
                               "GB/s": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
                               "copies_rotated": g_copies})
        # the roofline's kernel: the largest launch
        dom_desc = max(per_launch, key=lambda d: d["algorithmic_bytes_per_launch"])
        achieved = dom_desc["GB/s"]
        dom_desc = dict(dom_desc)
        dom_desc["every_launch"] = per_launch
    elif kind == "gemm_q8":
        # the int8 product alone (its activations quantized once, before the
        # graph), the same rotation and timing
        h0 = handles[0][0]
        for j in range(len(mats)):
            Q.qmv_quantize_q8(xs[j], xqs[j], dxs[j])

        def launch(i):
            Q.qmv_gemm_q8(handles[i % ncopies][0], xqs[0], dxs[0], ys[0])
        dom_ms = timed_steps(launch, steps, warmup, stream, use_graph, args.warm_seconds)
        achieved = step_flops / (dom_ms * 1e-3) / 1e12
        log(f"int8 product alone: {dom_ms * 1e3:.3f} us per launch (h {h0.rows}x{h0.cols})")
        dom_desc = {"int8_ops_per_launch": step_flops, "us_per_launch": round(dom_ms * 1e3, 3),
                    "bf16_peak_fraction": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = value
        dom_desc = {"algorithmic_bytes_per_launch": step_bytes if kind != "gemm" else None,
                    "flops_per_launch": step_flops if kind == "gemm" else None,
                    "us_per_launch": round(ms_step * 1e3, 3)}
    kname, ksrc = DOMINANT_KERNEL[name]
    traffic = traffic_from_profiles(name, ksrc)
    roof = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": kname, "launch": dom_desc,
            "launches_per_step": launches_per_step,
            "algorithmic_bytes_per_step": step_bytes, "flops_per_step": step_flops}
    cpu = None
    if cpu_budget > 0:
        log("timing the oracle on the host cores")
        cpu = cpu_baseline(kind, config, mats, batch, cpu_budget)
    for hs in handles:
        for h in hs:
            Q.qmv_destroy(h)
    del handles
    wl = {"workload": name, "description": desc, "config": config, "batch": batch,
          "matrices": [{"wtype": "Q8_0" if wt == Q8 else "Q4_0",
                        "scales": "f16" if sf else "f32", "rows": r, "cols": c}
                       for _, wt, sf, r, c in mats],
          "weight_copies_rotated": ncopies, "hip_graph": use_graph}
    return {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded; uniform quants and scales, N(0,1) "
                                "activations)",
        "config": wl, "roofline": roof, "cpu_baseline": cpu}


def run_writer(args, name, desc, config, mats, stream, cpu_budget):
    """The weight writer as a step: one qmv_quantize_weights call over a
    float32 matrix (rotated copies, >= 512 MB), captured in a graph."""
    import torch
    from block_quant_weight_amd import qmv as Q
    m, wt, sf, r, c = mats[0]
    step_bytes, _ = step_work("writer", mats, 1)
    search = "search" in name
    rule = Q.QMV_Q4_SEARCH if search else Q.QMV_Q4_ROUND
    w = torch.from_numpy(writer_weights(config, m, r, c)).cuda()
    ncopies = max(2, -(-ROTATE_BYTES // (4 * r * c)))
    ws = [w] + [w.clone() for _ in range(ncopies - 1)]
    n = Q.qmv_span(wt, sf, r, c)["min_span"]
    image = torch.empty(n, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 20
    log(f"workload {name}: {desc}; {ncopies} input copies; "
        f"{steps} steps after {warmup} warm-up")
    Q.qmv_quantize_weights(wt, sf, ws[0], image, status=status, rule=rule)
    torch.cuda.synchronize()
    if int(status[0].item()) != 0:
        raise RuntimeError("writer reported an unstorable scale")

    def step(i):
        Q.qmv_quantize_weights(wt, sf, ws[i % ncopies], image, status=status, rule=rule)
    use_graph = not args.no_graph
    ms_step = timed_steps(step, steps, warmup, stream, use_graph, args.warm_seconds)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kname, ksrc = DOMINANT_KERNEL[name]
    launch = {"algorithmic_bytes_per_launch": step_bytes, "us_per_launch": round(ms_step * 1e3, 3)}
    if search:
        # bound by float32 arithmetic, not by memory
        ops = SEARCH_OPS_PER_BLOCK * r * c // 32
        achieved = ops / (ms_step * 1e-3) / 1e12
        launch["f32_ops_per_launch"] = ops
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(F32_OPS_PEAK_T, 3),
                "unit": "Tops/s (float32, unfused)", "frac": round(achieved / F32_OPS_PEAK_T, 4),
                "traffic": traffic_from_profiles(name, ksrc), "kernel": kname,
                "launch": launch, "launches_per_step": 1,
                "algorithmic_bytes_per_step": step_bytes, "flops_per_step": ops}
    else:
        roof = {"bound": "hbm", "achieved": round(value, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles(name, ksrc), "kernel": kname,
                "launch": launch, "launches_per_step": 1,
                "algorithmic_bytes_per_step": step_bytes, "flops_per_step": None}
    cpu = None
    if cpu_budget > 0:
        log("timing the oracle on the host cores")
        cpu = cpu_baseline("writer_search" if search else "writer", config, mats, 1, cpu_budget)
    wl = {"workload": name, "description": desc, "config": config, "batch": 1,
          "matrices": [{"wtype": "Q8_0" if wt == Q8 else "Q4_0", "scales": "f16" if sf else "f32",
                        "rows": r, "cols": c}],
          "input_copies_rotated": ncopies, "hip_graph": use_graph}
    return {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; N(0,1) float32 weights)", "config": wl,
        "roofline": roof, "cpu_baseline": cpu}


def timed_steps(step, steps, warmup, stream, use_graph, warm_seconds):
    """ms per step of step(i) for i in [warmup, warmup + steps): warmup
    eager calls, then (use_graph) one captured graph of the timed steps,
    replayed untimed for at least warm_seconds and then once under HIP events
    on the launching stream (without a graph: the steps themselves, repeated
    for the warm-up time, then once timed)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                step(warmup + i)
        run = g.replay
    else:
        def run():
            for i in range(steps):
                step(warmup + i)
    t0 = time.perf_counter()
    while True:
        run()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_seconds:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# Read-ceiling sizes: the algorithmic bytes of each GEMV configuration's
# largest launch, plus a spread of sizes around them.
READ_SIZES = [1 << 18, 1 << 20, 1 << 22, 1 << 23, 1 << 24, 1 << 25, 1 << 26, 1 << 27, 1 << 28]


def read_ceiling(nbytes, stream, args, steps=None):
    """GB/s of qmv_read_probe over nbytes, each launch on a different part of
    a buffer of >= 512 MB (every read from HBM), timed like a workload."""
    import torch
    from block_quant_weight_amd import qmv as Q
    n = (nbytes + 255) // 256 * 256
    copies = max(2, -(-ROTATE_BYTES // n))
    buf = torch.empty(copies * n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    nb = nbytes // 16 * 16
    if steps is None:
        steps = 1000 if nbytes < (64 << 20) else 100

    def step(i):
        k = i % copies
        Q.qmv_read_probe(buf[k * n:(k + 1) * n], nb, sink)
    ms = timed_steps(step, steps, 5, stream, not args.no_graph, min(args.warm_seconds, 0.2))
    del buf
    return {"bytes": nb, "us_per_read": round(ms * 1e3, 3), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": copies}


def read_stream(args, stream):
    """The read ceiling over READ_SIZES and the GEMV configurations' launch sizes."""
    sizes = sorted(set(READ_SIZES + [b for b in GEMV_LAUNCH_BYTES.values()]))
    res = [read_ceiling(b, stream, args) for b in sizes]
    for r in res:
        log(f"read ceiling {r['bytes']:>11,d} B: {r['us_per_read']:9.3f} us, {r['GB/s']:7.1f} GB/s")
    best = max(res, key=lambda r: r["GB/s"])
    return {"metric": "read ceiling GB/s (qmv_read_probe)", "value": best["GB/s"], "unit": "GB/s",
            "n_gpus": 1, "higher_is_better": True, "config": {"workload": "read_stream"},
            "ceilings": res}


MFMA_FLOPS = 32 * 32 * 16 * 2  # one v_mfma_f32_32x32x16_f16


def mfma_rate(args, stream, iters=4096, reps=5):
    """Back-to-back rate of the prefill product's matrix-core instruction
    (qmv_mfma_probe) at one and two waves per SIMD, on constant and on
    pseudo-random operands: TFLOP/s from the launches' HIP-event time, the
    cycles per product and the clock from the waves' own counters."""
    import torch
    from block_quant_weight_amd import qmv as Q
    res = []
    for wps in (1, 2):
        waves = 1024 * wps
        clocks = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
        sink = torch.zeros(64 * waves, dtype=torch.float32, device="cuda")
        for rnd in (0, 1):
            for _ in range(2):
                Q.qmv_mfma_probe(rnd, wps, iters, clocks, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                Q.qmv_mfma_probe(rnd, wps, iters, clocks, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            c = clocks.view(-1, 2).double().cpu()
            cyc, ticks = c[:, 0].mean().item(), c[:, 1].mean().item()
            products = 8 * iters
            r = {"waves_per_simd": wps, "operands": "random" if rnd else "constant",
                 "us_per_launch": round(ms * 1e3, 2),
                 "TFLOP/s": round(MFMA_FLOPS * products * waves / (ms * 1e-3) / 1e12, 1),
                 "frac_of_peak": round(MFMA_FLOPS * products * waves / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "cycles_per_product_per_wave": round(cyc / products, 2),
                 "clock_GHz": round(cyc / (ticks / 100e6) / 1e9, 3)}
            res.append(r)
            log(f"mfma rate, {wps} wave(s) per SIMD, {r['operands']} operands: {r['TFLOP/s']:.0f} TFLOP/s, "
                f"{r['cycles_per_product_per_wave']:.1f} cycles per product per wave, clock {r['clock_GHz']:.2f} GHz")
    best = max((r for r in res if r["operands"] == "random"), key=lambda r: r["TFLOP/s"])
    return {"metric": "matrix-core rate TFLOP/s (qmv_mfma_probe, random operands)", "value": best["TFLOP/s"],
            "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True, "config": {"workload": "mfma_rate"},
            "rates": res}


def gemv_launch_bytes(name):
    """Algorithmic bytes of each launch of a GEMV workload's step."""
    desc, kind, config, mats, batch = workload(name)
    groups = launch_groups(name, mats)
    gated = name == "decode_layer_gated"
    return [step_work(kind, [mats[j] for j in gr], batch, [list(range(len(gr)))], gated)[0]
            for gr in groups]


GEMV_WORKLOADS = ("q8_gemv_512", "q4_gemv_4096", "decode_layer", "lm_head_b1", "lm_head_b64")
GEMV_LAUNCH_BYTES = {}
for _n in GEMV_WORKLOADS:
    for _k, _b in enumerate(gemv_launch_bytes(_n)):
        GEMV_LAUNCH_BYTES[(_n, _k)] = _b

# the default run: every configuration, headline first in importance
ALL = ["q8_gemv_512", "q4_gemv_4096", "decode_layer", "gemm_q4_14336x4096",
       "gemm_q8_4096x14336", "lm_head_b1", "lm_head_b64", "embed_64"]
HEADLINE = "lm_head_b1"


def with_ceiling(rec, name, args, stream):
    """Adds the read ceiling at each launch's byte count to a GEMV record."""
    roof = rec["roofline"]
    launches = roof["launch"].get("every_launch") or [dict(roof["launch"], **{"GB/s": roof["achieved"]})]
    out = []
    for k, ln in enumerate(launches):
        c = read_ceiling(GEMV_LAUNCH_BYTES[(name, k)], stream, args)
        out.append({"matrices": ln.get("matrices", [0]), "bytes": c["bytes"],
                    "launch_GB/s": ln["GB/s"], "ceiling_GB/s": c["GB/s"],
                    "ceiling_us": c["us_per_read"],
                    "frac_of_ceiling": round(ln["GB/s"] / c["GB/s"], 4)})
        log(f"{name} launch {k}: {ln['GB/s']:.1f} GB/s against a read ceiling of "
            f"{c['GB/s']:.1f} GB/s at {c['bytes']:,d} B")
    roof["read_ceiling"] = out


def with_mfma_ceiling(rec, ceiling):
    """Adds the matrix-core instruction's own rate on random operands at two
    waves per SIMD (the product's occupancy) to a prefill GEMM record."""
    c = next(r for r in ceiling["rates"] if r["operands"] == "random" and r["waves_per_simd"] == 2)
    roof = rec["roofline"]
    roof["mfma_ceiling"] = {"TFLOP/s": c["TFLOP/s"], "clock_GHz": c["clock_GHz"],
                            "frac_of_ceiling": round(roof["achieved"] / c["TFLOP/s"], 4),
                            "probe": "qmv_mfma_probe, v_mfma_f32_32x32x16_f16 back to back, random operands"}
    log(f"{rec['config']['workload']}: {roof['achieved']:.1f} TFLOP/s against the matrix cores' "
        f"{c['TFLOP/s']:.1f} TFLOP/s on random operands")


def summary(rec):
    wl = rec["config"]
    return {"config": wl.get("config"), "description": wl.get("description"),
            "value": rec["value"], "unit": rec["unit"], "ms_per_step": rec["ms_per_step"],
            "steps": rec["steps"], "roofline": rec["roofline"],
            "cpu_baseline": rec["cpu_baseline"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=None,
                    help="seconds of oracle time per workload (default 10 for one "
                         "workload, 3 each for the default run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed replays of the step graph before timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the product runs on a single MI355X; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    # One side stream for warm-up, capture and timing: the library keeps its
    # split-K workspace per stream, so the capture stream must be warmed up.
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    if args.workload != "all":
        budget = 0.0 if args.no_cpu_baseline else (args.cpu_budget or 10.0)
        rec = measure(args.workload, args, stream, budget)
        print(json.dumps(rec), flush=True)
        return
    budget = 0.0 if args.no_cpu_baseline else (args.cpu_budget or 3.0)
    recs = {}
    for name in ALL:
        log(f"=== {name}")
        recs[name] = measure(name, args, stream, budget)
        if name in GEMV_WORKLOADS:
            with_ceiling(recs[name], name, args, stream)
        if name.startswith("gemm_"):
            if "mfma" not in recs:
                recs["mfma"] = mfma_rate(args, stream)
            with_mfma_ceiling(recs[name], recs["mfma"])
        torch.cuda.empty_cache()
    recs.pop("mfma", None)
    head = dict(recs[HEADLINE])
    head["configs"] = {name: summary(r) for name, r in recs.items()}
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
