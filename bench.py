#!/usr/bin/env python3
"""Benchmark of the GALE 1-bit routed-expert matmul on one MI355X.

Step = one decode token (batch 1) through the full resident stack of
DeepSeek-V4-Flash-shaped routed experts: 43 layers x 256 experts x {w1, w3, w2}
(33,024 packed matrices, 46.0 GB in HBM), each layer routing the token to its
top-6 experts and combining their SwiGLU FFN outputs.  Inputs are seeded
synthetic data of the model card's shapes (no weights or datasets are used).

Reported:
  value        packed expert-weight bytes touched per token (258 experts) / step time, GB/s
  tokens_per_s steps per second
  roofline     the GEMV kernel at its sustained launch shape: one launch over 1024
               distinct [2048, 4096] matrices of the resident stack (w1 and w3 of 512
               experts), one token each, timed with HIP events; algorithmic bytes
               1,405,952 per matrix
  cpu_baseline the fp64 oracle on the host for a bounded sample of the same step
               (its outputs also check the GPU step at full size)
  stream_ceiling  a plain elementwise kernel (negate, fp32) over a 1 GiB buffer: the
               HBM rate a trivial streaming kernel reaches on this device; it is also the
               known-size reference that scales the HBM byte counters behind "traffic"

"traffic" is read from profiles/gemv_kernel_traffic.txt, written from two rocprofv3
--pmc runs (FETCH_SIZE, WRITE_SIZE) of this script; it is reported only while the
SHA-256 of the GEMV kernel sources still matches the one recorded there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HIDDEN, INTER, EXPERTS, TOPK = 4096, 2048, 256, 6
W13_BYTES = 1_393_664          # one [2048, 4096] matrix, 41 outliers per row
W2_BYTES = 1_392_640           # one [4096, 2048] matrix, 20 outliers per row
EXPERT_BYTES = 2 * W13_BYTES + W2_BYTES
GEMV_UNIT_BYTES = W13_BYTES + 2 * HIDDEN + 2 * INTER   # weights + fp16 x + fp16 y
HBM_PEAK_GBPS = 8000.0
GEMV_WARM_CALLS = 10
DECODE_BATCHES = (1, 4, 16, 32)
PREFILL_TOKENS = 2048
PREFILL_FLOP = 2 * TOPK * PREFILL_TOKENS * 3 * INTER * HIDDEN      # dense-equivalent, 618.5 GFLOP
MFMA_FP16_PEAK_TFLOPS = 2500.0
CEIL_BYTES = 1 << 30            # one side of the streaming-ceiling kernel
GEMV_SOURCES = ("gale_gemv.hip", "gale_gemv_core.h", "gale_decode.h", "gale_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_kernel_traffic.txt")


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, "quantized_expert_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(n_mats: int):
    """HBM bytes per sustained-GEMV launch from the committed counter summary, or None
    when it is absent, was taken at another launch size, or predates the kernel sources."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ":" in l)
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("source_sha256") != gemv_source_hash() or int(kv.get("matrices_per_launch", -1)) != n_mats:
            return None
        return int(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_stack(q, synth, layers: int, seed: int, dev):
    """Generate, pack and keep the resident stack; returns per-layer expert tables and
    the flat list of the [2048, 4096] matrices (w1, w3 of every expert, in memory order)
    for the sustained GEMV."""
    import torch
    tables, w13_all = [], []
    for l in range(layers):
        b13 = synth.gen_matrix_bank(seed, [(l, e, m) for e in range(EXPERTS) for m in (0, 1)], INTER, HIDDEN,
                                    device=dev)
        s13, c13 = q.pack_device(INTER, HIDDEN, 2 * EXPERTS, b13["signs"], b13["block_scales"])
        del b13["signs"], b13["block_scales"]
        b2 = synth.gen_matrix_bank(seed, [(l, e, 2) for e in range(EXPERTS)], HIDDEN, INTER, device=dev)
        s2, c2 = q.pack_device(HIDDEN, INTER, EXPERTS, b2["signs"], b2["block_scales"])
        del b2["signs"], b2["block_scales"]
        nw13, ns13 = INTER * HIDDEN // 32, INTER * HIDDEN // 128
        nw2, ns2 = HIDDEN * INTER // 32, HIDDEN * INTER // 128

        def mat13(i):
            return q.PackedMatrix(INTER, HIDDEN, s13[i * nw13:(i + 1) * nw13], c13[i * ns13:(i + 1) * ns13],
                                  b13["row_scales"], b13["row_ptr"], b13["out_cols"][i], b13["out_vals"][i])

        def mat2(i):
            return q.PackedMatrix(HIDDEN, INTER, s2[i * nw2:(i + 1) * nw2], c2[i * ns2:(i + 1) * ns2],
                                  b2["row_scales"], b2["row_ptr"], b2["out_cols"][i], b2["out_vals"][i])

        experts = [(mat13(2 * e), mat13(2 * e + 1), mat2(e)) for e in range(EXPERTS)]
        tables.append(q.expert_table(experts))
        w13_all.extend(m for e in experts for m in e[:2])
        if l % 8 == 7 or l == layers - 1:
            torch.cuda.synchronize()
            log(f"stack: {l + 1}/{layers} layers resident, "
                f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")
    return tables, w13_all


def time_events(fn, reps: int):
    """Average milliseconds per call of fn over reps calls, HIP events on the current stream."""
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def cpu_baseline(synth, O, seed, xs, logits, gpu_y, n_layers):
    """Oracle on the host for the first n_layers of the step; returns timing and parity."""
    import numpy as np
    from threadpoolctl import threadpool_info
    t_total, errs = 0.0, []
    for l in range(n_layers):
        lg = logits[l].cpu().numpy()
        x = xs[l].cpu().numpy()
        idx, _ = O.route(lg, TOPK)
        mats = {}
        for e in idx[0]:
            e = int(e)
            mats[e] = tuple(synth.gen_matrix(seed, (l, e, m), r, c).numpy()
                            for m, r, c in ((0, INTER, HIDDEN), (1, INTER, HIDDEN), (2, HIDDEN, INTER)))
        t0 = time.perf_counter()
        yref, _, _ = O.moe(lambda e: mats[e], lg, x, k=TOPK)
        t_total += time.perf_counter() - t0
        errs.append(float(O.rel_l2(gpu_y[l].float().cpu().numpy().astype(np.float64), yref).max()))
    per_token = t_total / n_layers * 43
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return per_token, threads, max(errs)


SWEEP_SHAPES = ((2048, 4096, 0.01), (2048, 4096, 0.02), (2048, 4096, 0.03), (2048, 4096, 0.05),
                (3072, 7168, 0.01), (7168, 3072, 0.01))


def packed_matrix_bytes(rows: int, cols: int, frac: float) -> int:
    """Bytes of one packed matrix: signs, fp16 block scales, uint16 outlier columns,
    int4 outlier values, fp16 row scales (round(frac * cols) outliers per row)."""
    import synth
    nnz = rows * synth.n_outliers(cols, frac)
    return rows * cols // 8 + rows * cols // 128 * 2 + 2 * nnz + (nnz + 1) // 2 + 2 * rows


def sweep_gemv(q, synth, lib, dev, seed, reps: int, warm_s: float):
    """Sustained GEMV (one launch over >= 1 GB of distinct matrices, one token each) across
    outlier budgets and matrix shapes: GB/s of algorithmic bytes against bits per weight."""
    import torch
    res = []
    for rows, cols, frac in SWEEP_SHAPES:
        unit = packed_matrix_bytes(rows, cols, frac)
        # a power of two of at least 512 matrices and 1 GB per set: the persistent workgroups'
        # runs of units then start on matrix boundaries, as in the main measurement
        n = 512
        while n * unit < (1 << 30):
            n *= 2
        sets = []
        for k in range(2):                       # two disjoint sets, alternated
            b = synth.gen_matrix_bank(seed, [(0x50000 + k, rows, int(frac * 1000), i) for i in range(n)], rows, cols,
                                      outlier_frac=frac, device=dev)
            sg, sc = q.pack_device(rows, cols, n, b["signs"], b["block_scales"])
            del b["signs"], b["block_scales"]
            nw, ns = rows * cols // 32, rows * cols // 128
            mats = [q.PackedMatrix(rows, cols, sg[i * nw:(i + 1) * nw], sc[i * ns:(i + 1) * ns], b["row_scales"],
                                   b["row_ptr"], b["out_cols"][i], b["out_vals"][i]) for i in range(n)]
            sets.append((q.matrix_table(mats), mats, sg, sc, b))
        from synth import gen_x
        xg = torch.stack([gen_x(seed, (0x51000 + i,), 1, cols, device=dev) for i in range(n)])
        rec = q.prepare_activations(xg)
        yg = torch.empty(n, 1, rows, dtype=torch.float16, device=dev)
        flip = [0]
        stage = q.gale_outlier_stage_flag(sets[0][0].outliers_per_row)

        def call():
            t = sets[flip[0]][0]
            flip[0] ^= 1
            rc = lib.gale_expert_gemv(rows, cols, t.ptr(), n, rec.data_ptr(), q.GALE_F16, 0, 1, yg.data_ptr(),
                                      q.GALE_F16, None, 0, q.GALE_X_PREPARED | stage,
                                      torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(lib.gale_last_error().decode())

        t_w = time.time()                       # steady clocks first, as for the main measurement
        while time.time() - t_w < warm_s:
            for _ in range(8):
                call()
            torch.cuda.synchronize()
        for _ in range(GEMV_WARM_CALLS):
            call()
        torch.cuda.synchronize()
        ms = time_events(call, reps)
        bytes_launch = n * (unit + 2 * cols + 2 * rows)
        gbps = bytes_launch / (ms * 1e-3) / 1e9
        bpw = 8.0 * unit / (rows * cols)
        log(f"sweep: [{rows}, {cols}] outliers {frac:.0%} ({bpw:.3f} b/w): {n} matrices in {ms * 1e3:.1f} us -> "
            f"{gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
        res.append({"rows": rows, "cols": cols, "outlier_frac": frac, "bits_per_weight": round(bpw, 4),
                    "outlier_stage": stage >> q.GALE_OUTLIER_STAGE_SHIFT,
                    "matrices_per_launch": n, "avg_launch_us": round(ms * 1e3, 2), "gbps": round(gbps, 1),
                    "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        del sets, rec, yg, xg
        torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=43)
    ap.add_argument("--gemv-mats", type=int, default=1024)
    ap.add_argument("--gemv-reps", type=int, default=50)
    ap.add_argument("--device-warm-s", type=float, default=1.0)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--cpu-layers", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the sustained GEMV at outlier budgets 1/2/3/5 %% and the DeepSeek-V4-Pro shapes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (the whole 46 GB stack fits one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    import quantized_expert_gemv_amd as q
    import synth
    from synth import config_seed, gen_logits_normal, gen_logits_zipf, gen_x

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lib = q.lib()
    dev = torch.device("cuda:0")
    seed = config_seed(4)
    L = args.layers

    t0 = time.time()
    tables, w13_all = build_stack(q, synth, L, seed, dev)
    log(f"stack built in {time.time() - t0:.1f}s")

    # ---- sustained GEMV: one launch over n distinct resident matrices, one token each
    n = min(args.gemv_mats, len(w13_all) // 2)
    sets = [q.matrix_table(w13_all[i * n:(i + 1) * n]) for i in range(2)]     # two disjoint sets, alternated
    xg = torch.stack([gen_x(seed, (0x30000 + i,), 1, HIDDEN, device=dev) for i in range(n)])
    rec = q.prepare_activations(xg)
    yg = torch.empty(n, 1, INTER, dtype=torch.float16, device=dev)
    gemv_args = [(INTER, HIDDEN, t.ptr(), n, rec.data_ptr(), q.GALE_F16, 0, 1, yg.data_ptr(), q.GALE_F16, None, 0,
                  q.GALE_X_PREPARED) for t in sets]
    flip = [0]

    def gemv_call():
        a = gemv_args[flip[0]]
        flip[0] ^= 1
        rc = lib.gale_expert_gemv(*a, torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(lib.gale_last_error().decode())

    # The device reaches its steady clocks only after some time under load: stream the
    # sustained-GEMV pool for a while before any timed region.
    t_w = time.time()
    while time.time() - t_w < args.device_warm_s:
        for _ in range(16):
            gemv_call()
        torch.cuda.synchronize()
    for _ in range(GEMV_WARM_CALLS):
        gemv_call()
    torch.cuda.synchronize()
    ms_gemv = time_events(gemv_call, args.gemv_reps)
    gemv_gbps = n * GEMV_UNIT_BYTES / (ms_gemv * 1e-3) / 1e9
    log(f"sustained GEMV: {n} matrices in {ms_gemv * 1e3:.1f} us -> {gemv_gbps:.0f} GB/s "
        f"({100 * gemv_gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    sweep = sweep_gemv(q, synth, lib, dev, seed, args.gemv_reps, args.device_warm_s) if args.sweep else None


    xs = [gen_x(seed, (0x10000 + l,), 1, HIDDEN, device=dev) for l in range(L)]
    logits = [gen_logits_normal(seed, (0x20000 + l,), 1, EXPERTS, device=dev) for l in range(L)]
    ys = [torch.empty(1, HIDDEN, dtype=torch.float16, device=dev) for _ in range(L)]
    idxs = [torch.empty(1, TOPK, dtype=torch.int32, device=dev) for _ in range(L)]
    wts = [torch.empty(1, TOPK, dtype=torch.float32, device=dev) for _ in range(L)]
    ws = torch.empty(q.moe_workspace_bytes(1, EXPERTS, TOPK, HIDDEN, INTER), dtype=torch.uint8, device=dev)
    args_per_layer = [(HIDDEN, INTER, tables[l].ptr(), EXPERTS, logits[l].data_ptr(), TOPK, xs[l].data_ptr(), 1,
                       ys[l].data_ptr(), idxs[l].data_ptr(), wts[l].data_ptr(), ws.data_ptr(), ws.numel(), 0)
                      for l in range(L)]

    def step():
        st = torch.cuda.current_stream().cuda_stream
        for a in args_per_layer:
            rc = lib.gale_moe_layer_fwd(*a, st)
            if rc:
                raise RuntimeError(lib.gale_last_error().decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    y_eager = [y.clone() for y in ys]
    ms_eager = time_events(step, args.steps)
    torch.cuda.synchronize()
    log(f"eager step: {ms_eager * 1e3:.1f} us/token")

    ms_graph = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        ok = True
        for r in range(3):
            for y in ys:
                y.zero_()
            g.replay()
            torch.cuda.synchronize()
            ok = ok and all(torch.equal(a, b) for a, b in zip(ys, y_eager))
            step()                                  # eager work between replays
            torch.cuda.synchronize()
        if ok:
            for _ in range(args.warmup):
                g.replay()
            ms_graph = time_events(g.replay, args.steps)
            log(f"graph step: {ms_graph * 1e3:.1f} us/token")
        else:
            log("graph replay differs from eager: graph timing not used")
    torch.cuda.synchronize()

    ms_step = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    bytes_per_token = 43 * TOPK * EXPERT_BYTES * L // 43
    gbps = bytes_per_token / (ms_step * 1e-3) / 1e9

    # ---- one MoE layer at decode batches of 1, 4, 16 and 32 tokens (N(0,1) logits, top-6):
    #      the layers of the stack in turn, so every call streams its experts from HBM
    import numpy as np
    batches = []
    for T in DECODE_BATCHES:
        xb = [gen_x(seed, (0x60000 + T, l), T, HIDDEN, device=dev) for l in range(L)]
        lb = [gen_logits_normal(seed, (0x60000 + T, l), T, EXPERTS, device=dev) for l in range(L)]
        yb = torch.empty(T, HIDDEN, dtype=torch.float16, device=dev)
        wsb = torch.empty(q.moe_workspace_bytes(T, EXPERTS, TOPK, HIDDEN, INTER), dtype=torch.uint8, device=dev)
        uniq = [int(np.unique(torch.topk(lb[l], TOPK, dim=1).indices.cpu().numpy()).size) for l in range(L)]
        cur = [0]

        def layer_call():
            l = cur[0]
            cur[0] = (l + 1) % L
            rc = lib.gale_moe_layer_fwd(HIDDEN, INTER, tables[l].ptr(), EXPERTS, lb[l].data_ptr(), TOPK,
                                        xb[l].data_ptr(), T, yb.data_ptr(), None, None, wsb.data_ptr(), wsb.numel(),
                                        0, torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(lib.gale_last_error().decode())

        for _ in range(L):
            layer_call()
        torch.cuda.synchronize()
        cur[0] = 0
        reps = 2 * L
        ms_layer = time_events(layer_call, reps)
        u_mean = sum(uniq[i % L] for i in range(reps)) / reps
        gb = u_mean * EXPERT_BYTES / (ms_layer * 1e-3) / 1e9
        batches.append({"tokens": T, "us_per_layer": round(ms_layer * 1e3, 2), "unique_experts": round(u_mean, 1),
                        "gbps": round(gb, 1), "frac_of_peak": round(gb / HBM_PEAK_GBPS, 4),
                        "tokens_per_s_per_layer": round(T / (ms_layer * 1e-3), 1)})
        log(f"decode layer T={T}: {ms_layer * 1e3:.1f} us, {u_mean:.1f} experts -> {gb:.0f} GB/s "
            f"({100 * gb / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
        del wsb

    # ---- grouped prefill: one layer of the stack, 2048 tokens, Zipf(1.1)-skewed top-6
    xp = gen_x(seed, (0x40000,), PREFILL_TOKENS, HIDDEN, device=dev)
    lgp = gen_logits_zipf(seed, (0x40000,), PREFILL_TOKENS, EXPERTS, device=dev)
    ypf = torch.empty(PREFILL_TOKENS, HIDDEN, dtype=torch.float16, device=dev)
    wsp = torch.empty(q.moe_workspace_bytes(PREFILL_TOKENS, EXPERTS, TOPK, HIDDEN, INTER, 0), dtype=torch.uint8,
                      device=dev)

    def prefill():
        rc = lib.gale_moe_layer_fwd(HIDDEN, INTER, tables[0].ptr(), EXPERTS, lgp.data_ptr(), TOPK, xp.data_ptr(),
                                    PREFILL_TOKENS, ypf.data_ptr(), None, None, wsp.data_ptr(), wsp.numel(), 0,
                                    torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(lib.gale_last_error().decode())

    for _ in range(2):
        prefill()
    torch.cuda.synchronize()
    ms_prefill = time_events(prefill, args.prefill_reps)
    prefill_tflops = PREFILL_FLOP / (ms_prefill * 1e-3) / 1e12
    log(f"grouped prefill: {PREFILL_TOKENS} tokens in {ms_prefill:.3f} ms -> "
        f"{PREFILL_TOKENS / ms_prefill * 1e3:.0f} tokens/s, {prefill_tflops:.1f} dense-equivalent TFLOP/s")
    del wsp

    # ---- streaming ceiling: a plain elementwise kernel of known size (read 1 GiB, write 1 GiB)
    src = torch.ones(CEIL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    ms_ceil = time_events(lambda: torch.neg(src, out=dst), 10)
    ceil_gbps = 2 * CEIL_BYTES / (ms_ceil * 1e-3) / 1e9
    del src, dst
    log(f"streaming ceiling (elementwise negate, 2 x 1 GiB): {ceil_gbps:.0f} GB/s")
    traffic = recorded_traffic(n)

    out = {
        "metric": "packed-weight GB/s & % HBM peak; tokens/s per 43-layer MoE expert stack",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp4-e2m1 MFMA (exact 0/1 sign planes, 4-term fp8 activation split), fp32 accumulate, fp16 io",
        "data": "synthetic (seeded DeepSeek-V4-Flash-shaped GALE 1-bit experts; no weights)",
        "config": {"workload": f"decode batch 1 through the resident {L}-layer GALE expert stack "
                               f"({L} x 256 experts x w1/w3 [2048,4096] + w2 [4096,2048], "
                               f"{L * EXPERTS * EXPERT_BYTES / 1e9:.2f} GB), top-6 routing per layer",
                   "layers": L, "experts": EXPERTS, "top_k": TOPK, "batch": 1, "hidden": HIDDEN,
                   "inter": INTER, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(1e3 / ms_step, 2),
        "hbm_frac_step": round(gbps / HBM_PEAK_GBPS, 4),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "bytes_per_token": bytes_per_token,
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "gemv_kernel<1,4,false,512,2> (fp4 sign-plane MFMA GEMV)",
                     "launch": f"{n} distinct [2048,4096] matrices (w1, w3 of {n // 2} experts) x 1 token, "
                               f"prepared activations; two disjoint sets alternated",
                     "bytes_per_launch": n * GEMV_UNIT_BYTES, "avg_launch_us": round(ms_gemv * 1e3, 2),
                     "source_sha256": gemv_source_hash()[:16]},
        "decode_batches": {"workload": "one MoE layer (256 experts, N(0,1) logits, top-6), the stack's layers in "
                                       "turn; GB/s on the unique experts' packed bytes", "batches": batches},
        "prefill": {"workload": f"one layer (256 experts), {PREFILL_TOKENS} tokens x hidden {HIDDEN} fp16, "
                                f"Zipf(1.1) top-6 routing, grouped path",
                    "ms": round(ms_prefill, 4), "tokens_per_s": round(PREFILL_TOKENS / ms_prefill * 1e3, 1),
                    "dense_equiv_tflops": round(prefill_tflops, 2),
                    "frac_of_fp16_mfma_peak": round(prefill_tflops / MFMA_FP16_PEAK_TFLOPS, 4)},
        "gemv_sweep": sweep,
        "stream_ceiling": {"value": round(ceil_gbps, 1), "unit": "GB/s",
                           "kernel": "torch.neg fp32, read 1 GiB + write 1 GiB"},
    }

    if not args.no_cpu:
        import oracle as O
        per_tok, threads, err = cpu_baseline(synth, O, seed, xs, logits, ys, min(args.cpu_layers, L))
        out["cpu_baseline"] = {"value": round(bytes_per_token / per_tok / 1e9, 4), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "tokens_per_s": round(1.0 / per_tok, 5),
                               "sample": f"1 token through {min(args.cpu_layers, L)} layers (route + 6 fp64 "
                                         f"dequantize/matvec FFNs each), scaled to 43 layers"}
        out["parity_rel_l2_sampled_layers"] = err
        log(f"cpu oracle: {per_tok:.1f} s/token; GPU vs oracle rel-L2 {err:.2e}")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
