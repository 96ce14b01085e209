#!/usr/bin/env python3
"""Benchmark of the compressed-weight product on one MI355X.

Headline (one JSON line on stdout): decode GEMV of the Llama-70B gate/up
projection, K = 8192 inputs x N = 28672 outputs, group RTN 4-bit, groups of
64 with fp16 scale + offset, bf16 activations, batch 1.  A step is one
launch of that GEMV on the next copy of a rotating pool of distinct packed
weights (>= 2 GiB, larger than the 256 MB Infinity Cache plus L2, so every
step streams its bytes from HBM).  value = compressed bytes per step x steps
/ wall time of the timed region (inputs resident in HBM, bracketed by
torch.cuda.synchronize()).

Also reported:
  roofline      HBM bytes/launch (algorithmic: codes + meta) / average kernel
                time measured with HIP events on the launch stream, against the
                8 TB/s HBM3E peak; `traffic` comes from the committed rocprofv3
                FETCH_SIZE/WRITE_SIZE summary when it matches the current kernel
                source, else null.
  cpu_baseline  the fp64 CPU oracle (unpack codes, rebuild W_hat, multiply) on a
                bounded sample of rows of the same matrix.
  rows          every other row of the hot path, timed the same way: batch 16,
                the mixed-width layer shapes, the binary low-rank GEMV, prefill
                GEMM in both formats (MFMA utilisation), whole-layer tok/s
                equivalents.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = ["compressed_gemv_amd/csrc/gemv_kernels.hpp", "compressed_gemv_amd/csrc/gemv_group.hip",
                  "compressed_gemv_amd/csrc/common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_b1_gate_8192x28672_4b_g64.md")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """Bytes/launch from the committed pmc summary, if it matches the source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--pool-gib", type=float, default=2.0)
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one plain 1 GiB device copy (pmc calibration)")
    ap.add_argument("--only", default="",
                    help="comma-separated substrings: measure only the rows whose names contain one (profiling)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read reference")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(the product shards by output rows with no exchange; see the design notes). "
                         "Run with --gpus 1.\n")
        sys.exit(2)

    import numpy as np
    import torch

    import compressed_gemv_amd as cg
    from workloads import LAYER_SHAPES, MIXED_SETS, N_LAYERS, ATTN, layer_weights, layer_x, binlr_factors

    cg.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(a):
        return to_dev(a.view(np.int16)).view(torch.bfloat16)

    def pool_of(tensors, nbytes):
        n = max(2, int(args.pool_gib * (1 << 30) // nbytes) + 1)
        return [tuple(t.clone() for t in tensors) for _ in range(n)]

    def capture(fn, idx):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in idx:
                    fn(i)
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        return g

    def time_launches(fn, steps, warmup, period=None):
        """(wall seconds, event seconds) over exactly `steps` launches after `warmup`.

        The `steps` launches (launch i on rotating-pool copy i) are captured
        into one HIP graph and replayed once inside the timed region, so the
        host's per-call cost (Python binding, two launches for the binary
        path) never starves the GPU and the region holds a single graph
        launch; past 4096 steps, a graph of `period` launches is replayed
        several times plus one of the remainder.  The capture is replayed
        once untimed.  Events are recorded on the stream the kernels run on.
        """
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        if steps <= 4096:
            graphs = [capture(fn, range(steps))]
        else:
            period = min(period or 1, steps)
            reps, rem = divmod(steps, period)
            g = capture(fn, range(period))
            graphs = [g] * reps + ([capture(fn, range(rem))] if rem else [])
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, e0.elapsed_time(e1) * 1e-3

    # ------------------------------------------------------------ headline
    K, N = LAYER_SHAPES["gate"]
    bits, group = 4, 64
    log(f"generating gate weights {N}x{K}")
    W = layer_weights("gate")
    codes, meta = cg.qpack_group(to_dev(W), bits, group)
    nbytes = codes.numel() + meta.numel() * 4
    assert nbytes == 132_120_576
    pool = pool_of((codes, meta), nbytes)
    x = bf16(layer_x(K, 1))
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def step(i):
        c, m = pool[i % len(pool)]
        cg.qgemv_group(c, m, N, K, bits, group, x, y=y)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    wall, ev = time_launches(step, args.steps, args.warmup, period=len(pool))
    value = nbytes * args.steps / wall / 1e9
    achieved = nbytes * args.steps / ev / 1e9
    log(f"headline: {wall / args.steps * 1e6:.2f} us/step wall, {ev / args.steps * 1e6:.2f} us/launch events, "
        f"{achieved:.0f} GB/s")
    del pool
    torch.cuda.empty_cache()

    rows = {}
    if not args.no_rows:
        only = [o for o in args.only.split(",") if o]
        rows = measure_rows(cg, torch, np, dev, W, to_dev, bf16, pool_of, time_launches, log,
                            LAYER_SHAPES, MIXED_SETS, N_LAYERS, ATTN, layer_weights, layer_x, binlr_factors,
                            lambda name: not only or any(o in name for o in only))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(np, W, bits, group, log)
    ceiling = None if args.no_ceiling else stream_ceiling(cg, torch, dev, time_launches, log)

    traffic = committed_traffic()
    out = {
        "metric": "compressed-weight GEMV GB/s (% HBM peak) at 8192x28672, batch 1",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode GEMV, Llama-70B gate/up projection K=8192 x N=28672, group-RTN 4-bit, "
                        "groups of 64 with fp16 scale+offset, bf16 activations, batch 1",
            "K": K, "N": N, "bits": bits, "group": group, "batch": 1,
            "compressed_bytes_per_step": nbytes,
            "rotating_pool_copies": max(2, int(args.pool_gib * (1 << 30) // nbytes) + 1),
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "timed_region": "one HIP graph of all steps, replayed once between two torch.cuda.synchronize()",
            "tok_s_equivalent_80_layers_4b_g64": round(value * 1e9 / (N_LAYERS * layer_bytes(4, 64, 4, 64)), 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "gemv_b1_kernel<4,64,bf16>",
            "per_launch_us": round(ev / args.steps * 1e6, 3),
            "timing": "achieved = algorithmic bytes / per_launch_us, per_launch_us = HIP-event time of the "
                      "timed region (graph of all steps, on the launch stream) / steps; value uses the "
                      "wall-clock time of the same region",
            "streaming_read_ceiling": ceiling,
            "frac_of_measured_ceiling": (round(achieved / ceiling["read_132MB_GBps"], 4) if ceiling else None),
            "kernel_source_sha": kernel_source_sha(),
        },
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


def _group_bytes(N, K, bits, group):
    return N * K * bits // 8 + N * (K // group) * 4


def layer_bytes(attn_bits, attn_group, mlp_bits, mlp_group):
    from workloads import LAYER_SHAPES, ATTN
    tot = 0
    for name, (K, N) in LAYER_SHAPES.items():
        if name in ATTN:
            tot += _group_bytes(N, K, attn_bits, attn_group)
        else:
            tot += _group_bytes(N, K, mlp_bits, mlp_group)
    return tot


KV_STEPS = 1000          # key-cache rows: 1000 calls (tens of ms), as the GEMV rows
STREAM_PASSES = 2000     # streaming-read reference: 132 MB passes per timed region


def measure_rows(cg, torch, np, dev, W_gate, to_dev, bf16, pool_of, time_launches, log,
                 LAYER_SHAPES, MIXED_SETS, N_LAYERS, ATTN, layer_weights, layer_x, binlr_factors, want):
    """Every other row of the hot path; want(name) selects rows (all by default)."""
    rows = {}
    # 2000 launches per row (tens of ms): a sustained HBM stream runs ~10 %
    # faster for its first ~2 ms and then dips while the chip's power
    # management settles, so windows of a few ms mix in that transient
    steps, warm = 2000, 20

    def gemv_row(name, W, bits, group, B):
        N, K = W.shape
        codes, meta = cg.qpack_group(to_dev(W), bits, group)
        nbytes = codes.numel() + meta.numel() * 4
        pool = pool_of((codes, meta), nbytes)
        x = bf16(layer_x(K, B))
        y = torch.empty((B, N), dtype=torch.float32, device=dev)

        def f(i):
            c, m = pool[i % len(pool)]
            cg.qgemv_group(c, m, N, K, bits, group, x, y=y)
        wall, ev = time_launches(f, steps, warm, period=len(pool))
        gbs = nbytes * steps / ev / 1e9
        del pool
        torch.cuda.empty_cache()
        return {"us": round(ev / steps * 1e6, 3), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / 8000.0, 2), "bytes": nbytes}

    # batch 16 on the headline shape
    if want("gemv_4b_g64_gate_B16"):
        rows["gemv_4b_g64_gate_B16"] = gemv_row("gate", W_gate, 4, 64, 16)
        log("B16:", rows["gemv_4b_g64_gate_B16"])
    # whole 4-bit layer set at batch 1, and the mixed-width sets
    for label, spec in [("4b_g64", {"attn_bits": 4, "mlp_bits": 4, "group": 64})] + list(MIXED_SETS.items()):
        if not (want(f"layer_set_{label}_B1") or want(f"layer_set_{label}_B1_grouped")):
            continue
        per = {}
        t_layer = 0.0
        for name in ["q", "k", "v", "o", "gate", "up", "down"]:
            bits = spec["attn_bits"] if name in ATTN else spec["mlp_bits"]
            Wn = W_gate if name in ("gate", "up") else layer_weights(name)
            r = gemv_row(name, Wn, bits, spec["group"], 1)
            per[name] = r
            t_layer += r["us"]
        layer_b = sum(v["bytes"] for v in per.values())
        rows[f"layer_set_{label}_B1"] = {
            "sum_kernel_us_per_layer": round(t_layer, 2),
            "GB/s": round(layer_b / (t_layer * 1e-6) / 1e9, 1),
            "tok_s_equivalent_80_layers": round(1.0 / (N_LAYERS * t_layer * 1e-6), 1),
            "per_matrix": per,
        }
        log(label, rows[f"layer_set_{label}_B1"]["GB/s"], "GB/s")
    # the layer sets at their batches above 1 (4-bit set at 16, the mixed
    # widths at 8): every token of the batch shares one pass over the weights
    for label, spec, B in ([("4b_g64", {"attn_bits": 4, "mlp_bits": 4, "group": 64}, 16)]
                           + [(lb, sp, 8) for lb, sp in MIXED_SETS.items()]):
        name = f"layer_set_{label}_B{B}"
        if not (want(name) or want(name + "_grouped")):
            continue
        per = {}
        t_layer = 0.0
        for mat in ["q", "k", "v", "o", "gate", "up", "down"]:
            bits = spec["attn_bits"] if mat in ATTN else spec["mlp_bits"]
            Wn = W_gate if mat in ("gate", "up") else layer_weights(mat)
            per[mat] = gemv_row(mat, Wn, bits, spec["group"], B)
            t_layer += per[mat]["us"]
        layer_b = sum(v["bytes"] for v in per.values())
        rows[name] = {
            "sum_kernel_us_per_layer": round(t_layer, 2),
            "GB/s": round(layer_b / (t_layer * 1e-6) / 1e9, 1),
            "batch": B,
            "tok_s_80_layers": round(B / (N_LAYERS * t_layer * 1e-6), 1),
            "per_matrix": per,
        }
        log(name, rows[name]["GB/s"], "GB/s")
    # each layer set with q/k/v in one launch and gate/up in one launch
    def grouped_row(specs, bits, group, B=1):
        """specs: [(name, W)] sharing K; one grouped launch per step."""
        K = specs[0][1].shape[1]
        packed = [cg.qpack_group(to_dev(W), bits, group) + (W.shape[0],) for _, W in specs]
        nbytes = sum(c.numel() + m.numel() * 4 for c, m, _ in packed)
        pool = pool_of(tuple(t for c, m, _ in packed for t in (c, m)), nbytes)
        x = bf16(layer_x(K, B))
        ys = [torch.empty((B, n), dtype=torch.float32, device=dev) for _, _, n in packed]

        def f(i):
            p = pool[i % len(pool)]
            cg.qgemv_group_multi([(p[2 * j], p[2 * j + 1], packed[j][2]) for j in range(len(packed))], K, bits,
                                 group, x, ys=ys)
        wall, ev = time_launches(f, steps, warm, period=len(pool))
        del pool
        torch.cuda.empty_cache()
        return {"us": round(ev / steps * 1e6, 3), "GB/s": round(nbytes * steps / ev / 1e9, 1), "bytes": nbytes}

    sets = [("4b_g64", {"attn_bits": 4, "mlp_bits": 4, "group": 64})] + list(MIXED_SETS.items())
    for (label, spec), B in [(st, 1) for st in sets] + [(sets[0], 16)] + [(st, 8) for st in sets[1:]]:
        name = f"layer_set_{label}_B{B}_grouped"
        if not want(name) or f"layer_set_{label}_B{B}" not in rows:
            continue
        gsz = spec["group"]
        g_qkv = grouped_row([(n, layer_weights(n)) for n in ("q", "k", "v")], spec["attn_bits"], gsz, B)
        g_gu = grouped_row([("gate", W_gate), ("up", W_gate)], spec["mlp_bits"], gsz, B)
        per = rows[f"layer_set_{label}_B{B}"]["per_matrix"]
        t_layer = g_qkv["us"] + per["o"]["us"] + g_gu["us"] + per["down"]["us"]
        layer_b = g_qkv["bytes"] + per["o"]["bytes"] + g_gu["bytes"] + per["down"]["bytes"]
        rows[name] = {
            "sum_kernel_us_per_layer": round(t_layer, 2),
            "GB/s": round(layer_b / (t_layer * 1e-6) / 1e9, 1),
            ("tok_s_equivalent_80_layers" if B == 1 else "tok_s_80_layers"):
                round(B / (N_LAYERS * t_layer * 1e-6), 1),
            "launches": {"qkv": g_qkv, "o": per["o"], "gate_up": g_gu, "down": per["down"]},
        }
        log(f"grouped layer set {label}:", rows[name]["GB/s"], "GB/s")
    # the headline shape with its outlier channels kept aside in fp16 (0.1 %
    # of K = 8 channels); bytes = codes + meta + side columns
    def outlier_row(W, bits, group, n_out, B):
        N, K = W.shape
        codes, meta, side, idx = cg.qpack_group_outlier(to_dev(W), bits, group, n_out)
        nbytes = codes.numel() + meta.numel() * 4 + side.numel() * 2
        pool = pool_of((codes, meta, side), nbytes)
        x = bf16(layer_x(K, B))
        y = torch.empty((B, N), dtype=torch.float32, device=dev)

        def f(i):
            c, m, sd = pool[i % len(pool)]
            cg.qgemv_group_outlier(c, m, sd, idx, N, K, bits, group, x, y=y)

        def f_plain(i):   # the same codes without the side term, timed just before
            c, m, _ = pool[i % len(pool)]
            cg.qgemv_group(c, m, N, K, bits, group, x, y=y)
        _, ev_plain = time_launches(f_plain, steps, warm, period=len(pool))
        wall, ev = time_launches(f, steps, warm, period=len(pool))
        gbs = nbytes * steps / ev / 1e9
        del pool
        torch.cuda.empty_cache()
        return {"us": round(ev / steps * 1e6, 3), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / 8000.0, 2), "bytes": nbytes, "n_out": n_out,
                "plain_gemv_us_same_pool": round(ev_plain / steps * 1e6, 3)}

    for B in (1, 16):
        if not want(f"gemv_4b_g64_gate_outlier8_B{B}"):
            continue
        rows[f"gemv_4b_g64_gate_outlier8_B{B}"] = outlier_row(W_gate, 4, 64, 8, B)
        log(f"outlier B{B}:", rows[f"gemv_4b_g64_gate_outlier8_B{B}"])
    # the headline shape with per-group codebooks (default 8-book dictionary);
    # bytes = codes + meta + one book id per group
    def codebook_row(W, bits, group, B):
        N, K = W.shape
        books = cg.qcodebook_default(bits).to(dev)
        codes, meta, ids = cg.qpack_group_cb(to_dev(W), bits, group, books)
        nbytes = codes.numel() + meta.numel() * 4 + ids.numel()
        pool = pool_of((codes, meta, ids), nbytes)
        x = bf16(layer_x(K, B))
        y = torch.empty((B, N), dtype=torch.float32, device=dev)

        def f(i):
            c, m, k = pool[i % len(pool)]
            cg.qgemv_group_cb(c, m, k, books, N, K, bits, group, x, y=y)

        def f_plain(i):   # the same codes read as plain RTN codes, timed just before
            c, m, _ = pool[i % len(pool)]
            cg.qgemv_group(c, m, N, K, bits, group, x, y=y)
        _, ev_plain = time_launches(f_plain, steps, warm, period=len(pool))
        wall, ev = time_launches(f, steps, warm, period=len(pool))
        gbs = nbytes * steps / ev / 1e9
        del pool
        torch.cuda.empty_cache()
        return {"us": round(ev / steps * 1e6, 3), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / 8000.0, 2), "bytes": nbytes, "books": int(books.shape[0]),
                "plain_gemv_us_same_pool": round(ev_plain / steps * 1e6, 3)}

    for bits, B in [(4, 1), (4, 16), (2, 1)]:
        if not want(f"gemv_{bits}b_g64_gate_codebook_B{B}"):
            continue
        rows[f"gemv_{bits}b_g64_gate_codebook_B{B}"] = codebook_row(W_gate, bits, 64, B)
        log(f"codebook {bits}b B{B}:", rows[f"gemv_{bits}b_g64_gate_codebook_B{B}"])
    # attention logits from quantized keys (random rotation + Lloyd-Max codes
    # + QJL sign bits): 8 KV heads x 131072 keys (a 128K context), 4 grouped
    # queries per head; bytes = codes + signs + norms.  For scale, the same
    # logits from unquantized keys with torch (bf16 and fp32 batched matmul).
    def kv_row(bits, H=8, n=131072, nq=4):
        rng = np.random.default_rng(np.random.SeedSequence([0, 9, bits]))
        Pi = to_dev(cg.qtq_rotation(rng.standard_normal((128, 128))))
        S = to_dev(rng.standard_normal((128, 128)))
        SPi = cg.qtq_project(S, Pi)
        delta, table = cg.qtq_centroids(128, bits - 1)
        Kf = torch.randn((H * n, 128), device=dev, generator=torch.Generator(device=dev).manual_seed(bits))
        c, sg, nm = cg.qtq_quant_keys(Kf, bits, Pi, S, delta, table)
        Qv = torch.randn((H, nq, 128), device=dev, generator=torch.Generator(device=dev).manual_seed(100 + bits))
        nbytes = c.numel() * 4 + sg.numel() * 4 + nm.numel() * 4
        pool = pool_of((c, sg, nm), nbytes)
        out = torch.empty((H, nq, n), dtype=torch.float32, device=dev)
        ws = torch.empty(H * nq * 132 * 4, dtype=torch.uint8, device=dev)

        def f(i):
            a, b_, m_ = pool[i % len(pool)]
            cg.qtq_logits(a, b_, m_, n, H, bits, delta, table, Pi, SPi, Qv, out=out, ws=ws)
        wall, ev = time_launches(f, KV_STEPS, 10, period=len(pool))
        del pool
        torch.cuda.empty_cache()
        us = ev / KV_STEPS * 1e6
        base = {}
        Kh = Kf.view(H, n, 128)
        for label, dt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
            kd = Kh.to(dt).contiguous()
            qt = Qv.to(dt).transpose(1, 2).contiguous()
            kp = pool_of((kd,), kd.numel() * kd.element_size())
            for i in range(3):
                torch.bmm(kp[i % len(kp)][0], qt)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(40):
                torch.bmm(kp[i % len(kp)][0], qt)
            e1.record()
            torch.cuda.synchronize()
            base[label] = round(e0.elapsed_time(e1) * 1e3 / 40, 2)
            del kp, kd
            torch.cuda.empty_cache()
        del Kf
        return {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 8e12, 2), "bytes": nbytes,
                "keys_per_s": round(H * n / (us * 1e-6) / 1e9, 2), "unit_keys_per_s": "1e9",
                "torch_bf16_keys_us": base["bf16"], "torch_fp32_keys_us": base["fp32"],
                "speedup_vs_fp32": round(base["fp32"] / us, 2), "speedup_vs_bf16": round(base["bf16"] / us, 2)}

    for kb in (4, 3):
        if not want(f"kv_logits_{kb}bit_h8_n131072_q4"):
            continue
        rows[f"kv_logits_{kb}bit_h8_n131072_q4"] = kv_row(kb)
        log(f"kv logits {kb}-bit:", rows[f"kv_logits_{kb}bit_h8_n131072_q4"])

    # attention output over quantized values (3-bit codes), the same heads,
    # context and queries; bytes = codes + norms + the weights P read.  For
    # scale, torch's batched matmul of P with the unquantized values.
    def kv_attend_row(bits, H=8, n=131072, nq=4):
        rng = np.random.default_rng(np.random.SeedSequence([0, 10, bits]))
        Pi = to_dev(cg.qtq_rotation(rng.standard_normal((128, 128))))
        delta, table = cg.qtq_centroids(128, bits)
        Vf = torch.randn((H * n, 128), device=dev, generator=torch.Generator(device=dev).manual_seed(200 + bits))
        c, nm = cg.qtq_quant_values(Vf, bits, Pi, delta, table)
        Pw = torch.softmax(torch.randn((H, nq, n), device=dev), dim=2).contiguous()
        nbytes = c.numel() * 4 + nm.numel() * 4 + Pw.numel() * 4
        pool = pool_of((c, nm), c.numel() * 4 + nm.numel() * 4)
        out = torch.empty((H, nq, 128), dtype=torch.float32, device=dev)
        ws = torch.empty(cg.qtq_attend_ws(n, H, nq), dtype=torch.uint8, device=dev)

        def f(i):
            a, m_ = pool[i % len(pool)]
            cg.qtq_attend(a, m_, n, H, bits, delta, table, Pi, Pw, out=out, ws=ws)
        wall, ev = time_launches(f, KV_STEPS, 10, period=len(pool))
        del pool
        torch.cuda.empty_cache()
        us = ev / KV_STEPS * 1e6
        base = {}
        for label, dt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
            vd = Vf.view(H, n, 128).to(dt).contiguous()
            pd = Pw.to(dt).contiguous()
            vp = pool_of((vd,), vd.numel() * vd.element_size())
            for i in range(3):
                torch.bmm(pd, vp[i % len(vp)][0])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(40):
                torch.bmm(pd, vp[i % len(vp)][0])
            e1.record()
            torch.cuda.synchronize()
            base[label] = round(e0.elapsed_time(e1) * 1e3 / 40, 2)
            del vp, vd, pd
            torch.cuda.empty_cache()
        del Vf
        return {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 8e12, 2), "bytes": nbytes,
                "torch_bf16_values_us": base["bf16"], "torch_fp32_values_us": base["fp32"],
                "speedup_vs_fp32": round(base["fp32"] / us, 2), "speedup_vs_bf16": round(base["bf16"] / us, 2)}

    if want("kv_attend_3bit_h8_n131072_q4"):
        rows["kv_attend_3bit_h8_n131072_q4"] = kv_attend_row(3)
        log("kv attend 3-bit:", rows["kv_attend_3bit_h8_n131072_q4"])
    # mixed widths at batch 8 (MLP shape)
    for bits in (3, 2):
        if want(f"gemv_{bits}b_g32_gate_B8"):
            rows[f"gemv_{bits}b_g32_gate_B8"] = gemv_row("gate", W_gate, bits, 32, 8)
    for bits in (6, 5):
        if want(f"gemv_{bits}b_g32_q_B8"):
            rows[f"gemv_{bits}b_g32_q_B8"] = gemv_row("q", layer_weights("q"), bits, 32, 8)

    # binary low-rank GEMV
    for (K, N, r) in [(8192, 28672, 4096), (8192, 8192, 2048)]:
        if not want(f"binlr_gemv_{K}x{N}_r{r}_B1"):
            continue
        U, V, s1, s2 = binlr_factors(K, N, r)
        ub, vb = cg.qpack_binlr(to_dev(U), to_dev(V))
        nbytes = (r * (N + K)) // 8 + 2 * (N + K)
        pool = pool_of((ub, vb), ub.numel() * 4 + vb.numel() * 4)
        s1d, s2d = to_dev(s1.view(np.int16)), to_dev(s2.view(np.int16))
        x = bf16(layer_x(K, 1, config=4))
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        ws = torch.empty(cg.qbinlr_sizes(N, K, r, 1)[2], dtype=torch.uint8, device=dev)

        def f(i):
            a, b = pool[i % len(pool)]
            cg.qgemv_binlr(a, b, s1d, s2d, N, K, r, x, y=y, ws=ws)
        wall, ev = time_launches(f, steps, warm, period=len(pool))
        gbs = nbytes * steps / ev / 1e9
        rows[f"binlr_gemv_{K}x{N}_r{r}_B1"] = {
            "us": round(ev / steps * 1e6, 3), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / 8000.0, 2),
            "bytes": nbytes,
            "tok_s_equivalent_5.35GB_model": round(gbs * 1e9 / 5.35e9, 1),
        }
        log("binlr", rows[f"binlr_gemv_{K}x{N}_r{r}_B1"])
        del pool
        torch.cuda.empty_cache()

    # prefill GEMM, both formats
    if not any(want(f"prefill_{lb}_M{M}") for lb in ("rtn_4b_g64", "binlr_r4096", "codebook_4b_g64")
               for M in (512, 4096)):
        return rows
    K, N = 8192, 28672
    codes, meta = cg.qpack_group(to_dev(W_gate), 4, 64)
    wq = cg.make_qweight_group(codes, meta, N, K, 4, 64)
    U, V, s1, s2 = binlr_factors(8192, 28672, 4096)
    ub, vb = cg.qpack_binlr(to_dev(U), to_dev(V))
    s1d, s2d = to_dev(s1.view(np.int16)), to_dev(s2.view(np.int16))
    wb = cg.make_qweight_binlr(ub, vb, s1d, s2d, N, K, 4096)
    books = cg.qcodebook_default(4).to(dev)
    cc, mc, kc = cg.qpack_group_cb(to_dev(W_gate), 4, 64, books)
    wcb = cg.make_qweight_group(cc, mc, N, K, 4, 64, book_ids=kc, books=books)
    for M in (512, 4096):
        X = bf16(layer_x(K, M, config=5))
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for label, w, flops in [("rtn_4b_g64", wq, 2.0 * M * N * K), ("binlr_r4096", wb, 2.0 * M * 4096 * (K + N)),
                                ("codebook_4b_g64", wcb, 2.0 * M * N * K)]:
            if not want(f"prefill_{label}_M{M}"):
                continue
            ws = None
            need = cg.qgemm_prefill_ws(w, M)
            if need:
                ws = torch.empty(need, dtype=torch.uint8, device=dev)
            it = 5 if M == 4096 else 10
            wall, ev = time_launches(lambda i: cg.qgemm_prefill(w, X, Y=Y, ws=ws), it, 2, period=1)
            tf = flops * it / ev / 1e12
            rows[f"prefill_{label}_M{M}"] = {"us": round(ev / it * 1e6, 1), "TFLOP/s": round(tf, 1),
                                             "mfma_util_vs_2.5PF": round(tf / 2500.0, 4)}
            log("prefill", label, M, rows[f"prefill_{label}_M{M}"])
    return rows


def cpu_baseline(np, W, bits, group, log):
    """The oracle as it stands, on a bounded sample of rows of the same matrix:
    unpack codes -> rebuild W_hat (fp64) and the fp64 product, timed
    separately, median of three runs, as GB/s of compressed bytes.  The
    offline quantize/pack of the sample is not timed.  BLAS runs on every core
    of this process's affinity set; the rebuild is numpy on one thread (as
    the oracle is written)."""
    import oracle
    from workloads import layer_x
    cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        limiter = threadpool_limits(limits=cores, user_api="blas")
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        limiter, blas = None, 1
    N, K = W.shape
    x = oracle.product.bf16_to_f64(layer_x(K, 1))
    per_row = K * bits // 8 + (K // group) * 4

    def packed(R):
        q, s, o = oracle.rtn.quantize(W[:R], bits, group)       # offline: not timed
        return oracle.fmt.pack_codes(q, bits), oracle.fmt.pack_meta(s, o)

    def timed(R, words, meta):
        t0 = time.perf_counter()
        W_hat = oracle.product.what_group(words, meta, R, K, bits, group)
        t1 = time.perf_counter()
        _ = oracle.product.matmul_ref(W_hat, x)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    # probe a small sample, then size the sample to ~4 s per run (three runs)
    R0 = min(N, 1024)
    a0, b0 = timed(R0, *packed(R0))
    R = int(min(N, max(R0, R0 * 4.0 / max(a0 + b0, 1e-3))))
    words, meta = packed(R)
    runs = [timed(R, words, meta) for _ in range(3)]
    rec = sorted(r[0] for r in runs)[1]
    mul = sorted(r[1] for r in runs)[1]
    tot = sorted(r[0] + r[1] for r in runs)[1]
    if limiter is not None:
        limiter.restore_original_limits()
    log(f"cpu oracle: {R} rows, rebuild {rec:.2f} s + product {mul:.2f} s (median of 3), {cores} cores, {cpu_model}")
    return {
        "value": round(R * per_row / tot / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{R} of {N} rows of the same 8192x28672 4-bit g64 matrix ({R * per_row} compressed bytes), "
                  f"median of 3 runs: unpack + rebuild W_hat in fp64 {rec:.3f} s (numpy, one thread) + fp64 "
                  f"product {mul:.3f} s (BLAS, {blas} threads)",
        "cpu_model": cpu_model,
        "affinity_cores": int(cores),
        "blas_threads": int(blas),
        "rebuild_s": round(rec, 4),
        "product_s": round(mul, 4),
        "rows": int(R),
    }


def stream_ceiling(cg, torch, dev, time_launches, log):
    """Read rate this GPU's HBM gives a plain read-only stream of 16-byte
    nontemporal loads (the library's streaming-read kernel): 132 MB passes
    (the headline launch's size) over a 2 GiB rotating pool, timed the same
    way as the headline, and 4 GiB passes; the measured ceiling beside the
    8 TB/s specification."""
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    n = 132_120_576
    chunks = [buf[i * n:(i + 1) * n] for i in range((2 << 30) // n + 1)]
    _, ev = time_launches(lambda i: cg.qstream_read(chunks[i % len(chunks)], sink), STREAM_PASSES, 20,
                          period=len(chunks))
    small = n * STREAM_PASSES / ev / 1e9
    _, ev = time_launches(lambda i: cg.qstream_read(buf, sink), 40, 2)
    big = buf.numel() * 40 / ev / 1e9
    del buf, chunks
    torch.cuda.empty_cache()
    log(f"streaming read: {small:.0f} GB/s per 132 MB pass, {big:.0f} GB/s over 4 GiB")
    return {"read_132MB_GBps": round(small, 1), "read_4GiB_GBps": round(big, 1),
            "method": "qstream_read (16-byte nontemporal loads, grid-stride, 2048x256 threads, nothing written), "
                      "HIP events over one graph of back-to-back passes"}


if __name__ == "__main__":
    main()
