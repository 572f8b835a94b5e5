#!/usr/bin/env python3
"""Throughput of the QSA hot path on one MI355X.

One step = one pass of the whole prefill path over one sequence of 262,144
tokens (pool every block -> compressed indexer + top-k_B -> sparse core
attention; bf16, 16 query / 2 KV heads, K = 2048, r = 4), with every input
resident in HBM before the timed region.  `value` is prefill tokens/s.  The
decode half of the metric (batch 8, 1,048,576 cached tokens each, one new
token per sequence: pool the new block -> indexer + top-k -> split attention)
is timed the same way and reported under "decode".

Stage times come from HIP events recorded on the stream the kernels run on
(torch's current stream).  The roofline object describes the stage that
takes the most time.  The CPU oracle is timed on a bounded uniform sample of
the same workload's rows on this host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA prefill tokens/s @256K and decode tokens/s @1M ctx, 1 MI355X; % roofline"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PEAK_HBM_GBS = 8000.0       # HBM3E, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--prefill-cfg", default="cfg2")
    ap.add_argument("--decode-cfg", default="cfg4d")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="uniformly spaced prefill rows the CPU oracle computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, copy a buffer of MIB MiB with a plain device copy "
                         "(3 times), so that a counter run can scale FETCH_SIZE / WRITE_SIZE "
                         "by a kernel of known traffic")
    return ap.parse_args()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` recorded from rocprofv3 counter runs in
    profiles/traffic.txt, if the kernel's source still has the recorded
    sha256 (else None: the counters describe another version)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        if kv.get("kernel") != kernel:
            continue
        src = os.path.join(ROOT, kv["source"])
        if not os.path.exists(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv["sha256"]:
            return None
        return int(kv["traffic_bytes"])
    return None


def sum_nb(n, r=4):
    """sum over rows i < n of floor((i+1)/r): the indexer's (row, block) pairs."""
    q, rem = divmod(n, r)
    return r * q * (q - 1) // 2 + q * (rem + 1)


def bench_prefill(args, torch, qsa, inputs):
    d = inputs.make(args.prefill_cfg, seed=2, backend="torch")
    p = qsa.params()
    B, n, hq, hkv = d["B"], d["n"], d["hq"], d["hkv"]
    kB = qsa.k_blocks(p)
    nb = n // p.r
    dev = d["q"].device
    kbar = torch.empty((B, nb, 128), dtype=d["k_idx"].dtype, device=dev)
    idx = torch.empty((B, n, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["q"])
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.dtype_code(d["q_idx"]), B, n, nb,
                                                    False))
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(record):
        if record:
            ev[0].record(stream)
        qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, nb, stream)
        if record:
            ev[1].record(stream)
        qsa.qsa_index_topk(p, d["q_idx"], kbar, idx, cnt, ws, 0, None, stream)
        if record:
            ev[2].record(stream)
        qsa.qsa_sparse_attn_prefill(p, d["q"], d["k"], d["v"], idx, cnt, out, 0, 0.0, stream)
        if record:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    st = [0.0, 0.0, 0.0]
    tot = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        ev[3].synchronize()
        st[0] += ev[0].elapsed_time(ev[1])
        st[1] += ev[1].elapsed_time(ev[2])
        st[2] += ev[2].elapsed_time(ev[3])
        tot += ev[0].elapsed_time(ev[3])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    K = args.steps
    ms = tot / K
    st = [s / K for s in st]
    # algorithmic work
    pairs = sum_nb(n, p.r) * B
    c = cnt.to(torch.int64)
    pos = torch.arange(n, device=dev, dtype=torch.int64)
    tails = ((pos + 1) % p.r).sum().item() * B
    slots = int(c.sum().item()) * p.r + tails  # sum |T_i|
    elt = 2
    idx_flop = 1024.0 * pairs
    attn_bytes = (hkv * 2 * 128 * elt * slots + 2 * B * n * hq * 128 * elt +
                  4 * int(c.sum().item()) + 4 * B * n)
    pool_bytes = B * (n * 128 * elt + nb * 128 * elt)
    res = dict(n=n, B=B, ms=ms, wall_ms=wall * 1000 / K, stage_ms=st, pairs=pairs, slots=slots,
               idx_tflops=idx_flop / (st[1] * 1e-3) / 1e12,
               attn_gbs=attn_bytes / (st[2] * 1e-3) / 1e9,
               pool_gbs=pool_bytes / (st[0] * 1e-3) / 1e9,
               idx_flop=idx_flop, attn_bytes=attn_bytes, pool_bytes=pool_bytes,
               tok_s=B * n / (ms * 1e-3))
    return res, d


def bench_decode(args, torch, qsa, inputs):
    d = inputs.make(args.decode_cfg, seed=4, backend="torch")
    p = qsa.params()
    B, L, hq, hkv = d["B"], d["n"], d["hq"], d["hkv"]
    kB = qsa.k_blocks(p)
    nb = L // p.r
    dev = d["q"].device
    kbar = torch.empty((B, nb, 128), dtype=d["k_idx"].dtype, device=dev)
    qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, nb)
    seq_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    idx = torch.empty((B, 1, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, 1), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["q"])
    ws_i = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.dtype_code(d["q_idx"]), B, 1, nb,
                                                      True))
    ws_a = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, 1, hq, hkv))
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(record):
        if record:
            ev[0].record(stream)
        # the newest block completes at this step: pool it into the cache
        # (calls go to the current stream: the capture stream under a graph)
        qsa.qsa_pool_keys(p, d["k_idx"], kbar, nb - 1, nb)
        if record:
            ev[1].record(stream)
        qsa.qsa_index_topk(p, d["q_idx"], kbar, idx, cnt, ws_i, 0, seq_len)
        if record:
            ev[2].record(stream)
        qsa.qsa_sparse_attn_decode(p, d["q"], d["k"], d["v"], seq_len, idx, cnt, out, ws_a, 0.0)
        if record:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    K = args.decode_steps
    st = [0.0, 0.0, 0.0]
    tot = 0.0
    for _ in range(K):
        step(True)
        ev[3].synchronize()
        st[0] += ev[0].elapsed_time(ev[1])
        st[1] += ev[1].elapsed_time(ev[2])
        st[2] += ev[2].elapsed_time(ev[3])
        tot += ev[0].elapsed_time(ev[3])
    eager_ms = tot / K
    st = [s / K for s in st]
    # The same step captured once in a HIP graph and replayed: one submission
    # per step, so the GPU does not wait for the host between the calls.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(False)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(K):
        ev[0].record(stream)
        g.replay()
        ev[3].record(stream)
        ev[3].synchronize()
        tot += ev[0].elapsed_time(ev[3])
    ms = tot / K
    c = cnt.to(torch.int64)
    slots = int(c.sum().item()) * p.r + B * (L % p.r)
    elt = 2
    scan_bytes = B * nb * 128 * elt + B * nb * 4  # pooled keys read + one score per block
    gather_bytes = hkv * 2 * 128 * elt * slots
    io_bytes = B * (2 * hq * 128 * elt + 4 * 128 * elt + kB * 4)
    step_bytes = B * nb * 128 * elt + gather_bytes + io_bytes
    return dict(B=B, L=L, ms=ms, eager_ms=eager_ms, stage_ms=st, tok_s=B / (ms * 1e-3),
                step_bytes=step_bytes,
                scan_bytes=scan_bytes, gather_bytes=gather_bytes,
                step_gbs=step_bytes / (ms * 1e-3) / 1e9,
                index_gbs=scan_bytes / (st[1] * 1e-3) / 1e9)


def cpu_baseline(args, d, qsa_p):
    """The oracle on a uniform sample of the prefill rows, extrapolated."""
    import numpy as np
    import oracle
    import torch
    n = d["n"]
    S = max(1, min(args.cpu_rows, n))
    rows = np.unique(np.linspace(0, n - 1, S).astype(np.int64))

    def host(t):
        t = t.contiguous()
        return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.cpu().numpy()

    k_idx = host(d["k_idx"][0])
    q_idx = host(d["q_idx"][0])
    q = host(d["q"][0])
    k, v = host(d["k"][0]), host(d["v"][0])
    oracle.load()
    t0 = time.perf_counter()
    kbar = oracle.pool(k_idx)
    t_pool = time.perf_counter() - t0
    t1 = time.perf_counter()
    idx, cnt = oracle.index_rows(q_idx, kbar, rows)
    t_idx = time.perf_counter() - t1
    t2 = time.perf_counter()
    oracle.attend_rows(q, k, v, rows, idx, cnt)
    t_att = time.perf_counter() - t2
    total = t_pool + (t_idx + t_att) * n / rows.size
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return dict(value=n / total, unit="tokens/s", cores=cores, kind="oracle",
                sample="pool of all %d blocks + indexer/top-k/attention of %d uniformly spaced "
                       "rows of the %d-token prefill, extrapolated x%.1f; measured %.1f s" % (
                           n // 4, rows.size, n, n / rows.size, t_pool + t_idx + t_att))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    from trainable_sparse_attention_amd import inputs, qsa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    qsa.lib()
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: %d bytes read and %d bytes written per copy" % (
            nbytes, nbytes), file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()
    pre, d = bench_prefill(args, torch, qsa, inputs)
    print("[bench] prefill %s: %.3f ms/step (pool %.3f, index %.3f, attn %.3f ms)" % (
        args.prefill_cfg, pre["ms"], *pre["stage_ms"]), file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, d, qsa.params())
        print("[bench] cpu baseline %.1f tok/s (%s)" % (cpu["value"], cpu["sample"]),
              file=sys.stderr, flush=True)
    del d
    torch.cuda.empty_cache()
    dec = None
    if not args.no_decode:
        dec = bench_decode(args, torch, qsa, inputs)
        print("[bench] decode %s: %.3f ms/step as a graph replay; eager %.3f ms/step (pool %.3f, "
              "index %.3f, attn %.3f ms)" % (args.decode_cfg, dec["ms"], dec["eager_ms"],
                                             *dec["stage_ms"]), file=sys.stderr, flush=True)

    names = ["pool_keys", "index_topk", "sparse_attn_prefill"]
    dom = max(range(3), key=lambda i: pre["stage_ms"][i])
    if dom == 1:
        ach = pre["idx_tflops"]
        roof = dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=ach / PEAK_BF16_TFLOPS, traffic=None, kernel=names[dom])
    else:
        ach = pre["attn_gbs"] if dom == 2 else pre["pool_gbs"]
        roof = dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS,
                    traffic=recorded_traffic(names[dom]) if dom == 2 else None,
                    kernel=names[dom])
    line = {
        "metric": METRIC,
        "value": pre["tok_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "QSA prefill, batch 1, n=262144 tokens, K=2048, r=4, indexer "
                               "4x128 + 1x128 heads, attention 16 q / 2 kv heads, d=128, bf16",
                   "global_batch": pre["B"], "seq_len": pre["n"], "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": {
            "pool_keys": {"ms": pre["stage_ms"][0], "GB/s": pre["pool_gbs"],
                          "frac_hbm": pre["pool_gbs"] / PEAK_HBM_GBS},
            "index_topk": {"ms": pre["stage_ms"][1], "TFLOP/s": pre["idx_tflops"],
                           "frac_mfma": pre["idx_tflops"] / PEAK_BF16_TFLOPS,
                           "pairs": pre["pairs"]},
            "sparse_attn_prefill": {"ms": pre["stage_ms"][2], "GB/s": pre["attn_gbs"],
                                    "frac_hbm": pre["attn_gbs"] / PEAK_HBM_GBS,
                                    "sum_T": pre["slots"]},
        },
    }
    if dec is not None:
        line["decode"] = {
            "value": dec["tok_s"], "unit": "tokens/s", "ms_per_step": dec["ms"],
            "steps": args.decode_steps,
            "workload": "QSA decode, batch 8, 1048576 cached tokens per sequence, 1 new token",
            "timing": "one HIP graph replay per step (the three calls captured once)",
            "eager_ms_per_step": dec["eager_ms"],
            "eager_stage_ms": {"pool_keys": dec["stage_ms"][0], "index_topk": dec["stage_ms"][1],
                               "sparse_attn_decode": dec["stage_ms"][2]},
            "step_GB/s": dec["step_gbs"], "frac_hbm": dec["step_gbs"] / PEAK_HBM_GBS,
            "index_GB/s": dec["index_gbs"], "step_bytes": dec["step_bytes"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
