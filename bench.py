#!/usr/bin/env python3
"""Throughput of the QSA hot path on one MI355X.

One step = one pass of the whole prefill path over one sequence of 262,144
tokens (pool every block -> compressed indexer + top-k_B -> sparse core
attention; bf16, 16 query / 2 KV heads, K = 2048, r = 4), with every input
resident in HBM before the timed region.  `value` is prefill tokens/s.  The
decode half of the metric (batch 8, 1,048,576 cached tokens each, one new
token per sequence: pool the new block -> indexer + top-k -> split attention)
is timed the same way and reported under "decode"; further decode workloads
(batch 64 at 256K; batch 4 at 1M with 4 new tokens per step, the pages'
setting) under "decode_more".

Timing: HIP events recorded on the stream the kernels run on (torch's current
stream) around every step and stage.  Before each timed step an untimed
512 MB read evicts L2 and the memory-side cache, so every step starts cold;
the same steps back to back without it are reported under "unflushed".  The
graphics clock is sampled on a host thread during the timed steps.

The roofline object describes the kernel that takes the most time (the
prefill attention) against the bf16 MFMA peak with its algorithmic FLOPs; its
gathers are placed against a measured ceiling: a memory-only replay of the
same gathers (include/qsa_probe.h), swept over waves per CU and chunks in
flight.  The CPU oracle is timed on a bounded uniform sample of the same
workload's rows on this host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA prefill tokens/s @256K and decode tokens/s @1M ctx, 1 MI355X; % roofline"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PEAK_HBM_GBS = 8000.0       # HBM3E, MI355X
FLUSH_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--prefill-cfg", default="prefill_256k")
    ap.add_argument("--decode-cfg", default="decode_8x1m")
    ap.add_argument("--more-decode", default="decode_64x256k,decode_4x1m_next4",
                    help="comma-separated further decode workloads ('' for none)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense GQA comparison (chunked prefill and decode)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training kernels (distillation, backward)")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="uniformly spaced prefill rows the CPU oracle computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, copy a buffer of MIB MiB with a plain device copy "
                         "(3 times), so that a counter run can scale FETCH_SIZE / WRITE_SIZE "
                         "by a kernel of known traffic")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class ClockSampler:
    """Samples device 0's graphics clock as the power-management firmware
    reports it (amdsmi GPU metrics: the per-XCD current gfxclk) every few ms
    on a host thread while the timed steps run, and reports min / median /
    max MHz of the raw readings.  Informative only, and not the clock the
    kernels hold: on these parts the firmware's readings lag and sit far
    below it (157 MHz idle, about 400 MHz under a matrix-multiply load),
    while the GRBM counters show 1.9-2.4 GHz inside the kernels
    (profiles/qsa_clock_mfma.md).  Any failure is recorded, not raised."""

    def __init__(self):
        self.vals, self.err, self._stop = [], None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:
            self._smi, self.err = None, str(e)[:120]

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        xs = m.get("current_gfxclks")
        if not isinstance(xs, (list, tuple)):
            xs = [m.get("current_gfxclk")]
        return [x for x in xs if isinstance(x, (int, float)) and x > 0]

    def __enter__(self):
        import threading
        self.vals = []
        if self._smi is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    self.vals.extend(self._read())
                except Exception as e:
                    self.err = str(e)[:120]
                    return
                self._stop.wait(0.005)

        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *a):
        if self._stop is not None:
            self._stop.set()
            self._t.join()

    def summary(self):
        v = sorted(self.vals)
        if not v:
            return {"error": self.err or "no samples"}
        return {"source": "amdsmi GPU metrics, current gfxclk per XCD (firmware reading, not "
                          "the kernels' clock; see profiles/qsa_clock_mfma.md)",
                "gfx_mhz_min": v[0], "gfx_mhz_median": v[len(v) // 2], "gfx_mhz_max": v[-1],
                "samples": len(v)}


def recorded_traffic(kernel):
    """Bytes per launch of `kernel` from beyond L2 (MALL or HBM) recorded from
    rocprofv3 counter runs in profiles/traffic.txt, if the kernel's source
    still has the recorded sha256 (else None: the counters describe another
    version)."""
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


class Flusher:
    """An untimed read of a 512 MB buffer between timed steps: L2 (4 MB per
    XCD) and the 256 MB memory-side cache then hold none of the step's
    inputs, and the previous step's dirty outputs have been written back (a
    read leaves clean lines, so the timed step pays for no write-back)."""

    def __init__(self, torch, enabled):
        self.buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda") \
            if enabled else None

    def __call__(self):
        if self.buf is not None:
            self.acc = self.buf.sum()


def time_steps(torch, stream, stages, K, flush):
    """Run K steps (each a list of stage callables) with events around every
    stage; flush() before each step, outside the events.  Returns
    (mean step ms, mean ms per stage)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
    st = [0.0] * len(stages)
    tot = 0.0
    torch.cuda.synchronize()
    for _ in range(K):
        flush()
        ev[0].record(stream)
        for i, f in enumerate(stages):
            f()
            ev[i + 1].record(stream)
        ev[-1].synchronize()
        for i in range(len(stages)):
            st[i] += ev[i].elapsed_time(ev[i + 1])
        tot += ev[0].elapsed_time(ev[-1])
    torch.cuda.synchronize()
    return tot / K, [s / K for s in st]


def bench_prefill(args, torch, qsa, inputs, flush):
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
    stages = [lambda: qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, nb, stream),
              lambda: qsa.qsa_index_topk(p, d["q_idx"], kbar, idx, cnt, ws, 0, None, stream),
              lambda: qsa.qsa_sparse_attn_prefill(p, d["q"], d["k"], d["v"], idx, cnt, out, 0,
                                                  0.0, stream)]
    for _ in range(args.warmup):
        for f in stages:
            f()
    torch.cuda.synchronize()
    clocks = ClockSampler()
    t0 = time.perf_counter()
    with clocks:
        ms, st = time_steps(torch, stream, stages, args.steps, flush)
    wall = time.perf_counter() - t0
    ms_u, st_u = time_steps(torch, stream, stages, args.steps, lambda: None)
    # algorithmic work
    pairs = sum_nb(n, p.r) * B
    c = cnt.to(torch.int64)
    pos = torch.arange(n, device=dev, dtype=torch.int64)
    tails = ((pos + 1) % p.r).sum().item() * B
    slots = int(c.sum().item()) * p.r + tails  # sum |T_i|
    elt = 2
    idx_flop = 1024.0 * pairs
    attn_flop = 4.0 * 128 * hq * slots
    gather_bytes = hkv * 2 * 128 * elt * slots
    attn_bytes = gather_bytes + 2 * B * n * hq * 128 * elt + 4 * int(c.sum().item()) + 4 * B * n
    pool_bytes = B * (n * 128 * elt + nb * 128 * elt)
    res = dict(n=n, B=B, ms=ms, wall_ms=wall * 1000 / args.steps, stage_ms=st, pairs=pairs,
               slots=slots, idx_flop=idx_flop, attn_flop=attn_flop, attn_bytes=attn_bytes,
               gather_bytes=gather_bytes, pool_bytes=pool_bytes, tok_s=B * n / (ms * 1e-3),
               ms_unflushed=ms_u, stage_ms_unflushed=st_u, clocks=clocks.summary())
    probe = None
    if not args.no_probe:
        probe = probe_sweep(torch, qsa, p, d, idx, cnt, flush, stream)
    return res, d, probe


def probe_sweep(torch, qsa, p, d, idx, cnt, flush, stream):
    """Memory-only replay of the attention's gathers over waves per CU and
    chunks in flight per wave; each point is the best of two cold runs."""
    B, n, hkv = d["B"], d["n"], d["hkv"]
    sink = torch.empty(B * n * hkv, dtype=torch.int32, device="cuda")
    pts = []
    for w, depth in [(8, 1), (8, 2), (8, 4), (12, 2), (16, 1), (16, 2), (16, 4), (0, 4)]:
        best = None
        for _ in range(2):
            ms, _ = time_steps(torch, stream, [lambda: qsa.qsa_probe_gather(
                p, d["k"], d["v"], idx, cnt, sink, waves_per_cu=w, depth=depth,
                stream=stream)], 1, flush)
            best = ms if best is None else min(best, ms)
        pts.append({"waves_per_cu": w, "depth": depth, "ms": best})
        log("gather probe: %s waves/CU, depth %d: %.3f ms" % (w or "max", depth, best))
    return pts


def bench_decode(name, args, torch, qsa, inputs, flush, shared=False):
    """One decode step per sequence batch: pool the blocks the new tokens
    complete, select, attend.  shared: the step's new tokens share the one
    selection made at the first new token (index reuse)."""
    d = inputs.make(name, seed=4, backend="torch")
    p = qsa.params()
    B, L, n_q, hq, hkv = d["B"], d["n"], d["n_q"], d["hq"], d["hkv"]
    kB = qsa.k_blocks(p)
    nb = L // p.r
    dev = d["q"].device
    kbar = torch.empty((B, nb, 128), dtype=d["k_idx"].dtype, device=dev)
    qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, nb)
    seq_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    n_sel = 1 if shared else n_q
    # a shared selection is made for the first new token: its lengths end there
    sel_len = torch.full((B,), L - n_q + 1, dtype=torch.int32, device=dev) if shared else seq_len
    q_idx_sel = d["q_idx"][:, :1].contiguous() if shared else d["q_idx"]
    idx = torch.empty((B, n_sel, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n_sel), dtype=torch.int32, device=dev)
    out = torch.empty_like(d["q"])
    ws_i = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.dtype_code(d["q_idx"]), B, n_sel,
                                                      nb, True))
    ws_a = qsa.workspace(qsa.qsa_sparse_attn_decode_workspace(p, B, n_q, hq, hkv))
    stream = torch.cuda.current_stream()
    # the blocks the new tokens complete are pooled into the cache
    b0, b1 = (L - n_q) // p.r, L // p.r
    # calls go to the current stream: the capture stream under a graph
    attend = qsa.qsa_sparse_attn_decode_shared if shared else qsa.qsa_sparse_attn_decode
    stages = [lambda: qsa.qsa_pool_keys(p, d["k_idx"], kbar, b0, b1),
              lambda: qsa.qsa_index_topk(p, q_idx_sel, kbar, idx, cnt, ws_i, 0, sel_len),
              lambda: attend(p, d["q"], d["k"], d["v"], seq_len, idx, cnt, out, ws_a, 0.0)]
    for _ in range(args.warmup):
        for f in stages:
            f()
    torch.cuda.synchronize()
    K = args.decode_steps
    eager_ms, st = time_steps(torch, stream, stages, K, flush)
    # The same step captured once in a HIP graph and replayed: one submission
    # per step, so the GPU does not wait for the host between the calls.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for f in stages:
            f()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in stages:
            f()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    ms, _ = time_steps(torch, stream, [g.replay], K, flush)
    ms_u, _ = time_steps(torch, stream, [g.replay], K, lambda: None)
    c = cnt.to(torch.int64)
    pos = L - n_q + torch.arange(n_q, device=dev, dtype=torch.int64)
    if shared:  # each token: the shared blocks + tokens from the first token's block edge
        start = (L - n_q + 1) // p.r * p.r
        slots = int(c.sum().item()) * p.r * n_q + int((pos + 1 - start).sum().item()) * B
    else:
        tails = int(((pos + 1) % p.r).sum().item()) * B
        slots = int(c.sum().item()) * p.r + tails
    elt = 2
    scan_bytes = B * nb * 128 * elt + B * n_q * nb * 4  # pooled keys once + scores
    gather_bytes = hkv * 2 * 128 * elt * slots
    io_bytes = B * n_q * (2 * hq * 128 * elt + 4 * 128 * elt + kB * 4)
    step_bytes = B * nb * 128 * elt + gather_bytes + io_bytes
    return dict(name=name + ("_shared" if shared else ""), base=name, B=B, L=L, n_q=n_q, ms=ms, ms_unflushed=ms_u, eager_ms=eager_ms,
                stage_ms=st, tok_s=B * n_q / (ms * 1e-3), step_bytes=step_bytes,
                scan_bytes=scan_bytes, gather_bytes=gather_bytes,
                step_gbs=step_bytes / (ms * 1e-3) / 1e9,
                index_gbs=scan_bytes / (st[1] * 1e-3) / 1e9)


def bench_dense_comparison(args, torch, qsa, inputs, flush):
    """The pages' kernel comparison ([glide] "QSA Ablations and Efficiency",
    Figure 6(c,d)): (c) chunked prefill, one 16K-token chunk at the end of a
    context of L tokens, batch 1: QSA (pool the chunk's blocks, index + top-k
    for the chunk's rows, sparse attention) against dense causal GQA
    attention of the same rows; (d) decode at batch 4 with 4 new tokens per
    sequence at 1M: the QSA step against dense attention of the 4 tokens."""
    d = inputs.make("prefill_1m", seed=6, backend="torch")
    p = qsa.params()
    n, hq, hkv = d["n"], d["hq"], d["hkv"]
    kB = qsa.k_blocks(p)
    dev = d["q"].device
    stream = torch.cuda.current_stream()
    kbar = torch.empty((1, n // p.r, 128), dtype=torch.bfloat16, device=dev)
    qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, n // p.r)
    C = 16384
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, 1, C, n // p.r, False))
    idx = torch.empty((1, C, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, C), dtype=torch.int32, device=dev)
    out = torch.empty((1, C, hq, 128), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty_like(out)
    rows = []
    for L in [131072, 262144, 524288, 1048576]:
        p0 = L - C
        qi = d["q_idx"][:, p0:L]
        qq = d["q"][:, p0:L]
        stages = [lambda: qsa.qsa_pool_keys(p, d["k_idx"], kbar, p0 // p.r, L // p.r, stream),
                  lambda: qsa.qsa_index_topk(p, qi, kbar, idx, cnt, ws, p0, None, stream),
                  lambda: qsa.qsa_sparse_attn_prefill(p, qq, d["k"], d["v"], idx, cnt, out, p0,
                                                      0.0, stream)]
        dense = [lambda: qsa.qsa_dense_attn_prefill(qq, d["k"], d["v"], out_d, p0, 0.0, stream)]
        for f in stages + dense:
            f()
        ms_q, st_q = time_steps(torch, stream, stages, 3, flush)
        ms_d, _ = time_steps(torch, stream, dense, 2, flush)
        flop_d = 4.0 * 128 * hq * (C * p0 + C * (C + 1) / 2)
        rows.append({"context": L, "chunk": C, "qsa_ms": ms_q,
                     "qsa_stage_ms": {"pool_keys": st_q[0], "index_topk": st_q[1],
                                      "sparse_attn_prefill": st_q[2]},
                     "dense_ms": ms_d, "dense_TFLOP/s": flop_d / (ms_d * 1e-3) / 1e12,
                     "dense_frac_mfma": flop_d / (ms_d * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "speedup": ms_d / ms_q})
        log("chunked prefill, 16K chunk at %d: QSA %.3f ms (pool %.3f, index %.3f, attn %.3f), "
            "dense %.3f ms (%.0f TFLOP/s): %.2fx" % (L, ms_q, *st_q, ms_d,
                                                    flop_d / (ms_d * 1e-3) / 1e12, ms_d / ms_q))
    del d, kbar, ws, idx, cnt, out, out_d
    torch.cuda.empty_cache()
    # decode, batch 4, 4 new tokens per sequence, 1M context: dense attention
    dd = inputs.make("decode_4x1m_next4", seed=4, backend="torch")
    B, L, n_q = dd["B"], dd["n"], dd["n_q"]
    seq_len = torch.full((B,), L, dtype=torch.int32, device=dev)
    out = torch.empty_like(dd["q"])
    ws = qsa.workspace(qsa.qsa_dense_attn_decode_workspace(B, n_q, hkv, L))
    step = [lambda: qsa.qsa_dense_attn_decode(dd["q"], dd["k"], dd["v"], seq_len, out, ws)]
    for f in step:
        f()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step[0]()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step[0]()
    gr.replay()
    ms_dd, _ = time_steps(torch, stream, [gr.replay], args.decode_steps, flush)
    kv_bytes = B * hkv * L * 128 * 2 * 2
    log("dense decode, batch 4 x 4 new tokens at 1M: %.4f ms (%.0f GB/s of K/V)" % (
        ms_dd, kv_bytes / (ms_dd * 1e-3) / 1e9))
    return {"chunked_prefill": rows,
            "decode_b4_next4_1m": {"dense_ms": ms_dd,
                                   "dense_GB/s": kv_bytes / (ms_dd * 1e-3) / 1e9,
                                   "dense_frac_hbm": kv_bytes / (ms_dd * 1e-3) / 1e9 /
                                   PEAK_HBM_GBS}}


def bench_training(args, torch, qsa, inputs, flush):
    """The training kernels at a training context length ([hub] "Key ideas",
    native-trainability bullet): stage-1 indexer distillation (loss and
    gradients against the dense teacher), the pooling backward that carries
    the pooled-key gradient to the raw indexer keys, and the stage-2
    sparse-attention backward.  The forward (pool, select, attend) runs once,
    untimed; the gradient buffers the kernels add into are cleared inside
    the timed step."""
    d = inputs.make("train_32k", seed=8, backend="torch")
    p = qsa.params()
    B, n, hq, hkv = d["B"], d["n"], d["hq"], d["hkv"]
    kB = qsa.k_blocks(p)
    nb = n // p.r
    dev = d["q"].device
    stream = torch.cuda.current_stream()
    kbar = torch.empty((B, nb, 128), dtype=torch.bfloat16, device=dev)
    qsa.qsa_pool_keys(p, d["k_idx"], kbar, 0, nb, stream)
    idx = torch.empty((B, n, kB), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n), dtype=torch.int32, device=dev)
    ws = qsa.workspace(qsa.qsa_index_topk_workspace(p, qsa.QSA_BF16, B, n, nb, False))
    qsa.qsa_index_topk(p, d["q_idx"], kbar, idx, cnt, ws, 0, None, stream)
    out = torch.empty_like(d["q"])
    qsa.qsa_sparse_attn_prefill(p, d["q"], d["k"], d["v"], idx, cnt, out, 0, 0.0, stream)
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    dout = (torch.randn(out.shape, generator=g, device=dev) * 0.1).to(torch.bfloat16)
    loss = torch.empty((B, n), dtype=torch.float32, device=dev)
    dq_idx = torch.empty((B, n, 4, 128), dtype=torch.float32, device=dev)
    dkbar = torch.empty((B, nb, 128), dtype=torch.float32, device=dev)
    dk_idx = torch.empty((B, n, 128), dtype=torch.float32, device=dev)
    dq = torch.empty((B, n, hq, 128), dtype=torch.float32, device=dev)
    dk = torch.empty((B, hkv, n, 128), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    wsb = qsa.workspace(qsa.qsa_sparse_attn_backward_workspace(p, B, n, 0, hq))
    wsd = qsa.workspace(qsa.qsa_index_distill_workspace(p, B, n, 0))
    stages = [lambda: (dkbar.zero_(), dk.zero_(), dv.zero_()),
              lambda: qsa.qsa_index_distill(p, d["q"], d["k"], d["q_idx"], kbar, loss, dq_idx,
                                            dkbar, wsd, 0, 0.0, stream),
              lambda: qsa.qsa_pool_keys_backward(p, dkbar, dk_idx, 0, nb, stream),
              lambda: qsa.qsa_sparse_attn_backward(p, d["q"], d["k"], d["v"], idx, cnt, out,
                                                   dout, dq, dk, dv, wsb, 0, 0.0, stream)]
    for _ in range(max(1, args.warmup)):
        for f in stages:
            f()
    K = max(1, min(args.steps, 3))
    ms, _ = time_steps(torch, stream, stages, K, flush)
    # each call timed on its own (events between calls inside one step can
    # be stamped early after a long kernel); the gradient buffers are
    # cleared, untimed, before every call that adds into them
    st = [time_steps(torch, stream, [stages[0]], K, flush)[0]]
    for i in (1, 2, 3):
        t = 0.0
        for _ in range(K):
            stages[0]()
            t += time_steps(torch, stream, [stages[i]], 1, flush)[0]
        st.append(t / K)
    c = cnt.to(torch.int64)
    pos = torch.arange(n, device=dev, dtype=torch.int64)
    slots = int(c.sum().item()) * p.r + int(((pos + 1) % p.r).sum().item()) * B
    # (row, gathered block) pairs of the backward's key side: the selected
    # blocks and each row's incomplete block
    bwd_pairs = int(c.sum().item()) + int(((pos + 1) % p.r != 0).sum().item()) * B
    pairs = sum_nb(n, p.r) * B
    causal = B * n * (n + 1) // 2
    # algorithmic work: the teacher's logits once (2 d flops per head and
    # key), the student's scores and its two gradients (3 x 2 d per indexer
    # head and block); the backward's five products per head and gathered
    # key (logits recomputed, dP, dV, dQ, dK)
    distill_flop = 2.0 * 128 * hq * causal + 3 * 2.0 * 128 * 4 * pairs
    bwd_flop = 10.0 * 128 * hq * slots
    # algorithmic gathers of the backward: the query side reads each
    # gathered key's K row twice and its V row once (256 bytes each, per KV
    # head); the key side reads the Q and dO rows of the KV head's hq / hkv
    # query heads for every (row, block) pair
    bwd_gather = 768.0 * slots * hkv + 2 * 256.0 * hq * bwd_pairs
    pool_bwd_bytes = B * (nb * 128 * 4 + n * 128 * 4)
    res = {"workload": inputs.describe("train_32k"), "ms_per_step": ms,
           "stage_ms": {"clear_gradients": st[0], "index_distill": st[1],
                        "pool_keys_backward": st[2], "sparse_attn_backward": st[3]},
           "index_distill": {"TFLOP/s": distill_flop / (st[1] * 1e-3) / 1e12,
                             "frac_mfma": distill_flop / (st[1] * 1e-3) / 1e12 /
                             PEAK_BF16_TFLOPS, "flop": distill_flop},
           "sparse_attn_backward": {"TFLOP/s": bwd_flop / (st[3] * 1e-3) / 1e12,
                                    "frac_mfma": bwd_flop / (st[3] * 1e-3) / 1e12 /
                                    PEAK_BF16_TFLOPS, "flop": bwd_flop, "sum_T": slots,
                                    "gather_bytes": bwd_gather,
                                    "gather_GB/s": bwd_gather / (st[3] * 1e-3) / 1e9},
           "pool_keys_backward": {"GB/s": pool_bwd_bytes / (st[2] * 1e-3) / 1e9,
                                  "frac_hbm": pool_bwd_bytes / (st[2] * 1e-3) / 1e9 /
                                  PEAK_HBM_GBS},
           "mean_loss": float(loss.mean().item())}
    log("training kernels %s: %.3f ms/step (clear %.3f, distill %.3f = %.1f TFLOP/s, pool bwd "
        "%.4f, attn bwd %.3f = %.1f TFLOP/s, %.0f GB/s of gathers)" % (
            "train_32k", ms, st[0], st[1], res["index_distill"]["TFLOP/s"], st[2], st[3],
            res["sparse_attn_backward"]["TFLOP/s"], res["sparse_attn_backward"]["gather_GB/s"]))
    return res


def decode_record(inputs, dec, steps):
    return {
        "value": dec["tok_s"], "unit": "tokens/s", "ms_per_step": dec["ms"],
        "steps": steps, "workload": inputs.describe(dec["base"]) + (
            "; the new tokens share one selection made at the first (index reuse)"
            if dec["name"] != dec["base"] else ""),
        "timing": "one HIP graph replay per step (the three calls captured once), "
                  "untimed 512 MB read before each step",
        "ms_per_step_unflushed": dec["ms_unflushed"],
        "eager_ms_per_step": dec["eager_ms"],
        "eager_stage_ms": {"pool_keys": dec["stage_ms"][0], "index_topk": dec["stage_ms"][1],
                           "sparse_attn_decode": dec["stage_ms"][2]},
        "step_bytes": dec["step_bytes"], "step_GB/s": dec["step_gbs"],
        "frac_hbm": dec["step_gbs"] / PEAK_HBM_GBS, "index_GB/s": dec["index_gbs"]}


def cpu_baseline(args, d):
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
        log("copy calibration: %d bytes read and %d bytes written per copy" % (nbytes, nbytes))
        del src, dst
        torch.cuda.empty_cache()
    flush = Flusher(torch, not args.no_flush)
    pre, d, probe = bench_prefill(args, torch, qsa, inputs, flush)
    log("prefill %s: %.3f ms/step (pool %.3f, index %.3f, attn %.3f ms); unflushed %.3f ms "
        "(pool %.3f, index %.3f, attn %.3f ms)" % (args.prefill_cfg, pre["ms"], *pre["stage_ms"],
                                                   pre["ms_unflushed"],
                                                   *pre["stage_ms_unflushed"]))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, d)
        log("cpu baseline %.1f tok/s (%s)" % (cpu["value"], cpu["sample"]))
    del d
    torch.cuda.empty_cache()
    decs = []
    if not args.no_decode:
        names = [args.decode_cfg] + [x for x in args.more_decode.split(",") if x]
        runs = [(x, False) for x in names] + [(x, True) for x in names
                                              if inputs.CONFIGS[x].get("n_new", 1) > 1]
        for name, shared in runs:
            dec = bench_decode(name, args, torch, qsa, inputs, flush, shared)
            log("decode %s: %.4f ms/step as a graph replay (unflushed %.4f); eager %.4f ms/step "
                "(pool %.4f, index %.4f, attn %.4f ms)" % (dec["name"], dec["ms"],
                                                           dec["ms_unflushed"],
                                                           dec["eager_ms"], *dec["stage_ms"]))
            decs.append(dec)
            torch.cuda.empty_cache()

    train = None
    if not args.no_train:
        train = bench_training(args, torch, qsa, inputs, flush)
        torch.cuda.empty_cache()

    cmp_ = None
    if not args.no_dense:
        cmp_ = bench_dense_comparison(args, torch, qsa, inputs, flush)
        qsa_dec = {x["name"]: x["ms"] for x in decs}
        if "decode_4x1m_next4_shared" in qsa_dec:
            dm = cmp_["decode_b4_next4_1m"]
            for name in ("decode_4x1m_next4", "decode_4x1m_next4_shared"):
                dm[name + "_ms"] = qsa_dec[name]
                dm["speedup_" + name] = dm["dense_ms"] / qsa_dec[name]

    st = pre["stage_ms"]
    attn_ms = st[2]
    attn_tflops = pre["attn_flop"] / (attn_ms * 1e-3) / 1e12
    gather = {"algorithmic_bytes": pre["gather_bytes"],
              "achieved_GB/s": pre["gather_bytes"] / (attn_ms * 1e-3) / 1e9,
              "l2_miss_bytes": recorded_traffic("sparse_attn_prefill")}
    if probe:
        best = min(probe, key=lambda x: x["ms"])
        own = [x for x in probe if x["waves_per_cu"] == 8 and x["depth"] == 1][0]
        gather.update({"ceiling_ms": best["ms"],
                       "ceiling_config": {"waves_per_cu": best["waves_per_cu"],
                                          "depth": best["depth"]},
                       "ceiling_GB/s": pre["gather_bytes"] / (best["ms"] * 1e-3) / 1e9,
                       "attn_frac_of_ceiling": best["ms"] / attn_ms,
                       "probe_at_attn_config_ms": own["ms"], "probe": probe})
    # end to end: the step's lower bound over the measured step time, with
    # the indexer at the MFMA peak, the pooling at the HBM peak and the
    # attention at the larger of its MFMA time and its gather time
    idx_b = pre["idx_flop"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    pool_b = pre["pool_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
    attn_mfma_b = pre["attn_flop"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    hbm_form = idx_b + max(attn_mfma_b, pre["gather_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3) + pool_b
    e2e = {"t_bound_hbm_form_ms": hbm_form,
           "note": "the gathers at the HBM peak bound the step above its measured time: "
                   "most gathers are served by L2 and the memory-side cache"}
    if "ceiling_ms" in gather:
        t_bound = idx_b + max(attn_mfma_b, gather["ceiling_ms"]) + pool_b
        e2e.update({"t_bound_ms": t_bound, "frac": t_bound / pre["ms"],
                    "gather_term": "the measured gather ceiling (probe, %.3f ms)"
                                   % gather["ceiling_ms"]})
    roof = dict(bound="mfma", achieved=attn_tflops, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=attn_tflops / PEAK_BF16_TFLOPS, traffic=gather["l2_miss_bytes"],
                kernel="sparse_attn_prefill", flop=pre["attn_flop"],
                traffic_kind="bytes read and written beyond L2 (served by the memory-side "
                             "cache or HBM), from rocprofv3 FETCH_SIZE / WRITE_SIZE")
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
        "config": {"workload": inputs.describe(args.prefill_cfg), "global_batch": pre["B"],
                   "seq_len": pre["n"], "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing": "HIP events per step on the kernels' stream; an untimed 512 MB read before "
                  "each timed step evicts the caches" if not args.no_flush else
                  "HIP events, back to back",
        "unflushed": {"ms_per_step": pre["ms_unflushed"],
                      "tokens/s": pre["B"] * pre["n"] / (pre["ms_unflushed"] * 1e-3),
                      "stage_ms": dict(zip(["pool_keys", "index_topk", "sparse_attn_prefill"],
                                           pre["stage_ms_unflushed"]))},
        "clocks": pre["clocks"],
        "end_to_end": e2e,
        "stages": {
            "pool_keys": {"ms": st[0], "GB/s": pre["pool_bytes"] / (st[0] * 1e-3) / 1e9,
                          "frac_hbm": pre["pool_bytes"] / (st[0] * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "index_topk": {"ms": st[1],
                           "TFLOP/s": pre["idx_flop"] / (st[1] * 1e-3) / 1e12,
                           "frac_mfma": pre["idx_flop"] / (st[1] * 1e-3) / 1e12 /
                           PEAK_BF16_TFLOPS, "pairs": pre["pairs"]},
            "sparse_attn_prefill": {"ms": attn_ms, "TFLOP/s": attn_tflops,
                                    "frac_mfma": attn_tflops / PEAK_BF16_TFLOPS,
                                    "sum_T": pre["slots"], "gather": gather},
        },
    }
    if cmp_ is not None:
        line["qsa_vs_dense"] = cmp_
    if train is not None:
        line["training"] = train
    if decs:
        line["decode"] = decode_record(inputs, decs[0], args.decode_steps)
        if len(decs) > 1:
            line["decode_more"] = {x["name"]: decode_record(inputs, x, args.decode_steps)
                                   for x in decs[1:]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
