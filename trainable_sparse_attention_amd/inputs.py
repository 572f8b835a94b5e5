"""Seeded synthetic inputs for the QSA path.

This module only draws random numbers, scales them, rounds them to the
storage type and copies scaled query vectors into chosen key slots
("planted matches").  It holds none of the method's arithmetic, imports
nothing else from this package, and serves the HIP path and the CPU oracle
alike, which then receive identical bytes.

Value recipe (the same for every configuration): every element of q_idx,
k_idx, q, k, v is drawn standard normal in float32 and divided by sqrt(128),
then rounded round-to-nearest-even to the storage type.  The draw order is
q_idx, k_idx, q, k, v, then the planting draws.

Planting: a planted match pairs a query row i with a block b it can see
(only rows that see more than k_B blocks).  Every token of block b gets, on
the indexer dims that are not position-rotated (64..127), k_idx = c *
q_idx[i, h] for a random indexer head h, and zeros on the rotated dims
(0..63), so the match does not depend on the distance between i and b; in
the attention KV head g of a random query head a, k[g, token] = 4 c *
q[i, a].  c is drawn uniform in [2, 4] (the 4K-token float32 workload uses
c = 4 exactly).  Decode workloads plant against the last new query of each
sequence.

Two generators exist: ``numpy`` (Philox on the host; used by the CPU tests
and the small GPU parity cases) and ``torch`` (Philox on the GPU through
torch's device generator; used for the large configurations, where drawing
several GB on the host would take minutes).  Each is deterministic for a
given seed; they do not produce the same values as each other.
"""
import math

import numpy as np

R, K_TOP, H_IDX, D_IDX, ROPE_DIMS, THETA, D_HEAD = 4, 2048, 4, 128, 64, 10000.0, 128

# The workloads: prefill rows are positions 0..n-1 of each sequence; a decode
# sequence holds n tokens, the last n_new of which are the new queries (the
# pages' decode benchmark takes 4 new tokens per step: 1 + 3 drafts).
CONFIGS = {
    "prefill_4k_fp32": dict(mode="prefill", B=1, n=4096, hq=4, hkv=1, dtype="fp32",
                            planted=16, plant_c=4.0),
    "prefill_64k": dict(mode="prefill", B=1, n=65536, hq=16, hkv=2, dtype="bf16", planted=256),
    "prefill_256k": dict(mode="prefill", B=1, n=262144, hq=16, hkv=2, dtype="bf16",
                         planted=256),
    "decode_64x256k": dict(mode="decode", B=64, n=262144, hq=16, hkv=2, dtype="bf16",
                           planted=64),
    "prefill_1m": dict(mode="prefill", B=1, n=1048576, hq=16, hkv=2, dtype="bf16",
                       planted=1024),
    "decode_8x1m": dict(mode="decode", B=8, n=1048576, hq=16, hkv=2, dtype="bf16",
                        planted=1024),
    "decode_4x1m_next4": dict(mode="decode", B=4, n=1048576, n_new=4, hq=16, hkv=2,
                              dtype="bf16", planted=1024),
    # one training step's kernels at a training context length: indexer
    # distillation (dense teacher) and the sparse-attention backward
    "train_32k": dict(mode="prefill", B=1, n=32768, hq=16, hkv=2, dtype="bf16", planted=0,
                      train=True),
}


def describe(name):
    """The workload's sizes in words."""
    c = CONFIGS[name]
    dt = "bf16" if c["dtype"] == "bf16" else "float32"
    heads = "indexer 4x128 query heads + 1x128 key head, attention %d q / %d kv heads, d=128" % (
        c["hq"], c["hkv"])
    if c.get("train"):
        return "QSA training kernels (indexer distillation against the dense teacher, " \
               "pooling backward, sparse-attention backward), batch %d, n=%d tokens, K=2048, " \
               "r=4, %s, %s" % (c["B"], c["n"], heads, dt)
    if c["mode"] == "prefill":
        return "QSA prefill, batch %d, n=%d tokens, K=2048, r=4, %s, %s" % (c["B"], c["n"],
                                                                         heads, dt)
    return "QSA decode, batch %d, %d cached tokens per sequence, %d new token(s), K=2048, " \
           "r=4, %s, %s" % (c["B"], c["n"], c.get("n_new", 1), heads, dt)


def k_blocks(K=K_TOP, r=R):
    return -(-K // r)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round-to-nearest-even); returns the
    bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _plant_rows(rng, mode, n, planted, kB, r):
    """Planted (row, block) pairs of one sequence."""
    if mode == "decode":
        rows = np.full(planted, n - 1, dtype=np.int64)
    else:
        lo = kB * r + (r - 1)  # first row that sees more than kB blocks
        rows = rng.integers(lo, n, size=planted, dtype=np.int64)
    nvis = (rows + 1) // r
    blocks = (rng.random(planted) * nvis).astype(np.int64)
    return rows, blocks


def make(cfg="prefill_4k_fp32", seed=0, backend="numpy", device="cuda", overrides=None):
    """Inputs of one configuration.

    Returns a dict with the shapes and
      q_idx [B][n_q][4][128], k_idx [B][n][128], q [B][n_q][hq][128],
      k, v [B][hkv][n][128]  (n_q = n for prefill, n_new (default 1) for
      decode: the queries of positions n - n_q .. n - 1),
      plants: list of (seq, row, block, idx_head, attn_head, c).
    numpy backend: float32 arrays or bf16 bit patterns (uint16).
    torch backend: torch tensors on `device` (float32 or bfloat16)."""
    spec = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    if overrides:
        spec.update(overrides)
    mode, B, n, hq, hkv = spec["mode"], spec["B"], spec["n"], spec["hq"], spec["hkv"]
    planted = spec.get("planted", 0)
    plant_c = spec.get("plant_c", None)
    r = spec.get("r", R)
    kB = k_blocks(spec.get("K", K_TOP), r)
    n_q = n if mode == "prefill" else spec.get("n_new", 1)
    bf16 = spec["dtype"] == "bf16"
    inv = 1.0 / math.sqrt(128.0)
    shapes = dict(q_idx=(B, n_q, H_IDX, D_IDX), k_idx=(B, n, D_IDX), q=(B, n_q, hq, D_HEAD),
                  k=(B, hkv, n, D_HEAD), v=(B, hkv, n, D_HEAD))
    out = dict(spec=spec, mode=mode, B=B, n=n, n_q=n_q, hq=hq, hkv=hkv, r=r, kB=kB,
               dtype=spec["dtype"], seed=seed)

    if backend == "numpy":
        rng = np.random.Generator(np.random.Philox(seed))
        arrs = {}
        for name in ("q_idx", "k_idx", "q", "k", "v"):
            arrs[name] = (rng.standard_normal(shapes[name], dtype=np.float32) * np.float32(inv))
        plants = []
        for b in range(B):
            rows, blocks = _plant_rows(rng, mode, n, planted, kB, r)
            heads = rng.integers(0, H_IDX, size=planted)
            aheads = rng.integers(0, hq, size=planted)
            cs = rng.uniform(2.0, 4.0, size=planted) if plant_c is None else \
                np.full(planted, plant_c)
            for t in range(planted):
                i, blk, h, a, c = int(rows[t]), int(blocks[t]), int(heads[t]), int(aheads[t]), \
                    float(cs[t])
                qi = n_q - 1 if mode == "decode" else i
                g = (a * hkv) // hq
                for tok in range(blk * r, blk * r + r):
                    arrs["k_idx"][b, tok, :ROPE_DIMS] = 0.0
                    arrs["k_idx"][b, tok, ROPE_DIMS:] = np.float32(c) * \
                        arrs["q_idx"][b, qi, h, ROPE_DIMS:]
                    arrs["k"][b, g, tok, :] = np.float32(4.0 * c) * arrs["q"][b, qi, a, :]
                plants.append((b, i, blk, h, a, c))
        for name in arrs:
            out[name] = f32_to_bf16_bits(arrs[name]) if bf16 else np.ascontiguousarray(arrs[name])
        out["plants"] = plants
        return out

    if backend == "torch":
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        tdt = torch.bfloat16 if bf16 else torch.float32
        res = {}
        for name in ("q_idx", "k_idx", "q", "k", "v"):
            shp = shapes[name]
            t = torch.empty(shp, dtype=tdt, device=device)
            flat = t.view(-1, shp[-1])
            step = max(1, (1 << 26) // shp[-1])  # draw in chunks of 64M values
            for s in range(0, flat.shape[0], step):
                e = min(flat.shape[0], s + step)
                blk = torch.randn((e - s, shp[-1]), generator=g, device=device,
                                  dtype=torch.float32)
                blk.mul_(inv)
                flat[s:e].copy_(blk)
            res[name] = t
        prng = np.random.Generator(np.random.Philox(seed + 1_000_003))
        plants = []
        for b in range(B):
            rows, blocks = _plant_rows(prng, mode, n, planted, kB, r)
            heads = prng.integers(0, H_IDX, size=planted)
            aheads = prng.integers(0, hq, size=planted)
            cs = prng.uniform(2.0, 4.0, size=planted) if plant_c is None else \
                np.full(planted, plant_c)
            for t in range(planted):
                i, blk, h, a, c = int(rows[t]), int(blocks[t]), int(heads[t]), int(aheads[t]), \
                    float(cs[t])
                qi = n_q - 1 if mode == "decode" else i
                gk = (a * hkv) // hq
                src_i = res["q_idx"][b, qi, h, :].float() * c
                src_i[:ROPE_DIMS] = 0.0
                src_a = res["q"][b, qi, a, :].float() * (4.0 * c)
                res["k_idx"][b, blk * r:blk * r + r, :] = src_i.to(tdt)[None, :]
                res["k"][b, gk, blk * r:blk * r + r, :] = src_a.to(tdt)[None, :]
                plants.append((b, i, blk, h, a, c))
        out.update(res)
        out["plants"] = plants
        return out

    raise ValueError("backend must be 'numpy' or 'torch'")


def small(B=1, n=64, hq=4, hkv=1, dtype="fp32", planted=0, r=R, K=K_TOP, seed=0,
          mode="prefill", plant_c=None):
    """Inputs with custom (small) shapes, numpy backend."""
    spec = dict(mode=mode, B=B, n=n, hq=hq, hkv=hkv, dtype=dtype, planted=planted, r=r, K=K)
    if plant_c is not None:
        spec["plant_c"] = plant_c
    return make(spec, seed=seed, backend="numpy")
