"""Seeded synthetic inputs for the five workloads (numpy only).

This module holds no quantization arithmetic.  Both the GPU tests/bench and
the CPU oracle draw their inputs from here.  bf16 tensors are returned as
uint16 bit patterns (numpy has no bf16); they are the round-to-nearest-even
bf16 images of float32 draws.

Workloads (synthetic stand-ins for the LLM weights, activations and KV caches
the pages evaluate on):
  c1  fp32 [256, 1024]: N(0,1), exactly round(1% of N) positions (uniform,
      without replacement) multiplied by 20.
  c2  bf16 [14336, 4096] (out x in): Student-t(df=4) * 0.02; per-input-column
      importance lognormal(0, 1), float32 [4096].
  c3  bf16 [8192, 4096] (tokens x channels): N(0,1); 8 distinct channels x50.
  c4  bf16 [8192, 8192]: half of the 16-element blocks (a random permutation)
      are U(-1, 1); the others are Laplace(0, 0.1) with one spike of +-1.0 at
      a uniform position inside the block.
  c5  bf16 [64, 32, 4096, 128] viewed as [64*32*4096, 128]: N(0,1) times a
      per-head scale s_h ~ lognormal(0, 0.5) (32 values shared across the
      batch); in each batch slice round(0.1% of its elements) positions x30.
"""
import concurrent.futures as cf

import numpy as np

SHAPES = {
    "c1": (256, 1024),
    "c2": (14336, 4096),
    "c3": (8192, 4096),
    "c4": (8192, 8192),
    "c5": (64 * 32 * 4096, 128),
}


def f32_to_bf16_bits(f):
    """Round-to-nearest-even bf16 bit patterns of a float32 array (finite)."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def c1(rows=256, cols=1024, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n = rows * cols
    k = int(round(0.01 * n))
    pos = rng.choice(n, size=k, replace=False)
    x.reshape(-1)[pos] *= np.float32(20.0)
    return x


def c2(rows=14336, cols=4096, seed=2):
    """Returns (weights as bf16 bits, importance float32 [cols])."""
    rng = np.random.default_rng(seed)
    imp = rng.lognormal(0.0, 1.0, size=cols).astype(np.float32)
    out = np.empty((rows, cols), np.uint16)
    step = 1024
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        t = rng.standard_t(4, size=(r1 - r0, cols)).astype(np.float32) * np.float32(0.02)
        out[r0:r1] = f32_to_bf16_bits(t)
    return out, imp


def c3(rows=8192, cols=4096, seed=3, n_outlier_channels=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    ch = rng.choice(cols, size=min(n_outlier_channels, cols), replace=False)
    x[:, ch] *= np.float32(50.0)
    return f32_to_bf16_bits(x)


def c4(rows=8192, cols=8192, seed=4, block=16):
    rng = np.random.default_rng(seed)
    nb = rows * cols // block
    uniform_blocks = np.zeros(nb, bool)
    uniform_blocks[rng.permutation(nb)[: nb // 2]] = True
    x = np.empty((nb, block), np.float32)
    nu = int(uniform_blocks.sum())
    x[uniform_blocks] = rng.uniform(-1.0, 1.0, size=(nu, block)).astype(np.float32)
    ns = nb - nu
    spiky = rng.laplace(0.0, 0.1, size=(ns, block)).astype(np.float32)
    where = rng.integers(0, block, size=ns)
    sign = np.where(rng.integers(0, 2, size=ns) == 1, np.float32(1.0), np.float32(-1.0))
    spiky[np.arange(ns), where] = sign
    x[~uniform_blocks] = spiky
    return f32_to_bf16_bits(x.reshape(rows, cols)), uniform_blocks


def c5(batch=64, heads=32, seq=4096, head_dim=128, seed=5, threads=16):
    """KV-cache-shaped tensor as [batch*heads*seq, head_dim] bf16 bits."""
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(batch + 1)
    head_scale = np.random.default_rng(kids[batch]).lognormal(0.0, 0.5, size=heads).astype(np.float32)
    per_b = heads * seq * head_dim
    out = np.empty(batch * per_b, np.uint16)

    def one(b):
        rng = np.random.default_rng(kids[b])
        x = rng.standard_normal((heads, seq * head_dim), dtype=np.float32)
        x *= head_scale[:, None]
        x = x.reshape(-1)
        k = int(round(0.001 * per_b))
        pos = rng.choice(per_b, size=k, replace=False)
        x[pos] *= np.float32(30.0)
        out[b * per_b:(b + 1) * per_b] = f32_to_bf16_bits(x)

    with cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(batch)))
    return out.reshape(batch * heads * seq, head_dim)


def rows_sample(x, n_rows, seed=0):
    """A reproducible sorted sample of row indices of a 2-D tensor."""
    rng = np.random.default_rng(seed)
    n_rows = min(n_rows, x.shape[0])
    return np.sort(rng.choice(x.shape[0], size=n_rows, replace=False))
