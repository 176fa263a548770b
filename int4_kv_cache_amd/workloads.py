"""Seeded synthetic inputs for the SAW-INT4 append/gather path.

This module draws random numbers and lays out slot mappings; it holds none of
the method's arithmetic (no rotation, no quantisation, no packing), so that
the oracle and the HIP path can both be fed from it without sharing any code
that computes a result.

Five workloads, shaped like the serving scenarios the pages talk about
(decode at up to 256 concurrent requests and long contexts: gist.science
summary of SAW-INT4, §4 "Risultati Sperimentali"; 8 KV heads x head_dim 128,
fp16 K/V in: youngju.dev reading, fused-kernel diagram):

  tiny     64 tokens of one sequence, 2 heads, N(0,1), channels 3 and 77 of
           every head x16, h=128, K+V, page 16, identity slots, 4 extra pages
           that nothing addresses (sentinel pages)
  decode   256 sequences x 1 token, 8 heads, 36 layers called one by one,
           N(0,1) + 4 fixed channels per (layer, head, tensor) x20, h=128,
           K-only, page 16, 256 distinct slots scattered over 2^20 slots
  prefill  32 x 4096 tokens, 8 heads, Student-t(4) + 2 % of the
           (head, channel) pairs x10, h=128, K+V, page 16, pages from a
           seeded free-list permutation
  sweep    64 x 1024 tokens, 8 heads, the decode recipe (one layer), page 16,
           free-list pages; run for h in {32, 64, 128} x {none, K, K+V}
  long     64 x 32768 tokens, 8 heads, N(0,1) + 4 fixed channels per
           (head, tensor) x32, h=128, K+V, page 32, shuffled free list

Draw recipe (numpy PCG64 via default_rng, seeded from a SeedSequence key):
  values    key (seed, workload id, 0, layer, tensor, chunk); chunks of 4096
            tokens; standard normal drawn as float32, Student-t as float64
            then cast to float32; each chunk is [n, H, D] in C order
  outliers  key (seed, workload id, 1, layer, tensor); multipliers applied in
            float32; the scaled values are cast once to fp16 (round to
            nearest even)
  slots     key (seed, workload id, 2)
Any token range of any tensor can be regenerated on its own, which is what the
full-size tests use to check sampled tokens.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 4096
ROT_NONE, ROT_K, ROT_KV = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int               # stable id used in seed keys
    n_seq: int
    seq_len: int           # tokens per sequence appended by one call
    H: int
    D: int
    P: int                 # page size (tokens per page)
    N_pg: int              # pages in the pool
    h: int                 # Hadamard block size
    rot_mode: int          # ROT_NONE / ROT_K / ROT_KV
    values: str            # "normal" or "student_t4"
    outliers: tuple        # ("channels", (c0, c1, ...), factor) |
                           # ("per_head", count, factor) | ("fraction", frac, factor)
    placement: str         # "identity" | "scatter" | "free_list"
    layers: int = 1
    seed: int = 0

    @property
    def T(self):
        return self.n_seq * self.seq_len

    @property
    def n_slots(self):
        return self.N_pg * self.P

    def bytes_per_token(self):
        """Algorithmic HBM bytes per token of one append (or one gather):
        fp16 K and V, packed codes and fp16 scales of K and V, int64 slot."""
        return self.H * (2 * self.D * 2 + 2 * (self.D // 2) + 2 * 2) + 8


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 2, 128, 16, 8, 128, ROT_KV, "normal",
                     ("channels", (3, 77), 16.0), "identity"),
    "decode": Workload("decode", 2, 256, 1, 8, 128, 16, 65536, 128, ROT_K, "normal",
                       ("per_head", 4, 20.0), "scatter", layers=36),
    "prefill": Workload("prefill", 3, 32, 4096, 8, 128, 16, 8192, 128, ROT_KV,
                        "student_t4", ("fraction", 0.02, 10.0), "free_list"),
    "sweep": Workload("sweep", 4, 64, 1024, 8, 128, 16, 4096, 128, ROT_KV, "normal",
                      ("per_head", 4, 20.0), "free_list"),
    "long": Workload("long", 5, 64, 32768, 8, 128, 32, 65536, 128, ROT_KV, "normal",
                     ("per_head", 4, 32.0), "free_list"),
}

SWEEP_VARIANTS = [(h, mode) for h in (32, 64, 128) for mode in (ROT_NONE, ROT_K, ROT_KV)]


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def outlier_multipliers(wl, layer, tensor):
    """float32 [H, D] multipliers (1 or the outlier factor) for tensor 0 = K, 1 = V."""
    kind = wl.outliers[0]
    mult = np.ones((wl.H, wl.D), dtype=np.float32)
    rng = np.random.default_rng([wl.seed, wl.wid, 1, layer, tensor])
    if kind == "channels":
        _, chans, f = wl.outliers
        mult[:, list(chans)] = np.float32(f)
    elif kind == "per_head":
        _, count, f = wl.outliers
        for hd in range(wl.H):
            ch = rng.choice(wl.D, size=count, replace=False)
            mult[hd, ch] = np.float32(f)
    elif kind == "fraction":
        _, frac, f = wl.outliers
        n = int(round(frac * wl.H * wl.D))
        flat = rng.choice(wl.H * wl.D, size=n, replace=False)
        mult.reshape(-1)[flat] = np.float32(f)
    else:
        raise ValueError(kind)
    return mult


def _chunk(wl, layer, tensor, c, mult):
    lo = c * CHUNK
    n = min(CHUNK, wl.T - lo)
    rng = np.random.default_rng([wl.seed, wl.wid, 0, layer, tensor, c])
    if wl.values == "normal":
        x = rng.standard_normal((n, wl.H, wl.D), dtype=np.float32)
    elif wl.values == "student_t4":
        x = rng.standard_t(4.0, size=(n, wl.H, wl.D)).astype(np.float32)
    else:
        raise ValueError(wl.values)
    x *= mult[None]
    return x.astype(np.float16)


def tensor(wl, which, layer=0, lo=0, hi=None):
    """fp16 [hi-lo, H, D] of K (which=0) or V (which=1) for tokens [lo, hi)."""
    hi = wl.T if hi is None else hi
    if not (0 <= lo <= hi <= wl.T):
        raise ValueError("token range out of bounds")
    out = np.empty((hi - lo, wl.H, wl.D), dtype=np.float16)
    if hi == lo:
        return out
    mult = outlier_multipliers(wl, layer, which)
    c0, c1 = lo // CHUNK, (hi - 1) // CHUNK

    def fill(c):
        x = _chunk(wl, layer, which, c, mult)
        a = max(lo, c * CHUNK)
        b = min(hi, c * CHUNK + len(x))
        out[a - lo:b - lo] = x[a - c * CHUNK:b - c * CHUNK]

    if c1 == c0:
        fill(c0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(c0, c1 + 1)))
    return out


def kv(wl, layer=0, lo=0, hi=None):
    return tensor(wl, 0, layer, lo, hi), tensor(wl, 1, layer, lo, hi)


def slot_mapping(wl):
    """int64 [T] slot of every token (slot = page * P + offset)."""
    T = wl.T
    rng = np.random.default_rng([wl.seed, wl.wid, 2])
    if wl.placement == "identity":
        return np.arange(T, dtype=np.int64)
    if wl.placement == "scatter":
        return rng.choice(wl.n_slots, size=T, replace=False).astype(np.int64)
    if wl.placement == "free_list":
        pages_per_seq = -(-wl.seq_len // wl.P)
        if pages_per_seq * wl.n_seq > wl.N_pg:
            raise ValueError("pool too small for the free list")
        perm = rng.permutation(wl.N_pg).astype(np.int64)
        s = np.repeat(np.arange(wl.n_seq, dtype=np.int64), wl.seq_len)
        t = np.tile(np.arange(wl.seq_len, dtype=np.int64), wl.n_seq)
        page = perm[s * pages_per_seq + t // wl.P]
        return page * wl.P + t % wl.P
    raise ValueError(wl.placement)


def pool_shapes(N_pg, P, H, D):
    """Shapes and dtypes of the four pool arrays (K codes, V codes, K scales, V scales)."""
    return ((N_pg, P, H, D // 2), np.uint8), ((N_pg, P, H), np.float16)
