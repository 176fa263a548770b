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

Decode attention over the paged INT4 cache reads a pool that is already full;
its inputs (AttnWorkload, attn_inputs) are drawn directly as pool contents:
codes, fp16 scales, fp16 queries, block tables and context lengths. They are
not produced by the write path, so no attention input comes out of the kernels
under test. Recipe, key (seed, workload id, 3, part[, chunk]):
  lengths   part 0: integers uniform in [lo, hi] (or a fixed list)
  pages     part 1: a permutation of the pool; sequence b takes the next
            ceil(L_b / P) pages; unused table entries are -1; with
            masked > 0 that many in-range entries (chosen uniformly) are set
            to -1 as well
  codes     part 2 (K) / 3 (V), per chunk of 4096 pages: every nibble drawn
            independently from 0.96 x a discretised normal on [-8, 7] with
            sd 2.7 (the spread of codes of a rotated vector whose largest
            entry maps to 7) + 0.04 x uniform on [-8, 7] (so that every code,
            -8 included, occurs), sampled through a 65536-entry byte table
  scales    part 4 (K) / 5 (V): fp16 of base[head] * lognormal(0, 0.3), base
            0.35, and 20x that on two heads per tensor (outlier heads)
  queries   part 6: fp16 standard normal [B, Hq, D]; queries for another
            number of query heads Hq' over the same pool: key
            (seed, workload id, 3, 6, Hq')
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


# --------------------------------------------------------------------------
# Decode attention over a filled INT4 pool
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    wid: int
    B: int                 # sequences, one query token each
    Hq: int                # query heads
    H: int                 # KV heads (Hq % H == 0)
    D: int
    P: int                 # page size
    ctx: tuple             # ("uniform", lo, hi) | ("list", (L0, L1, ...))
    h: int                 # Hadamard block size the pool was written with
    rot_mode: int
    spare_pages: int = 64  # pool pages no sequence uses
    masked: int = 0        # in-range block-table entries replaced by -1
    seed: int = 0

    @property
    def G(self):
        return self.Hq // self.H

    def bytes_per_token(self):
        """Algorithmic HBM bytes per cached token read by one decode step:
        K and V codes and fp16 scales of every KV head."""
        return self.H * (2 * (self.D // 2) + 2 * 2)


ATTN_WORKLOADS = {
    # The decode workload's shape (256 concurrent requests, 8 KV heads of
    # 128, page 16, K-only rotation) with 32 query heads (4 per KV head) and
    # contexts of 1 to 8000 tokens.
    "attn": AttnWorkload("attn", 6, 256, 32, 8, 128, 16, ("uniform", 1, 8000), 128, ROT_K),
    # Long contexts: the long append workload's shape (64 sequences of 32768
    # tokens, page 32) read by one decode step, 2.2 GB of K/V per layer.
    "attn_long": AttnWorkload("attn_long", 9, 64, 32, 8, 128, 32, ("uniform", 32768, 32768),
                              128, ROT_K),
    # Small cases the oracle finishes in seconds: ragged lengths around the
    # 16-token tiles and 32-token steps, an empty context and masked pages.
    "attn_small": AttnWorkload("attn_small", 7, 9, 32, 8, 128, 16,
                               ("list", (0, 1, 15, 16, 17, 33, 100, 700, 1300)), 128,
                               ROT_KV, masked=3),
}


def attn_lengths(wl):
    kind = wl.ctx[0]
    if kind == "uniform":
        rng = np.random.default_rng([wl.seed, wl.wid, 3, 0])
        return rng.integers(wl.ctx[1], wl.ctx[2] + 1, size=wl.B).astype(np.int32)
    if kind == "list":
        L = np.asarray(wl.ctx[1], dtype=np.int32)
        if len(L) != wl.B:
            raise ValueError("length list does not match B")
        return L
    raise ValueError(kind)


def _code_table():
    """uint8 [65536]: a 16-bit uniform draw -> one code byte whose two nibbles
    are independent draws from the code distribution described above."""
    v = np.arange(-8, 8, dtype=np.float64)
    w = np.exp(-0.5 * (v / 2.7) ** 2)
    w = 0.96 * w / w.sum() + 0.04 / 16.0
    cdf = np.cumsum(w)
    u = (np.arange(256, dtype=np.float64) + 0.5) / 256.0
    nib = np.searchsorted(cdf, u).clip(0, 15) - 8          # [256] value for each byte draw
    lo = (nib.astype(np.int64) & 0xF)
    hi = (nib.astype(np.int64) & 0xF)
    idx = np.arange(65536)
    return (lo[idx & 0xFF] | (hi[idx >> 8] << 4)).astype(np.uint8)


def attn_inputs(wl):
    """Seeded inputs of one decode-attention step. Returns a dict of numpy
    arrays: q fp16 [B, Hq, D]; k_codes, v_codes uint8 [N_pg, P, H, D/2];
    k_scales, v_scales fp16 [N_pg, P, H]; block_tables int32 [B, max_pages];
    context_lens int32 [B]."""
    L = attn_lengths(wl)
    npages = -(-L.astype(np.int64) // wl.P)
    N_pg = int(npages.sum()) + wl.spare_pages
    max_pages = max(1, int(npages.max()) if len(npages) else 1)
    rng = np.random.default_rng([wl.seed, wl.wid, 3, 1])
    perm = rng.permutation(N_pg).astype(np.int32)
    bt = np.full((wl.B, max_pages), -1, dtype=np.int32)
    start = np.concatenate([[0], np.cumsum(npages)[:-1]]).astype(np.int64)
    for b in range(wl.B):
        bt[b, :npages[b]] = perm[start[b]:start[b] + npages[b]]
    if wl.masked:
        live = np.argwhere(np.arange(max_pages)[None, :] < npages[:, None])
        pick = rng.choice(len(live), size=min(wl.masked, len(live)), replace=False)
        bt[live[pick, 0], live[pick, 1]] = -1

    table = _code_table()
    half = wl.D // 2
    codes = []
    for part in (2, 3):
        out = np.empty((N_pg, wl.P, wl.H, half), dtype=np.uint8)
        flat = out.reshape(N_pg, -1)
        per = 4096

        def fill(c, part=part, flat=flat):
            lo, hi = c * per, min(N_pg, (c + 1) * per)
            r = np.random.default_rng([wl.seed, wl.wid, 3, part, c])
            draw = r.integers(0, 65536, size=(hi - lo, flat.shape[1]), dtype=np.uint16)
            flat[lo:hi] = table[draw]

        n_chunks = -(-N_pg // per)
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(n_chunks)))
        codes.append(out)

    scales = []
    for part in (4, 5):
        r = np.random.default_rng([wl.seed, wl.wid, 3, part])
        base = np.full(wl.H, 0.35, dtype=np.float64)
        base[r.choice(wl.H, size=min(2, wl.H), replace=False)] *= 20.0
        ln = r.lognormal(0.0, 0.3, size=(N_pg, wl.P, wl.H))
        scales.append((ln * base[None, None, :]).astype(np.float16))

    return {"q": attn_queries(wl), "k_codes": codes[0], "v_codes": codes[1],
            "k_scales": scales[0], "v_scales": scales[1], "block_tables": bt,
            "context_lens": L}


def attn_queries(wl, Hq=None):
    """The queries of an attention workload alone, fp16 [B, Hq, D] (part 6 of
    the recipe); with another Hq they are a fresh draw for the same pool (the
    pool does not depend on the number of query heads)."""
    Hq = wl.Hq if Hq is None else Hq
    r = np.random.default_rng([wl.seed, wl.wid, 3, 6] + ([] if Hq == wl.Hq else [Hq]))
    return r.standard_normal((wl.B, Hq, wl.D), dtype=np.float32).astype(np.float16)
