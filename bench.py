"""Benchmark of the fused Hadamard + INT4 paged append (sawkv) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]
    python bench.py --workload attn     (decode attention over the INT4 pool)
    python bench.py --workload attn_long  (the same over 64 contexts of 32768 tokens)
    python bench.py --workload concurrency  (rotated vs naive INT4 across 1..256
                                             concurrent decodes)
    python bench.py --heads 1   (one GPU's share of the 8 KV heads under TP-8)

The default workload is the long-context batch: 64 sequences x 32768 tokens,
8 KV heads x 128, page 32 in a shuffled pool, K and V rotated with h = 128.
One step = one sawkv_quantize_append call over the workload's batch (rotate,
token-wise INT4, pack, scatter into the paged pool: the whole write path).
Inputs are generated, uploaded and resident in HBM before timing starts;
after the warm-up steps, launches of the same step run for at least 100 ms
(reported under "settle") so that the timed steps start at steady clocks.
Prints ONE JSON line. Alongside the step it times, on the same batch:
  * the naive-INT4 control (sawkv_naive_int4_append), interleaved with the
    rotated kernel over 9 rounds, for the rotate-vs-naive ratio and its
    bootstrap 95 % interval;
  * the same two kernels with cold caches (an untimed 1 GiB read before every
    timed launch);
  * the read-back (sawkv_dequant_gather) of the same slots, back to back and
    cold;
  * the append's access-pattern control (sawkv_append_pattern_control: the
    same loads and stores, no arithmetic), writing to the mapped slots and to
    token order, interleaved with the append: the bandwidth the append's
    pattern reaches at all on this device;
  * (prefill, sweep) the uncompressed fp16 cache write and token-wise INT8
    append / read-back, with INT8's reconstruction error;
  * the CPU oracle on a bounded sample of the same batch (a baseline only).
Roofline: achieved HBM GB/s of the append kernel (algorithmic bytes per launch
over the event-timed average launch) against the MI355X HBM3E peak, 8 TB/s.

With --workload attn one step is one sawkv_decode_attention call over 256
sequences whose contexts already sit in the INT4 pool (at this size the lean
split: every 16-token step of the batch divided evenly over the resident
waves, the query preparation folded in; then the merge of the partials); its
bytes are the K and V codes and scales of every context token, the queries,
the outputs and the block tables.
"""
import argparse
import dataclasses
import hashlib
import json
import mmap
import multiprocessing
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from int4_kv_cache_amd import workloads as W  # noqa: E402

METRIC = ("GB/s and tokens/s of fused Hadamard+INT4 paged append; % HBM peak; "
          "vs naive INT4")
HBM_PEAK_GBPS = 8000.0
ROT_NAME = {0: "none", 1: "k", 2: "kv"}
KERNEL_SRC = [os.path.join(ROOT, "int4_kv_cache_amd", "csrc", f)
              for f in ("sawkv.hip", "sawkv_append.hpp", "sawkv_device.hpp")]
ATTN_SRC = [os.path.join(ROOT, "int4_kv_cache_amd", "csrc", f)
            for f in ("sawkv_attn.hip", "sawkv_device.hpp")]
ATTN_METRIC = ("GB/s and decode tokens/s of attention over the paged INT4 KV cache "
               "(fused dequant); % HBM peak; vs naive INT4")


def kernel_source_hash(srcs=KERNEL_SRC):
    h = hashlib.sha256()
    for p in srcs:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, srcs=KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash(srcs):
        return None
    return ent.get("bytes_per_launch")


def describe(wl, h, rot):
    vals = {"normal": "N(0,1)", "student_t4": "Student-t(4)"}[wl.values]
    return (f"{wl.name}: {wl.n_seq} seq x {wl.seq_len} tok, {wl.H} KV heads x {wl.D}, "
            f"{vals} + outliers {wl.outliers}, h={h}, rot={ROT_NAME[rot]}, page {wl.P}, "
            f"{wl.placement} slots, {wl.layers} layer(s)")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_FORK_SHARED = {}   # inputs and pools the forked oracle workers inherit


def _shared_zeros(shape, dtype):
    """Zeroed array in anonymous shared memory: forked workers write into the
    parent's pages."""
    n = int(np.prod(shape))
    buf = mmap.mmap(-1, max(n * np.dtype(dtype).itemsize, 1))
    return np.frombuffer(buf, dtype=dtype, count=n).reshape(shape)


def _worker_ready(_):
    return os.getpid()


def _oracle_chunk(bounds):
    from oracle import sawint4 as O
    a, b = bounds
    m = _FORK_SHARED
    O.quantize_append(m["k"][a:b], m["v"][a:b], m["slots"][a:b], m["kc"], m["vc"], m["ks"],
                      m["vs"], h=m["h"], rot_mode=m["rot"])
    return b - a


def cpu_baseline(wl, h, rot, sample_tokens):
    """The oracle, untuned, on the first `sample_tokens` tokens of the batch
    (encode K and V and scatter into host pools): (i) one process; (ii) one
    forked process per available core (at most 16), each on a contiguous
    chunk of the tokens, writing disjoint slots of one shared host pool.
    Runs before this process touches the GPU (the workers are forked)."""
    from oracle import sawint4 as O
    k, v = W.kv(wl, 0, 0, sample_tokens)
    slots = W.slot_mapping(wl)[:sample_tokens]
    code_shape = (wl.N_pg, wl.P, wl.H, wl.D // 2)
    scale_shape = (wl.N_pg, wl.P, wl.H)
    bytes_sample = sample_tokens * wl.bytes_per_token()

    n_proc = max(1, min(16, len(os.sched_getaffinity(0))))
    _FORK_SHARED.update(k=k, v=v, slots=slots, h=h, rot=rot,
                        kc=_shared_zeros(code_shape, np.uint8),
                        vc=_shared_zeros(code_shape, np.uint8),
                        ks=_shared_zeros(scale_shape, np.float16),
                        vs=_shared_zeros(scale_shape, np.float16))
    edges = np.linspace(0, sample_tokens, n_proc + 1).astype(np.int64)
    chunks = [(int(edges[i]), int(edges[i + 1])) for i in range(n_proc)]
    with multiprocessing.get_context("fork").Pool(n_proc) as pool:
        pool.map(_worker_ready, range(n_proc), chunksize=1)     # workers up before the clock
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_chunk, chunks, chunksize=1))
        dt_n = time.perf_counter() - t0
    assert done == sample_tokens

    kc = np.zeros(code_shape, np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros(scale_shape, np.float16)
    vs = np.zeros_like(ks)
    t0 = time.perf_counter()
    O.quantize_append(k, v, slots, kc, vc, ks, vs, h=h, rot_mode=rot)
    dt_1 = time.perf_counter() - t0
    m = _FORK_SHARED
    same = bool(np.array_equal(kc, m["kc"]) and np.array_equal(vc, m["vc"])
                and np.array_equal(ks.view(np.uint16), m["ks"].view(np.uint16))
                and np.array_equal(vs.view(np.uint16), m["vs"].view(np.uint16)))
    _FORK_SHARED.clear()
    return {"value": round(bytes_sample / dt_n / 1e9, 4), "unit": "GB/s", "cores": n_proc,
            "kind": "oracle", "tokens_per_s": round(sample_tokens / dt_n, 1),
            "sample_tokens": sample_tokens,
            "seconds": round(dt_n, 3),
            "sample": f"first {sample_tokens} tokens of the {wl.name} batch (K and V), numpy "
                      f"float32 oracle, {n_proc} forked processes on contiguous token chunks "
                      f"writing disjoint slots of one shared host pool",
            "single_process": {"value": round(bytes_sample / dt_1 / 1e9, 4), "cores": 1,
                               "tokens_per_s": round(sample_tokens / dt_1, 1),
                               "seconds": round(dt_1, 2)},
            "pools_equal_across_legs": same,
            "cpu_model": _cpu_model(), "numpy": np.__version__}

LLC_BYTES = 256 * 1024 * 1024    # MI355X last-level (Infinity) cache


def settle_clocks(torch, fn, min_ms=100.0):
    """Launch `fn` until at least `min_ms` of wall time has passed (synchronised),
    so that the timed steps that follow start at steady clocks."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        if ms >= min_ms:
            return {"launches": n, "ms": round(ms, 1), "min_ms": min_ms}


def bootstrap_ratio_ci(a, b, n=2000, seed=0):
    """95 % bootstrap interval of median(a) / median(b)."""
    rng = np.random.default_rng(seed)
    boots = [np.median(rng.choice(a, len(a))) / np.median(rng.choice(b, len(b)))
             for _ in range(n)]
    return [round(float(np.percentile(boots, 2.5)), 4), round(float(np.percentile(boots, 97.5)), 4)]


def pct(a):
    """p5 / median / p95 of a list of ms, in us."""
    return {q: round(float(np.percentile(a, v)) * 1e3, 2)
            for q, v in (("p5", 5), ("median", 50), ("p95", 95))}


class Flush:
    """An untimed 1 GiB device read before each timed launch (more than the
    256 MB last-level cache plus L2; a read leaves only clean lines)."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.buf = torch.ones(256 * 1024 * 1024, dtype=torch.int32, device=dev)
        self.sum = torch.empty((1,), dtype=torch.int64, device=dev)

    def cold(self, fns, n, stream):
        torch = self.torch
        res = {name: [] for name in fns}
        for _ in range(n):
            for name, fn in fns.items():
                torch.sum(self.buf, dim=(0,), dtype=torch.int64, out=self.sum[0])
                c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c0.record(stream)
                fn()
                c1.record(stream)
                torch.cuda.synchronize()
                res[name].append(c0.elapsed_time(c1))
        return res


def pattern_ceiling(S, torch, wl, kv, slots, pools, step_rot, timed, bytes_step, n_ab):
    """The append's loads and stores with no arithmetic (the access-pattern
    control), at the workload's slots and in token order, interleaved with
    the rotated append over 5 rounds on the same inputs and pools."""
    k, v = kv
    fns = {"same_pattern": S.PatternControlCall(k, v, slots, *pools, placement="slots"),
           "token_order": S.PatternControlCall(k, v, slots, *pools, placement="token_order"),
           "append": step_rot}
    for fn in fns.values():
        for _ in range(5):
            fn()
    ms = {name: [] for name in fns}
    for _ in range(5):
        for name, fn in fns.items():
            ms[name].append(timed(fn, n_ab))
    med = {name: float(np.median(v_)) for name, v_ in ms.items()}
    gb = {name: bytes_step / (m * 1e-3) / 1e9 for name, m in med.items()}
    step_rot()                      # leave the pools holding the append's codes
    torch.cuda.synchronize()
    return {"same_pattern_GBps": round(gb["same_pattern"], 1),
            "token_order_GBps": round(gb["token_order"], 1),
            "append_GBps_interleaved": round(gb["append"], 1),
            "append_over_same_pattern": round(gb["append"] / gb["same_pattern"], 4),
            "same_pattern_us": round(med["same_pattern"] * 1e3, 2),
            "token_order_us": round(med["token_order"] * 1e3, 2),
            "append_us": round(med["append"] * 1e3, 2),
            "rounds": 5, "steps_per_round": n_ab,
            "note": ("sawkv_append_pattern_control: the append's grid, loads and stores with "
                     "none of the method's arithmetic; same_pattern writes the mapped slots, "
                     "token_order writes row t*H + head (contiguous pages)")}


def mse_gpu(torch, out, ref):
    d = out.double() - ref.double()
    return float((d * d).mean().item())


def sweep_variants(S, torch, wl, kv, slots, timed, stream):
    """Block size x rotation ablation on one tensor pair: time of the append
    and reconstruction MSE of K and V after append + gather."""
    k, v = kv
    pools = S.alloc_pools(wl.N_pg, wl.P, wl.H, wl.D, k.device)
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    res = []
    bytes_call = wl.T * wl.bytes_per_token()
    for h in (16, 32, 64, 128):
        for rot in ("none", "k", "kv"):
            fn = lambda: S.quantize_append(k, v, slots, *pools, h=h, rot=rot, stream=stream)
            for _ in range(20):
                fn()
            ms = float(np.median([timed(fn, 100) for _ in range(5)]))
            S.dequant_gather(*pools, slots, h=h, rot=rot, k_out=ko, v_out=vo, stream=stream)
            torch.cuda.synchronize()
            res.append({"h": h, "rotation": rot, "append_us": round(ms * 1e3, 2),
                        "GBps": round(bytes_call / (ms * 1e-3) / 1e9, 1),
                        "mse_k": mse_gpu(torch, ko, k), "mse_v": mse_gpu(torch, vo, v)})
    return res


def controls(S, torch, wl, kv, slots, timed, stream, h, rot):
    """The caches the INT4 cache is compared against, on the same batch: the
    uncompressed fp16 paged write and token-wise INT8 (rotated as the INT4
    run, and naive), each with its bytes per token, GB/s, and the INT8
    reconstruction MSE."""
    k, v = kv
    T, H, D = k.shape
    res = {}
    kc = torch.empty((wl.N_pg, wl.P, H, D), dtype=torch.float16, device=k.device)
    vc = torch.empty_like(kc)
    fn = lambda: S.cache_append(k, v, slots, kc, vc, stream=stream)
    for _ in range(10):
        fn()
    ms = float(np.median([timed(fn, 50) for _ in range(5)]))
    b = T * (H * (2 * D * 2 + 2 * D * 2) + 8)
    res["fp16_cache_append"] = {"us": round(ms * 1e3, 2), "bytes_per_token": b // T,
                                "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
    del kc, vc
    pools8 = S.alloc_int8_pools(wl.N_pg, wl.P, H, D, k.device)
    b8 = T * (H * (2 * D * 2 + 2 * D + 2 * 2) + 8)
    for name, r in (("int8_" + ROT_NAME[rot], ROT_NAME[rot]), ("int8_none", "none")):
        fn = lambda: S.int8_append(k, v, slots, *pools8, h=h, rot=r, stream=stream)
        for _ in range(10):
            fn()
        ms = float(np.median([timed(fn, 50) for _ in range(5)]))
        ko, vo = S.int8_gather(*pools8, slots, h=h, rot=r, stream=stream)
        gfn = lambda: S.int8_gather(*pools8, slots, h=h, rot=r, k_out=ko, v_out=vo,
                                    stream=stream)
        gms = float(np.median([timed(gfn, 50) for _ in range(3)]))
        torch.cuda.synchronize()
        res[name] = {"append_us": round(ms * 1e3, 2), "bytes_per_token": b8 // T,
                     "append_GBps": round(b8 / (ms * 1e-3) / 1e9, 1),
                     "gather_us": round(gms * 1e3, 2),
                     "gather_GBps": round(b8 / (gms * 1e-3) / 1e9, 1),
                     "mse_k": mse_gpu(torch, ko, k), "mse_v": mse_gpu(torch, vo, v)}
    return res


def decode_extras(torch, step_rot, timed, stream, wl, layers, step_prepared):
    """For comparison with the one-launch step: one call per layer (eager,
    through the checking binding and through prepared calls that only
    launch), and the same per-layer calls replayed from one HIP graph."""
    eager_ms = timed(step_rot, 200)
    prepared_ms = timed(step_prepared, 200)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step_rot()           # warm the side stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step_rot()
    torch.cuda.synchronize()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(side)
    for _ in range(200):
        g.replay()
    e1.record(side)
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / 200
    return {"layer_calls_per_step": layers,
            "eager_us_per_step": round(eager_ms * 1e3, 2),
            "eager_us_per_layer_call": round(eager_ms * 1e3 / layers, 3),
            "prepared_us_per_step": round(prepared_ms * 1e3, 2),
            "prepared_us_per_layer_call": round(prepared_ms * 1e3 / layers, 3),
            "graph_us_per_step": round(graph_ms * 1e3, 2),
            "graph_us_per_layer_call": round(graph_ms * 1e3 / layers, 3),
            "graph_tokens_per_s": round(wl.T / (graph_ms * 1e-3), 1)}


def attn_bytes(wl, x):
    """Algorithmic HBM bytes of one decode-attention step: K and V codes and
    scales of every context token, block-table entries, context lengths,
    queries in and outputs out."""
    L = x["context_lens"].astype(np.int64)
    pages = (L + wl.P - 1) // wl.P
    return int(L.sum() * wl.bytes_per_token() + pages.sum() * 4 + wl.B * 4
               + 2 * wl.B * wl.Hq * wl.D * 2)


def attn_cpu_baseline(wl, x, h, rot, budget_s=12.0):
    """The float64 oracle, untuned, on the first sequences of the batch until
    about `budget_s` seconds of work."""
    from oracle import sawint4 as O
    t0 = time.perf_counter()
    n, toks = 0, 0
    while n < wl.B and time.perf_counter() - t0 < budget_s:
        O.paged_decode_attention(x["q"][n:n + 1], x["k_codes"], x["k_scales"], x["v_codes"],
                                 x["v_scales"], x["block_tables"][n:n + 1],
                                 x["context_lens"][n:n + 1], h=h, rot_mode=rot)
        toks += int(x["context_lens"][n])
        n += 1
    dt = time.perf_counter() - t0
    gbps = toks * wl.bytes_per_token() / dt / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "decode_tokens_per_s": round(n / dt, 2), "seconds": round(dt, 2),
            "sample": f"first {n} of {wl.B} sequences ({toks} context tokens) of the "
                      f"{wl.name} batch, numpy float64 oracle, single thread"}


def bench_attention(args):
    import torch
    from int4_kv_cache_amd import sawkv as S

    wl = W.ATTN_WORKLOADS[args.workload]
    if args.heads:
        # one GPU's share under tensor parallelism over KV heads: the same
        # contexts and queries per KV head, fewer KV heads
        wl = dataclasses.replace(wl, H=args.heads, Hq=wl.Hq // wl.H * args.heads)
    h = args.h or wl.h
    rot = {"none": 0, "k": 1, "kv": 2}[args.rot] if args.rot else wl.rot_mode
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    x = W.attn_inputs(wl)
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in x.items()}
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    L = x["context_lens"]
    maxc = int(L.max())
    stream = torch.cuda.current_stream()
    call = S.AttentionCall(d["q"], pools, d["block_tables"], d["context_lens"], maxc, h=h,
                           rot=ROT_NAME[rot])
    naive = S.AttentionCall(d["q"], pools, d["block_tables"], d["context_lens"], maxc, h=h,
                            rot="none", workspace=call.workspace)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(args.warmup):
        call()
    settle = settle_clocks(torch, call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    event_ms = e0.elapsed_time(e1) / args.steps
    nbytes = attn_bytes(wl, x)
    gbps = nbytes / (wall_ms * 1e-3) / 1e9
    achieved = nbytes / (event_ms * 1e-3) / 1e9

    rounds, n_ab = 9, max(20, args.steps // 4)
    rot_ms, naive_ms = [], []
    for _ in range(rounds):
        naive_ms.append(timed(naive, n_ab))
        rot_ms.append(timed(call, n_ab))
    ratio = float(np.median(rot_ms) / np.median(naive_ms))
    ratio_ci = bootstrap_ratio_ci(rot_ms, naive_ms)

    # cold caches: an untimed 1 GiB read before every timed call (the pool of
    # a shard, or of a small batch, fits the 256 MB last-level cache between
    # back-to-back calls)
    flush = Flush(torch, dev)
    cold = flush.cold({"naive": naive, "rot": call}, 15, stream)
    del flush
    cold_out = {"rot_us": pct(cold["rot"]), "naive_us": pct(cold["naive"]),
                "rot_over_naive": round(float(np.median(cold["rot"]) / np.median(cold["naive"])), 4),
                "GBps_rot_median": round(nbytes / (np.median(cold["rot"]) * 1e-3) / 1e9, 1),
                "launches": 15,
                "flush": "1 GiB device read before every timed call (not timed)"}

    # other query-head groupings on the same pool (fresh queries): 8 per KV
    # head (64 query heads, as Llama-2-70B) and 1 (multi-head attention)
    groupings = []
    for hq in (8 * wl.H, wl.H):
        qg = torch.from_numpy(W.attn_queries(wl, hq)).to(dev)
        cg = S.AttentionCall(qg, pools, d["block_tables"], d["context_lens"], maxc, h=h,
                             rot=ROT_NAME[rot])
        ng = S.AttentionCall(qg, pools, d["block_tables"], d["context_lens"], maxc, h=h,
                             rot="none", workspace=cg.workspace)
        for _ in range(10):
            cg()
            ng()
        gr, gn = [], []
        for _ in range(5):
            gn.append(timed(ng, 50))
            gr.append(timed(cg, 50))
        gb = attn_bytes(dataclasses.replace(wl, Hq=hq), x)
        groupings.append({"query_heads": hq, "kv_heads": wl.H,
                          "us": round(float(np.median(gr)) * 1e3, 2),
                          "GBps": round(gb / (np.median(gr) * 1e-3) / 1e9, 1),
                          "rot_over_naive": round(float(np.median(gr) / np.median(gn)), 4)})
        del cg, ng, qg

    traffic = measured_traffic(wl.name, ATTN_SRC) if not args.heads else None
    out = {
        "metric": ATTN_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": (f"{wl.name}: {wl.B} sequences x 1 query token, contexts uniform "
                                f"in [{wl.ctx[1]}, {wl.ctx[2]}] ({int(L.sum())} tokens, max "
                                f"{maxc}), {wl.Hq} query / {wl.H} KV heads x {wl.D}, page "
                                f"{wl.P}, INT4 pool rotation {ROT_NAME[rot]} h={h}"),
                   "sequences": wl.B, "context_tokens": int(L.sum()), "max_context": maxc,
                   "query_heads": wl.Hq, "kv_heads": wl.H, "head_dim": wl.D,
                   "page_size": wl.P, "rotation": ROT_NAME[rot], "block_size_h": h,
                   "parallelism": "single GPU"},
        "step": ("sawkv_decode_attention: split-context kernel (query prep folded in) + "
                 "merge (2 launches)"),
        "decode_tokens_per_s": round(wl.B / (wall_ms * 1e-3), 1),
        "context_tokens_per_s": round(int(L.sum()) / (wall_ms * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "kernel": "one sawkv_decode_attention call (attn_lean_pair_kernel, or "
                               "attn_chunk_pair_kernel below the lean split's sizes, + "
                               "attn_combine_kernel)"},
        "vs_naive": {"rot_ms_median": round(float(np.median(rot_ms)), 5),
                     "naive_ms_median": round(float(np.median(naive_ms)), 5),
                     "rot_over_naive": round(ratio, 4), "rot_over_naive_ci95": ratio_ci,
                     "rounds": rounds, "steps_per_round": n_ab},
        "settle": settle,
        "cold": cold_out,
        "cache_resident": nbytes <= LLC_BYTES,
        "other_head_groupings": groupings,
        "workspace_bytes": int(call.workspace.numel()),
        "kernel_source_hash": kernel_source_hash(ATTN_SRC),
    }
    if not args.no_cpu:
        print("[bench] cpu baseline: oracle attention on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = attn_cpu_baseline(wl, x, h, rot)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def measured_step(torch, S, c, app, layer_pools, d, maxc, wa, ws, layers, n):
    """One whole decode step at concurrency c per rotation mode, captured into
    a HIP graph and replayed: the layered append, then each layer's attention
    over its own pool copy (one shared workspace; the calls run in order on
    one stream). The graph's last output is checked against an eager run of
    the same step after every timing round."""
    stream = torch.cuda.current_stream()
    q, bt, cl = d["q"][:c], d["block_tables"][:c], d["context_lens"][:c]
    out = {r: torch.empty_like(q) for r in ("k", "none")}
    att = {r: [S.AttentionCall(q, lp, bt, cl, maxc, h=wa.h, rot=r, out=out[r], workspace=ws)
               for lp in layer_pools] for r in ("k", "none")}

    def step(r):
        app[r]()
        for a in att[r]:
            a()

    graphs = {}
    for r in ("k", "none"):
        step(r)                                   # eager, outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        torch.cuda.synchronize()
        graphs[r] = g

    def check(r):
        graphs[r].replay()
        torch.cuda.synchronize()
        got = out[r].clone()
        step(r)
        torch.cuda.synchronize()
        if not torch.equal(got, out[r]):
            raise RuntimeError(f"graph replay of the decode step differs from eager ({r})")

    def timed(r):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            graphs[r].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for r in ("k", "none"):
        for _ in range(3):
            graphs[r].replay()
        check(r)
    rot, naive = [], []
    for _ in range(9):
        naive.append(timed("none"))
        rot.append(timed("k"))
        check("k")
        check("none")
    return {"rot_us": round(float(np.median(rot)) * 1e3, 2),
            "naive_us": round(float(np.median(naive)) * 1e3, 2),
            "rot_over_naive": round(float(np.median(rot) / np.median(naive)), 4),
            "rot_over_naive_ci95": bootstrap_ratio_ci(rot, naive),
            "launches_per_step": 1 + 2 * layers, "replays_per_round": n, "rounds": 9}


def bench_concurrency(args):
    """The pages' serving claim, measured on this path: rotated INT4 against
    plain (naive) INT4 across concurrency levels. Per decode step at
    concurrency c: the 36 layers' appends of c new tokens in one launch
    (decode recipe, K-only rotation), and decode attention of the c sequences
    over their cached contexts (attn recipe, first c sequences), timed on one
    layer's pool; the step estimate is append + 36 x attention. The whole step
    is also measured: the append launch and 36 attention calls, each layer
    reading its own copy of the pool (so the layers do not share cached
    lines), captured into one HIP graph per rotation mode and replayed back
    to back (its output checked against the same step run eagerly)."""
    import torch
    from int4_kv_cache_amd import sawkv as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    wl = W.WORKLOADS["decode"]
    layers = wl.layers
    print(f"[bench] generating decode + attn inputs", file=sys.stderr, flush=True)
    slots = torch.from_numpy(W.slot_mapping(wl)).to(dev)
    kvs = []
    for layer in range(layers):
        k, v = W.kv(wl, layer)
        kvs.append((torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)))
    pools = [S.alloc_pools(wl.N_pg, wl.P, wl.H, wl.D, dev) for _ in range(layers)]
    wa = W.ATTN_WORKLOADS["attn"]
    x = W.attn_inputs(wa)
    d = {k_: torch.from_numpy(np.ascontiguousarray(v_)).to(dev) for k_, v_ in x.items()}
    apools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    # one pool copy per layer for the measured step (36 x 1.1 GB)
    layer_pools = [apools] + [tuple(t.clone() for t in apools) for _ in range(layers - 1)]
    ws = torch.empty(S.attention_workspace_size(wa.B, wa.Hq, wa.H, int(x["context_lens"].max())),
                     dtype=torch.uint8, device=dev)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    levels = []
    t_start = time.perf_counter()
    settle = None
    for c in (1, 4, 16, 64, 256):
        kv_c = [(k_[:c], v_[:c]) for k_, v_ in kvs]
        app = {r: S.LayersCall(kv_c, slots[:c], pools, h=wl.h, rot=r) for r in ("k", "none")}
        L = x["context_lens"][:c]
        maxc = int(L.max())
        att = {r: S.AttentionCall(d["q"][:c], apools, d["block_tables"][:c],
                                  d["context_lens"][:c], maxc, h=wa.h, rot=r)
               for r in ("k", "none")}
        res = {}
        if settle is None:
            settle = settle_clocks(torch, att["k"])
        for name, calls in (("append", app), ("attention", att)):
            for fn in calls.values():
                for _ in range(20):
                    fn()
            rot, naive = [], []
            n = max(20, args.steps // 10)
            for _ in range(9):
                naive.append(timed(calls["none"], n))
                rot.append(timed(calls["k"], n))
            res[name] = {"rot_us": round(float(np.median(rot)) * 1e3, 3),
                         "naive_us": round(float(np.median(naive)) * 1e3, 3),
                         "rot_over_naive": round(float(np.median(rot) / np.median(naive)), 4),
                         "rot_over_naive_ci95": bootstrap_ratio_ci(rot, naive)}
        step_rot = res["append"]["rot_us"] + layers * res["attention"]["rot_us"]
        step_naive = res["append"]["naive_us"] + layers * res["attention"]["naive_us"]
        measured = measured_step(torch, S, c, app, layer_pools, d, maxc, wa, ws, layers,
                                 max(10, args.steps // 100))
        levels.append({"concurrency": c, "context_tokens": int(L.sum()),
                       "append_36_layers": res["append"], "attention_one_layer": res["attention"],
                       "step_estimate_us": {"rot": round(step_rot, 2), "naive": round(step_naive, 2),
                                            "rot_over_naive": round(step_rot / step_naive, 4)},
                       "step_measured_us": measured,
                       "tokens_per_s": round(c / (measured["rot_us"] * 1e-6), 1),
                       "tokens_per_s_estimate": round(c / (step_rot * 1e-6), 1)})
        print(f"[bench] concurrency {c}: step {measured['rot_us']:.1f} us measured "
              f"(naive {measured['naive_us']:.1f}; estimate {step_rot:.1f} / {step_naive:.1f})",
              file=sys.stderr, flush=True)
    wall = time.perf_counter() - t_start
    top = levels[-1]
    out = {
        "metric": "decode tokens/s of the INT4 KV path (36-layer append + attention) across "
                  "concurrency; rotated vs naive INT4",
        "value": top["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 20,
        "ms_per_step": round(top["step_measured_us"]["rot_us"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": ("concurrency sweep: decode recipe (8 KV heads x 128, 36 layers, "
                                "K-only rotation h=128) for the appends, attn recipe (32 query "
                                "heads, contexts uniform in [1, 8000], page 16) for attention; "
                                "step = the 36-layer append launch + 36 attention calls, one "
                                "pool copy per layer, replayed from a HIP graph (value); "
                                "step estimate = 36-layer append + 36 x one layer's attention"),
                   "levels": [l["concurrency"] for l in levels], "parallelism": "single GPU"},
        "levels": levels,
        "settle": settle,
        "seconds": round(wall, 1),
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="long",
                    choices=["prefill", "decode", "sweep", "long", "attn", "attn_long",
                             "concurrency"])
    ap.add_argument("--h", type=int, default=None)
    ap.add_argument("--heads", type=int, default=None,
                    help="KV heads per GPU (e.g. 1 or 2: the TP-8 / TP-4 share of 8 heads; 'attn' keeps the query heads per KV head)")
    ap.add_argument("--rot", default=None, choices=["none", "k", "kv"])
    ap.add_argument("--cpu-sample", type=int, default=131072)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the append/gather path has no exchange "
              "step, so a multi-GPU figure is not produced (run with --gpus 1).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    if args.workload in ("attn", "attn_long"):
        bench_attention(args)
        return
    if args.workload == "concurrency":
        bench_concurrency(args)
        return

    wl = W.WORKLOADS[args.workload]
    if args.heads:
        # one GPU's share under tensor parallelism over KV heads (8 heads / TP-n)
        wl = dataclasses.replace(wl, H=args.heads)
    h = args.h or wl.h
    rot = {"none": 0, "k": 1, "kv": 2}[args.rot] if args.rot else wl.rot_mode

    # the CPU leg forks its workers, so it runs before anything touches the GPU
    cpu = None
    if not args.no_cpu:
        n = min(args.cpu_sample, wl.T)
        print(f"[bench] cpu baseline: oracle on {n} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, h, rot, n)
        print(f"[bench] cpu baseline done: {cpu['value']} GB/s on {cpu['cores']} processes, "
              f"{cpu['single_process']['value']} GB/s on one", file=sys.stderr, flush=True)

    import torch
    from int4_kv_cache_amd import sawkv as S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = wl.layers

    print(f"[bench] generating {describe(wl, h, rot)}", file=sys.stderr, flush=True)
    slots = torch.from_numpy(W.slot_mapping(wl)).to(dev)
    kvs = []
    for layer in range(layers):
        k, v = W.kv(wl, layer)
        kvs.append((torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)))
        del k, v
    pools = [S.alloc_pools(wl.N_pg, wl.P, wl.H, wl.D, dev) for _ in range(layers)]
    naive_pools = pools   # the control writes the same bytes to the same rows
    stream = torch.cuda.current_stream()   # every launch below goes to the current stream

    def per_layer_rot():
        for layer in range(layers):
            S.quantize_append(kvs[layer][0], kvs[layer][1], slots, *pools[layer], h=h,
                              rot=ROT_NAME[rot])

    if layers > 1:
        # a decode step: every layer's append in one launch (arguments marshalled once)
        step_rot = S.LayersCall(kvs, slots, pools, h=h, rot=ROT_NAME[rot])
        step_naive = S.LayersCall(kvs, slots, naive_pools, h=h, rot="none")
    else:
        # arguments checked and marshalled once; each call only launches
        step_rot = S.AppendCall(kvs[0][0], kvs[0][1], slots, *pools[0], h=h, rot=ROT_NAME[rot])
        step_naive = S.NaiveAppendCall(kvs[0][0], kvs[0][1], slots, *naive_pools[0])

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n      # ms per step

    tokens = wl.T                      # new tokens per step (each appended to every layer)
    bytes_step = wl.T * wl.bytes_per_token() * layers
    read_bytes = wl.T * (wl.H * 2 * wl.D * 2 + 8) * layers       # fp16 K, V and slots

    # warm-up, clock settle, then the timed K steps (wall clock bracketed by
    # synchronize; events on the launch stream)
    for _ in range(args.warmup):
        step_rot()
    settle = settle_clocks(torch, step_rot)
    print(f"[bench] settle: {settle['launches']} launches in {settle['ms']} ms; timing "
          f"{args.steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step_rot()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    event_ms = e0.elapsed_time(e1) / args.steps
    gbps = bytes_step / (wall_ms * 1e-3) / 1e9
    achieved = bytes_step / (event_ms * 1e-3) / 1e9

    # rotated vs naive: interleaved rounds on the same inputs and pools
    rounds = 9
    n_ab = max(20, args.steps // 4)
    rot_ms, naive_ms = [], []
    for _ in range(rounds):
        naive_ms.append(timed(step_naive, n_ab))
        rot_ms.append(timed(step_rot, n_ab))
    ratio = float(np.median(rot_ms) / np.median(naive_ms))
    ratio_ci = bootstrap_ratio_ci(rot_ms, naive_ms)
    print(f"[bench] rot/naive {ratio:.4f} {ratio_ci}", file=sys.stderr, flush=True)

    # cold caches: every timed launch follows an untimed read of 1 GiB (larger
    # than the 256 MB last-level cache plus L2), which leaves only clean lines
    # behind (a fill would leave dirty ones, whose write-back lands in the timed
    # launch); rotated and naive interleaved
    flush = Flush(torch, dev)
    n_cold = 30 if wl.T * layers <= 262144 else 10
    cold = flush.cold({"naive": step_naive, "rot": step_rot}, n_cold, stream)
    cold_out = {"rot_us": pct(cold["rot"]), "naive_us": pct(cold["naive"]),
                "rot_over_naive": round(float(np.median(cold["rot"]) / np.median(cold["naive"])), 4),
                "GBps_rot_median": round(bytes_step / (np.median(cold["rot"]) * 1e-3) / 1e9, 1),
                "launches": n_cold,
                "flush": "1 GiB device read before every timed launch (not timed)"}

    # read-back of the same slots: back to back, then cold
    outs = [(torch.empty_like(kvs[l][0]), torch.empty_like(kvs[l][1])) for l in range(layers)]
    gcalls = [S.GatherCall(*pools[l], slots, outs[l][0], outs[l][1], h=h, rot=ROT_NAME[rot])
              for l in range(layers)]

    def gather_fn():
        for c in gcalls:
            c()
    for _ in range(3):
        gather_fn()
    g_ms = timed(gather_fn, max(20, args.steps // 2))
    g_cold = flush.cold({"gather": gather_fn}, n_cold, stream)["gather"]
    g_read = wl.T * (wl.H * 2 * (wl.D // 2 + 2) + 8) * layers       # codes, scales, slots
    print(f"[bench] gather {g_ms * 1e3:.1f} us back to back, {np.median(g_cold) * 1e3:.1f} us "
          f"cold", file=sys.stderr, flush=True)

    # the append's own access pattern with no arithmetic, interleaved with the
    # append: at the workload's slots and in token order
    attainable = {}
    if layers == 1:
        attainable = pattern_ceiling(S, torch, wl, kvs[0], slots, pools[0], step_rot, timed,
                                     bytes_step, n_ab)
    del flush

    extra = {}
    if args.workload == "sweep":
        extra["variants"] = sweep_variants(S, torch, wl, kvs[0], slots, timed, stream)
    if args.workload == "decode":
        prepared = [S.AppendCall(kvs[layer][0], kvs[layer][1], slots, *pools[layer], h=h,
                                 rot=ROT_NAME[rot]) for layer in range(layers)]

        def per_layer_prepared():
            for call in prepared:
                call()
        extra["decode"] = decode_extras(torch, per_layer_rot, timed, stream, wl, layers,
                                        per_layer_prepared)
    if args.workload in ("sweep", "long", "prefill"):
        ko, vo = outs[0]
        extra["mse"] = {"k": mse_gpu(torch, ko, kvs[0][0]), "v": mse_gpu(torch, vo, kvs[0][1])}
    if args.workload in ("prefill", "sweep"):
        extra["controls"] = controls(S, torch, wl, kvs[0], slots, timed, stream, h, rot)
    del outs, gcalls

    # attainable-bandwidth context on this machine: a 256 MiB device copy (torch)
    cbuf = torch.empty(64 * 1024 * 1024, dtype=torch.int32, device=dev)
    cdst = torch.empty_like(cbuf)
    cdst.copy_(cbuf)
    c_ms = timed(lambda: cdst.copy_(cbuf), 50)
    attainable["copy_256MiB_GBps"] = round(2 * cbuf.numel() * 4 / (c_ms * 1e-3) / 1e9, 1)
    attainable["copy_note"] = "torch device-to-device copy on the same GPU, context only"
    del cbuf, cdst

    # the committed counters cover the workloads at their own shapes only
    traffic = measured_traffic(args.workload) if not args.heads else None
    resident = read_bytes <= LLC_BYTES
    # every timed call rewrites the same rows of codes and scales: when those
    # rows fit the last-level cache, back-to-back calls can leave part of the
    # writes there (the cold figures start from a flushed cache)
    rows_bytes = wl.T * wl.H * (wl.D // 2 + 2) * 2 * layers
    out = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": describe(wl, h, rot), "tokens_per_step": tokens,
                   "layers_appended_per_token": layers,
                   "heads": wl.H, "head_dim": wl.D, "block_size_h": h,
                   "rotation": ROT_NAME[rot], "page_size": wl.P, "pages": wl.N_pg,
                   "layers_per_step": layers, "parallelism": "single GPU",
                   "cpu_sample_tokens": None if cpu is None else cpu["sample_tokens"]},
        "step": ("sawkv_quantize_append_layers: every layer of the decode step in one launch"
                 if layers > 1 else
                 "sawkv_quantize_append over the batch (rotate, token-wise INT4, pack, "
                 "paged scatter)"),
        "tokens_per_s": round(tokens / (wall_ms * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "cache_resident": resident,
        "rewritten_rows_fit_llc": rows_bytes <= LLC_BYTES,
        "settle": settle,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_step,
                     "event_us_per_launch": round(event_ms * 1e3, 2),
                     "kernel": ("sawkv::append_layers_kernel" if layers > 1
                                else "sawkv::append_kernel"),
                     **({"frac_of_same_pattern":
                         round(achieved / attainable["same_pattern_GBps"], 4)}
                        if "same_pattern_GBps" in attainable else {})},
        "vs_naive": {"rot_ms_median": round(float(np.median(rot_ms)), 5),
                     "naive_ms_median": round(float(np.median(naive_ms)), 5),
                     "rot_over_naive": round(ratio, 4),
                     "rot_over_naive_ci95": ratio_ci,
                     "naive_GBps": round(bytes_step / (np.median(naive_ms) * 1e-3) / 1e9, 2),
                     "rounds": rounds, "steps_per_round": n_ab},
        "gather": {"ms_per_step": round(g_ms, 5),
                   "GBps": round(bytes_step / (g_ms * 1e-3) / 1e9, 2),
                   "tokens_per_s": round(tokens / (g_ms * 1e-3), 1),
                   "cache_resident": g_read <= LLC_BYTES,
                   "cold": {"us": pct(g_cold),
                            "GBps_median": round(bytes_step / (np.median(g_cold) * 1e-3) / 1e9, 1),
                            "launches": n_cold,
                            "flush": "1 GiB device read before every timed launch (not timed)"}},
        "cold": cold_out,
        "attainable": attainable,
        "kernel_source_hash": kernel_source_hash(),
        **extra,
    }
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
