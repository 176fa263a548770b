"""GPU parity of decode attention over the paged INT4 pools (sawkv_decode_attention,
called through the C ABI) against the float64 oracle.

Tolerance, per output element of sequence b and query head j (derived from the
kernel's arithmetic; Vmax bounds |V_t| over the context, Bmax bounds the
log2-unit logits' L1 magnitude):

    |got - ref| <= 2^-10 |ref| + Vmax * (2^-14 + 2^-17 * Bmax)

  * 2^-10 |ref|: the final fp16 rounding (half an ulp is <= 2^-11 |ref|).
  * Vmax * 2^-14: the value side. The weights p * s_v enter the matrix cores as
    fp16 hi + lo (relative error <= 2^-22), products with the codes are exact,
    float32 accumulation rounds once per matrix-core product of 32 token
    slots (twice per 16-token step where the hi and the lo weights enter as
    two products into one accumulator, eight queries per head in head pairs:
    at most 128 roundings, 2^-17 relative, over a chunk of 1024 tokens), and
    the +8 code bias is removed with a float32 running sum (<= 2^-17 relative
    over a chunk, times 8).
  * Vmax * 2^-17 * Bmax: the logits. The query enters as fp16 hi + lo
    (<= 2^-22 relative per channel); the bias constant and five float32
    roundings of sums bounded by 23 * sum |q'| * 8 give an absolute logit
    error below 2^-19 * Bmax (log2 units), and a logit error d moves the
    softmax average by at most 2 ln 2 * d * Vmax.
  Bmax = sm_scale * log2(e) * max_t s_k,t * 8 * ||R q||_1 (R the rotation
  when keys are rotated); Vmax = 8 * max_t s_v,t, times sqrt(h) when values
  are rotated (an error in the rotated basis grows by at most sqrt(h) in one
  channel after the inverse rotation).
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import scipy.linalg

from oracle import sawint4 as O
from int4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

ROTS = {O.ROT_NONE: "none", O.ROT_K: "k", O.ROT_KV: "kv"}
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    from int4_kv_cache_amd import sawkv as S   # raises if libsawkv.so is missing
    return torch, S


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_dev(env, x):
    torch, _ = env
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}


def run_gpu(env, x, max_context, h, rot, sm_scale=None, q=None):
    torch, S = env
    d = to_dev(env, x)
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    out = S.decode_attention(d["q"] if q is None else q, pools, d["block_tables"],
                             d["context_lens"], max_context, h=h, rot=ROTS[rot],
                             sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_oracle(x, h, rot, seqs=None, sm_scale=None, max_context=None):
    L = np.asarray(x["context_lens"]).astype(np.int64)
    if max_context is not None:
        L = np.clip(L, 0, max_context)
    seqs = np.arange(len(L)) if seqs is None else np.asarray(seqs)
    return O.paged_decode_attention(x["q"][seqs], x["k_codes"], x["k_scales"], x["v_codes"],
                                    x["v_scales"], x["block_tables"][seqs], L[seqs], h=h,
                                    rot_mode=rot, sm_scale=sm_scale)


def tolerance(x, h, rot, seqs, ref, sm_scale=None, max_context=None):
    """Per-element bound from the module docstring."""
    q = x["q"][seqs].astype(np.float64)
    B, Hq, D = q.shape
    n_pg, P, H, _ = x["k_codes"].shape
    G = Hq // H
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    if rot != O.ROT_NONE:
        blk = np.kron(np.eye(D // h), scipy.linalg.hadamard(h) / math.sqrt(h))
        q = q @ blk.T
    l1 = np.abs(q).sum(-1)                                     # [B, Hq]
    tol = np.zeros_like(ref)
    ks = x["k_scales"].reshape(n_pg * P, H).astype(np.float64)
    vs = x["v_scales"].reshape(n_pg * P, H).astype(np.float64)
    vfac = 8.0 * (math.sqrt(h) if rot == O.ROT_KV else 1.0)
    for i, b in enumerate(seqs):
        L = int(x["context_lens"][b])
        if max_context is not None:
            L = min(max(L, 0), max_context)
        t = np.arange(L)
        pages = x["block_tables"][b][t // P].astype(np.int64)
        ok = (pages >= 0) & (pages < n_pg)
        slots = (pages * P + t % P)[ok]
        if len(slots) == 0:
            continue
        for j in range(Hq):
            kv = j // G
            bmax = abs(sm) * LOG2E * ks[slots, kv].max() * 8.0 * l1[i, j]
            vmax = vfac * vs[slots, kv].max()
            tol[i, j] = vmax * (2.0 ** -14 + 2.0 ** -17 * bmax)
    return 2.0 ** -10 * np.abs(ref) + tol


def check(got, ref, tol, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    ratio = err / np.maximum(tol, 1e-300)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    say(f"{what}: max err {err.max():.3g}, max err/tol {ratio.max():.3g} at {worst}, "
        f"median |ref| {np.median(np.abs(ref)):.3g}")
    assert ratio.max() <= 1.0, f"{what}: error {err[worst]:.4g} > tol {tol[worst]:.4g} at {worst}"


def small(**kw):
    return dataclasses.replace(W.ATTN_WORKLOADS["attn_small"], **kw)


# --------------------------------------------------------------------------
# small cases: every output element against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("rot", [O.ROT_NONE, O.ROT_K, O.ROT_KV])
@pytest.mark.parametrize("h", [16, 32, 64, 128])
def test_small_all_rotations(env, rot, h):
    wl = small(h=h, rot_mode=rot)
    x = W.attn_inputs(wl)
    maxc = int(x["context_lens"].max())
    say(f"attn_small rot={ROTS[rot]} h={h} L={x['context_lens'].tolist()}")
    got = run_gpu(env, x, maxc, h, rot)
    ref = run_oracle(x, h, rot)
    check(got, ref, tolerance(x, h, rot, np.arange(wl.B), ref), f"small rot={rot} h={h}")
    assert np.array_equal(got[0], np.zeros_like(got[0]))          # empty context


@pytest.mark.parametrize("rot,h", [(O.ROT_NONE, 128), (O.ROT_K, 128), (O.ROT_KV, 128),
                                   (O.ROT_KV, 32)])
def test_few_sequences_long_contexts(env, rot, h):
    """Few sequences, long contexts: more than 16 chunks of 128 tokens over 128
    output vectors, the case where the merge of the chunks runs one wave per
    output vector; one empty context among them."""
    wl = small(B=4, ctx=("list", (6000, 0, 2500, 4100)), wid=40, masked=2, h=h, rot_mode=rot)
    x = W.attn_inputs(wl)
    say(f"attn few long contexts rot={ROTS[rot]} h={h} L={x['context_lens'].tolist()}")
    got = run_gpu(env, x, 6000, h, rot)
    ref = run_oracle(x, h, rot)
    check(got, ref, tolerance(x, h, rot, np.arange(wl.B), ref), f"long ctx rot={rot} h={h}")
    assert np.array_equal(got[1], np.zeros_like(got[1]))


# at most four queries per KV head and an even H run the head-pair kernel
# (G = 1 and 2 with repeated query slots: (8, 8), (16, 8), (2, 2), (12, 6);
# G = 4: (8, 2), (16, 4), (24, 6), (64, 16)); an odd H, or eight queries per
# KV head on a grid this shallow, the single-head kernel ((64, 8), (4, 1),
# (3, 3), (6, 3), (24, 3))
@pytest.mark.parametrize("Hq,H", [(8, 8), (16, 8), (64, 8), (4, 1), (2, 2), (12, 6),
                                  (8, 2), (16, 4), (24, 6), (64, 16), (3, 3), (6, 3),
                                  (24, 3)])
def test_group_sizes(env, Hq, H):
    wl = small(Hq=Hq, H=H, wid=8 + Hq + H)
    x = W.attn_inputs(wl)
    say(f"attn G={Hq // H} Hq={Hq} H={H}")
    got = run_gpu(env, x, int(x["context_lens"].max()), 128, O.ROT_KV)
    ref = run_oracle(x, 128, O.ROT_KV)
    check(got, ref, tolerance(x, 128, O.ROT_KV, np.arange(wl.B), ref), f"G={Hq // H}")


def widen_tables(x, max_context):
    """Block tables padded with -1 to ceil(max_context / P) columns (the
    bound the call checks; pages past a context's end are never read)."""
    P = x["k_codes"].shape[1]
    need = -(-max_context // P)
    bt = x["block_tables"]
    if bt.shape[1] < need:
        pad = np.full((bt.shape[0], need - bt.shape[1]), -1, dtype=bt.dtype)
        bt = np.concatenate([bt, pad], axis=1)
    return dict(x, block_tables=bt)


# Eight queries per KV head over an even head count, the short, masked
# attn_small contexts (0 to 1300 tokens, so the oracle stays cheap) under a
# large max_context: 50000 keeps the chunk form, where nine sequences give too
# few blocks for the head-pair kernel, so the single-head kernel runs
# (512-token chunks); 2^17 and 2^19 take the lean split, whose head-pair
# kernel for eight queries runs the pipelined step loop over ranges that hold
# several of these sequences each.
@pytest.mark.parametrize("max_context,P,rot,h", [
    (50000, 16, O.ROT_KV, 128), (50000, 16, O.ROT_NONE, 128), (1 << 17, 16, O.ROT_K, 16),
    (1 << 17, 16, O.ROT_KV, 64), (1 << 17, 32, O.ROT_KV, 32), (1 << 17, 64, O.ROT_K, 128),
    (1 << 19, 16, O.ROT_KV, 128), (1 << 19, 16, O.ROT_K, 64)])
def test_eight_queries_per_head_in_pairs(env, max_context, P, rot, h):
    wl = small(Hq=64, H=8, P=P, wid=90 + P + h)
    x = widen_tables(W.attn_inputs(wl), max_context)
    say(f"attn G=8 head pairs max_context={max_context} P={P} rot={ROTS[rot]} h={h}")
    got = run_gpu(env, x, max_context, h, rot)
    ref = run_oracle(x, h, rot)
    check(got, ref, tolerance(x, h, rot, np.arange(wl.B), ref),
          f"G=8 pairs max_context={max_context} P={P}")


# an odd head count runs the single-head kernel; with four queries per KV
# head its query rotation spans 16 lanes of 8 channels (three fused cross-lane
# stages, then one more), every block size h
@pytest.mark.parametrize("Hq,H", [(4, 1), (12, 3)])
@pytest.mark.parametrize("h", [16, 32, 64])
def test_single_head_kernel_block_sizes(env, Hq, H, h):
    wl = small(Hq=Hq, H=H, h=h, rot_mode=O.ROT_KV, wid=70 + Hq + h)
    x = W.attn_inputs(wl)
    say(f"attn single-head G={Hq // H} H={H} h={h}")
    got = run_gpu(env, x, int(x["context_lens"].max()), h, O.ROT_KV)
    ref = run_oracle(x, h, O.ROT_KV)
    check(got, ref, tolerance(x, h, O.ROT_KV, np.arange(wl.B), ref), f"single-head H={H} h={h}")


@pytest.mark.parametrize("P", [32, 64])
def test_page_sizes(env, P):
    wl = small(P=P, wid=20 + P)
    x = W.attn_inputs(wl)
    say(f"attn P={P}")
    got = run_gpu(env, x, int(x["context_lens"].max()), 128, O.ROT_K)
    ref = run_oracle(x, 128, O.ROT_K)
    check(got, ref, tolerance(x, 128, O.ROT_K, np.arange(wl.B), ref), f"P={P}")


def test_lengths_beyond_max_context_and_negative(env):
    x = W.attn_inputs(small())
    x["context_lens"] = np.array([0, 1, 15, -5, 17, 33, 100, 700, 1300], dtype=np.int32)
    maxc = 650
    say("attn lengths clipped to max_context=650, one negative")
    got = run_gpu(env, x, maxc, 128, O.ROT_KV)
    ref = run_oracle(x, 128, O.ROT_KV, max_context=maxc)
    check(got, ref, tolerance(x, 128, O.ROT_KV, np.arange(9), ref, max_context=maxc), "clip")
    assert np.array_equal(got[3], np.zeros_like(got[3]))


def test_zero_max_context_gives_zeros(env):
    x = W.attn_inputs(small())
    say("attn max_context=0")
    got = run_gpu(env, x, 0, 128, O.ROT_KV)
    assert np.array_equal(got, np.zeros_like(got))


def test_strided_q_and_custom_scale(env):
    torch, S = env
    x = W.attn_inputs(small())
    big = torch.zeros((9, 48, 128), dtype=torch.float16, device="cuda")
    big[:, 5:37] = torch.from_numpy(x["q"]).cuda()
    q = big[:, 5:37]                                       # row stride 48*128
    for sm in (0.05, -0.2):
        say(f"attn strided q, sm_scale={sm}")
        got = run_gpu(env, x, 1300, 64, O.ROT_KV, sm_scale=sm, q=q)
        ref = run_oracle(x, 64, O.ROT_KV, sm_scale=sm)
        check(got, ref, tolerance(x, 64, O.ROT_KV, np.arange(9), ref, sm_scale=sm),
              f"sm={sm}")


# (32 query heads: head pairs of four queries; 64 with a deep grid: head
# pairs of eight, see test_eight_queries_per_head_in_pairs)
@pytest.mark.parametrize("Hq,max_context", [(32, 1300), (64, 1 << 17)])
def test_peaked_softmax_outlier_heads(env, Hq, max_context):
    """Scales 20x larger on two heads per tensor make the softmax nearly
    one-hot there; sharpen further with a large sm_scale."""
    x = widen_tables(W.attn_inputs(small(Hq=Hq)), max_context)
    say(f"attn sm_scale=1.0 (peaked) Hq={Hq} max_context={max_context}")
    got = run_gpu(env, x, max_context, 128, O.ROT_K, sm_scale=1.0)
    ref = run_oracle(x, 128, O.ROT_K, sm_scale=1.0)
    check(got, ref, tolerance(x, 128, O.ROT_K, np.arange(9), ref, sm_scale=1.0),
          f"peaked Hq={Hq}")


# --------------------------------------------------------------------------
# end to end: the product write path fills the pool, attention reads it
# --------------------------------------------------------------------------

def test_append_then_attention(env):
    """K/V of the sweep recipe written by sawkv_quantize_append on the GPU and
    by the oracle on the CPU; the pools must agree byte for byte, and the
    attention over them must match the oracle's attention over its own pool."""
    torch, S = env
    wl = dataclasses.replace(W.WORKLOADS["sweep"], n_seq=4, seq_len=700, N_pg=4096)
    k, v = W.kv(wl)
    slots = W.slot_mapping(wl)
    for rot in (O.ROT_K, O.ROT_KV):
        say(f"append then attention rot={ROTS[rot]}")
        kc, vc, ks, vs = S.alloc_pools(wl.N_pg, wl.P, wl.H, wl.D, "cuda", code_fill=0,
                                       scale_bits_fill=0)
        S.quantize_append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                          torch.from_numpy(slots).cuda(), kc, vc, ks, vs, h=128, rot=ROTS[rot])
        okc = np.zeros((wl.N_pg, wl.P, wl.H, wl.D // 2), np.uint8)
        ovc = okc.copy()
        oks = np.zeros((wl.N_pg, wl.P, wl.H), np.float16)
        ovs = oks.copy()
        O.quantize_append(k, v, slots, okc, ovc, oks, ovs, 128, rot)
        assert kc.cpu().numpy().tobytes() == okc.tobytes()
        assert vs.cpu().numpy().tobytes() == ovs.tobytes()
        # pages of sequence s are the free-list pages its tokens were written to
        pages = (slots // wl.P).reshape(wl.n_seq, wl.seq_len)[:, ::wl.P].astype(np.int32)
        L = np.array([700, 1, 350, 699], dtype=np.int32)
        rng = np.random.default_rng(5)
        q = rng.standard_normal((wl.n_seq, 4 * wl.H, wl.D)).astype(np.float16)
        x = {"q": q, "k_codes": okc, "v_codes": ovc, "k_scales": oks, "v_scales": ovs,
             "block_tables": pages, "context_lens": L}
        got = S.decode_attention(torch.from_numpy(q).cuda(), (kc, vc, ks, vs),
                                 torch.from_numpy(pages).cuda(), torch.from_numpy(L).cuda(), 700,
                                 h=128, rot=ROTS[rot])
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        ref = run_oracle(x, 128, rot)
        check(got, ref, tolerance(x, 128, rot, np.arange(4), ref), f"e2e rot={rot}")


# --------------------------------------------------------------------------
# the lean split: from 40 960 steps of 16 tokens (B * ceil(max_context / 16))
# up to 1024 sequences with an even KV-head count, the step's 16-token steps
# are split evenly over the device's resident waves; a wave's range spans
# sequence ends, several short sequences, or (past 64 steps) more than 64
# pages, and with fewer steps than waves most ranges are empty
# --------------------------------------------------------------------------

def lens_case(env, Hq, lens, max_context, P=16, h=128, rot=O.ROT_K, seqs=None, wid=90,
              masked=3):
    wl = small(B=len(lens), Hq=Hq, ctx=("list", tuple(int(v) for v in lens)), P=P, h=h,
               rot_mode=rot, wid=wid, masked=masked)
    x = widen_tables(W.attn_inputs(wl), max_context)
    L = x["context_lens"]
    say(f"attn lens case B={len(L)} Hq={Hq} P={P} tokens={int(np.clip(L, 0, None).sum())} "
        f"max_context={max_context} rot={ROTS[rot]} h={h}")
    got = run_gpu(env, x, max_context, h, rot)
    sel = np.arange(len(L)) if seqs is None else np.asarray(seqs)
    ref = run_oracle(x, h, rot, seqs=sel, max_context=max_context)
    check(got[sel], ref, tolerance(x, h, rot, sel, ref, max_context=max_context),
          f"lens case B={len(L)} Hq={Hq} P={P}")
    return got


@pytest.mark.parametrize("Hq", [8, 32, 64])
def test_lean_many_short_sequences(env, Hq):
    # 1024 sequences of 0-300 tokens (about one in seven empty): ranges of
    # about 13 steps cross several sequences each
    rng = np.random.default_rng(Hq)
    lens = np.where(rng.random(1024) < 0.15, 0, rng.integers(1, 301, size=1024))
    lens[-3:] = 0                                   # empty sequences at the end
    got = lens_case(env, Hq, lens, 768, wid=91 + Hq)
    assert not got[lens == 0].any()


def test_lean_page_64_kv_rotation(env):
    rng = np.random.default_rng(3)
    lens = np.where(rng.random(1024) < 0.1, 0, rng.integers(1, 301, size=1024))
    lens_case(env, 32, lens, 768, P=64, rot=O.ROT_KV, h=32, wid=94)


def test_lean_fewer_steps_than_waves(env):
    # 64 sequences of 0-40 tokens under max_context 16384: about 90 steps for
    # hundreds of waves per head pair
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 41, size=64)
    lens[:2] = 0
    lens_case(env, 32, lens, 16384, rot=O.ROT_KV, h=64, wid=95)


@pytest.mark.parametrize("Hq", [32, 64])
def test_lean_ranges_over_many_pages(env, Hq):
    # 32 contexts of 24 000-32 768 tokens with 16-token pages: 80-130 steps
    # per wave, so ranges span more than 64 pages (page ids held 64 at a time)
    rng = np.random.default_rng(Hq + 1)
    lens = rng.integers(24000, 32769, size=32)
    seqs = np.unique(np.r_[np.argmin(lens), np.argmax(lens), rng.choice(32, 2, replace=False)])
    lens_case(env, Hq, lens, 32768, seqs=seqs, wid=96 + Hq, masked=0)


# Two or four KV heads (one GPU's share of an eight-head model at tensor
# parallelism 4 or 2): the head pairs' lean kernels run the pipelined step
# loop for every grouping. 1024 short sequences under max_context 768 (a few
# steps per wave: pieces of one step and up, odd and even counts, ranges
# crossing several sequences), then 96 contexts of 24 000-32 768 tokens over
# two heads and 64 over four (ranges of about 90 and 120 steps, over more than
# 64 pages, so the page ids change windows mid-range).
@pytest.mark.parametrize("Hq,H", [(2, 2), (4, 2), (8, 2), (16, 2), (4, 4), (16, 4)])
def test_lean_few_kv_heads_short(env, Hq, H):
    rng = np.random.default_rng(Hq + 7 * H)
    lens = np.where(rng.random(1024) < 0.15, 0, rng.integers(1, 301, size=1024))
    wl = small(B=1024, Hq=Hq, H=H, ctx=("list", tuple(int(v) for v in lens)),
               rot_mode=O.ROT_KV, wid=120 + Hq + H)
    x = widen_tables(W.attn_inputs(wl), 768)
    say(f"attn lean B=1024 Hq={Hq} H={H}")
    got = run_gpu(env, x, 768, 128, O.ROT_KV)
    ref = run_oracle(x, 128, O.ROT_KV, max_context=768)
    check(got, ref, tolerance(x, 128, O.ROT_KV, np.arange(1024), ref, max_context=768),
          f"lean Hq={Hq} H={H}")
    assert not got[lens == 0].any()


@pytest.mark.parametrize("Hq,H,B", [(4, 2, 96), (8, 2, 96), (16, 4, 64)])
def test_lean_few_kv_heads_long(env, Hq, H, B):
    rng = np.random.default_rng(Hq + 9 * H)
    lens = rng.integers(24000, 32769, size=B)
    wl = small(B=B, Hq=Hq, H=H, ctx=("list", tuple(int(v) for v in lens)), rot_mode=O.ROT_K,
               wid=130 + Hq + H, masked=0)
    x = widen_tables(W.attn_inputs(wl), 32768)
    say(f"attn lean B={B} Hq={Hq} H={H} long contexts")
    got = run_gpu(env, x, 32768, 128, O.ROT_K)
    seqs = np.unique(np.r_[np.argmin(lens), np.argmax(lens), rng.choice(B, 2, replace=False)])
    ref = run_oracle(x, 128, O.ROT_K, seqs=seqs)
    check(got[seqs], ref, tolerance(x, 128, O.ROT_K, seqs, ref), f"lean long Hq={Hq} H={H}")


# odd KV-head counts (a tensor-parallel shard's one or three heads): one wave per
# (range, head), from 128 steps per wave if every context had max_context
# tokens; 1024 sequences of 0-300 tokens under max_context 8192 leave most of
# the 3072 (one head) or 1024 (three heads) waves per head with one step or none;
# every group size of the single-head lean kernel (1, 2, 4 and 8 queries per head)
@pytest.mark.parametrize("Hq,H", [(4, 1), (8, 1), (12, 3), (1, 1), (2, 1), (6, 3)])
def test_lean_single_head(env, Hq, H):
    rng = np.random.default_rng(Hq + H)
    lens = np.where(rng.random(1024) < 0.15, 0, rng.integers(1, 301, size=1024))
    wl = small(B=1024, Hq=Hq, H=H, ctx=("list", tuple(int(v) for v in lens)),
               rot_mode=O.ROT_KV, wid=100 + Hq)
    x = widen_tables(W.attn_inputs(wl), 8192)
    say(f"attn lean single-head B=1024 Hq={Hq} H={H}")
    got = run_gpu(env, x, 8192, 128, O.ROT_KV)
    ref = run_oracle(x, 128, O.ROT_KV, max_context=8192)
    check(got, ref, tolerance(x, 128, O.ROT_KV, np.arange(1024), ref, max_context=8192),
          f"lean single-head Hq={Hq} H={H}")


def test_lean_single_head_ranges_over_many_pages(env):
    # 64 contexts of 30 000-32 768 tokens over 3 KV heads with 16-token pages
    # (131 072 steps at most, 128 per wave for 1024 waves per head): about 120
    # steps per wave, so a range's 32-token steps cross the 64-page
    # boundary of its page ids (a step's two tiles on either side of it)
    rng = np.random.default_rng(31)
    lens = rng.integers(30000, 32769, size=64)
    wl = small(B=64, Hq=12, H=3, ctx=("list", tuple(int(v) for v in lens)), rot_mode=O.ROT_K,
               wid=113, masked=0)
    x = widen_tables(W.attn_inputs(wl), 32768)
    say("attn lean single-head B=64 Hq=12 H=3 long contexts")
    got = run_gpu(env, x, 32768, 128, O.ROT_K)
    seqs = np.unique(np.r_[np.argmin(lens), np.argmax(lens), rng.choice(64, 2, replace=False)])
    ref = run_oracle(x, 128, O.ROT_K, seqs=seqs)
    check(got[seqs], ref, tolerance(x, 128, O.ROT_K, seqs, ref), "lean single-head long")


# Seeded random configurations over the dispatch space: head counts even and
# odd, 1 to 8 queries per KV head, page sizes, block sizes, rotations, batch
# sizes and max_context bounds from tight to loose (which choose between the
# chunk form's chunk lengths, the head-pair and single-head kernels, and the
# lean split). Contexts are short and partly empty, with some masked pages, so
# the oracle checks every output element.
def random_case(seed):
    rng = np.random.default_rng([2026, seed])
    H = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([16, 32, 48, 64]))
    h = int(rng.choice([16, 32, 64, 128]))
    rot = int(rng.choice([O.ROT_NONE, O.ROT_K, O.ROT_KV]))
    B = int(rng.choice([1, 7, 40, 96, 256]))
    lens = rng.integers(1, 400, size=B)
    lens[rng.random(B) < 0.1] = 0
    lens[rng.random(B) < 0.05] = rng.integers(400, 3000)
    maxc = int(rng.choice([max(int(lens.max()), 1), 16384, 32768]))
    return H, G, P, h, rot, lens, maxc


@pytest.mark.parametrize("seed", range(24))
def test_random_configurations(env, seed):
    H, G, P, h, rot, lens, maxc = random_case(seed)
    wl = small(B=len(lens), Hq=G * H, H=H, P=P, h=h, rot_mode=rot,
               ctx=("list", tuple(int(v) for v in lens)), wid=200 + seed,
               masked=min(3, int((lens > 0).sum())))
    x = widen_tables(W.attn_inputs(wl), maxc)
    say(f"attn random case {seed}: B={len(lens)} H={H} G={G} P={P} h={h} rot={ROTS[rot]} "
        f"max_context={maxc} tokens={int(lens.sum())}")
    got = run_gpu(env, x, maxc, h, rot)
    ref = run_oracle(x, h, rot, max_context=maxc)
    check(got, ref, tolerance(x, h, rot, np.arange(len(lens)), ref, max_context=maxc),
          f"random case {seed}")
    assert not got[lens == 0].any()


def test_more_sequences_than_the_lean_split_takes(env):
    # 1025 sequences: the chunk form
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 64, size=1025)
    lens_case(env, 32, lens, 768, wid=99)


# More than 1024 sequences take the chunk form. Contexts of 0-700 tokens give
# pieces of every step count up to 44, odd and even, exact multiples of 16 and
# one token past them; max_context sets the grid: 768 with eight queries per
# KV head is the head-pair kernel's pipelined step loop (two steps per pass,
# loads past the end of a chunk issued with an empty range) in 512-token
# chunks with the first loads before the query preparation; 3000 gives
# 1024-token chunks (512 for three KV heads) and more than 12 288 blocks, so
# the first loads follow the query preparation, for the pipelined head-pair
# kernel, the plain one (four queries per head) and the single-head kernel
# (three KV heads).
@pytest.mark.parametrize("Hq,H,max_context,rot", [(64, 8, 768, O.ROT_K), (64, 8, 3000, O.ROT_KV),
                                                  (32, 8, 3000, O.ROT_K), (12, 3, 3000, O.ROT_KV)])
def test_chunk_form_more_than_1024_sequences(env, Hq, H, max_context, rot):
    rng = np.random.default_rng(max_context + Hq)
    lens = rng.integers(0, 701, size=1100)
    lens[:44] = 16 * np.arange(44)
    lens[44:88] = 16 * np.arange(44) + 1
    wl = small(B=1100, Hq=Hq, H=H, ctx=("list", tuple(int(v) for v in lens)), rot_mode=rot,
               wid=97 + Hq, masked=3)
    x = widen_tables(W.attn_inputs(wl), max_context)
    say(f"attn chunk form B=1100 Hq={Hq} H={H} max_context={max_context} rot={ROTS[rot]}")
    got = run_gpu(env, x, max_context, 128, rot)
    ref = run_oracle(x, 128, rot, max_context=max_context)
    check(got, ref, tolerance(x, 128, rot, np.arange(1100), ref, max_context=max_context),
          f"chunk form B=1100 Hq={Hq} H={H} max_context={max_context}")
    assert not got[lens == 0].any()


# --------------------------------------------------------------------------
# full size: 256 sequences, contexts up to 8000, sampled against the oracle
# --------------------------------------------------------------------------

# 256 and 128 sequences: the lean split; 64: the chunk form (512-token chunks)
@pytest.mark.parametrize("B", [256, 128, 64])
def test_full_size_sampled(env, B):
    wl = W.ATTN_WORKLOADS["attn"]
    x = W.attn_inputs(wl)
    if B < wl.B:
        x = dict(x, q=x["q"][:B], block_tables=x["block_tables"][:B],
                 context_lens=x["context_lens"][:B])
    L = x["context_lens"]
    maxc = int(L.max())
    say(f"attn full size B={B} tokens={int(L.sum())} max={maxc}")
    got = run_gpu(env, x, maxc, wl.h, wl.rot_mode)
    rng = np.random.default_rng(B)
    seqs = np.unique(np.r_[np.argmin(L), np.argmax(L), rng.choice(B, 4, replace=False)])
    ref = run_oracle(x, wl.h, wl.rot_mode, seqs=seqs)
    check(got[seqs], ref, tolerance(x, wl.h, wl.rot_mode, seqs, ref), f"full sampled B={B}")
    assert np.all(np.isfinite(got))


def test_long_contexts_sampled(env):
    """64 contexts of 32768 tokens (page 32, 64 chunks per sequence): three
    sequences against the oracle, every output finite."""
    wl = W.ATTN_WORKLOADS["attn_long"]
    x = W.attn_inputs(wl)
    maxc = int(x["context_lens"].max())
    say(f"attn long contexts B={wl.B} L={maxc} P={wl.P}")
    got = run_gpu(env, x, maxc, wl.h, wl.rot_mode)
    seqs = np.array([0, 31, 63])
    ref = run_oracle(x, wl.h, wl.rot_mode, seqs=seqs)
    check(got[seqs], ref, tolerance(x, wl.h, wl.rot_mode, seqs, ref), "long sampled")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("Hq", [8, 64])
def test_long_contexts_other_groupings_sampled(env, Hq):
    """The 64 x 32768-token pool read by one and by eight query heads per KV
    head (head pairs with repeated query slots, resp. head pairs of 16
    queries), three sequences against the oracle, every output finite."""
    wl = dataclasses.replace(W.ATTN_WORKLOADS["attn_long"], Hq=Hq)
    x = W.attn_inputs(wl)
    maxc = int(x["context_lens"].max())
    say(f"attn long contexts Hq={Hq} B={wl.B} L={maxc} P={wl.P}")
    got = run_gpu(env, x, maxc, wl.h, wl.rot_mode)
    seqs = np.array([0, 31, 63])
    ref = run_oracle(x, wl.h, wl.rot_mode, seqs=seqs)
    check(got[seqs], ref, tolerance(x, wl.h, wl.rot_mode, seqs, ref), f"long Hq={Hq} sampled")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("Hq", [8, 64])
def test_full_size_other_groupings_sampled(env, Hq):
    """The full 256-sequence pool read by one query head per KV head (G = 1,
    head pairs with repeated query slots) and by eight (G = 8, head pairs of
    16 queries), sampled against the oracle; then the first 64 sequences (a
    shallow grid: first loads issued before the query preparation, and G = 8
    on the single-head kernel)."""
    wl = dataclasses.replace(W.ATTN_WORKLOADS["attn"], Hq=Hq)
    x = W.attn_inputs(wl)
    L = x["context_lens"]
    rng = np.random.default_rng(Hq)
    for B in (wl.B, 64):
        xb = dict(x, q=x["q"][:B], block_tables=x["block_tables"][:B], context_lens=L[:B])
        maxc = int(L[:B].max())
        say(f"attn full pool Hq={Hq} B={B} max={maxc}")
        got = run_gpu(env, xb, maxc, wl.h, wl.rot_mode)
        seqs = np.unique(np.r_[np.argmax(L[:B]), rng.choice(B, 3, replace=False)])
        ref = run_oracle(xb, wl.h, wl.rot_mode, seqs=seqs)
        check(got[seqs], ref, tolerance(xb, wl.h, wl.rot_mode, seqs, ref),
              f"Hq={Hq} B={B} sampled")
        assert np.all(np.isfinite(got))


def test_workspace_reused_with_shorter_contexts(env):
    """One workspace for two calls: the first over long contexts fills every
    chunk slot with partials, the second over shorter contexts of the same
    layout (same B and max_context) must merge only its own chunks, not the
    first call's partials left in the slots past its contexts' ends."""
    torch, S = env
    wl = small(B=4, ctx=("list", (6000, 5990, 6000, 5000)), wid=41, masked=0)
    x = W.attn_inputs(wl)
    d = to_dev(env, x)
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    ws = torch.empty(S.attention_workspace_size(wl.B, wl.Hq, wl.H, 6000), dtype=torch.uint8,
                     device="cuda")
    for lens in ((6000, 5990, 6000, 5000), (700, 0, 2500, 17)):
        L = np.array(lens, dtype=np.int32)
        say(f"attn workspace reuse, contexts {lens}")
        got = S.decode_attention(d["q"], pools, d["block_tables"], torch.from_numpy(L).cuda(),
                                 6000, h=wl.h, rot="kv", workspace=ws)
        torch.cuda.synchronize()
        xb = dict(x, context_lens=L)
        ref = run_oracle(xb, wl.h, O.ROT_KV)
        check(got.cpu().numpy(), ref, tolerance(xb, wl.h, O.ROT_KV, np.arange(wl.B), ref),
              f"reuse {lens}")
