"""GPU parity of the controls (uncompressed paged cache write, token-wise INT8
append and read-back), called through the C ABI, against the CPU oracle.

Byte-exact: INT8 codes and scales, the INT8 read-back's fp16 output and the
copied 16-bit cache rows must equal the oracle's; slots nobody maps keep
their sentinel bytes.
"""
import sys

import numpy as np
import pytest

import oracle as O
from int4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

ROTS = {O.ROT_NONE: "none", O.ROT_K: "k", O.ROT_KV: "kv"}


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    from int4_kv_cache_amd import sawkv as S
    return torch, S


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def slots_with_holes(rng, T, n_slots):
    s = rng.permutation(n_slots)[:T].astype(np.int64)
    s[::97] = -1
    s[5::101] = n_slots + 3
    return s


def run_int8(env, k, v, slots, n_pg, P, h, rot):
    torch, S = env
    H, D = k.shape[1], k.shape[2]
    kc, vc, ks, vs = S.alloc_int8_pools(n_pg, P, H, D)
    kc.fill_(0x55)
    vc.fill_(0x55)
    ks.view(torch.int16).fill_(-1)
    vs.view(torch.int16).fill_(-1)
    dk, dv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    ds = torch.from_numpy(slots).cuda()
    S.int8_append(dk, dv, ds, kc, vc, ks, vs, h=h, rot=ROTS[rot])
    gk, gv = S.int8_gather(kc, vc, ks, vs, ds, h=h, rot=ROTS[rot])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (kc, vc, ks, vs, gk, gv)]


def oracle_int8(k, v, slots, n_pg, P, h, rot):
    H, D = k.shape[1], k.shape[2]
    kc = np.full((n_pg, P, H, D), 0x55, np.int8)
    vc = kc.copy()
    ks = np.full((n_pg, P, H), 0xFFFF, np.uint16).view(np.float16)
    vs = ks.copy()
    O.int8_append(k, v, slots, kc, vc, ks, vs, h=h, rot_mode=rot)
    gk, gv = O.int8_gather(kc, vc, ks, vs, slots, h=h, rot_mode=rot)
    return [kc, vc, ks, vs, gk, gv]


def assert_same(got, want, what):
    names = ("k codes", "v codes", "k scales", "v scales", "k read-back", "v read-back")
    for name, g, w in zip(names, got, want):
        g, w = np.asarray(g), np.asarray(w)
        if g.tobytes() != w.tobytes():
            gb, wb = g.view(np.uint8).reshape(-1), w.view(np.uint8).reshape(-1)
            bad = np.nonzero(gb != wb)[0]
            raise AssertionError(f"{what} {name}: {len(bad)} bytes differ, first {bad[:8]}")


@pytest.mark.parametrize("rot", [O.ROT_NONE, O.ROT_K, O.ROT_KV])
@pytest.mark.parametrize("h", [16, 32, 64, 128])
def test_int8_all_block_sizes(env, h, rot):
    rng = np.random.default_rng(h + 10 * rot)
    T, H, n_pg, P = 1000, 8, 80, 16
    wl = W.WORKLOADS["sweep"]
    k, v = W.kv(wl, 0, 0, T)
    slots = slots_with_holes(rng, T, n_pg * P)
    say(f"int8 h={h} rot={ROTS[rot]}")
    assert_same(run_int8(env, k, v, slots, n_pg, P, h, rot),
                oracle_int8(k, v, slots, n_pg, P, h, rot), f"int8 h={h} rot={rot}")


# seeded random shapes, block sizes, rotations and magnitudes
@pytest.mark.parametrize("seed", range(8))
def test_int8_random_configurations(env, seed):
    rng = np.random.default_rng([2026, 8, seed])
    H = int(rng.choice([1, 2, 3, 8, 13]))
    T = int(rng.integers(1, 2001))
    P = int(rng.choice([1, 8, 16]))
    h = int(rng.choice([16, 32, 64, 128]))
    rot = int(rng.choice([O.ROT_NONE, O.ROT_K, O.ROT_KV]))
    mag = float(rng.choice([1e-4, 1.0, 300.0]))
    k = np.clip(rng.standard_normal((T, H, 128)) * mag, -6e4, 6e4).astype(np.float16)
    v = np.clip(rng.standard_t(4, (T, H, 128)) * mag, -6e4, 6e4).astype(np.float16)
    n_pg = (T + P - 1) // P + 2
    slots = slots_with_holes(rng, T, n_pg * P)
    say(f"int8 random {seed}: H={H} T={T} P={P} h={h} rot={ROTS[rot]} mag={mag}")
    assert_same(run_int8(env, k, v, slots, n_pg, P, h, rot),
                oracle_int8(k, v, slots, n_pg, P, h, rot), f"int8 random {seed}")


def test_int8_edge_values(env):
    rng = np.random.default_rng(2)
    T, H, D = 64, 2, 128
    k = np.zeros((T, H, D), np.float16)
    k[1] = 60000.0                                    # large, constant
    k[2, :, 7] = np.float16(1e-5)                     # fp16-subnormal scale, clamps
    k[3] = (rng.standard_normal((H, D)) * 1e-4).astype(np.float16)
    k[4] = np.float16(-65504.0)
    k[5:] = (rng.standard_normal((T - 5, H, D)) * 3).astype(np.float16)
    v = k[::-1].copy()
    slots = np.arange(T, dtype=np.int64)
    for rot in (O.ROT_NONE, O.ROT_KV):
        say(f"int8 edge values rot={ROTS[rot]}")
        assert_same(run_int8(env, k, v, slots, 8, 16, 128, rot),
                    oracle_int8(k, v, slots, 8, 16, 128, rot), f"int8 edges rot={rot}")


def test_int8_prefill_sampled(env):
    """Full prefill batch on the GPU; a seeded sample of 4096 tokens checked."""
    torch, S = env
    wl = W.WORKLOADS["prefill"]
    k, v = W.kv(wl)
    slots = W.slot_mapping(wl)
    say(f"int8 prefill T={wl.T}")
    kc, vc, ks, vs = S.alloc_int8_pools(wl.N_pg, wl.P, wl.H, wl.D)
    dk, dv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    S.int8_append(dk, dv, torch.from_numpy(slots).cuda(), kc, vc, ks, vs, h=128, rot="kv")
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(0).choice(wl.T, 4096, replace=False))
    flat_kc = kc.view(-1, wl.H, wl.D)[torch.from_numpy(slots[pick]).cuda()].cpu().numpy()
    flat_ks = ks.view(-1, wl.H)[torch.from_numpy(slots[pick]).cuda()].cpu().numpy()
    q, s = O.encode8_vectors(k[pick], 128, True)
    assert flat_kc.tobytes() == q.tobytes()
    assert flat_ks.tobytes() == s.tobytes()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_cache_append_copies_rows(env, dtype):
    torch, S = env
    rng = np.random.default_rng(3)
    T, H, D, n_pg, P = 700, 8, 128, 64, 16
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    bits_k = rng.integers(0, 65536, size=(T, 3 * H, D)).astype(np.uint16)   # fused QKV-like
    big = torch.from_numpy(bits_k.view(np.int16)).cuda().view(tdt)
    k, v = big[:, H:2 * H], big[:, 2 * H:]                                   # strided views
    slots = slots_with_holes(rng, T, n_pg * P)
    kc = torch.full((n_pg, P, H, D), 7.0, dtype=tdt, device="cuda")
    vc = torch.full((n_pg, P, H, D), 7.0, dtype=tdt, device="cuda")
    say(f"cache append {dtype}")
    S.cache_append(k, v, torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    want_k = np.full((n_pg, P, H, D), 0, np.uint16)
    want_v = want_k.copy()
    want_k[...] = kc.new_full((1,), 7.0).view(torch.int16).cpu().numpy().view(np.uint16)[0]
    want_v[...] = want_k[0, 0, 0, 0]
    O.cache_append(bits_k[:, H:2 * H], bits_k[:, 2 * H:], slots, want_k, want_v)
    assert kc.view(torch.int16).cpu().numpy().view(np.uint16).tobytes() == want_k.tobytes()
    assert vc.view(torch.int16).cpu().numpy().view(np.uint16).tobytes() == want_v.tobytes()


# ---- access-pattern control of the INT4 append ----

def pattern_rows(x):
    """What sawkv_append_pattern_control writes per vector (its documented
    definition, no method arithmetic): word c of the 64-byte row = xor of the
    four uint32 words of the input row's 16-byte piece c; value bits = word 0
    xor (word 0 >> 16), low 16 bits."""
    T, H, D = x.shape
    w = np.ascontiguousarray(x).view(np.uint32).reshape(T, H, 16, 4)
    row = w[..., 0] ^ w[..., 1] ^ w[..., 2] ^ w[..., 3]
    val = ((row[..., 0] ^ (row[..., 0] >> 16)) & 0xFFFF).astype(np.uint16)
    return row.astype(np.uint32).view(np.uint8).reshape(T, H, 64), val


@pytest.mark.parametrize("placement", ["slots", "token_order"])
@pytest.mark.parametrize("H,T", [(8, 1000), (3, 77), (8, 262144)])
def test_append_pattern_control(env, placement, H, T):
    """The control writes its documented bytes to the append's rows (or to
    token order) and nothing else; 262 144 tokens x 8 heads is 1 GiB of K and
    V, where K and V blocks alternate in dispatch order."""
    torch, S = env
    rng = np.random.default_rng(T + H)
    k = rng.standard_normal((T, H, 128), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((T, H, 128), dtype=np.float32).astype(np.float16) * np.float16(3)
    n_pg, P = -(-T // 16) + 3, 16
    n_slots = n_pg * P
    slots = slots_with_holes(rng, T, n_slots)
    say(f"pattern control {placement} H={H} T={T}")
    dk, dv, ds = (torch.from_numpy(a).cuda() for a in (k, v, slots))
    pools = S.alloc_pools(n_pg, P, H, 128, "cuda", code_fill=0xAA, scale_bits_fill=-1)
    S.append_pattern_control(dk, dv, ds, *pools, placement=placement)
    torch.cuda.synchronize()
    got = [p.cpu().numpy().reshape(n_slots, H, -1) if i < 2 else
           p.cpu().numpy().view(np.uint16).reshape(n_slots, H) for i, p in enumerate(pools)]
    if placement == "slots":
        ok = (slots >= 0) & (slots < n_slots)
        rows = slots[ok]
    else:
        ok = np.ones(T, bool)
        rows = np.arange(T)
    for x, codes, vals in ((k, got[0], got[2]), (v, got[1], got[3])):
        want_rows, want_vals = pattern_rows(x)
        want_c = np.full((n_slots, H, 64), 0xAA, np.uint8)
        want_v = np.full((n_slots, H), 0xFFFF, np.uint16)
        want_c[rows] = want_rows[ok]
        want_v[rows] = want_vals[ok]
        assert codes.tobytes() == want_c.tobytes()
        assert vals.tobytes() == want_v.tobytes()
