"""Pins of the oracle's decode attention over the paged INT4 cache.

Each test checks the oracle against something that is not the oracle: torch's
float64 scaled-dot-product attention on dense tensors that the test builds
itself, scipy's Hadamard matrix, closed forms, and invariances that any
correct implementation has (physical page order, masking, rotating q instead
of un-rotating every key).
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
from int4_kv_cache_amd import workloads as W


def signed(codes):
    """uint8 packed nibbles -> int64 codes, low nibble first (written here,
    independently of the oracle's unpacking)."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.stack([c & 15, c >> 4], axis=-1).reshape(*c.shape[:-1], 2 * c.shape[-1])
    return np.where(out >= 8, out - 16, out)


def dense_dequant(codes, scales, h, rotated):
    """float64 vectors via an explicit block-diagonal Hadamard matrix."""
    y = signed(codes).astype(np.float64) * np.asarray(scales, np.float16).astype(np.float64)[..., None]
    if not rotated:
        return y
    D = y.shape[-1]
    blk = np.kron(np.eye(D // h), scipy.linalg.hadamard(h).astype(np.float64))
    # integer +-1 matrix: the products and sums are exact in float64; then one
    # division by sqrt(h). H is symmetric, so this applies H^T = H^-1 per block.
    return (y @ blk) / np.sqrt(np.float64(h))


def random_dense(rng, B, Lmax, H, D):
    codes = rng.integers(0, 256, size=(2, B, Lmax, H, D // 2), dtype=np.uint8)
    scales = (rng.lognormal(-1.0, 0.5, size=(2, B, Lmax, H))).astype(np.float16)
    return codes, scales


def scatter_into_pool(rng, codes, scales, L, P, spare=3):
    """Write dense per-sequence tokens into a paged pool through a random page
    permutation; return pool arrays and the block table."""
    _, B, Lmax, H, half = codes.shape
    npg = [-(-int(x) // P) for x in L]
    N_pg = sum(npg) + spare
    perm = rng.permutation(N_pg)
    kc = rng.integers(0, 256, size=(N_pg, P, H, half), dtype=np.uint8)     # garbage
    vc = rng.integers(0, 256, size=(N_pg, P, H, half), dtype=np.uint8)
    ks = np.full((N_pg, P, H), np.float16(np.nan))                         # garbage
    vs = np.full((N_pg, P, H), np.float16(np.inf))
    bt = np.full((B, max(1, max(npg))), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        for i in range(npg[b]):
            bt[b, i] = perm[k]
            k += 1
        for t in range(int(L[b])):
            pg, off = bt[b, t // P], t % P
            kc[pg, off], vc[pg, off] = codes[0, b, t], codes[1, b, t]
            ks[pg, off], vs[pg, off] = scales[0, b, t], scales[1, b, t]
    return kc, vc, ks, vs, bt


def sdpa(q, K, V, L, sm_scale):
    """torch float64 attention, one query token per sequence, GQA by repeating
    KV heads; rows of an empty context are zero."""
    B, Hq, D = q.shape
    H = K.shape[2]
    G = Hq // H
    Lmax = K.shape[1]
    qt = torch.from_numpy(q.astype(np.float64)).unsqueeze(2)                       # B Hq 1 D
    kt = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)     # B Hq L D
    vt = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    mask = torch.arange(Lmax)[None, :] < torch.from_numpy(np.asarray(L))[:, None]
    out = torch.zeros(B, Hq, D, dtype=torch.float64)
    for b in range(B):
        if L[b] == 0:
            continue
        o = torch.nn.functional.scaled_dot_product_attention(
            qt[b:b + 1], kt[b:b + 1], vt[b:b + 1], attn_mask=mask[b][None, None, None, :],
            scale=sm_scale)
        out[b] = o[0, :, 0, :]
    return out.numpy()


@pytest.mark.parametrize("rot,h,G,P", [(O.ROT_NONE, 128, 4, 16), (O.ROT_K, 128, 2, 16),
                                        (O.ROT_KV, 32, 8, 32), (O.ROT_KV, 16, 1, 16)])
def test_attention_matches_torch_sdpa(rot, h, G, P):
    rng = np.random.default_rng(10 + rot + h + G)
    B, H, D = 4, 2, 128
    L = np.array([0, 1, 37, 70])
    codes, scales = random_dense(rng, B, int(L.max()), H, D)
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, L, P)
    q = rng.standard_normal((B, H * G, D)).astype(np.float16)
    sm = 1.0 / np.sqrt(D)
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt, L, h=h, rot_mode=rot)
    K = dense_dequant(codes[0], scales[0], h, rot in (O.ROT_K, O.ROT_KV))
    V = dense_dequant(codes[1], scales[1], h, rot == O.ROT_KV)
    want = sdpa(q, K, V, L, sm)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_dequant_exact_is_exact():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(50, 64), dtype=np.uint8)
    s = rng.lognormal(0, 2, size=50).astype(np.float16)
    for h in (16, 32, 64, 128):
        assert np.array_equal(O.dequant_exact(codes, s, h, True), dense_dequant(codes, s, h, True))
    assert np.array_equal(O.dequant_exact(codes, s, 128, False), dense_dequant(codes, s, 128, False))


def test_dequant_exact_rounds_to_the_read_back():
    """fp16 of the exact dequantised vector is within one fp16 ulp of the
    read-back path's output (which rounds c_h to float32 first)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((200, 128)) * 3).astype(np.float16)
    for h in (32, 128):
        codes, s = O.encode_vectors(x, h, True)
        exact16 = O.dequant_exact(codes, s, h, True).astype(np.float16)
        back = O.decode_vectors(codes, s, h, True)
        d = np.abs(exact16.view(np.int16).astype(np.int32) - back.view(np.int16).astype(np.int32))
        assert d.max() <= 1


def test_single_token_returns_its_value():
    rng = np.random.default_rng(5)
    codes, scales = random_dense(rng, 1, 1, 2, 128)
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, [1], 16)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt, [1], h=128, rot_mode=O.ROT_NONE)
    v = signed(codes[1, 0, 0]) * np.float64(scales[1, 0, 0])[:, None]        # [H, D]
    assert np.array_equal(got[0], np.repeat(v, 2, axis=0))


def test_equal_keys_average_the_values():
    rng = np.random.default_rng(6)
    B, L, H = 1, 45, 1
    codes, scales = random_dense(rng, B, L, H, 128)
    codes[0, 0, :] = codes[0, 0, 0]
    scales[0, 0, :] = scales[0, 0, 0]
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, [L], 16)
    q = rng.standard_normal((1, 3, 128)).astype(np.float16)
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt, [L], h=128, rot_mode=O.ROT_NONE)
    v = signed(codes[1, 0, :, 0]) * scales[1, 0, :, 0].astype(np.float64)[:, None]
    np.testing.assert_allclose(got[0], np.repeat(v.mean(axis=0)[None], 3, axis=0), rtol=1e-13)


def test_two_tokens_logistic_closed_form():
    """Two tokens: weight of token 1 = 1 / (1 + exp(-(s1 - s0)))."""
    rng = np.random.default_rng(7)
    codes, scales = random_dense(rng, 1, 2, 1, 128)
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, [2], 16)
    q = rng.standard_normal((1, 1, 128)).astype(np.float16)
    sm = 0.3
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt, [2], h=128, rot_mode=O.ROT_NONE,
                                   sm_scale=sm)
    kv = signed(codes[:, 0, :, 0]) * scales[:, 0, :, 0].astype(np.float64)[..., None]   # [2, 2, D]
    s = sm * (kv[0] @ q[0, 0].astype(np.float64))
    a = 1.0 / (1.0 + np.exp(-(s[1] - s[0])))
    np.testing.assert_allclose(got[0, 0], (1 - a) * kv[1, 0] + a * kv[1, 1], rtol=1e-12, atol=1e-14)


def test_rotating_q_equals_unrotating_keys():
    """(R q) . (q_codes s) == q . (R^T (q_codes s)): the identity a kernel
    uses to read rotated keys without un-rotating them."""
    rng = np.random.default_rng(8)
    L, H, D, h = 60, 1, 128, 64
    codes, scales = random_dense(rng, 1, L, H, D)
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, [L], 16)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt, [L], h=h, rot_mode=O.ROT_K)
    Hm = np.kron(np.eye(D // h), scipy.linalg.hadamard(h) / np.sqrt(h))
    qr = Hm @ q[0, 0].astype(np.float64)
    kr = signed(codes[0, 0, :, 0]) * scales[0, 0, :, 0].astype(np.float64)[:, None]
    s = (kr @ qr) / np.sqrt(D)
    w = np.exp(s - s.max())
    v = signed(codes[1, 0, :, 0]) * scales[1, 0, :, 0].astype(np.float64)[:, None]
    np.testing.assert_allclose(got[0, 0], (w / w.sum()) @ v, rtol=1e-12, atol=1e-14)


def test_physical_page_order_does_not_matter():
    x = W.attn_inputs(W.ATTN_WORKLOADS["attn_small"])
    a = O.paged_decode_attention(x["q"], x["k_codes"], x["k_scales"], x["v_codes"], x["v_scales"],
                                 x["block_tables"], x["context_lens"], h=128, rot_mode=O.ROT_KV)
    N = x["k_codes"].shape[0]
    perm = np.random.default_rng(9).permutation(N)          # new page i holds old page perm[i]
    inv = np.argsort(perm)
    bt = x["block_tables"].copy()
    live = bt >= 0
    bt[live] = inv[bt[live]]
    b = O.paged_decode_attention(x["q"], x["k_codes"][perm], x["k_scales"][perm],
                                 x["v_codes"][perm], x["v_scales"][perm], bt,
                                 x["context_lens"], h=128, rot_mode=O.ROT_KV)
    assert np.array_equal(a, b)


def test_masked_page_equals_dropping_its_tokens():
    rng = np.random.default_rng(11)
    P, H, L = 16, 2, 64
    codes, scales = random_dense(rng, 1, L, H, 128)
    kc, vc, ks, vs, bt = scatter_into_pool(rng, codes, scales, [L], P)
    q = rng.standard_normal((1, 4, 128)).astype(np.float16)
    bt_m = bt.copy()
    bt_m[0, 1] = -1                                    # tokens 16..31 masked
    got = O.paged_decode_attention(q, kc, ks, vc, vs, bt_m, [L], h=128, rot_mode=O.ROT_KV)
    keep = np.r_[0:16, 32:64]
    kc2, vc2, ks2, vs2, bt2 = scatter_into_pool(rng, codes[:, :, keep], scales[:, :, keep], [48], P)
    want = O.paged_decode_attention(q, kc2, ks2, vc2, vs2, bt2, [48], h=128, rot_mode=O.ROT_KV)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    bt_all = np.full_like(bt, -1)
    z = O.paged_decode_attention(q, kc, ks, vc, vs, bt_all, [L], h=128, rot_mode=O.ROT_KV)
    assert np.array_equal(z, np.zeros_like(z))


def test_default_scale_is_inverse_sqrt_d():
    x = W.attn_inputs(W.ATTN_WORKLOADS["attn_small"])
    args = (x["q"][:6], x["k_codes"], x["k_scales"], x["v_codes"], x["v_scales"],
            x["block_tables"][:6], x["context_lens"][:6])
    a = O.paged_decode_attention(*args, h=128, rot_mode=O.ROT_K)
    b = O.paged_decode_attention(*args, h=128, rot_mode=O.ROT_K, sm_scale=1 / np.sqrt(128))
    assert np.array_equal(a, b)
