"""Pins of the CPU oracle to facts other than itself (CPU only).

Sources of the pins:
  * the Hadamard matrix: scipy's Sylvester construction and the matrix's own
    defining identities (H H^T = h I, symmetry, +-1 entries, closed-form
    columns), since the pages name a Hadamard rotation that is orthogonal
    and undoable (youngju.dev reading, "The Rotation Trick - Block-Diagonal
    Hadamard"; gist.science SAW-INT4 summary, §2 BDR items 1-2);
  * IEEE rounding: exact rational arithmetic (tests/exact_fp.py);
  * worked cases derived by hand from the readings of the scale, code and
    packing steps (tests/golden/closed_forms.txt);
  * a brute-force scalar encoder in exact arithmetic on tiny inputs;
  * the pages' qualitative claims: token-wise append never touches other
    slots, rotation lowers the INT4 reconstruction error on outlier data.
"""
from fractions import Fraction
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import sawint4 as O
from tests.exact_fp import F16, F32, f16_bits, f32_bits, rint_even, rn
from int4_kv_cache_amd import workloads as W

HS = [2, 4, 8, 16, 32, 64, 128]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# the transform
# --------------------------------------------------------------------------

@pytest.mark.parametrize("h", HS)
def test_fwht_equals_dense_sylvester_on_integers(h):
    """F_h x == (I_{D/h} (x) H_h) x, exactly, on integer inputs (no rounding
    anywhere, so any dropped term, sign or index error shows)."""
    rng = np.random.default_rng(h)
    D = 128
    x = rng.integers(-1000, 1000, size=(5, D)).astype(np.float32)
    Hh = scipy.linalg.hadamard(h).astype(np.float64)
    dense = np.kron(np.eye(D // h), Hh)
    want = x.astype(np.float64) @ dense.T
    got = O.fwht_blocks(x, h)
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("h", HS)
def test_fwht_matrix_is_hadamard(h):
    """The matrix the oracle applies: +-1 entries, symmetric, H H^T = h I,
    equal to the recursive Sylvester definition H_2n = [[H, H], [H, -H]]."""
    M = np.stack([O.fwht_blocks(np.eye(h, dtype=np.float32)[j], h) for j in range(h)], axis=1)
    M = M.astype(np.int64)
    assert set(np.unique(M)) <= {-1, 1}
    assert np.array_equal(M, M.T)
    assert np.array_equal(M @ M.T, h * np.eye(h, dtype=np.int64))
    S = np.array([[1]], dtype=np.int64)
    while S.shape[0] < h:
        S = np.block([[S, S], [S, -S]])
    assert np.array_equal(M, S)


def test_fwht_one_hot_closed_form():
    """Column j of Sylvester H_128 is (-1)^popcount(i & j)."""
    for j in (0, 1, 5, 77, 127):
        e = np.zeros(128, np.float32)
        e[j] = 1
        got = O.fwht_blocks(e, 128)
        want = np.array([(-1) ** bin(i & j).count("1") for i in range(128)], np.float32)
        assert np.array_equal(got, want)


def test_fwht_stage_order_pinned():
    """The reading fixes the stride order 1, 2, ..., h/2 (float32 rounding after
    each stage). Hand derivation for x = [2^15, 2^-9, 2^-9, 0], h = 4:
      stride 1: [2^15 + 2^-9 -> 2^15 (tie, even), 2^15 - 2^-9, 2^-9, 2^-9]
      stride 2: [2^15 + 2^-9 -> 2^15, 2^15, 2^15 - 2^-9, 2^15 - 2^-8]
    The descending order would give [2^15, 2^15 - 2^-9, 2^15, 2^15 - 2^-8]."""
    x = np.array([2.0 ** 15, 2.0 ** -9, 2.0 ** -9, 0.0], np.float32)
    got = O.fwht_blocks(x, 4)
    want = np.array([2.0 ** 15, 2.0 ** 15, 2.0 ** 15 - 2.0 ** -9, 2.0 ** 15 - 2.0 ** -8], np.float32)
    assert np.array_equal(got, want)


def test_blocks_do_not_mix():
    """h < D: each block of h channels transforms on its own."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    y = O.fwht_blocks(x, 32)
    for b in range(4):
        assert np.array_equal(y[:, 32 * b:32 * (b + 1)], O.fwht_blocks(x[:, 32 * b:32 * (b + 1)], 32))


@pytest.mark.parametrize("h", HS)
def test_c_h_is_correctly_rounded(h):
    """c_h = float32 nearest to 1/sqrt(h): |c - 1/sqrt(h)| <= half an ulp,
    checked in exact arithmetic: (c - u/2)^2 <= 1/h <= (c + u/2)^2."""
    c = Fraction(float(O.c_h(h)))
    assert rn(c) == c
    e = math.floor(math.log2(float(c)))
    u = Fraction(2) ** (e - 23)
    assert (c - u / 2) ** 2 <= Fraction(1, h) <= (c + u / 2) ** 2


def test_c_h_bit_patterns():
    """fp32(sqrt 2) = 0x3FB504F3; 1/sqrt(2^k) is sqrt 2 scaled by a power of two,
    so the constants share its mantissa."""
    assert f32_bits(O.c_h(128)) == 0x3DB504F3
    assert f32_bits(O.c_h(64)) == 0x3E000000
    assert f32_bits(O.c_h(32)) == 0x3E3504F3


@pytest.mark.parametrize("h", [32, 64, 128])
def test_rotation_preserves_norm(h):
    rng = np.random.default_rng(h + 1)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    y = O.rotate(x, h)
    nx = np.linalg.norm(x.astype(np.float64), axis=-1)
    ny = np.linalg.norm(y.astype(np.float64), axis=-1)
    assert np.all(np.abs(ny - nx) <= 2e-6 * nx)


def test_rotation_norm_exact_for_h64_on_integers():
    rng = np.random.default_rng(7)
    x = rng.integers(-50, 50, size=(16, 128)).astype(np.float32)
    y = O.rotate(x, 64)
    assert np.array_equal(np.sum(y.astype(np.float64) ** 2, -1), np.sum(x.astype(np.float64) ** 2, -1))


@pytest.mark.parametrize("h", HS)
def test_round_trip(h):
    """F_h(F_h(x)) = h x exactly on integers; the normalised rotation is its
    own inverse to within float32 rounding (exact for h = 64, c = 1/8)."""
    rng = np.random.default_rng(11 + h)
    xi = rng.integers(-100, 100, size=(8, 128)).astype(np.float32)
    assert np.array_equal(O.fwht_blocks(O.fwht_blocks(xi, h), h), xi * h)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    back = O.rotate(O.rotate(x, h), h)
    assert np.max(np.abs(back - x)) <= 4 * np.finfo(np.float32).eps * np.max(np.abs(x))
    if h == 64:
        assert np.array_equal(O.rotate(O.rotate(xi, 64), 64), xi)


# --------------------------------------------------------------------------
# rounding of the library conversions the oracle relies on
# --------------------------------------------------------------------------

def test_numpy_f16_conversion_is_rne():
    cases = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -26,
             1.5 * 2.0 ** -24, 2.5 * 2.0 ** -24, 65519.0, 0.037880719, 6.1e-5]
    for v in cases:
        got = np.float32(v).astype(np.float16)
        want = rn(Fraction(float(np.float32(v))), F16)
        assert float(got) == float(want), v
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(65520.0).astype(np.float16))


def test_numpy_f32_division_and_rint():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(2000).astype(np.float32)
    b = (rng.standard_normal(2000).astype(np.float32) + np.float32(3.0))
    q = a / b
    for i in range(0, 2000, 37):
        assert Fraction(float(q[i])) == rn(Fraction(float(a[i])) / Fraction(float(b[i])))
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 7.5, -7.5], np.float32)
    assert np.array_equal(np.rint(x), np.array([0, 2, 2, -0, -2, -2, 8, -8], np.float32))


def test_no_flush_to_zero():
    tiny = np.float32(1e-40)
    assert tiny * np.float32(1.0) != 0
    assert np.float32(1e-38) / np.float32(1000.0) != 0


# --------------------------------------------------------------------------
# scale, codes, packing: worked cases
# --------------------------------------------------------------------------

def _load_golden(name="closed_forms.txt"):
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        cur = {}
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition("=")
            key, val = key.strip(), val.strip()
            if key == "case":
                if cur:
                    cases.append(cur)
                cur = {"case": val}
            else:
                cur[key] = val
        if cur:
            cases.append(cur)
    return cases


def _expand(spec, D):
    """'v0 v1 ... | fill' -> float list of length D."""
    head, _, fill = spec.partition("|")
    vals = [float(eval(t, {"__builtins__": {}})) for t in head.split()]
    fillv = float(eval(fill.strip(), {"__builtins__": {}})) if fill.strip() else 0.0
    return vals + [fillv] * (D - len(vals))


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["case"])
def test_golden_closed_forms(case):
    D = 128
    x = np.array(_expand(case["x"], D), np.float16)
    h = int(case.get("h", "128"))
    rot = case.get("rotate", "no") == "yes"
    codes, s16 = O.encode_vectors(x[None], h, rot)
    if "scale_bits" in case:
        assert f16_bits(float(s16[0])) == int(case["scale_bits"], 16)
    if "codes" in case:
        want = [int(t) for t in _expand(case["codes"], D)]
        assert O.unpack_nibbles(codes)[0].tolist() == want
    if "bytes" in case:
        want = [int(t, 16) for t in case["bytes"].split()]
        assert codes[0, :len(want)].tolist() == want


def test_one_hot_rotated_closed_form():
    """x = 3 e_5, h = 128: y_i = (-1)^popcount(i & 5) fl(3 c), every code is
    +-7 in that sign pattern, s = f16(fl(fl(3c) / 7)) (exact arithmetic)."""
    x = np.zeros(128, np.float16)
    x[5] = 3
    codes, s16 = O.encode_vectors(x[None], 128, True)
    c = Fraction(float(O.c_h(128)))
    y = rn(3 * c)
    s = rn(rn(y / 7), F16)
    assert Fraction(float(s16[0])) == s
    sign = [(-1) ** bin(i & 5).count("1") for i in range(128)]
    assert O.unpack_nibbles(codes)[0].tolist() == [7 * g for g in sign]


def test_constant_vector_closed_form():
    """x = 0.5 * 1: F x = [64, 0, ..., 0], y0 = 64 c (exact scaling), codes [7, 0, ...]."""
    x = np.full(128, 0.5, np.float16)
    codes, s16 = O.encode_vectors(x[None], 128, True)
    c = Fraction(float(O.c_h(128)))
    assert Fraction(float(s16[0])) == rn(rn(64 * c / 7), F16)
    assert O.unpack_nibbles(codes)[0].tolist() == [7] + [0] * 127


def test_exact_multiples_give_exact_codes():
    rng = np.random.default_rng(9)
    for s in (0.25, 2.0 ** -10, 4.0):
        k = rng.integers(-7, 8, size=128)
        k[0] = 7
        x = (k * s).astype(np.float16)
        codes, s16 = O.encode_vectors(x[None], 128, False)
        assert float(s16[0]) == s
        assert O.unpack_nibbles(codes)[0].tolist() == k.tolist()


def test_pack_unpack_round_trip_all_codes():
    q = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8).reshape(1, -1)
    b = O.pack_nibbles(q)
    assert b.shape == (1, 256)
    for j in range(256):
        lo, hi = q[0, 2 * j], q[0, 2 * j + 1]
        assert b[0, j] == ((int(lo) & 15) | ((int(hi) & 15) << 4))
    assert np.array_equal(O.unpack_nibbles(b), q)


# --------------------------------------------------------------------------
# brute force on tiny inputs (exact rational arithmetic, scalar loops)
# --------------------------------------------------------------------------

def _brute_encode(xs, h, rotate):
    x = [Fraction(float(v)) for v in xs]
    if rotate:
        s = 1
        while s < h:
            nx = list(x)
            for i in range(len(x)):
                if i % (2 * s) < s:
                    nx[i] = rn(x[i] + x[i + s])
                    nx[i + s] = rn(x[i] - x[i + s])
            x = nx
            s *= 2
        c = Fraction(float(O.c_h(h)))
        x = [rn(v * c) for v in x]
    amax = max(abs(v) for v in x)
    s16 = rn(rn(amax / 7), F16)
    if s16 == math.inf:
        s16 = Fraction(65504)
    if s16 == 0:
        return [0] * len(x), s16
    q = [max(-8, min(7, rint_even(rn(v / s16)))) for v in x]
    return q, s16


@pytest.mark.parametrize("h,rotate", [(8, True), (8, False), (4, True), (16, True), (2, True)])
def test_brute_force_tiny(h, rotate):
    rng = np.random.default_rng(100 + h)
    D = 16
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-7, 4)
        x = rng.standard_normal(D) * scale
        if trial % 5 == 0:
            x[rng.integers(D)] *= 50
        x = np.clip(x, -60000, 60000).astype(np.float16)   # finite inputs only
        codes, s16 = O.encode_vectors(x[None], h, rotate)
        q, s = _brute_encode(x, h, rotate)
        assert Fraction(float(s16[0])) == s, (trial, x)
        assert O.unpack_nibbles(codes)[0].tolist() == q, (trial, x)


# --------------------------------------------------------------------------
# edge cases of the scale
# --------------------------------------------------------------------------

def test_zero_vector():
    codes, s16 = O.encode_vectors(np.zeros((1, 128), np.float16), 128, True)
    assert float(s16[0]) == 0 and not np.any(codes)
    out = O.decode_vectors(codes, s16, 128, True)
    assert np.all(out == 0)


def test_scale_underflow_to_zero():
    """amax = 2^-24 (smallest fp16): amax/7 rounds to fp16 zero -> codes 0."""
    x = np.zeros((1, 128), np.float16)
    x[0, 3] = np.float16(2.0 ** -24)
    codes, s16 = O.encode_vectors(x, 128, False)
    assert float(s16[0]) == 0 and not np.any(codes)


def test_subnormal_scale_needs_clamp():
    """amax = 10 * 2^-24: s32 = 1.43 * 2^-24 -> f16 subnormal 2^-24, so
    y/s = 10 rounds to 10 and the clamp makes it 7."""
    x = np.zeros((1, 128), np.float16)
    x[0, 0] = np.float16(10 * 2.0 ** -24)
    x[0, 1] = np.float16(-3 * 2.0 ** -24)
    codes, s16 = O.encode_vectors(x, 128, False)
    assert float(s16[0]) == 2.0 ** -24
    assert O.unpack_nibbles(codes)[0, :2].tolist() == [7, -3]


def test_scale_saturation_and_minus_eight():
    """x = -65504 * 1, h = 128: y0 = -128 * 65504 * c, amax/7 > 65504, so the
    scale saturates to 65504 and y0/s = -11.3 clamps to -8."""
    x = np.full((1, 128), -65504.0, np.float16)
    codes, s16 = O.encode_vectors(x, 128, True)
    assert float(s16[0]) == 65504.0
    q = O.unpack_nibbles(codes)[0]
    assert q[0] == -8 and np.all(q[1:] == 0)


# --------------------------------------------------------------------------
# append / gather semantics
# --------------------------------------------------------------------------

def _pools(n_pg, P, H, D):
    kc = np.full((n_pg, P, H, D // 2), 0xAA, np.uint8)
    vc = kc.copy()
    ks = np.full((n_pg, P, H), 0xFFFF, np.uint16).view(np.float16)
    vs = ks.copy()
    return kc, vc, ks, vs


def test_append_touches_only_mapped_slots():
    rng = np.random.default_rng(1)
    T, H, D, P, n_pg = 40, 2, 128, 16, 8
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.choice(n_pg * P, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = n_pg * P + 5            # out of range: skipped
    pools = _pools(n_pg, P, H, D)
    O.quantize_append(k, v, slots, *pools, h=128, rot_mode=O.ROT_KV)
    kc, vc, ks, vs = pools
    written = np.zeros(n_pg * P, bool)
    ok = (slots >= 0) & (slots < n_pg * P)
    written[slots[ok]] = True
    for arr in (kc, vc):
        flat = arr.reshape(n_pg * P, -1)
        assert np.all(flat[~written] == 0xAA)
    for arr in (ks, vs):
        flat = arr.reshape(n_pg * P, -1).view(np.uint16)
        assert np.all(flat[~written] == 0xFFFF)
        assert not np.any(flat[written] == 0xFFFF)


def test_one_call_equals_per_token_calls():
    rng = np.random.default_rng(2)
    T, H, D, P, n_pg = 24, 3, 128, 8, 6
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.choice(n_pg * P, size=T, replace=False).astype(np.int64)
    a = _pools(n_pg, P, H, D)
    b = _pools(n_pg, P, H, D)
    O.quantize_append(k, v, slots, *a, h=64, rot_mode=O.ROT_KV)
    for t in range(T):
        O.quantize_append(k[t:t + 1], v[t:t + 1], slots[t:t + 1], *b, h=64, rot_mode=O.ROT_KV)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_gather_independent_of_page_permutation():
    rng = np.random.default_rng(4)
    T, H, D, P, n_pg = 64, 2, 128, 16, 4
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    outs = []
    for perm in (np.arange(n_pg), rng.permutation(n_pg)):
        t = np.arange(T)
        slots = (perm[t // P] * P + t % P).astype(np.int64)
        pools = _pools(n_pg, P, H, D)
        O.quantize_append(k, v, slots, *pools, h=128, rot_mode=O.ROT_KV)
        outs.append(O.dequant_gather(*pools, slots, h=128, rot_mode=O.ROT_KV))
    for a, b in zip(outs[0], outs[1]):
        assert a.tobytes() == b.tobytes()


def test_gather_invalid_slots_zero_rows():
    rng = np.random.default_rng(6)
    T, H, D, P, n_pg = 8, 2, 128, 4, 4
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = np.arange(T, dtype=np.int64)
    pools = _pools(n_pg, P, H, D)
    O.quantize_append(k, k, slots, *pools, h=128, rot_mode=O.ROT_KV)
    g = slots.copy()
    g[2] = -1
    g[5] = n_pg * P
    ko, vo = O.dequant_gather(*pools, g, h=128, rot_mode=O.ROT_KV)
    assert np.all(ko[2] == 0) and np.all(vo[5] == 0)
    assert np.any(ko[1] != 0)


def test_identity_mapping_gives_token_order():
    rng = np.random.default_rng(8)
    T, H, D, P, n_pg = 32, 2, 128, 16, 2
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    pools = _pools(n_pg, P, H, D)
    O.quantize_append(k, k, np.arange(T, dtype=np.int64), *pools, h=128, rot_mode=O.ROT_KV)
    codes, s16 = O.encode_vectors(k, 128, True)
    assert pools[0].reshape(T, H, D // 2).tobytes() == codes.tobytes()
    assert pools[2].reshape(T, H).tobytes() == s16.tobytes()


def test_k_only_mode():
    """Keys-only rotation: K codes equal the K+V run's K codes, V codes equal
    the naive run's V codes (gist.science summary §4: rotating the keys alone
    is enough)."""
    rng = np.random.default_rng(10)
    T, H, D, P, n_pg = 16, 2, 128, 16, 1
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = np.arange(T, dtype=np.int64)
    runs = {}
    for mode in (O.ROT_NONE, O.ROT_K, O.ROT_KV):
        pools = _pools(n_pg, P, H, D)
        O.quantize_append(k, v, slots, *pools, h=128, rot_mode=mode)
        runs[mode] = pools
    assert runs[O.ROT_K][0].tobytes() == runs[O.ROT_KV][0].tobytes()
    assert runs[O.ROT_K][2].tobytes() == runs[O.ROT_KV][2].tobytes()
    assert runs[O.ROT_K][1].tobytes() == runs[O.ROT_NONE][1].tobytes()
    assert runs[O.ROT_K][3].tobytes() == runs[O.ROT_NONE][3].tobytes()


def test_gather_reconstruction_bound():
    """Read-back error per element is at most half a quantisation step
    (s/2 in the rotated basis; the orthonormal inverse keeps the 2-norm) plus
    fp16 rounding of the output."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    for rot in (False, True):
        codes, s16 = O.encode_vectors(x, 128, rot)
        out = O.decode_vectors(codes, s16, 128, rot).astype(np.float64)
        err = np.linalg.norm(out - x.astype(np.float64), axis=-1)
        bound = 0.5 * s16.astype(np.float64) * np.sqrt(128) * (1 + 1e-3) \
            + 2.0 ** -11 * np.linalg.norm(x.astype(np.float64), axis=-1) * 2
        assert np.all(err <= bound)


def _pack_by_hand(q):
    """Two's-complement nibbles, element 2k in the low nibble of byte k."""
    return np.array([(q[2 * k] & 15) | ((q[2 * k + 1] & 15) << 4) for k in range(len(q) // 2)],
                    np.uint8)


def _f32_staged_fwht(y, h):
    """F_h by butterfly stages (strides 1, 2, ..., h/2), every sum rounded to
    float32 with exact rational arithmetic: used only to show that a case
    tells the scale-first order apart."""
    y = [rn(Fraction(v)) for v in y]
    s = 1
    while s < h:
        for i in range(len(y)):
            if i % (2 * s) < s:
                a, b = y[i], y[i + s]
                y[i], y[i + s] = rn(a + b), rn(a - b)
        s *= 2
    return y


@pytest.mark.parametrize("case", _load_golden("read_back.txt"), ids=lambda c: c["case"])
def test_golden_read_back_rounding_order(case):
    """decode_vectors = f16(f32(c_h * F_h(q * s))) on every channel, with the
    exact value from the explicit Sylvester matrix and rational arithmetic.
    The case holds a channel where f32(c_h * s * F) is an fp16 midpoint, so
    rounding once straight to fp16, or applying c_h before the butterflies,
    gives other bits (checked here too)."""
    h = int(case["h"])
    q = [int(t) for t in case["codes"].split()]
    assert len(q) == 128
    s_bits = int(case["scale_bits"], 16)
    s16 = np.array([s_bits], np.uint16).view(np.float16)
    s = Fraction(float(s16[0]))
    out = O.decode_vectors(_pack_by_hand(q)[None], s16, h, True)[0]

    Hm = np.kron(np.eye(128 // h, dtype=np.int64), scipy.linalg.hadamard(h).astype(np.int64))
    F = Hm @ np.array(q, np.int64)
    c = Fraction(float(O.c_h(h)))
    want = [f16_bits(float(rn(rn(c * s * int(f)), F16))) for f in F]
    assert [f16_bits(float(v)) for v in out] == want

    e = int(case["elem"])
    assert int(F[e]) == int(case["F"])
    assert f32_bits(float(rn(c * s * int(F[e])))) == int(case["f32_bits"], 16)
    assert want[e] == int(case["want_bits"], 16)
    other = int(case["other_bits"], 16)
    assert f16_bits(float(rn(c * s * int(F[e]), F16))) == other          # one rounding
    scaled_first = _f32_staged_fwht([rn(c * rn(qi * s)) for qi in q], h)
    assert f16_bits(float(rn(scaled_first[e], F16))) == other            # c_h first


def test_mse_closed_form():
    """mse(x_hat, x) = sum of squared differences / number of elements, in
    float64: x on a 2^-4 grid, x_hat = x + k * 2^-8 (both exact in fp16), so
    the exact value is sum(k^2) * 2^-16 / N; every partial sum is a multiple
    of 2^-16 below 2^15, so float64 accumulation is exact and the oracle must
    return this value exactly."""
    rng = np.random.default_rng(31)
    shape = (64, 4, 128)
    N = int(np.prod(shape))
    x = (rng.integers(-64, 64, size=shape) * 2.0 ** -4).astype(np.float16)
    k = rng.integers(-255, 256, size=shape)
    k[rng.random(shape) < 0.3] = 0
    x_hat = (x.astype(np.float64) + k * 2.0 ** -8).astype(np.float16)
    assert np.array_equal(x_hat.astype(np.float64) - x.astype(np.float64), k * 2.0 ** -8)
    exact = Fraction(int(np.sum(k.astype(np.int64) ** 2)), 2 ** 16 * N)
    got = O.mse(x_hat, x)
    assert Fraction(got) == exact
    # the case tells apart a mean of |d| and a float16 accumulation
    assert Fraction(float(np.mean(np.abs(k * 2.0 ** -8)))) != exact
    d16 = x_hat - x
    assert Fraction(float(np.sum(d16 * d16, dtype=np.float16)) / N) != exact
    # and the sum over a whole tensor, not a mean over rows of their sums
    assert O.mse(x_hat[:1], x[:1]) == float(
        Fraction(int(np.sum(k[:1].astype(np.int64) ** 2)), 2 ** 16 * (N // 64)))


# --------------------------------------------------------------------------
# the pages' accuracy claim, on the synthetic recipes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "sweep", "long"])
def test_rotation_lowers_mse_on_outlier_data(name):
    """Rotation spreads outlier channels so the 16-level grid fits better
    (youngju.dev reading, "The Rotation Trick"; gist.science §2 BDR item 1):
    MSE(rotated) < MSE(naive) for K and for V on every recipe."""
    wl = W.WORKLOADS[name]
    n = min(wl.T, 1024)
    k, v = W.kv(wl, 0, 0, n)
    for x in (k, v):
        naive = O.decode_vectors(*O.encode_vectors(x, 128, False), 128, False)
        m_naive = O.mse(naive, x)
        for h in (32, 64, 128):
            rot = O.decode_vectors(*O.encode_vectors(x, h, True), h, True)
            assert O.mse(rot, x) < m_naive, (name, h)
