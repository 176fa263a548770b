"""Pins of the control oracles (token-wise INT8, uncompressed paged cache).

Checked against exact rational arithmetic (tests/exact_fp.py), closed forms,
scipy's Hadamard matrix and the INT4 path; nothing here re-types the
oracle's own formulas in numpy.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O
from int4_kv_cache_amd import workloads as W
from tests.exact_fp import F16, F32, rint_even, rn


def brute_int8(x16, rotate_it, h):
    """Exact-arithmetic encoder of one fp16 vector: transform stage by stage
    with float32 rounding, then scale and codes from the definitions."""
    y = [Fraction(float(v)) for v in np.asarray(x16, dtype=np.float16)]
    D = len(y)
    if rotate_it:
        s = 1
        while s < h:
            for i in range(D):
                if i % (2 * s) < s:
                    a, b = y[i], y[i + s]
                    y[i], y[i + s] = rn(a + b), rn(a - b)
            s *= 2
        ch = rn(1 / Fraction(float(np.sqrt(np.float64(h)))))   # c_h = f32(1/sqrt h)
        y = [rn(v * ch) for v in y]
    amax = max(abs(v) for v in y)
    s32 = rn(amax / 127)
    s16 = rn(s32, F16)
    if s16 == float("inf") or s16 > 65504:
        s16 = Fraction(65504)
    if s16 == 0:
        return [0] * D, s16
    q = [min(127, max(-128, rint_even(rn(v / s16)))) for v in y]
    return q, s16


@pytest.mark.parametrize("rotate_it,h", [(False, 128), (True, 16), (True, 128)])
def test_int8_encoder_matches_exact_arithmetic(rotate_it, h):
    rng = np.random.default_rng(20 + h + rotate_it)
    for _ in range(12):
        x = (rng.standard_normal(128) * rng.choice([1e-3, 1.0, 30.0])).astype(np.float16)
        x[rng.integers(0, 128)] *= np.float16(8)
        q, s = O.encode8_vectors(x, h, rotate_it)
        qq, ss = brute_int8(x, rotate_it, h)
        assert Fraction(float(s)) == ss
        assert q.astype(int).tolist() == qq


def test_int8_one_hot_and_zero():
    x = np.zeros(128, np.float16)
    q, s = O.encode8_vectors(x, 128, False)
    assert s == 0 and not q.any()
    x[5] = np.float16(-3.0)
    q, s = O.encode8_vectors(x, 128, False)
    # s = f16(3/127); q5 = rint(-3 / s) lands on -127 (3/127 is an fp16 rounding away)
    assert float(s) == float(rn(rn(Fraction(3, 127)), F16))
    assert q[5] == int(rint_even(rn(Fraction(-3) / Fraction(float(s)))))
    assert abs(int(q[5]) + 127) <= 1 and np.count_nonzero(q) == 1


def test_int8_large_inputs_and_clamp():
    # fp16 inputs cannot saturate an INT8 scale (|y| <= 65504 sqrt(128) < 127 * 65504):
    # a constant vector rotates to one channel of ~679 000 and s = f16(679 000 / 127)
    x = np.full(128, 60000.0, np.float16)
    y = O.rotate(x.astype(np.float32), 128)
    q, s = O.encode8_vectors(x, 128, True)
    assert Fraction(float(s)) == rn(rn(Fraction(float(y[0])) / 127), F16)
    assert q[0] == min(127, int(rint_even(rn(Fraction(float(y[0])) / Fraction(float(s))))))
    assert not q[1:].any()
    # an fp16-subnormal scale: the quotient can exceed 127 and must clamp
    x = np.zeros(128, np.float16)
    x[0] = np.float16(1e-5)                 # amax / 127 ~ 1.3 fp16 subnormal steps
    q, s = O.encode8_vectors(x, 128, False)
    assert Fraction(float(s)) == Fraction(1, 2 ** 24)
    assert rint_even(rn(Fraction(float(x[0])) / Fraction(float(s)))) > 127
    assert q[0] == 127


def test_int8_round_trip_error_bound():
    """Unrotated: |x - q s| <= s / 2 for every channel (codes never clamp here)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((500, 128)) * 4).astype(np.float16)
    q, s = O.encode8_vectors(x, 128, False)
    back = O.decode8_vectors(q, s, 128, False).astype(np.float64)
    exact = q.astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.array_equal(back, exact.astype(np.float16).astype(np.float64))
    err = np.abs(x.astype(np.float64) - exact)
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 + 1e-12)


def test_int8_rotated_read_back_two_roundings():
    """Rotated read-back = f16(f32(c_h * f32(F(q) * s))) with F(q) exact: compare
    with scipy's matrix in float64 within the two float32 roundings."""
    rng = np.random.default_rng(4)
    q = rng.integers(-128, 128, size=(64, 128)).astype(np.int8)
    s = rng.lognormal(-2, 1, size=64).astype(np.float16)
    for h in (16, 64, 128):
        got = O.decode8_vectors(q, s, h, True).astype(np.float64)
        blk = np.kron(np.eye(128 // h), scipy.linalg.hadamard(h))
        Fq = q.astype(np.float64) @ blk                      # exact integers
        assert np.all(np.abs(Fq) <= 2 ** 14)
        ref = Fq * s.astype(np.float64)[:, None] / np.sqrt(h)
        tol = np.abs(ref) * 2.0 ** -10 + 1e-30
        assert np.all(np.abs(got - ref) <= tol + np.abs(ref) * 2.0 ** -22)


def test_int8_much_finer_than_int4():
    wl = W.WORKLOADS["sweep"]
    k, v = W.kv(wl, 0, 0, 2048)
    for rot in (False, True):
        q8, s8 = O.encode8_vectors(k, 128, rot)
        back8 = O.decode8_vectors(q8, s8, 128, rot)
        c4, s4 = O.encode_vectors(k, 128, rot)
        back4 = O.decode_vectors(c4, s4, 128, rot)
        assert O.mse(back8, k) * 100 < O.mse(back4, k)


def test_int8_append_and_gather_semantics():
    rng = np.random.default_rng(6)
    T, H, D, n_pg, P = 40, 2, 128, 6, 16
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.permutation(n_pg * P)[:T].astype(np.int64)
    slots[3] = -1
    slots[7] = n_pg * P + 5
    kc = np.full((n_pg, P, H, D), 77, np.int8)
    vc = kc.copy()
    ks = np.full((n_pg, P, H), 9, np.float16)
    vs = ks.copy()
    O.int8_append(k, v, slots, kc, vc, ks, vs, h=128, rot_mode=O.ROT_K)
    ok = (slots >= 0) & (slots < n_pg * P)
    flat = kc.reshape(-1, H, D)
    untouched = np.ones(n_pg * P, bool)
    untouched[slots[ok]] = False
    assert np.all(flat[untouched] == 77)
    qk, sk = O.encode8_vectors(k[ok], 128, True)
    qv, sv = O.encode8_vectors(v[ok], 128, False)
    assert np.array_equal(flat[slots[ok]], qk)
    assert np.array_equal(vc.reshape(-1, H, D)[slots[ok]], qv)
    gk, gv = O.int8_gather(kc, vc, ks, vs, slots, h=128, rot_mode=O.ROT_K)
    assert not gk[~ok].any() and not gv[~ok].any()
    assert np.array_equal(gk[ok], O.decode8_vectors(qk, sk, 128, True))


def test_cache_append_copies_bits():
    rng = np.random.default_rng(7)
    T, H, D, n_pg, P = 30, 4, 128, 4, 16
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.integers(0, 65536, size=(T, H, D)).astype(np.uint16)   # any 16-bit pattern (bf16)
    slots = rng.permutation(n_pg * P)[:T].astype(np.int64)
    slots[0] = -2
    kc = np.zeros((n_pg, P, H, D), np.float16)
    vc = np.zeros((n_pg, P, H, D), np.uint16)
    O.cache_append(k, v, slots, kc, vc)
    flat_k, flat_v = kc.reshape(-1, H, D), vc.reshape(-1, H, D)
    for t in range(1, T):
        assert flat_k[slots[t]].tobytes() == k[t].tobytes()
        assert flat_v[slots[t]].tobytes() == v[t].tobytes()
    written = np.zeros(n_pg * P, bool)
    written[slots[1:]] = True
    assert not flat_k[~written].any() and not flat_v[~written].any()
