"""Property tests of the CPU oracle on arbitrary fp16 vectors (hypothesis).

The properties are the ones the method fixes whatever the input (youngju.dev
reading of SAW-INT4, "Why Naive INT4 Breaks" for token-wise symmetric INT4 on
16 levels; "The Rotation Trick - Block-Diagonal Hadamard" for an orthogonal,
undoable rotation), checked against exact arithmetic or closed forms rather
than against the oracle's own formulas:

  * codes lie in [-8, 7]; -8 and |q| = 8 rounding only occur with a scale that
    saturated or fell into the fp16 subnormal range;
  * the stored scale is the fp16 rounding of the float32 quotient amax / 7
    (checked in exact rational arithmetic), saturated to 65504;
  * outside the clamp, each channel of the (rotated) vector is reproduced by
    q * s within s / 2 plus the float32 rounding of the quotient;
  * the packed bytes unpack to the codes, and the read-back of an append is
    the decode of the encode;
  * the unnormalised transform applied twice is h times the identity on
    integer inputs (exact), and the normalised one preserves the norm.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

from oracle import sawint4 as O
from tests.exact_fp import F16, rn

D = 128
f16_vectors = hnp.arrays(
    np.float16, (D,),
    elements=st.floats(min_value=-65504, max_value=65504, allow_nan=False,
                       allow_infinity=False, width=16))
block_sizes = st.sampled_from([16, 32, 64, 128])
SETTINGS = settings(max_examples=150, deadline=None)


@SETTINGS
@given(x=f16_vectors, h=block_sizes, rotate_it=st.booleans())
def test_scale_and_code_range(x, h, rotate_it):
    codes, s16 = O.encode_vectors(x[None], h, rotate_it)
    q = O.unpack_nibbles(codes)[0].astype(np.int64)
    assert q.min() >= -8 and q.max() <= 7
    y = O.rotate(x.astype(np.float32)[None], h)[0] if rotate_it else x.astype(np.float32)
    amax = max(abs(Fraction(float(v))) for v in y)
    want = rn(rn(amax / 7), F16)
    want = min(want, Fraction(65504)) if want != float("inf") else Fraction(65504)
    assert Fraction(float(s16[0])) == want
    s = float(s16[0])
    if s == 0.0:
        assert not q.any()
        return
    clamp_possible = s == 65504.0 or s < 6.103515625e-05
    if not clamp_possible:
        assert q.min() >= -7                      # |y / s| < 7.004 rounds to at most 7
        err = np.abs(y.astype(np.float64) - q * s)
        assert np.all(err <= s / 2 + np.abs(y.astype(np.float64)) * 2.0 ** -23 + 1e-30)


@SETTINGS
@given(x=f16_vectors, h=block_sizes, rotate_it=st.booleans())
def test_pack_and_read_back_consistent(x, h, rotate_it):
    codes, s16 = O.encode_vectors(x[None], h, rotate_it)
    q = O.unpack_nibbles(codes)
    assert np.array_equal(O.pack_nibbles(q), codes)
    # append into a one-page pool at slot 3, then read back
    kc = np.zeros((1, 4, 1, D // 2), np.uint8)
    ks = np.zeros((1, 4, 1), np.float16)
    slots = np.array([3], np.int64)
    rot = O.ROT_KV if rotate_it else O.ROT_NONE
    O.quantize_append(x[None, None], None, slots, kc, None, ks, None, h=h, rot_mode=rot)
    assert np.array_equal(kc[0, 3, 0], codes[0]) and ks[0, 3, 0] == s16[0]
    assert not kc[0, :3].any() and not ks[0, :3].any()
    back, _ = O.dequant_gather(kc, None, ks, None, slots, h=h, rot_mode=rot)
    want = O.decode_vectors(codes, s16, h, rotate_it)
    assert np.array_equal(back[0, 0].view(np.uint16), want[0].view(np.uint16))


@SETTINGS
@given(v=hnp.arrays(np.int64, (D,), elements=st.integers(-2 ** 12, 2 ** 12)), h=block_sizes)
def test_transform_twice_is_h_identity(v, h):
    x = v.astype(np.float32)
    twice = O.fwht_blocks(O.fwht_blocks(x, h), h).astype(np.float64)
    assert np.array_equal(twice, h * v.astype(np.float64))


@SETTINGS
@given(x=f16_vectors, h=block_sizes)
def test_rotation_preserves_norm(x, h):
    xf = x.astype(np.float64)
    y = O.rotate(x.astype(np.float32), h).astype(np.float64)
    n0, n1 = np.linalg.norm(xf), np.linalg.norm(y)
    assert abs(n1 - n0) <= 1e-5 * n0 + 1e-30
