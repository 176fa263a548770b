"""CPU oracle for the controls the INT4 cache is compared against.

TEST INFRASTRUCTURE, like oracle/sawint4.py: imported only by the tests, the
package smoke check and the benchmark's CPU-baseline leg; it shares no code
with the HIP library.

  * the uncompressed cache: each new token's 16-bit K/V rows copied to their
    slots of a paged fp16 (or bf16) pool. The pages' accuracy and throughput
    baseline is a BF16 cache (gist.science summary of SAW-INT4, §4 Risultati
    Sperimentali: accuracy and system throughput against BF16);
  * token-wise INT8: the same per-vector steps as the INT4 path with 256
    levels. The news page's table has a uniform INT8 row (ainews.cool, the
    comparison table under "技术深度解析"); here INT8 is token-wise, with the
    same optional block-diagonal rotation, so that only the code width
    differs from the INT4 path.

Readings (the pages give no formula for either control):
  * INT8 scale s = f16(f32(amax / 127)), saturating to 65504 as for INT4;
    codes q = clamp(rint_half_even(f32(y / s)), -128, 127); s == 0 gives 0;
    codes stored as int8, one byte per channel; pool [N_pg][P][H][D].
  * INT8 read-back: the Walsh-Hadamard transform of the integer codes (exact
    in float32: every partial sum is an integer of magnitude <= 2^14), times
    s, times c_h, each product rounded to float32, then fp16; without
    rotation f16(q * s) (exact product). (For INT4 the same order gives the
    same value as transforming q * s, since every sum there is exact too.)
"""
import numpy as np

from .sawint4 import F16, F16_MAX, F32, _rotated, _valid_slots, c_h, fwht_blocks, rotate


def token_scale8(y):
    """One fp16 scale per vector for 256 levels: s = f16(f32(amax / 127)),
    saturating to 65504."""
    y = np.asarray(y, dtype=F32)
    s32 = np.max(np.abs(y), axis=-1) / F32(127.0)
    with np.errstate(over="ignore"):
        s16 = s32.astype(F16)
    return np.where(np.isinf(s16), F16_MAX, s16).astype(F16)


def quantize8_with_scale(y, s16):
    """q = clamp(rint(f32(y / s)), -128, 127), half-to-even; s == 0 -> 0."""
    y = np.asarray(y, dtype=F32)
    sf = np.asarray(s16, dtype=F16).astype(F32)[..., None]
    zero = sf == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = y / np.where(zero, F32(1.0), sf)
    q = np.clip(np.rint(qf), -128, 127)
    q = np.where(zero, F32(0.0), q)
    return q.astype(np.int8)


def encode8_vectors(x, h, rotate_it):
    """fp16 vectors [..., D] -> (int8 codes [..., D], fp16 scales [...])."""
    x32 = np.asarray(x, dtype=F16).astype(F32)
    y = rotate(x32, h) if rotate_it else x32
    s16 = token_scale8(y)
    return quantize8_with_scale(y, s16), s16


def decode8_vectors(codes, s16, h, rotate_it):
    """Read-back of INT8 vectors: f16(f32(c_h * f32(F_h(q) * s))) when
    rotated (F_h(q) exact), else f16(q * s)."""
    q = np.asarray(codes, dtype=np.int8).astype(F32)
    sf = np.asarray(s16, dtype=F16).astype(F32)[..., None]
    if rotate_it:
        y = (fwht_blocks(q, h) * sf) * c_h(h)
    else:
        y = q * sf
    with np.errstate(over="ignore"):
        return y.astype(F16)


def int8_append(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, h=128, rot_mode=0):
    """Token-wise INT8 append, in place; pools: int8 [N_pg, P, H, D] codes,
    fp16 [N_pg, P, H] scales; invalid slots skipped (as for INT4)."""
    for name, x, codes, scales in (("k", k, k_codes, k_scales), ("v", v, v_codes, v_scales)):
        if x is None:
            continue
        n_pg, P, H, D = codes.shape
        flat_codes = codes.reshape(n_pg * P, H, D)
        flat_scales = scales.reshape(n_pg * P, H)
        ok, slots = _valid_slots(slot_mapping, n_pg * P)
        q, s16 = encode8_vectors(np.asarray(x)[ok], h, _rotated(rot_mode, name))
        flat_codes[slots[ok]] = q
        flat_scales[slots[ok]] = s16


def int8_gather(k_codes, v_codes, k_scales, v_scales, slot_mapping, h=128, rot_mode=0):
    """INT8 read-back at slot_mapping: fp16 [T, H, D] per tensor (None where
    the pool is None); invalid slots give zero rows."""
    out = []
    for name, codes, scales in (("k", k_codes, k_scales), ("v", v_codes, v_scales)):
        if codes is None:
            out.append(None)
            continue
        n_pg, P, H, D = codes.shape
        flat_codes = codes.reshape(n_pg * P, H, D)
        flat_scales = scales.reshape(n_pg * P, H)
        ok, slots = _valid_slots(slot_mapping, n_pg * P)
        res = np.zeros((len(slots), H, D), dtype=F16)
        res[ok] = decode8_vectors(flat_codes[slots[ok]], flat_scales[slots[ok]], h,
                                  _rotated(rot_mode, name))
        out.append(res)
    return tuple(out)


def cache_append(k, v, slot_mapping, k_cache, v_cache):
    """Uncompressed paged write: cache[slot] = the token's [H, D] rows of
    16-bit values (fp16 or bf16 bit patterns, copied unchanged), in place;
    invalid slots skipped."""
    for x, cache in ((k, k_cache), (v, v_cache)):
        if x is None:
            continue
        n_pg, P, H, D = cache.shape
        flat = cache.reshape(n_pg * P, H, D)
        ok, slots = _valid_slots(slot_mapping, n_pg * P)
        flat[slots[ok]] = np.asarray(x).view(cache.dtype)[ok]
