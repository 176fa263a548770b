"""CPU oracle for the SAW-INT4 KV-cache write path and its read-back.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the CPU
baseline leg of the benchmark import this module. The product path (the HIP
library and its Python binding) never imports, links or executes it, and this
module imports nothing from the product path.

The method, as the source pages describe it, and where each step comes from:

  [YJ]  youngju.dev reading of the SAW-INT4 preprint (the English and the
        Chinese transcriptions carry the same sections):
          "Why Naive INT4 Breaks"            -> one scale per token, 16 levels,
                                                quantise on arrival, append,
                                                never revisit past tokens
          "The Rotation Trick - Block-Diagonal Hadamard"
                                             -> orthogonal Hadamard rotation,
                                                undoable, applied within blocks
          "The System Is the Design - A Fused Kernel" (diagram)
                                             -> fp16 K,V in; rotate; token-wise
                                                INT4; append to a paged block
  [GS]  gist.science summary, "SAW-INT4: System-Aware 4-Bit KV-Cache
        Quantization for Real-World LLM Serving":
          §2 Metodologia (token-wise principle; BDR items 1-3)
                                             -> Hadamard rotation before
                                                quantisation, in independent
                                                blocks of size h
          §4 Risultati Sperimentali          -> h = 128; rotating keys only is
                                                enough

The pages leave the arithmetic open. The readings taken here (the plainest
ones the pages support) are:

  * Hadamard: Sylvester construction, natural order, no random signs; the
    un-normalised transform F_h is a sequence of butterfly stages with
    strides 1, 2, 4, ..., h/2, each butterfly (a, b) -> (a + b, a - b) rounded
    to float32; blocks are h contiguous channels of one head.
  * Normalisation: after the butterflies, one float32 multiply by
    c_h = float32(1/sqrt(h)).
  * Scale: one per (token, head, K|V) vector over all D channels:
    s = f16(f32(amax / 7)); an f16 overflow saturates to 65504.
  * Codes: q = clamp(rint(f32(y / s)), -8, 7), rint = half-to-even; s == 0
    gives all-zero codes.
  * Packing: two's-complement nibbles, element 2k in the low nibble of byte k.
  * Pool: slot = page * P + offset; codes [N_pg][P][H][D/2] uint8, scales
    [N_pg][P][H] float16, separate K and V pools; slot < 0 or slot >= N_pg*P
    is skipped (append) or gives a zero row (gather).
  * Read-back: y = q * s (exact in float32), the same butterflies, times c_h,
    then f16; without rotation just f16(q * s).

All floating-point work is IEEE float32 with round-to-nearest-even, done by
numpy element by element (no fused multiply-add, no flush-to-zero), so that
the codes a GPU must reproduce are fixed bit for bit.
"""

import numpy as np

F32 = np.float32
F16 = np.float16

ROT_NONE = 0   # naive token-wise INT4 (the control)
ROT_K = 1      # rotate keys only, values go through naive INT4
ROT_KV = 2     # rotate keys and values

F16_MAX = F16(65504.0)


def c_h(h):
    """float32 nearest to 1/sqrt(h) — the orthonormal scaling of the h x h
    Sylvester Hadamard matrix ([YJ] "The Rotation Trick": the rotation is
    orthogonal, hence undoable)."""
    return F32(1.0 / np.sqrt(np.float64(h)))


def _check_h(h, D):
    if h < 1 or (h & (h - 1)) != 0 or D % h != 0:
        raise ValueError(f"block size h={h} must be a power of two dividing D={D}")


def fwht_blocks(x, h):
    """Un-normalised block-diagonal Walsh-Hadamard transform F_h over the last
    axis, in float32, stage by stage ([GS] §2, BDR item 2: independent blocks
    of size h instead of one dense rotation).

    Stage with stride s (s = 1, 2, ..., h/2, in this order) replaces every
    pair (x[i], x[i+s]) with i mod 2s < s by (x[i] + x[i+s], x[i] - x[i+s]),
    each sum rounded to float32.  Because s < h and h is a multiple of 2s,
    every pair stays inside its block of h channels.
    """
    x = np.array(x, dtype=F32, copy=True)
    D = x.shape[-1]
    _check_h(h, D)
    lead = x.shape[:-1]
    s = 1
    while s < h:
        v = x.reshape(*lead, D // (2 * s), 2, s)   # index i = g*2s + half*s + c
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        s *= 2
    return x


def rotate(x, h):
    """y = f32(c_h * F_h(x)): the block-diagonal Hadamard rotation applied to
    each KV vector before quantisation ([GS] §2 BDR item 1; [YJ] "The Rotation
    Trick")."""
    return fwht_blocks(x, h) * c_h(h)


def token_scale(y):
    """One fp16 scale per vector ([YJ] "Why Naive INT4 Breaks": a scale of the
    token's own, not per channel; [GS] §2 token-wise principle).

    amax = max |y_i| over the whole vector; s = f16(f32(amax / 7)); +inf after
    the f16 rounding saturates to 65504.
    """
    y = np.asarray(y, dtype=F32)
    amax = np.max(np.abs(y), axis=-1)
    s32 = amax / F32(7.0)
    with np.errstate(over="ignore"):
        s16 = s32.astype(F16)
    s16 = np.where(np.isinf(s16), F16_MAX, s16).astype(F16)
    return s16


def quantize_with_scale(y, s16):
    """Symmetric INT4 codes on 16 levels ([YJ] "Why Naive INT4 Breaks"):
    q = clamp(rint(f32(y / s)), -8, 7) with half-to-even rounding, using the
    stored fp16 scale; a zero scale gives all-zero codes."""
    y = np.asarray(y, dtype=F32)
    sf = np.asarray(s16, dtype=F16).astype(F32)[..., None]
    zero = sf == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = y / np.where(zero, F32(1.0), sf)
    q = np.clip(np.rint(qf), -8, 7)
    q = np.where(zero, F32(0.0), q)
    return q.astype(np.int8)


def quantize(y):
    """Token-wise INT4 of each vector: returns (codes int8 [..., D], scale f16 [...])."""
    s16 = token_scale(y)
    return quantize_with_scale(y, s16), s16


def pack_nibbles(q):
    """Two's-complement nibbles, element 2k in the low nibble of byte k."""
    q = np.asarray(q, dtype=np.int8)
    lo = q[..., 0::2].astype(np.uint8) & 0x0F
    hi = q[..., 1::2].astype(np.uint8) & 0x0F
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b):
    """Inverse of pack_nibbles: uint8 [..., D/2] -> int8 [..., D] in [-8, 7]."""
    b = np.asarray(b, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    return q.astype(np.int8)


def _rotated(rot_mode, tensor):
    """[GS] §4: rotating only the keys is enough; the values then go through
    naive token-wise INT4."""
    if rot_mode not in (ROT_NONE, ROT_K, ROT_KV):
        raise ValueError(f"bad rot_mode {rot_mode}")
    if tensor == "k":
        return rot_mode in (ROT_K, ROT_KV)
    return rot_mode == ROT_KV


def encode_vectors(x, h, rotate_it):
    """fp16 vectors [..., D] -> (packed codes uint8 [..., D/2], scales f16 [...]).
    The per-vector body of the fused kernel in the [YJ] diagram: rotate (or
    not), then token-wise INT4, then pack."""
    x32 = np.asarray(x, dtype=F16).astype(F32)
    y = rotate(x32, h) if rotate_it else x32
    q, s16 = quantize(y)
    return pack_nibbles(q), s16


def decode_vectors(codes, s16, h, rotate_it):
    """Read-back of one vector set: y = q * s (exact in float32), inverse
    rotation (the same orthonormal Sylvester transform, its own inverse;
    [YJ] "The Rotation Trick": the rotation can be undone), then fp16."""
    q = unpack_nibbles(codes).astype(F32)
    y = q * np.asarray(s16, dtype=F16).astype(F32)[..., None]
    if rotate_it:
        y = rotate(y, h)
    with np.errstate(over="ignore"):
        return y.astype(F16)


def _valid_slots(slot_mapping, n_slots):
    s = np.asarray(slot_mapping, dtype=np.int64)
    return (s >= 0) & (s < n_slots), s


def quantize_append(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales,
                    h=128, rot_mode=ROT_KV):
    """Append T new tokens to the paged INT4 pools, in place.

    k, v          fp16 [T, H, D] (None skips that tensor; its pools are then unused)
    slot_mapping  int64 [T]; slot = page * P + offset
    k_codes ...   uint8 [N_pg, P, H, D/2]; k_scales ... f16 [N_pg, P, H]

    Each token is quantised on arrival with its own scale and written to its
    slot only; no other byte of the pools changes ([YJ] "Why Naive INT4
    Breaks": append without revisiting past tokens; [GS] §2 BDR item 3:
    one pass, no separate sweep over the cache).
    """
    for name, x, codes, scales in (("k", k, k_codes, k_scales), ("v", v, v_codes, v_scales)):
        if x is None:
            continue
        n_pg, P, H, half = codes.shape
        flat_codes = codes.reshape(n_pg * P, H, half)
        flat_scales = scales.reshape(n_pg * P, H)
        ok, slots = _valid_slots(slot_mapping, n_pg * P)
        packed, s16 = encode_vectors(np.asarray(x)[ok], h, _rotated(rot_mode, name))
        flat_codes[slots[ok]] = packed
        flat_scales[slots[ok]] = s16


def dequant_gather(k_codes, v_codes, k_scales, v_scales, slot_mapping, h=128,
                   rot_mode=ROT_KV):
    """Read the vectors at slot_mapping back from the pools: fp16 [T, H, D]
    per tensor (None where the pool is None); invalid slots give zero rows."""
    out = []
    for name, codes, scales in (("k", k_codes, k_scales), ("v", v_codes, v_scales)):
        if codes is None:
            out.append(None)
            continue
        n_pg, P, H, half = codes.shape
        flat_codes = codes.reshape(n_pg * P, H, half)
        flat_scales = scales.reshape(n_pg * P, H)
        ok, slots = _valid_slots(slot_mapping, n_pg * P)
        res = np.zeros((len(slots), H, 2 * half), dtype=F16)
        res[ok] = decode_vectors(flat_codes[slots[ok]], flat_scales[slots[ok]], h,
                                 _rotated(rot_mode, name))
        out.append(res)
    return out[0], out[1]


def mse(x_hat, x):
    """Mean squared reconstruction error, in float64, over all elements."""
    d = np.asarray(x_hat, dtype=np.float64) - np.asarray(x, dtype=np.float64)
    return float(np.mean(d * d))


# --------------------------------------------------------------------------
# Consumer of the pages: decode attention over the INT4 pool
# --------------------------------------------------------------------------

def dequant_exact(codes, s16, h, rotate_it):
    """Dequantised vectors in float64 without any final rounding: q * s, then
    (rotated tensors) the normalised Sylvester transform, its own inverse.
    The partial sums of F(q * s) are exact in float32; the 1/sqrt(h) factor is
    applied in float64."""
    q = unpack_nibbles(codes).astype(F32)
    y = q * np.asarray(s16, dtype=F16).astype(F32)[..., None]
    if rotate_it:
        return fwht_blocks(y, h).astype(np.float64) / np.sqrt(np.float64(h))
    return y.astype(np.float64)


def paged_decode_attention(q, k_codes, k_scales, v_codes, v_scales, block_tables,
                           context_lens, h=128, rot_mode=ROT_KV, sm_scale=None):
    """One decode step of attention over the paged INT4 cache, in float64.

    q             fp16 [B, Hq, D]; query head j reads KV head j // (Hq // H)
    k/v pools     as written by quantize_append
    block_tables  int [B, max_pages]: page of the sequence's p-th block
    context_lens  int [B]: tokens 0..L-1 live at page block_tables[b, t // P],
                  offset t % P; a page id outside the pool masks its tokens
    Returns float64 [B, Hq, D]: softmax(sm_scale * q . K_t) weighted sum of
    V_t over the context, with K_t, V_t the dequantised vectors in the
    original basis; an empty context gives zeros.

    The consumer of the paged INT4 cache: youngju.dev English page, "Why the
    KV Cache Is the Real Bottleneck" (decoding reads every cached K and V;
    serving engines keep paged layouts and fused attention), and ainews.cool,
    "技术深度解析" item 3 (dequantisation back to compute precision is
    normally fused into the attention kernel). The K and V rows are the
    exact dequantised vectors, so this is the plain definition of one decode
    step of softmax attention over them.
    """
    q = np.asarray(q, dtype=F16)
    B, Hq, D = q.shape
    n_pg, P, H, half = k_codes.shape
    G = Hq // H
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    kc = k_codes.reshape(n_pg * P, H, half)
    vc = v_codes.reshape(n_pg * P, H, half)
    ks = k_scales.reshape(n_pg * P, H)
    vs = v_scales.reshape(n_pg * P, H)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        t = np.arange(L)
        pages = np.asarray(block_tables[b], dtype=np.int64)[t // P]
        ok = (pages >= 0) & (pages < n_pg)
        slots = (pages * P + t % P)[ok]
        if len(slots) == 0:
            continue
        K = dequant_exact(kc[slots], ks[slots], h, _rotated(rot_mode, "k"))   # [n, H, D]
        V = dequant_exact(vc[slots], vs[slots], h, _rotated(rot_mode, "v"))
        for j in range(Hq):
            kv = j // G
            s = (K[:, kv, :] @ q[b, j].astype(np.float64)) * np.float64(sm_scale)
            w = np.exp(s - s.max())
            out[b, j] = (w / w.sum()) @ V[:, kv, :]
    return out
