"""Thin ctypes binding over libsawkv.so (C ABI in include/sawkv.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. Tensors are torch tensors on the ROCm device; torch
provides the memory and the current stream. Importing this module loads the
library and raises ImportError when it has not been built
(python -m int4_kv_cache_amd.build).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsawkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m int4_kv_cache_amd.build`")

lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EUNSUPPORTED, EALIGN, EHIP = 0, 1, 2, 3, 4
PLACE_SLOTS, PLACE_TOKEN_ORDER = 0, 1
ROT_NONE, ROT_K, ROT_KV = 0, 1, 2
ROT = {"none": ROT_NONE, "k": ROT_K, "kv": ROT_KV}

_p, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32


class LayerDesc(ctypes.Structure):
    """sawkv_layer_t"""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p)]


MAX_LAYERS = 64

lib.sawkv_quantize_append.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _i32,
                                      _p, _p, _p, _p, _i64, _i32, _i32, _i32, _p]
lib.sawkv_quantize_append.restype = ctypes.c_int
lib.sawkv_quantize_append_layers.argtypes = [ctypes.POINTER(LayerDesc), _i32, _i64, _i64, _p,
                                             _i64, _i32, _i32, _i64, _i32, _i32, _i32, _p]
lib.sawkv_quantize_append_layers.restype = ctypes.c_int
lib.sawkv_dequant_gather.argtypes = [_p, _p, _p, _p, _i64, _i32, _p, _i64, _i32, _i32,
                                     _p, _p, _i32, _i32, _p]
lib.sawkv_dequant_gather.restype = ctypes.c_int
lib.sawkv_naive_int4_append.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _i32,
                                        _p, _p, _p, _p, _i64, _i32, _p]
lib.sawkv_naive_int4_append.restype = ctypes.c_int
lib.sawkv_naive_int4_gather.argtypes = [_p, _p, _p, _p, _i64, _i32, _p, _i64, _i32, _i32,
                                        _p, _p, _p]
lib.sawkv_naive_int4_gather.restype = ctypes.c_int
lib.sawkv_decode_attention_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i64,
                                                      ctypes.POINTER(ctypes.c_size_t)]
lib.sawkv_decode_attention_workspace_size.restype = ctypes.c_int
lib.sawkv_decode_attention.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i32, _p, _i64, _p,
                                       _i64, _i32, _i32, _i32, _i64, ctypes.c_float, _i32, _i32,
                                       _p, _p, ctypes.c_size_t, _p]
lib.sawkv_decode_attention.restype = ctypes.c_int
lib.sawkv_decode_attention_noalloc.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i32, _p, _i64,
                                               _p, _i64, _i32, _i32, _i32, _i64, ctypes.c_float,
                                               _i32, _i32, _p, _p]
lib.sawkv_decode_attention_noalloc.restype = ctypes.c_int
NOALLOC_MAX_BYTES = 128 << 20    # SAWKV_NOALLOC_MAX_BYTES
lib.sawkv_cache_append.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _i32, _p, _p, _i64,
                                   _i32, _p]
lib.sawkv_cache_append.restype = ctypes.c_int
lib.sawkv_int8_append.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _i32, _p, _p, _p, _p,
                                  _i64, _i32, _i32, _i32, _p]
lib.sawkv_int8_append.restype = ctypes.c_int
lib.sawkv_int8_gather.argtypes = [_p, _p, _p, _p, _i64, _i32, _p, _i64, _i32, _i32, _p, _p, _i32,
                                  _i32, _p]
lib.sawkv_int8_gather.restype = ctypes.c_int
lib.sawkv_append_pattern_control.argtypes = [_p, _p, _i64, _i64, _p, _i64, _i32, _i32, _p, _p,
                                             _p, _p, _i64, _i32, _i32, _p]
lib.sawkv_append_pattern_control.restype = ctypes.c_int
lib.sawkv_status_string.argtypes = [ctypes.c_int]
lib.sawkv_status_string.restype = ctypes.c_char_p
lib.sawkv_last_error.argtypes = []
lib.sawkv_last_error.restype = ctypes.c_char_p
lib.sawkv_version.argtypes = []
lib.sawkv_version.restype = ctypes.c_int


class SawkvError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"sawkv status {status} ({lib.sawkv_status_string(status).decode()}): "
                         f"{detail}")


def _check(status):
    if status != OK:
        raise SawkvError(status, lib.sawkv_last_error().decode())


def _addr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _rot(rot):
    return ROT[rot] if isinstance(rot, str) else int(rot)


def _kv_geometry(x):
    """[T, H, D] fp16 view with unit channel stride and head stride D; returns
    (T, H, D, token stride in elements)."""
    if x.dtype != torch.float16 or x.dim() != 3:
        raise ValueError("K/V must be fp16 [T, H, D]")
    T, H, D = x.shape
    if x.stride(2) != 1 or (H > 1 and x.stride(1) != D):
        raise ValueError("K/V must have unit channel stride and head stride D")
    return T, H, D, x.stride(0)


def _pool_geometry(codes, scales):
    if codes.dtype != torch.uint8 or codes.dim() != 4 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8 [N_pg, P, H, D/2]")
    if scales.dtype != torch.float16 or tuple(scales.shape) != tuple(codes.shape[:3]) \
            or not scales.is_contiguous():
        raise ValueError("scales must be contiguous fp16 [N_pg, P, H]")
    return codes.shape


def _on_gpu(*tensors):
    """Every tensor handed to the library must live in device memory of one GPU."""
    devs = {t.device for t in tensors if t is not None}
    if any(d.type != "cuda" for d in devs):
        raise ValueError("every tensor must be on the GPU (device memory)")
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _slots(slot_mapping, T=None):
    """slot_mapping must be a contiguous int64 vector (of T entries when T is
    given): the library reads it as a packed array."""
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 \
            or not slot_mapping.is_contiguous() or (T is not None and slot_mapping.numel() != T):
        raise ValueError("slot_mapping must be a contiguous int64 [T]")
    return slot_mapping.numel()


def _pools_for(H, D, pairs):
    """Geometry (N_pg, P, H, D/2) shared by every present (codes, scales) pair;
    each pool's heads and row width must be those of the K/V rows it holds."""
    shape = None
    for codes, scales in pairs:
        g = tuple(_pool_geometry(codes, scales))
        if g[2:] != (H, D // 2):
            raise ValueError(f"pool [N_pg, P, H, D/2] = {list(g)} does not hold rows of "
                             f"H={H} heads x D={D}")
        if shape is not None and g != shape:
            raise ValueError(f"K and V pools differ in shape: {list(shape)} vs {list(g)}")
        shape = g
    if shape is None:
        raise ValueError("no pool given")
    return shape


def _kv_pair(k, v):
    """(T, H, D, k token stride, v token stride) of the present K/V tensors,
    which must agree in T, H and D."""
    if k is None and v is None:
        raise ValueError("k and v are both None")
    gk = _kv_geometry(k) if k is not None else None
    gv = _kv_geometry(v) if v is not None else None
    if gk is not None and gv is not None and gk[:3] != gv[:3]:
        raise ValueError(f"K {list(gk[:3])} and V {list(gv[:3])} differ in [T, H, D]")
    T, H, D = (gk or gv)[:3]
    return T, H, D, gk[3] if gk else 0, gv[3] if gv else 0


def alloc_pools(N_pg, P, H, D, device="cuda", code_fill=None, scale_bits_fill=None):
    """The four pool tensors (K codes, V codes, K scales, V scales)."""
    kc = torch.empty((N_pg, P, H, D // 2), dtype=torch.uint8, device=device)
    vc = torch.empty_like(kc)
    ks = torch.empty((N_pg, P, H), dtype=torch.float16, device=device)
    vs = torch.empty_like(ks)
    if code_fill is not None:
        kc.fill_(code_fill)
        vc.fill_(code_fill)
    if scale_bits_fill is not None:
        ks.view(torch.int16).fill_(scale_bits_fill)
        vs.view(torch.int16).fill_(scale_bits_fill)
    return kc, vc, ks, vs


def _present_pools(k, v, k_codes, v_codes, k_scales, v_scales):
    return [pair for x, pair in ((k, (k_codes, k_scales)), (v, (v_codes, v_scales)))
            if x is not None]


def _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, h, rot):
    T, H, D, ks_, vs_ = _kv_pair(k, v)
    pairs = _present_pools(k, v, k_codes, v_codes, k_scales, v_scales)
    N_pg, P = _pools_for(H, D, pairs)[:2]
    _slots(slot_mapping, T)
    _on_gpu(k, v, slot_mapping, *[t for pair in pairs for t in pair])
    return (_addr(k), _addr(v), ks_, vs_, _addr(slot_mapping), T, H, D,
            _addr(k_codes) if k is not None else None, _addr(v_codes) if v is not None else None,
            _addr(k_scales) if k is not None else None, _addr(v_scales) if v is not None else None,
            N_pg, P, h, _rot(rot))


def quantize_append(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *,
                    h=128, rot="kv", stream=None):
    """Fused rotate + token-wise INT4 + paged append (sawkv_quantize_append).
    k or v may be None to skip that tensor."""
    args = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, h, rot)
    _check(lib.sawkv_quantize_append(*args, _stream(stream)))


class AppendCall:
    """sawkv_quantize_append with its arguments checked and marshalled once:
    calling the object only launches (for loops of per-layer calls, where the
    per-call Python checks would otherwise exceed the kernel time). The
    tensors must stay alive and keep their storage while the object is used."""

    def __init__(self, k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *, h=128,
                 rot="kv"):
        self._args = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales,
                                  h, rot)
        self._keep = (k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales)

    def __call__(self, stream=None):
        _check(lib.sawkv_quantize_append(*self._args, _stream(stream)))


class _Prepared:
    """An entry point with its arguments checked and marshalled once: calling
    the object only launches. The tensors must stay alive and keep their
    storage while the object is used."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)))


def NaiveAppendCall(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales):
    """sawkv_naive_int4_append, prepared (see _Prepared)."""
    a = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, 128, "none")
    return _Prepared(lib.sawkv_naive_int4_append, a[:14],
                     (k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales))


def PatternControlCall(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *,
                       placement="slots"):
    """sawkv_append_pattern_control, prepared (see _Prepared)."""
    a = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, 128, "none")
    place = {"slots": PLACE_SLOTS, "token_order": PLACE_TOKEN_ORDER}[placement]
    return _Prepared(lib.sawkv_append_pattern_control, a[:14] + (place,),
                     (k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales))


def GatherCall(k_codes, v_codes, k_scales, v_scales, slot_mapping, k_out, v_out, *, h=128,
               rot="kv"):
    """sawkv_dequant_gather into given outputs, prepared (see _Prepared)."""
    N_pg, P, H, D, T, k_out, v_out = _gather_args(k_codes, v_codes, k_scales, v_scales,
                                                  slot_mapping, k_out, v_out, k_out is not None,
                                                  v_out is not None)
    want_k, want_v = k_out is not None, v_out is not None
    a = (_addr(k_codes) if want_k else None, _addr(v_codes) if want_v else None,
         _addr(k_scales) if want_k else None, _addr(v_scales) if want_v else None,
         N_pg, P, _addr(slot_mapping), T, H, D, _addr(k_out), _addr(v_out), h, _rot(rot))
    return _Prepared(lib.sawkv_dequant_gather, a,
                     (k_codes, v_codes, k_scales, v_scales, slot_mapping, k_out, v_out))


def quantize_append_layers(kv, slot_mapping, pools, *, h=128, rot="kv", stream=None):
    """One launch for several layers of a decode step
    (sawkv_quantize_append_layers). kv: list of (k, v) per layer (k or v may
    be None in every layer); pools: list of (k_codes, v_codes, k_scales,
    v_scales) per layer; all layers share shapes, strides and slot_mapping."""
    LayersCall(kv, slot_mapping, pools, h=h, rot=rot)(stream)


class LayersCall:
    """sawkv_quantize_append_layers with its arguments checked and marshalled
    once: calling the object only launches (for decode loops, where per-call
    Python work would otherwise exceed the kernel time). The tensors must stay
    alive and keep their storage while the object is used."""

    def __init__(self, kv, slot_mapping, pools, *, h=128, rot="kv"):
        self._args = _layers_args(kv, slot_mapping, pools, h, rot)
        self._keep = (kv, slot_mapping, pools)

    def __call__(self, stream=None):
        descs, n, ks_, vs_, slots, T, H, D, N_pg, P, h, rot = self._args
        _check(lib.sawkv_quantize_append_layers(descs, n, ks_, vs_, slots, T, H, D, N_pg, P, h,
                                                rot, _stream(stream)))


def _layers_args(kv, slot_mapping, pools, h, rot):
    n = len(kv)
    if n != len(pools) or not 1 <= n <= MAX_LAYERS:
        raise ValueError(f"need 1..{MAX_LAYERS} layers with one pool set each")
    k0, v0 = kv[0]
    T, H, D, ks_, vs_ = _kv_pair(k0, v0)
    pool = _pools_for(H, D, _present_pools(k0, v0, *pools[0]))
    _slots(slot_mapping, T)
    descs = (LayerDesc * n)()
    for i, ((k, v), (kc, vc, kss, vss)) in enumerate(zip(kv, pools)):
        # the C call takes one geometry for all layers: insist on it here
        if (k is None) != (k0 is None) or (v is None) != (v0 is None):
            raise ValueError("every layer must have the same k/v presence")
        for x, stride in ((k, ks_), (v, vs_)):
            if x is not None and _kv_geometry(x) != (T, H, D, stride):
                raise ValueError("every layer must have the same [T, H, D] and stride")
        if _pools_for(H, D, _present_pools(k, v, kc, vc, kss, vss)) != pool:
            raise ValueError("every layer's pools must have the same shape")
        descs[i] = LayerDesc(_addr(k), _addr(v),
                             _addr(kc) if k is not None else None,
                             _addr(vc) if v is not None else None,
                             _addr(kss) if k is not None else None,
                             _addr(vss) if v is not None else None)
    _on_gpu(slot_mapping, *[x for layer in kv for x in layer],
            *[t for layer_pools in pools for t in layer_pools])
    return (descs, n, ks_, vs_, _addr(slot_mapping), T, H, D, pool[0], pool[1], h, _rot(rot))


def naive_int4_append(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *,
                      stream=None):
    """The no-rotation control (sawkv_naive_int4_append)."""
    a = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, 128, "none")
    _check(lib.sawkv_naive_int4_append(*a[:14], _stream(stream)))


def append_pattern_control(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *,
                           placement="slots", stream=None):
    """The INT4 append's loads and stores with no arithmetic of the method
    (sawkv_append_pattern_control): placement "slots" writes where the append
    writes, "token_order" writes row t*H + head instead."""
    a = _append_args(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, 128, "none")
    place = {"slots": PLACE_SLOTS, "token_order": PLACE_TOKEN_ORDER}[placement]
    _check(lib.sawkv_append_pattern_control(*a[:14], place, _stream(stream)))


def _gather_args(k_codes, v_codes, k_scales, v_scales, slot_mapping, k_out, v_out, want_k,
                 want_v):
    if not (want_k or want_v):
        raise ValueError("neither K nor V wanted")
    pairs = [pair for want, pair in ((want_k, (k_codes, k_scales)), (want_v, (v_codes, v_scales)))
             if want]
    H, half = _pool_geometry(*pairs[0])[2:]
    N_pg, P, H, half = _pools_for(H, 2 * half, pairs)
    D = 2 * half
    T = _slots(slot_mapping)
    _on_gpu(slot_mapping, k_out, v_out, *[t for pair in pairs for t in pair])
    dev = (k_codes if want_k else v_codes).device
    if want_k and k_out is None:
        k_out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    if want_v and v_out is None:
        v_out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    for o in (k_out, v_out):
        if o is not None and (o.dtype != torch.float16 or tuple(o.shape) != (T, H, D)
                              or not o.is_contiguous()):
            raise ValueError("outputs must be contiguous fp16 [T, H, D]")
    return N_pg, P, H, D, T, (k_out if want_k else None), (v_out if want_v else None)


def dequant_gather(k_codes, v_codes, k_scales, v_scales, slot_mapping, *, h=128, rot="kv",
                   k_out=None, v_out=None, want_k=True, want_v=True, stream=None):
    """Dequantise + inverse-rotate the slots back to fp16 (sawkv_dequant_gather).
    Returns (k_out, v_out); a tensor not wanted is None."""
    N_pg, P, H, D, T, k_out, v_out = _gather_args(k_codes, v_codes, k_scales, v_scales,
                                                  slot_mapping, k_out, v_out, want_k, want_v)
    _check(lib.sawkv_dequant_gather(
        _addr(k_codes) if want_k else None, _addr(v_codes) if want_v else None,
        _addr(k_scales) if want_k else None, _addr(v_scales) if want_v else None,
        N_pg, P, _addr(slot_mapping), T, H, D, _addr(k_out), _addr(v_out), h, _rot(rot),
        _stream(stream)))
    return k_out, v_out


def naive_int4_gather(k_codes, v_codes, k_scales, v_scales, slot_mapping, *, k_out=None,
                      v_out=None, want_k=True, want_v=True, stream=None):
    N_pg, P, H, D, T, k_out, v_out = _gather_args(k_codes, v_codes, k_scales, v_scales,
                                                  slot_mapping, k_out, v_out, want_k, want_v)
    _check(lib.sawkv_naive_int4_gather(
        _addr(k_codes) if want_k else None, _addr(v_codes) if want_v else None,
        _addr(k_scales) if want_k else None, _addr(v_scales) if want_v else None,
        N_pg, P, _addr(slot_mapping), T, H, D, _addr(k_out), _addr(v_out), _stream(stream)))
    return k_out, v_out


def attention_workspace_size(B, Hq, H, max_context, D=128):
    """Bytes of workspace sawkv_decode_attention needs for these sizes."""
    n = ctypes.c_size_t(0)
    _check(lib.sawkv_decode_attention_workspace_size(B, Hq, H, D, max_context, ctypes.byref(n)))
    return n.value


def _attention_common(q, pools, block_tables, context_lens, max_context, h, rot, sm_scale,
                      out):
    """Checked and marshalled arguments of sawkv_decode_attention up to `out`
    (the workspace arguments excluded), out, and the workspace bytes needed."""
    k_codes, v_codes, k_scales, v_scales = pools
    N_pg, P, H, half = _pool_geometry(k_codes, k_scales)
    if tuple(_pool_geometry(v_codes, v_scales)) != (N_pg, P, H, half):
        raise ValueError("K and V pools must have the same shape")
    D = 2 * half
    if q.dtype != torch.float16 or q.dim() != 3 or q.shape[2] != D or q.stride(2) != 1 \
            or (q.shape[1] > 1 and q.stride(1) != D):
        raise ValueError("q must be fp16 [B, Hq, D] with unit channel stride and head stride D")
    B, Hq = q.shape[0], q.shape[1]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 \
            or block_tables.shape[0] != B or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [B, max_pages] with unit column stride")
    if B > 0 and block_tables.shape[1] < -(-max_context // P):
        raise ValueError(f"block_tables has {block_tables.shape[1]} columns, fewer than "
                         f"ceil(max_context / P) = {-(-max_context // P)}")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B \
            or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    if out.dtype != torch.float16 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp16 [B, Hq, D]")
    _on_gpu(q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens, out)
    need = attention_workspace_size(B, Hq, H, max_context, D)
    if sm_scale is None:
        sm_scale = 1.0 / float(D) ** 0.5
    bt_stride = block_tables.stride(0) if B > 0 else block_tables.shape[1]
    args = (_addr(q), q.stride(0) if B > 0 else Hq * D, _addr(k_codes), _addr(v_codes),
            _addr(k_scales), _addr(v_scales), N_pg, P, _addr(block_tables), bt_stride,
            _addr(context_lens), B, Hq, H, D, max_context, float(sm_scale), h, _rot(rot),
            _addr(out))
    return args, out, need


def _attention_args(q, pools, block_tables, context_lens, max_context, h, rot, sm_scale, out,
                    workspace):
    args, out, need = _attention_common(q, pools, block_tables, context_lens, max_context, h,
                                        rot, sm_scale, out)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _on_gpu(q, workspace)
    return args + (_addr(workspace), workspace.numel() * workspace.element_size()), out, \
        workspace


def decode_attention(q, pools, block_tables, context_lens, max_context, *, h=128, rot="k",
                     sm_scale=None, out=None, workspace=None, stream=None):
    """One decode step of attention over the paged INT4 pools
    (sawkv_decode_attention). pools = (k_codes, v_codes, k_scales, v_scales).
    Returns out, fp16 [B, Hq, D]."""
    args, out, _ = _attention_args(q, pools, block_tables, context_lens, max_context, h, rot,
                                   sm_scale, out, workspace)
    _check(lib.sawkv_decode_attention(*args, _stream(stream)))
    return out


def decode_attention_noalloc(q, pools, block_tables, context_lens, max_context, *, h=128,
                             rot="k", sm_scale=None, out=None, stream=None):
    """sawkv_decode_attention without a workspace: the library's static
    per-GPU scratch holds the partials (sawkv_decode_attention_noalloc).
    Calls that overlap in time on one GPU race. Returns out."""
    args, out, _ = _attention_common(q, pools, block_tables, context_lens, max_context, h, rot,
                                     sm_scale, out)
    _check(lib.sawkv_decode_attention_noalloc(*args, _stream(stream)))
    return out


class AttentionCall:
    """sawkv_decode_attention with arguments checked and marshalled once (and
    the workspace allocated once); calling the object only launches. The
    tensors must stay alive and keep their storage while the object is used."""

    def __init__(self, q, pools, block_tables, context_lens, max_context, *, h=128, rot="k",
                 sm_scale=None, out=None, workspace=None):
        self._args, self.out, self.workspace = _attention_args(
            q, pools, block_tables, context_lens, max_context, h, rot, sm_scale, out, workspace)
        self._keep = (q, pools, block_tables, context_lens)

    def __call__(self, stream=None):
        _check(lib.sawkv_decode_attention(*self._args, _stream(stream)))
        return self.out


# ---- controls: uncompressed cache write, token-wise INT8 ----

def alloc_int8_pools(N_pg, P, H, D, device="cuda"):
    """INT8 pools: codes int8 [N_pg, P, H, D] (K, V), scales fp16 [N_pg, P, H] (K, V)."""
    kc = torch.empty((N_pg, P, H, D), dtype=torch.int8, device=device)
    ks = torch.empty((N_pg, P, H), dtype=torch.float16, device=device)
    return kc, torch.empty_like(kc), ks, torch.empty_like(ks)


def _int8_pool_geometry(codes, scales):
    if codes.dtype != torch.int8 or codes.dim() != 4 or not codes.is_contiguous():
        raise ValueError("INT8 codes must be contiguous int8 [N_pg, P, H, D]")
    if scales.dtype != torch.float16 or tuple(scales.shape) != tuple(codes.shape[:3]) \
            or not scales.is_contiguous():
        raise ValueError("scales must be contiguous fp16 [N_pg, P, H]")
    return codes.shape


def _int8_pools_for(H, D, pairs):
    """Geometry (N_pg, P, H, D) shared by every present INT8 (codes, scales) pair."""
    shape = None
    for codes, scales in pairs:
        g = tuple(_int8_pool_geometry(codes, scales))
        if g[2:] != (H, D):
            raise ValueError(f"INT8 pool [N_pg, P, H, D] = {list(g)} does not hold rows of "
                             f"H={H} heads x D={D}")
        if shape is not None and g != shape:
            raise ValueError(f"K and V pools differ in shape: {list(shape)} vs {list(g)}")
        shape = g
    if shape is None:
        raise ValueError("no pool given")
    return shape


def cache_append(k, v, slot_mapping, k_cache, v_cache, *, stream=None):
    """Uncompressed paged write of 16-bit K/V rows (sawkv_cache_append)."""
    ref = k if k is not None else v
    if ref.dtype not in (torch.float16, torch.bfloat16) or ref.dim() != 3:
        raise ValueError("K/V must be fp16 or bf16 [T, H, D]")
    T, H, D = ref.shape
    strides = []
    for x, c in ((k, k_cache), (v, v_cache)):
        if x is None:
            strides.append(0)
            continue
        if x.dtype != ref.dtype or x.shape != ref.shape or x.stride(2) != 1 \
                or (H > 1 and x.stride(1) != D):
            raise ValueError("K/V must share shape and dtype, unit channel stride, head stride D")
        if c.dtype != ref.dtype or c.dim() != 4 or tuple(c.shape[2:]) != (H, D) \
                or not c.is_contiguous():
            raise ValueError("caches must be contiguous [N_pg, P, H, D] of the K/V dtype")
        strides.append(x.stride(0))
    cache = k_cache if k is not None else v_cache
    if k is not None and v is not None and tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("K and V caches differ in shape")
    _slots(slot_mapping, T)
    _on_gpu(k, v, slot_mapping, k_cache if k is not None else None,
            v_cache if v is not None else None)
    _check(lib.sawkv_cache_append(_addr(k), _addr(v), strides[0], strides[1],
                                  _addr(slot_mapping), T, H, D,
                                  _addr(k_cache) if k is not None else None,
                                  _addr(v_cache) if v is not None else None,
                                  cache.shape[0], cache.shape[1], _stream(stream)))


def int8_append(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, *, h=128, rot="none",
                stream=None):
    """Token-wise INT8 append (sawkv_int8_append)."""
    T, H, D, ks_, vs_ = _kv_pair(k, v)
    pairs = _present_pools(k, v, k_codes, v_codes, k_scales, v_scales)
    pool = _int8_pools_for(H, D, pairs)
    _slots(slot_mapping, T)
    _on_gpu(k, v, slot_mapping, *[t for pair in pairs for t in pair])
    _check(lib.sawkv_int8_append(
        _addr(k), _addr(v), ks_, vs_, _addr(slot_mapping), T, H, D,
        _addr(k_codes) if k is not None else None, _addr(v_codes) if v is not None else None,
        _addr(k_scales) if k is not None else None, _addr(v_scales) if v is not None else None,
        pool[0], pool[1], h, _rot(rot), _stream(stream)))


def int8_gather(k_codes, v_codes, k_scales, v_scales, slot_mapping, *, h=128, rot="none",
                k_out=None, v_out=None, want_k=True, want_v=True, stream=None):
    """INT8 read-back (sawkv_int8_gather). Returns (k_out, v_out)."""
    if not (want_k or want_v):
        raise ValueError("neither K nor V wanted")
    pairs = [pair for want, pair in ((want_k, (k_codes, k_scales)), (want_v, (v_codes, v_scales)))
             if want]
    H, D = _int8_pool_geometry(*pairs[0])[2:]
    N_pg, P, H, D = _int8_pools_for(H, D, pairs)
    T = _slots(slot_mapping)
    _on_gpu(slot_mapping, k_out, v_out, *[t for pair in pairs for t in pair])
    dev = (k_codes if want_k else v_codes).device
    if want_k and k_out is None:
        k_out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    if want_v and v_out is None:
        v_out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    k_out = k_out if want_k else None
    v_out = v_out if want_v else None
    for o in (k_out, v_out):
        if o is not None and (o.dtype != torch.float16 or tuple(o.shape) != (T, H, D)
                              or not o.is_contiguous()):
            raise ValueError("outputs must be contiguous fp16 [T, H, D]")
    _on_gpu(k_out, v_out)
    _check(lib.sawkv_int8_gather(
        _addr(k_codes) if want_k else None, _addr(v_codes) if want_v else None,
        _addr(k_scales) if want_k else None, _addr(v_scales) if want_v else None,
        N_pg, P, _addr(slot_mapping), T, H, D, _addr(k_out), _addr(v_out), h, _rot(rot),
        _stream(stream)))
    return k_out, v_out
