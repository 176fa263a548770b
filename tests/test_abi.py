"""The C ABI of libsawkv.so on the host (CPU only, no GPU).

Every call here either fails host-side validation or has T == 0, so nothing
is ever launched: validation runs before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sawkv.h")
# SAWKV_TEST_LIB: another build of the library to check (the host-only
# AddressSanitizer build of tests/test_host_asan.py)
LIB = os.environ.get("SAWKV_TEST_LIB") or os.path.join(ROOT, "int4_kv_cache_amd", "libsawkv.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EHIP = 0, 1, 2, 3, 4

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsawkv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sawkv_\w+)\s*\(", text)))


class LayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("k", "v", "k_codes", "v_codes", "k_scales", "v_scales")]


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.sawkv_quantize_append.argtypes = [p, p, i64, i64, p, i64, i32, i32, p, p, p, p, i64, i32,
                                        i32, i32, p]
    L.sawkv_dequant_gather.argtypes = [p, p, p, p, i64, i32, p, i64, i32, i32, p, p, i32, i32, p]
    L.sawkv_naive_int4_append.argtypes = [p, p, i64, i64, p, i64, i32, i32, p, p, p, p, i64,
                                          i32, p]
    L.sawkv_naive_int4_gather.argtypes = [p, p, p, p, i64, i32, p, i64, i32, i32, p, p, p]
    L.sawkv_quantize_append_layers.argtypes = [ctypes.POINTER(LayerDesc), i32, i64, i64, p, i64,
                                               i32, i32, i64, i32, i32, i32, p]
    L.sawkv_status_string.restype = ctypes.c_char_p
    L.sawkv_last_error.restype = ctypes.c_char_p
    return L


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) >= {"sawkv_quantize_append", "sawkv_dequant_gather",
                          "sawkv_naive_int4_append", "sawkv_naive_int4_gather",
                          "sawkv_status_string", "sawkv_last_error", "sawkv_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.sawkv_version() == 1
    for st, word in ((OK, b"ok"), (EINVAL, b"invalid"), (EUNSUPPORTED, b"unsupported"),
                     (EALIGN, b"misaligned"), (EHIP, b"HIP")):
        assert word in lib.sawkv_status_string(st)
    assert lib.sawkv_status_string(99) == b"unknown status"


# fake, suitably aligned addresses: never dereferenced, because every call
# below stops in validation or has T == 0
A = 0x100000
K, V, S, KC, VC, KS, VS = (A * i for i in range(1, 8))


def app(lib, **kw):
    a = dict(k=K, v=V, ks=1024, vs=1024, slots=S, T=64, H=8, D=128, kc=KC, vc=VC, kss=KS,
             vss=VS, npg=16, P=16, h=128, rot=2)
    a.update(kw)
    return lib.sawkv_quantize_append(a["k"], a["v"], a["ks"], a["vs"], a["slots"], a["T"],
                                     a["H"], a["D"], a["kc"], a["vc"], a["kss"], a["vss"],
                                     a["npg"], a["P"], a["h"], a["rot"], None)


def gat(lib, **kw):
    a = dict(kc=KC, vc=VC, kss=KS, vss=VS, npg=16, P=16, slots=S, T=64, H=8, D=128, ko=K,
             vo=V, h=128, rot=2)
    a.update(kw)
    return lib.sawkv_dequant_gather(a["kc"], a["vc"], a["kss"], a["vss"], a["npg"], a["P"],
                                    a["slots"], a["T"], a["H"], a["D"], a["ko"], a["vo"],
                                    a["h"], a["rot"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), EINVAL),
    (dict(H=0), EINVAL),
    (dict(D=64), EUNSUPPORTED),
    (dict(D=256), EUNSUPPORTED),
    (dict(P=0), EINVAL),
    (dict(npg=0), EINVAL),
    (dict(npg=1 << 40), EINVAL),
    (dict(h=48), EUNSUPPORTED),
    (dict(h=8), EUNSUPPORTED),
    (dict(h=256), EUNSUPPORTED),
    (dict(rot=3), EINVAL),
    (dict(rot=-1), EINVAL),
    (dict(T=1 << 31, H=1), EUNSUPPORTED),
    (dict(H=257, ks=257 * 128, vs=257 * 128), EUNSUPPORTED),
    (dict(ks=1 << 26), EUNSUPPORTED),
    (dict(slots=None), EINVAL),
    (dict(slots=S + 4), EALIGN),
    (dict(slots=S + 4, T=0), EALIGN),
    (dict(k=None, v=None), EINVAL),
    (dict(kc=None), EINVAL),
    (dict(vss=None), EINVAL),
    (dict(k=K + 8), EALIGN),
    (dict(vc=VC + 2), EALIGN),
    (dict(ks=1000), EINVAL),
    (dict(vs=1028), EALIGN),
])
def test_append_validation(lib, kw, status):
    assert app(lib, **kw) == status
    assert lib.sawkv_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(T=-5), EINVAL),
    (dict(D=96), EUNSUPPORTED),
    (dict(h=100), EUNSUPPORTED),
    (dict(ko=None, vo=None), EINVAL),
    (dict(kc=None), EINVAL),
    (dict(ko=K + 4), EALIGN),
    (dict(rot=7), EINVAL),
    (dict(slots=None), EINVAL),
])
def test_gather_validation(lib, kw, status):
    assert gat(lib, **kw) == status


def test_naive_entry_points_validate(lib):
    assert lib.sawkv_naive_int4_append(K, V, 1024, 1024, S, 64, 8, 64, KC, VC, KS, VS, 16, 16,
                                       None) == EUNSUPPORTED
    assert lib.sawkv_naive_int4_gather(KC, VC, KS, VS, 16, 16, S, 64, 8, 128, None, None,
                                       None) == EINVAL


def test_zero_tokens_launch_nothing(lib):
    assert app(lib, T=0) == OK
    assert app(lib, T=0, k=None, v=None, slots=None) == OK      # empty tensors: NULL data
    assert gat(lib, T=0, ko=None, vo=None, slots=None) == OK
    assert lib.sawkv_last_error() == b""
    assert app(lib, T=0, D=64) == EUNSUPPORTED                   # sizes still checked
    assert gat(lib, T=0) == OK
    assert app(lib, T=0, v=None, vc=None, vss=None, rot=1) == OK
    assert lib.sawkv_naive_int4_append(K, None, 1024, 0, S, 0, 8, 128, KC, None, KS, None, 4,
                                       16, None) == OK


def test_one_tensor_may_be_absent(lib):
    # V absent: its pool pointers are ignored (T = 0 keeps this launch-free)
    assert app(lib, T=0, v=None, vc=None, vss=None) == OK
    assert gat(lib, T=0, ko=None, kc=None, kss=None) == OK


def layers_call(lib, descs, n=None, T=256, slots=S, h=128, rot=1):
    arr = (LayerDesc * max(1, len(descs)))(*descs)
    return lib.sawkv_quantize_append_layers(arr if descs else None, len(descs) if n is None else n,
                                            1024, 1024, slots, T, 8, 128, 64, 16, h, rot, None)


def good_layer(i):
    base = A * (16 + 8 * i)
    return LayerDesc(base, base + A, base + 2 * A, base + 3 * A, base + 4 * A, base + 5 * A)


def test_layers_validation(lib):
    descs = [good_layer(i) for i in range(4)]
    assert layers_call(lib, [], n=0) == EINVAL                        # NULL array
    assert layers_call(lib, descs, n=0) == EINVAL
    assert layers_call(lib, [good_layer(i) for i in range(65)]) == EINVAL
    bad = list(descs)
    bad[2] = LayerDesc(bad[2].k, None, bad[2].k_codes, None, bad[2].k_scales, None)
    assert layers_call(lib, bad) == EINVAL                            # presence differs
    assert b"layer 2" in lib.sawkv_last_error()
    mis = list(descs)
    mis[3] = LayerDesc(mis[3].k + 8, mis[3].v, mis[3].k_codes, mis[3].v_codes,
                       mis[3].k_scales, mis[3].v_scales)
    assert layers_call(lib, mis) == EALIGN
    assert b"layer 3" in lib.sawkv_last_error()
    nul = list(descs)
    nul[1] = LayerDesc(nul[1].k, nul[1].v, None, nul[1].v_codes, nul[1].k_scales, nul[1].v_scales)
    assert layers_call(lib, nul) == EINVAL
    assert layers_call(lib, descs, h=40) == EUNSUPPORTED
    assert layers_call(lib, descs, T=0) == OK                          # nothing launched


# ---- decode attention: every call below stops in validation (the base case
# has a 1-byte workspace, which is the last check) or has B == 0 ----

Q, BT, CL, OUT, WS = (A * i for i in range(8, 13))


def attn(lib, **kw):
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sawkv_decode_attention.argtypes = [p, i64, p, p, p, p, i64, i32, p, i64, p, i64, i32,
                                           i32, i32, i64, ctypes.c_float, i32, i32, p, p,
                                           ctypes.c_size_t, p]
    a = dict(q=Q, qs=32 * 128, kc=KC, vc=VC, kss=KS, vss=VS, npg=64, P=16, bt=BT, bts=64,
             cl=CL, B=4, Hq=32, H=8, D=128, maxc=1000, sm=0.088, h=128, rot=1, out=OUT, ws=WS,
             wsb=1)
    a.update(kw)
    return lib.sawkv_decode_attention(a["q"], a["qs"], a["kc"], a["vc"], a["kss"], a["vss"],
                                      a["npg"], a["P"], a["bt"], a["bts"], a["cl"], a["B"],
                                      a["Hq"], a["H"], a["D"], a["maxc"], a["sm"], a["h"],
                                      a["rot"], a["out"], a["ws"], a["wsb"], None)


def attn_ws(lib, B=4, Hq=32, H=8, D=128, maxc=1000):
    lib.sawkv_decode_attention_workspace_size.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
        ctypes.POINTER(ctypes.c_size_t)]
    n = ctypes.c_size_t(0)
    st = lib.sawkv_decode_attention_workspace_size(B, Hq, H, D, maxc, ctypes.byref(n))
    return st, n.value


def test_attention_base_case_stops_at_workspace_size(lib):
    assert attn(lib) == EINVAL
    assert b"workspace" in lib.sawkv_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), EINVAL),
    (dict(H=0), EINVAL),
    (dict(Hq=30), EINVAL),
    (dict(Hq=24), EUNSUPPORTED),
    (dict(Hq=128), EUNSUPPORTED),
    (dict(D=64, qs=32 * 64), EUNSUPPORTED),
    (dict(H=512, Hq=512, qs=512 * 128), EUNSUPPORTED),
    (dict(maxc=-1), EINVAL),
    (dict(maxc=(1 << 30) + 1, bts=1 << 27), EUNSUPPORTED),
    (dict(P=0), EINVAL),
    (dict(P=8), EUNSUPPORTED),
    (dict(P=24), EUNSUPPORTED),
    (dict(npg=0), EINVAL),
    (dict(npg=1 << 31), EUNSUPPORTED),
    (dict(h=8), EUNSUPPORTED),
    (dict(rot=3), EINVAL),
    (dict(sm=float("inf")), EINVAL),
    (dict(sm=float("nan")), EINVAL),
    (dict(bts=62), EINVAL),
    (dict(qs=32 * 128 - 8), EINVAL),
    (dict(qs=32 * 128 + 4), EALIGN),
    (dict(q=None), EINVAL),
    (dict(bt=None), EINVAL),
    (dict(cl=None), EINVAL),
    (dict(out=None), EINVAL),
    (dict(ws=None), EINVAL),
    (dict(q=Q + 8), EALIGN),
    (dict(vss=VS + 2), EALIGN),
    (dict(ws=WS + 16), EALIGN),
    (dict(bt=BT + 2), EALIGN),
])
def test_attention_validation(lib, kw, status):
    assert attn(lib, **kw) == status
    assert lib.sawkv_last_error() != b""


def test_attention_empty_batch_reads_nothing(lib):
    assert attn(lib, B=0, q=None, kc=None, vc=None, kss=None, vss=None, bt=None, cl=None,
                out=None, ws=None, wsb=0) == OK


def test_attention_workspace_size(lib):
    st, n = attn_ws(lib)
    assert st == OK and n > 0 and n % 256 == 0
    # grows with the batch and the context; rejects what the call rejects
    assert attn_ws(lib, B=8)[1] > n
    assert attn_ws(lib, maxc=100000)[1] > n
    assert attn_ws(lib, Hq=24)[0] == EUNSUPPORTED
    assert attn_ws(lib, maxc=-3)[0] == EINVAL
    # a workspace one byte short of the reported size is refused
    assert attn(lib, wsb=n - 1) == EINVAL
    assert b"workspace" in lib.sawkv_last_error()


@pytest.mark.parametrize("B,H,maxc,C", [
    (256, 8, 8000, 1024),   # 16384 (sequence, chunk, head) items at 1024 tokens
    (64, 8, 32768, 1024),   # long contexts: 16384 items at 1024
    (192, 8, 8000, 512),    # 12288 items at 1024: 512-token chunks
    (16, 8, 8000, 128),     # halved while fewer than 8192 items, down to 128
    (1, 8, 3611, 64),       # fewer than 1024 items even at 128: 64-token chunks
])
def test_attention_workspace_follows_the_chunk_rule(lib, B, H, maxc, C):
    """The workspace holds float32 partials per (sequence, chunk, query head):
    a (max, sum) pair and a 128-channel output, each region 256-byte aligned;
    the chunk count is ceil(max_context / C) for the chunk length C the
    launch picks from the step's size."""
    Hq = 4 * H
    st, n = attn_ws(lib, B=B, Hq=Hq, H=H, maxc=maxc)
    assert st == OK
    nc = -(-maxc // C)
    align = lambda x: (x + 255) // 256 * 256
    assert n == align(B * nc * Hq * 2 * 4) + align(B * nc * Hq * 128 * 4)


@pytest.mark.parametrize("B,Hq,H,maxc,lean", [
    (1024, 32, 8, 640, True),     # 40 960 steps of 16 tokens: the lean split may run
    (1024, 32, 8, 624, False),    # 39 936 steps: the chunk form only
    (1025, 32, 8, 1000, False),   # more than 1024 sequences: the chunk form only
    (1024, 28, 7, 640, False),    # odd KV-head count: no head pairs, the chunk form only
])
def test_attention_workspace_covers_the_lean_split(lib, B, Hq, H, maxc, lean):
    """Where the lean split may run, the workspace also holds its layout: 8 bytes
    per sequence for the merge's view, then the partials of (sequence, wave)
    rows b + k, at most B + 4096 / (H / 2) of them per query head."""
    st, n = attn_ws(lib, B=B, Hq=Hq, H=H, maxc=maxc)
    assert st == OK
    align = lambda x: (x + 255) // 256 * 256
    rows = (B + 4096 // (H // 2)) * Hq
    lean_bytes = align(B * 8) + align(rows * 2 * 4) + align(rows * 128 * 4)
    if lean:
        assert n >= lean_bytes
    else:
        # the chunk form's layout alone: (max, sum) pairs and outputs of whole chunks
        per = n // (Hq * (2 + 128) * 4)
        assert n == align(per * Hq * 2 * 4) + align(per * Hq * 128 * 4)


# ---- controls: uncompressed cache write and token-wise INT8 (validation only) ----

def ctl(lib, name, **kw):
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    if name == "cache":
        f = lib.sawkv_cache_append
        f.argtypes = [p, p, i64, i64, p, i64, i32, i32, p, p, i64, i32, p]
        a = dict(k=K, v=V, ks=1024, vs=1024, slots=S, T=64, H=8, D=128, kc=KC, vc=VC, npg=16,
                 P=16)
        a.update(kw)
        return f(a["k"], a["v"], a["ks"], a["vs"], a["slots"], a["T"], a["H"], a["D"], a["kc"],
                 a["vc"], a["npg"], a["P"], None)
    if name == "append8":
        f = lib.sawkv_int8_append
        f.argtypes = [p, p, i64, i64, p, i64, i32, i32, p, p, p, p, i64, i32, i32, i32, p]
        a = dict(k=K, v=V, ks=1024, vs=1024, slots=S, T=64, H=8, D=128, kc=KC, vc=VC, kss=KS,
                 vss=VS, npg=16, P=16, h=128, rot=2)
        a.update(kw)
        return f(a["k"], a["v"], a["ks"], a["vs"], a["slots"], a["T"], a["H"], a["D"], a["kc"],
                 a["vc"], a["kss"], a["vss"], a["npg"], a["P"], a["h"], a["rot"], None)
    f = lib.sawkv_int8_gather
    f.argtypes = [p, p, p, p, i64, i32, p, i64, i32, i32, p, p, i32, i32, p]
    a = dict(kc=KC, vc=VC, kss=KS, vss=VS, npg=16, P=16, slots=S, T=64, H=8, D=128, ko=K, vo=V,
             h=128, rot=2)
    a.update(kw)
    return f(a["kc"], a["vc"], a["kss"], a["vss"], a["npg"], a["P"], a["slots"], a["T"], a["H"],
             a["D"], a["ko"], a["vo"], a["h"], a["rot"], None)


@pytest.mark.parametrize("name", ["cache", "append8", "gather8"])
@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), EINVAL),
    (dict(H=0), EINVAL),
    (dict(D=64), EUNSUPPORTED),
    (dict(npg=0), EINVAL),
    (dict(slots=None), EINVAL),
    (dict(slots=S + 4), EALIGN),
])
def test_control_validation(lib, name, kw, status):
    assert ctl(lib, name, **kw) == status
    assert lib.sawkv_last_error() != b""


def test_control_specific_validation(lib):
    assert ctl(lib, "cache", k=None, v=None) == EINVAL
    assert ctl(lib, "cache", k=K + 8) == EALIGN
    assert ctl(lib, "cache", ks=1000) == EINVAL
    assert ctl(lib, "cache", kc=None) == EINVAL
    assert ctl(lib, "append8", h=48) == EUNSUPPORTED
    assert ctl(lib, "append8", rot=5) == EINVAL
    assert ctl(lib, "append8", vss=VS + 2) == EALIGN
    assert ctl(lib, "gather8", ko=None, vo=None) == EINVAL
    assert ctl(lib, "gather8", kc=None) == EINVAL
    # T == 0 reads no pointer
    assert ctl(lib, "cache", T=0, k=None, v=None, kc=None, vc=None, slots=None) == OK
    assert ctl(lib, "append8", T=0, k=None, v=None, kc=None, vc=None, kss=None, vss=None,
               slots=None) == OK
    assert ctl(lib, "gather8", T=0, ko=None, vo=None, kc=None, vc=None, kss=None, vss=None,
               slots=None) == OK


@pytest.mark.parametrize("stride", [-8, -1024, -(1 << 40), 0, 8])
@pytest.mark.parametrize("which", ["k", "v"])
def test_input_stride_below_row_is_rejected_by_every_append(lib, stride, which):
    """A K or V token stride below H*D (negative included) is refused before
    any launch by every entry point that reads fp16 K/V rows."""
    kw = {"ks": stride} if which == "k" else {"vs": stride}
    assert app(lib, **kw) == EINVAL
    assert b"stride" in lib.sawkv_last_error()
    ks, vs = kw.get("ks", 1024), kw.get("vs", 1024)
    assert lib.sawkv_naive_int4_append(K, V, ks, vs, S, 64, 8, 128, KC, VC, KS, VS, 16, 16,
                                       None) == EINVAL
    arr = (LayerDesc * 2)(good_layer(0), good_layer(1))
    assert lib.sawkv_quantize_append_layers(arr, 2, ks, vs, S, 256, 8, 128, 64, 16, 128, 1,
                                            None) == EINVAL
    assert ctl(lib, "append8", **kw) == EINVAL
    assert ctl(lib, "cache", **kw) == EINVAL
    assert b"stride" in lib.sawkv_last_error()


def test_pattern_control_validation(lib):
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = lib.sawkv_append_pattern_control
    f.argtypes = [p, p, i64, i64, p, i64, i32, i32, p, p, p, p, i64, i32, i32, p]

    def call(**kw):
        a = dict(k=K, v=V, ks=1024, vs=1024, slots=S, T=64, H=8, D=128, kc=KC, vc=VC, kss=KS,
                 vss=VS, npg=16, P=16, place=0)
        a.update(kw)
        return f(a["k"], a["v"], a["ks"], a["vs"], a["slots"], a["T"], a["H"], a["D"], a["kc"],
                 a["vc"], a["kss"], a["vss"], a["npg"], a["P"], a["place"], None)

    assert call(place=2) == EINVAL
    assert call(place=-1) == EINVAL
    assert call(place=1, T=300, npg=16, P=16) == EINVAL       # token order needs T <= N_pg*P
    assert b"token order" in lib.sawkv_last_error()
    assert call(ks=-8) == EINVAL
    assert call(k=K + 8) == EALIGN
    assert call(D=64) == EUNSUPPORTED
    assert call(k=None, v=None) == EINVAL
    assert call(T=0, k=None, v=None, slots=None) == OK


def test_noalloc_attention_validation(lib):
    """The no-allocation decode attention: size checks happen before any HIP
    call; sizes whose partials exceed the static scratch are refused."""
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f = lib.sawkv_decode_attention_noalloc
    f.argtypes = [p, i64, p, p, p, p, i64, i32, p, i64, p, i64, i32, i32, i32, i64,
                  ctypes.c_float, i32, i32, p, p]

    def call(**kw):
        a = dict(q=Q, qs=32 * 128, kc=KC, vc=VC, kss=KS, vss=VS, npg=64, P=16, bt=BT,
                 bts=1 << 20, cl=CL, B=4, Hq=32, H=8, D=128, maxc=1000, sm=0.088, h=128, rot=1,
                 out=OUT)
        a.update(kw)
        return f(a["q"], a["qs"], a["kc"], a["vc"], a["kss"], a["vss"], a["npg"], a["P"],
                 a["bt"], a["bts"], a["cl"], a["B"], a["Hq"], a["H"], a["D"], a["maxc"],
                 a["sm"], a["h"], a["rot"], a["out"], None)

    st, need = attn_ws(lib, B=64, maxc=1 << 24)
    assert st == OK and need > 128 << 20
    assert call(B=64, maxc=1 << 24) == EUNSUPPORTED
    assert b"scratch" in lib.sawkv_last_error()
    assert call(Hq=24) == EUNSUPPORTED
    assert call(B=-1) == EINVAL
    assert call(B=0, q=None, kc=None, vc=None, kss=None, vss=None, bt=None, cl=None,
                out=None) == OK
