"""Host-side checks of the Python binding (CPU only, nothing is launched).

The binding must refuse, before calling the library, every tensor set whose
shapes would let a kernel index outside a buffer: pools that do not hold rows
of the K/V heads and width, K and V pools of different shapes, K and V of
different shapes, and tensors that are not in device memory.
"""
import os

import pytest

torch = pytest.importorskip("torch")

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "int4_kv_cache_amd", "libsawkv.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsawkv.so not built")


@pytest.fixture(scope="module")
def S():
    from int4_kv_cache_amd import sawkv
    return sawkv


def kv(T=16, H=8, D=128):
    return (torch.zeros((T, H, D), dtype=torch.float16),
            torch.zeros((T, H, D), dtype=torch.float16),
            torch.zeros((T,), dtype=torch.int64))


def pools(S, N_pg=4, P=16, H=8, D=128):
    return S.alloc_pools(N_pg, P, H, D, "cpu")


def test_cpu_tensors_are_refused(S):
    k, v, s = kv()
    with pytest.raises(ValueError, match="GPU"):
        S.quantize_append(k, v, s, *pools(S))
    with pytest.raises(ValueError, match="GPU"):
        S.naive_int4_append(k, v, s, *pools(S))
    with pytest.raises(ValueError, match="GPU"):
        S.dequant_gather(*pools(S), s)
    with pytest.raises(ValueError, match="GPU"):
        S.quantize_append_layers([(k, v)], s, [pools(S)])


@pytest.mark.parametrize("fn", ["quantize_append", "naive_int4_append"])
def test_pool_with_fewer_heads_is_refused(S, fn):
    k, v, s = kv(H=8)
    with pytest.raises(ValueError, match="heads"):
        getattr(S, fn)(k, v, s, *pools(S, H=4))


def test_pool_with_narrower_rows_is_refused(S):
    k, v, s = kv(H=8)
    kc, vc, ks, vs = pools(S)
    narrow = torch.zeros((4, 16, 8, 32), dtype=torch.uint8)
    with pytest.raises(ValueError, match="heads"):
        S.quantize_append(k, v, s, narrow, vc, ks, vs)


def test_smaller_v_pool_is_refused(S):
    k, v, s = kv()
    kc, _, ks, _ = pools(S, N_pg=4)
    _, vc, _, vs = pools(S, N_pg=2)
    with pytest.raises(ValueError, match="differ"):
        S.quantize_append(k, v, s, kc, vc, ks, vs)
    with pytest.raises(ValueError, match="differ"):
        S.dequant_gather(kc, vc, ks, vs, s)


def test_k_and_v_of_different_shapes_are_refused(S):
    k, _, s = kv(H=8)
    v = torch.zeros((16, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="differ"):
        S.quantize_append(k, v, s, *pools(S))


def test_layers_pool_mismatch_is_refused(S):
    k, v, s = kv()
    good = pools(S)
    with pytest.raises(ValueError, match="heads|same shape"):
        S.quantize_append_layers([(k, v), (k, v)], s, [good, pools(S, H=2)])


def test_int8_pool_mismatch_is_refused(S):
    k, v, s = kv()
    p8 = S.alloc_int8_pools(4, 16, 4, 128, "cpu")
    with pytest.raises(ValueError, match="heads"):
        S.int8_append(k, v, s, *p8)
    with pytest.raises(ValueError, match="GPU"):
        S.int8_append(k, v, s, *S.alloc_int8_pools(4, 16, 8, 128, "cpu"))


def test_attention_cpu_tensors_are_refused(S):
    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    cl = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        S.decode_attention(q, pools(S), bt, cl, 64)


def test_strided_slot_mapping_is_refused(S):
    # the library reads slot_mapping as a packed int64 array: a strided view
    # would hand it other tensors' values
    k, v, _ = kv()
    s = torch.zeros((32,), dtype=torch.int64)[::2]
    with pytest.raises(ValueError, match="contiguous int64"):
        S.quantize_append(k, v, s, *pools(S))
    with pytest.raises(ValueError, match="contiguous int64"):
        S.naive_int4_append(k, v, s, *pools(S))
    with pytest.raises(ValueError, match="contiguous int64"):
        S.dequant_gather(*pools(S), s)
    with pytest.raises(ValueError, match="contiguous int64"):
        S.quantize_append_layers([(k, v)], s, [pools(S)])
    with pytest.raises(ValueError, match="contiguous int64"):
        S.int8_append(k, v, s, *S.alloc_int8_pools(4, 16, 8, 128, "cpu"))
    with pytest.raises(ValueError, match="contiguous int64"):
        S.int8_gather(*S.alloc_int8_pools(4, 16, 8, 128, "cpu"), s)
    with pytest.raises(ValueError, match="contiguous int64"):
        S.cache_append(k, v, s, torch.zeros((4, 16, 8, 128), dtype=torch.float16),
                       torch.zeros((4, 16, 8, 128), dtype=torch.float16))


def test_slot_mapping_of_other_length_or_type_is_refused(S):
    k, v, _ = kv(T=16)
    with pytest.raises(ValueError, match="contiguous int64"):
        S.quantize_append(k, v, torch.zeros((15,), dtype=torch.int64), *pools(S))
    with pytest.raises(ValueError, match="contiguous int64"):
        S.quantize_append(k, v, torch.zeros((16,), dtype=torch.int32), *pools(S))


def test_attention_block_table_narrower_than_context_is_refused(S):
    # max_context 100 with 16-token pages needs 7 page ids per sequence
    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    bt = torch.zeros((2, 6), dtype=torch.int32)
    cl = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError, match="columns"):
        S.decode_attention(q, pools(S), bt, cl, 100)
    with pytest.raises(ValueError, match="columns"):
        S.decode_attention_noalloc(q, pools(S), bt, cl, 100)
    # a view of a wider table keeps its row stride but not its width
    wide = torch.zeros((2, 8), dtype=torch.int32)
    with pytest.raises(ValueError, match="columns"):
        S.decode_attention(q, pools(S), wide[:, :6], cl, 100)
    with pytest.raises(ValueError, match="GPU"):
        S.decode_attention(q, pools(S), wide[:, :7], cl, 100)
