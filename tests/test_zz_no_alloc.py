"""The decode-attention entry point that allocates nothing
(sawkv_decode_attention_noalloc, partials in the library's static per-GPU
scratch), called through the C ABI, against sawkv_decode_attention with a
caller workspace on the same inputs: the outputs must be identical bytes (the
same kernels run on the same data), on two calls in a row, the second one
smaller, so that it runs over what the first left in the scratch.
"""
import sys

import numpy as np
import pytest

from int4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


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


def _dev(torch, x):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}


def _both(env, d, B, max_context, h, rot):
    """(no-alloc output, workspace output) for the first B sequences."""
    torch, S = env
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    q, bt, cl = d["q"][:B], d["block_tables"][:B], d["context_lens"][:B]
    got = S.decode_attention_noalloc(q, pools, bt, cl, max_context, h=h, rot=rot)
    ref = S.decode_attention(q, pools, bt, cl, max_context, h=h, rot=rot)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("name,first,second", [
    ("attn", 256, 40),          # the lean split, then the chunk form on fewer sequences
    ("attn_small", 9, 4),       # ragged, empty and masked contexts
])
def test_noalloc_equals_workspace_call(env, name, first, second):
    torch, S = env
    wl = W.ATTN_WORKLOADS[name]
    x = W.attn_inputs(wl)
    d = _dev(torch, x)
    L = x["context_lens"]
    for B in (first, second):
        maxc = int(L[:B].max())
        need = S.attention_workspace_size(B, wl.Hq, wl.H, maxc)
        assert need <= S.NOALLOC_MAX_BYTES
        say(f"noalloc {name}: B={B} max_context={maxc} partials {need} bytes")
        got, ref = _both(env, d, B, maxc, wl.h, {0: "none", 1: "k", 2: "kv"}[wl.rot_mode])
        assert got.tobytes() == ref.tobytes(), f"{name} B={B}"


def test_noalloc_rejects_sizes_beyond_the_scratch(env):
    torch, S = env
    wl = W.ATTN_WORKLOADS["attn_small"]
    x = W.attn_inputs(wl)
    d = _dev(torch, x)
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    big = 1 << 22                   # max_context large enough to need > 128 MiB
    bt = torch.zeros((wl.B, big // wl.P), dtype=torch.int32, device="cuda")
    assert S.attention_workspace_size(wl.B, wl.Hq, wl.H, big) > S.NOALLOC_MAX_BYTES
    with pytest.raises(S.SawkvError) as e:
        S.decode_attention_noalloc(d["q"], pools, bt, d["context_lens"], big, h=wl.h)
    assert e.value.status == S.EUNSUPPORTED


@pytest.mark.parametrize("name", ["attn_small", "attn"])
def test_noalloc_replays_under_graph_capture(env, name):
    """The callers it is for: the no-alloc call captured into a HIP graph
    (after one eager call, which looks up the scratch address). Every replay,
    with fresh queries written in place beforehand and eager calls of both
    entry points in between, equals those eager calls byte for byte. The small
    batch runs the chunk form, the 256-sequence one the lean split."""
    torch, S = env
    wl = W.ATTN_WORKLOADS[name]
    x = W.attn_inputs(wl)
    d = _dev(torch, x)
    pools = (d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"])
    maxc = int(x["context_lens"].max())
    q = d["q"].clone()
    out = torch.empty_like(q)
    args = (pools, d["block_tables"], d["context_lens"], maxc)
    S.decode_attention_noalloc(q, *args, h=wl.h, rot="kv", out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.decode_attention_noalloc(q, *args, h=wl.h, rot="kv", out=out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for i in range(4):
        fresh = rng.standard_normal(tuple(q.shape)).astype(np.float16)
        q.copy_(torch.from_numpy(fresh).cuda())
        torch.cuda.synchronize()
        say(f"graph replay {i} ({name})")
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        eager = S.decode_attention_noalloc(q, *args, h=wl.h, rot="kv").cpu().numpy()
        ref = S.decode_attention(q, *args, h=wl.h, rot="kv").cpu().numpy()
        assert got.tobytes() == eager.tobytes(), f"replay {i} vs eager no-alloc call"
        assert got.tobytes() == ref.tobytes(), f"replay {i} vs workspace call"
