"""The seeded input generators (CPU only): determinism, chunk independence,
outlier placement and slot-mapping structure of every workload."""
import numpy as np
import pytest

from int4_kv_cache_amd import workloads as W


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_deterministic_and_range_independent(name):
    wl = W.WORKLOADS[name]
    n = min(wl.T, W.CHUNK + 300)
    a = W.tensor(wl, 0, 0, 0, n)
    b = W.tensor(wl, 0, 0, 0, n)
    assert a.dtype == np.float16 and a.shape == (n, wl.H, wl.D)
    assert a.tobytes() == b.tobytes()
    lo, hi = max(0, n - 500), n
    assert W.tensor(wl, 0, 0, lo, hi).tobytes() == a[lo:hi].tobytes()
    assert not np.array_equal(a, W.tensor(wl, 1, 0, 0, n))
    assert np.all(np.isfinite(a.astype(np.float32)))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_slot_mapping(name):
    wl = W.WORKLOADS[name]
    s = W.slot_mapping(wl)
    assert s.dtype == np.int64 and s.shape == (wl.T,)
    assert s.min() >= 0 and s.max() < wl.n_slots
    assert len(np.unique(s)) == wl.T
    assert np.array_equal(s, W.slot_mapping(wl))
    if wl.placement == "free_list":
        # tokens of one page are consecutive tokens of one sequence
        t = np.arange(wl.T)
        pos = t % wl.seq_len
        assert np.all(s % wl.P == pos % wl.P)
        page = s // wl.P
        first = page[::wl.P]
        assert np.all(page.reshape(-1, wl.P) == first[:, None])
    if wl.placement == "identity":
        assert np.array_equal(s, np.arange(wl.T))


def test_tiny_outlier_channels():
    wl = W.WORKLOADS["tiny"]
    k, v = W.kv(wl)
    for x in (k, v):
        mag = np.abs(x.astype(np.float32)).mean(axis=0)
        for hd in range(wl.H):
            top = set(np.argsort(mag[hd])[-2:].tolist())
            assert top == {3, 77}


def test_per_head_outliers_and_fraction():
    wl = W.WORKLOADS["decode"]
    m0 = W.outlier_multipliers(wl, 0, 0)
    m1 = W.outlier_multipliers(wl, 1, 0)
    assert np.all((m0 == 20).sum(axis=1) == 4)
    assert not np.array_equal(m0, m1)
    wp = W.WORKLOADS["prefill"]
    mp = W.outlier_multipliers(wp, 0, 0)
    assert (mp == 10).sum() == round(0.02 * wp.H * wp.D)


def test_bytes_per_token():
    assert W.WORKLOADS["prefill"].bytes_per_token() == 5160
    assert W.WORKLOADS["tiny"].bytes_per_token() == 1296
