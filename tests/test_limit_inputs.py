"""CPU checks of the index-limit input formulas (workloads): numpy on the host
and torch tensors (as on the device) give the same integers at the ends of
their ranges, and the degree recipe sums to the requested entry count."""
import numpy as np
import torch

import workloads as W

LIMIT = 2**31 - 2


def test_formulas_agree_between_numpy_and_torch():
    p = np.concatenate([np.arange(0, 1000), np.arange(LIMIT - 1000, LIMIT)]).astype(np.int64)
    for K in (1, 7, (1 << 24) + 3, LIMIT):
        a = W.hashed_cols(p, K)
        b = W.hashed_cols(torch.from_numpy(p), K).numpy()
        assert np.array_equal(a, b)
        assert a.min() >= 0 and a.max() < K
    f = W.small_int_features(p)
    assert np.array_equal(f, W.small_int_features(torch.from_numpy(p)).numpy())
    assert f.min() >= -1000 and f.max() <= 1000
    assert np.array_equal(f.astype(np.float32).astype(np.int64), f)      # exact in fp32
    i = np.arange(LIMIT - 10, LIMIT + 1, dtype=np.int64)
    assert np.array_equal(np.diff(W.alternating_rowptr(i)), i[:-1] % 2)   # odd rows hold one entry


def test_limit_degrees():
    M = 1 << 16
    d = W.limit_degrees(M, 40_000_000, 63, 1 << 20)
    assert d.sum() == 40_000_000 and d.min() >= 0 and d[-1] == 1 << 20
    light = np.setdiff1d(np.arange(M - 1), np.linspace(0, M - 2, 63).astype(np.int64))
    assert d[light].max() <= 700
    assert (d > 700).sum() == 64
