"""The K/V cache layouts documented in include/libdllm.h (keys in matrix-core
fragment order, values row-major) against the tests' unpacking into
[N, B, L, G, dh]: every (key, dim) placed by the documented formula must come
back at its own position."""

from __future__ import annotations

import numpy as np
import torch

from gpu_common import unpack_k, unpack_v


def _k_index(j, t, dh):
    # [j/32][t/16][j%32 + 32*((t/8)%2)][t%8]
    return (j // 32, t // 16, j % 32 + 32 * ((t // 8) % 2), t % 8)


def _v_index(j, t, dh):
    # [j][t]: row-major values
    return (j, t)


def _roundtrip(index, unpack, L32, G, dh, blk):
    vals = np.arange(L32 * G * dh, dtype=np.float64).reshape(L32, G, dh) + 1.0
    packed = np.zeros((1, 1, G) + blk, np.float64)
    for j in range(L32):
        for g in range(G):
            for t in range(dh):
                packed[(0, 0, g) + index(j, t, dh)] = vals[j, g, t]
    got = unpack(torch.from_numpy(packed))[0, 0]
    assert got.shape == vals.shape
    assert np.array_equal(got, vals)


def test_k_cache_layout_roundtrip():
    for L32, G, dh in ((64, 2, 64), (32, 1, 128)):
        _roundtrip(_k_index, unpack_k, L32, G, dh, (L32 // 32, dh // 16, 64, 8))


def test_v_cache_layout_roundtrip():
    for L32, G, dh in ((64, 2, 64), (32, 1, 128)):
        _roundtrip(_v_index, unpack_v, L32, G, dh, (L32, dh))
