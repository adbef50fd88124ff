"""Pins of the oracle's cached temporal convolution (the causal Mix-FFN's
temporal conv with the previous block's last frame kept): hand-worked values,
numpy's convolve, streaming = one-shot and block causality."""

import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "tconv_example.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("kt,bias", [(3, False), (2, False), (3, True)])
def test_hand_worked(kt, bias):
    g = golden()
    x = np.array(g["x"], dtype=np.float64)[None, :, :]          # (B=1, N=4 frames of 1 token, Ch=2)
    w = np.array(g[f"w_kt{kt}"], dtype=np.float64)
    b = np.array(g["bias"]) if bias else None
    y = oracle.temporal_conv(x, w, 1, g["block_frames"], bias=b)
    want = g["y_kt3_bias"] if bias else g[f"y_kt{kt}"]
    assert np.array_equal(y[0], np.array(want, dtype=np.float64))


def rand(seed, B, F, P, Ch):
    return np.random.default_rng(seed).standard_normal((B, F * P, Ch))


@pytest.mark.parametrize("kt", [2, 3])
def test_matches_numpy_convolve(kt):
    """Each block is numpy's convolution of the series [cached frame, block, 0]
    (valid part), per spatial position and channel."""
    B, F, P, Ch, bf = 2, 10, 3, 4, 3
    x = rand(1, B, F, P, Ch)
    w = np.random.default_rng(2).standard_normal((kt, Ch))
    y = oracle.temporal_conv(x, w, P, bf).reshape(B, F, P, Ch)
    xf = x.reshape(B, F, P, Ch)
    for b in range(B):
        for p in range(P):
            for c in range(Ch):
                for s in range(0, F, bf):
                    e = min(F, s + bf)
                    prev = xf[b, s - 1, p, c] if s > 0 else 0.0
                    series = np.concatenate([[prev], xf[b, s:e, p, c], [0.0]])
                    full = np.convolve(series, w[::-1, c], mode="valid")   # length e - s + 3 - kt
                    assert np.allclose(y[b, s:e, p, c], full[:e - s], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kt", [2, 3])
def test_streaming_equals_one_shot(kt):
    B, P, Ch, bf, nblk = 2, 5, 6, 2, 4
    x = rand(3, B, bf * nblk, P, Ch)
    w = np.random.default_rng(4).standard_normal((kt, Ch))
    bias = np.random.default_rng(5).standard_normal(Ch)
    one = oracle.temporal_conv(x, w, P, bf, bias=bias)
    cache = oracle.ConvCache(B, P, Ch)
    L = bf * P
    parts = []
    for j in range(nblk):
        xb = x[:, j * L:(j + 1) * L]
        again = oracle.temporal_conv_stream_block(cache, xb, w, P, bias=bias, save=False)
        parts.append(oracle.temporal_conv_stream_block(cache, xb, w, P, bias=bias, save=True))
        assert np.array_equal(again, parts[-1])          # save=0 reads the same cache, changes nothing
    assert np.array_equal(np.concatenate(parts, axis=1), one)
    assert cache.frames_done == bf * nblk
    assert np.array_equal(cache.last, x.reshape(B, bf * nblk, P, Ch)[:, -1])


def test_block_causality_and_reach():
    """Later blocks never reach earlier outputs; a block's last frame reaches only
    the next block's first frame (kernel 3) across the boundary."""
    B, F, P, Ch, bf = 1, 9, 2, 3, 3
    x = rand(6, B, F, P, Ch)
    w = np.random.default_rng(7).standard_normal((3, Ch))
    y = oracle.temporal_conv(x, w, P, bf).reshape(B, F, P, Ch)
    x2 = x.reshape(B, F, P, Ch).copy()
    x2[:, 5] += 1.0                                      # last frame of block 1
    y2 = oracle.temporal_conv(x2.reshape(B, F * P, Ch), w, P, bf).reshape(B, F, P, Ch)
    changed = [t for t in range(F) if not np.array_equal(y[:, t], y2[:, t])]
    assert changed == [4, 5, 6]                          # its own block's neighbours and frame 6 only
    x3 = x.reshape(B, F, P, Ch).copy()
    x3[:, 6] += 1.0                                      # first frame of block 2
    y3 = oracle.temporal_conv(x3.reshape(B, F * P, Ch), w, P, bf).reshape(B, F, P, Ch)
    assert [t for t in range(F) if not np.array_equal(y[:, t], y3[:, t])] == [6, 7]


def test_first_block_of_other_length_and_ragged_end():
    B, P, Ch = 1, 2, 2
    x = rand(8, B, 8, P, Ch)
    w = np.random.default_rng(9).standard_normal((3, Ch))
    y = oracle.temporal_conv(x, w, P, 3, first_block_frames=2)      # blocks of 2, 3, 3 frames
    xf = x.reshape(B, 8, P, Ch)
    parts = [oracle.temporal_conv_block(xf[:, 0:2], w)]
    parts.append(oracle.temporal_conv_block(xf[:, 2:5], w, xf[:, 1]))
    parts.append(oracle.temporal_conv_block(xf[:, 5:8], w, xf[:, 4]))
    assert np.array_equal(y.reshape(B, 8, P, Ch), np.concatenate(parts, axis=1))
    y7 = oracle.temporal_conv(x[:, :7 * P], w, P, 3)                 # blocks of 3, 3, 1 frames
    assert y7.shape == (B, 7 * P, Ch)


def test_linear_in_x_and_bias_shift():
    B, P, Ch, bf = 1, 3, 4, 4
    x, x2 = rand(10, B, 8, P, Ch), rand(11, B, 8, P, Ch)
    w = np.random.default_rng(12).standard_normal((3, Ch))
    f = lambda a: oracle.temporal_conv(a, w, P, bf)
    assert np.allclose(f(2.0 * x - x2), 2.0 * f(x) - f(x2), rtol=1e-13, atol=1e-13)
    bias = np.array([1.0, -2.0, 0.5, 3.0])
    assert np.allclose(oracle.temporal_conv(x, w, P, bf, bias=bias) - f(x), bias, rtol=0, atol=1e-13)
