"""Pins of the oracle's fused prologue: q/k RMSNorm over a token's C channels and
the (B, N, 3, C) q|k|v input, checked against hand-worked values, a library norm
and the invariants the reading implies."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROPE_3D = {"split": (2, 2, 4), "grid": (2, 3), "base": 100.0}


def frac(x):
    return float(Fraction(x))


def load_golden():
    with open(os.path.join(HERE, "golden", "qk_norm_example.json")) as f:
        return json.load(f)


def rand_qkv(seed, B, N, H, d):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, N, 3, H * d))


def test_norm_hand_worked():
    g = load_golden()["norm_only"]
    gamma = np.array([frac(x) for x in g["gamma"]])
    for case in g["cases"]:
        y = oracle.qk_rms_norm(np.array(case["x"], dtype=np.float64), gamma, case["norm_eps"])
        assert np.allclose(y, [frac(x) for x in case["y"]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("block_tokens,key", [(2, "out_block2"), (1, "out_block1")])
def test_fused_forward_hand_worked(block_tokens, key):
    g = load_golden()["attention"]
    qkv = np.stack([np.array(g["q"]), np.array(g["k"]), np.array(g["v"])], axis=1)[None].astype(np.float64)
    out = oracle.forward_qkv(qkv, g["heads"], 1, block_tokens, None, g["eps"],
                             q_gamma=np.array(g["gamma_q"], dtype=np.float64),
                             k_gamma=np.array(g["gamma_k"], dtype=np.float64), norm_eps=g["norm_eps"])
    want = np.array([[[frac(x) for x in head] for head in tok] for tok in g[key]])
    assert np.allclose(out[0], want, rtol=0, atol=1e-14)


def test_norm_matches_library_norm():
    """With norm_eps = 0 the norm is x * sqrt(C) / ||x||_2 (numpy's vector norm) times gamma."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7, 96)) * rng.uniform(0.1, 10.0, (5, 7, 1))
    gamma = rng.standard_normal(96)
    want = x * np.sqrt(96) / np.linalg.norm(x, axis=-1, keepdims=True) * gamma
    assert np.allclose(oracle.qk_rms_norm(x, gamma, 0.0), want, rtol=1e-13, atol=0)


def test_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 64))
    ones = np.ones(64)
    y = oracle.qk_rms_norm(x, ones, 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    c = rng.uniform(0.01, 100.0, (9, 1))
    assert np.allclose(oracle.qk_rms_norm(c * x, ones, 0.0), y, rtol=1e-13)
    # norm_eps moves the result toward zero: rms(y) = sqrt(ms / (ms + eps)) < 1
    y_eps = oracle.qk_rms_norm(x, ones, 0.5)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y_eps * y_eps, axis=-1)), np.sqrt(ms / (ms + 0.5)), rtol=1e-14)


def test_layout_without_norm_is_plain_forward():
    """No weights: the fused input is only a layout; q|k|v rows hold (H, d) heads in order."""
    B, N, H, d = 2, 24, 3, 8
    qkv = rand_qkv(5, B, N, H, d)
    q = qkv[:, :, 0].reshape(B, N, H, d)
    k = qkv[:, :, 1].reshape(B, N, H, d)
    v = qkv[:, :, 2].reshape(B, N, H, d)
    # element [b, n, 1, h*d + i] is k[b, n, h, i]
    assert k[1, 5, 2, 3] == qkv[1, 5, 1, 2 * d + 3]
    rope = {"split": (2, 2, 4), "grid": (2, 3), "base": 100.0}
    got = oracle.forward_qkv(qkv, H, 6, 2, rope)
    assert np.array_equal(got, oracle.forward(q, k, v, 6, 2, rope))


def test_norm_spans_all_heads():
    """The reading normalises over the token's C channels: scaling one head's k
    changes the other heads' outputs through the shared rms; without the norm it
    does not."""
    B, N, H, d = 1, 12, 3, 4
    qkv = rand_qkv(6, B, N, H, d)
    gq, gk = np.ones(H * d), np.ones(H * d)
    a = oracle.forward_qkv(qkv, H, 4, 1, None, q_gamma=gq, k_gamma=gk)
    b_in = qkv.copy()
    b_in[:, :, 1, 0:d] *= 10.0              # head 0 of k only
    b = oracle.forward_qkv(b_in, H, 4, 1, None, q_gamma=gq, k_gamma=gk)
    assert not np.allclose(a[:, :, 1:], b[:, :, 1:], rtol=1e-6)
    a0 = oracle.forward_qkv(qkv, H, 4, 1, None)
    b0 = oracle.forward_qkv(b_in, H, 4, 1, None)
    assert np.array_equal(a0[:, :, 1:], b0[:, :, 1:])


def test_token_scale_invariance_through_the_norm():
    """Scaling a token's k by c > 0 changes nothing once k is normalised (norm_eps
    = 0); scaling its q changes the output only through eps."""
    B, N, H, d = 1, 18, 2, 8
    qkv = rand_qkv(7, B, N, H, d)
    rng = np.random.default_rng(8)
    gq, gk = rng.standard_normal(H * d), rng.standard_normal(H * d)
    base = oracle.forward_qkv(qkv, H, 6, 1, ROPE_3D, q_gamma=gq, k_gamma=gk, norm_eps=0.0)
    c = rng.uniform(0.1, 10.0, (B, N, 1))
    sk = qkv.copy()
    sk[:, :, 1] *= c
    assert np.allclose(oracle.forward_qkv(sk, H, 6, 1, ROPE_3D, q_gamma=gq, k_gamma=gk, norm_eps=0.0),
                       base, rtol=1e-11, atol=1e-12)
    sq = qkv.copy()
    sq[:, :, 0] *= c
    assert np.allclose(oracle.forward_qkv(sq, H, 6, 1, ROPE_3D, q_gamma=gq, k_gamma=gk, norm_eps=0.0),
                       base, rtol=1e-7, atol=1e-9)
    # and without the norm, scaling k does change the result
    assert not np.allclose(oracle.forward_qkv(sk, H, 6, 1, ROPE_3D), oracle.forward_qkv(qkv, H, 6, 1, ROPE_3D))


def test_weight_applies_before_relu():
    """A negative weight flips the sign before phi: gamma_k = -1 gives the same
    result as normalised -k with weight +1."""
    B, N, H, d = 1, 12, 2, 4
    qkv = rand_qkv(9, B, N, H, d)
    neg = qkv.copy()
    neg[:, :, 1] *= -1.0
    one = np.ones(H * d)
    a = oracle.forward_qkv(qkv, H, 4, 1, None, q_gamma=one, k_gamma=-one)
    b = oracle.forward_qkv(neg, H, 4, 1, None, q_gamma=one, k_gamma=one)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    assert not np.allclose(a, oracle.forward_qkv(qkv, H, 4, 1, None, q_gamma=one, k_gamma=one))


def test_streaming_equals_one_shot():
    B, N, H, d, tpf, bf = 2, 24, 2, 8, 6, 1
    qkv = rand_qkv(10, B, N, H, d)
    rng = np.random.default_rng(11)
    gq, gk = rng.standard_normal(H * d), rng.standard_normal(H * d)
    one = oracle.forward_qkv(qkv, H, tpf, bf, ROPE_3D, q_gamma=gq, k_gamma=gk)
    st = oracle.StreamState(B, H, d)
    parts = [oracle.stream_block_qkv(st, qkv[:, i:i + tpf * bf], H, tpf, ROPE_3D, q_gamma=gq, k_gamma=gk)
             for i in range(0, N, tpf * bf)]
    assert np.allclose(np.concatenate(parts, axis=1), one, rtol=1e-12, atol=1e-13)


def test_zero_token_with_norm_eps():
    """A zero q row stays zero through the norm (norm_eps > 0) and reads out zero."""
    B, N, H, d = 1, 8, 2, 4
    qkv = rand_qkv(12, B, N, H, d)
    qkv[0, 3, 0] = 0.0
    out = oracle.forward_qkv(qkv, H, 4, 1, None, q_gamma=np.ones(H * d), k_gamma=np.ones(H * d))
    assert np.all(out[0, 3] == 0.0)
