"""Pins of the fp64 oracle backward against what the mathematics fixes.

The backward is checked against central finite differences of the forward
oracle (itself pinned in test_oracle_cpu.py), a different computation from the
analytic chain rule, and against exact structural properties: block causality
read backwards, linearity in the output gradient.
"""

import numpy as np
import pytest

import oracle

ROPE_3D = {"split": (2, 2, 4), "grid": (2, 3), "base": 100.0}
ROPE_1D = {"split": (8, 0, 0), "grid": (1, 1), "base": 10000.0}


def rand(seed, N, d, n=4):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((N, d)) for _ in range(n))


def loss(q, k, v, g, tpf, bf, rope, f0):
    return float(np.sum(g * oracle.forward_head(q, k, v, tpf, bf, rope, first_block_frames=f0)))


@pytest.mark.parametrize("tpf,frames,bf,f0,rope", [
    (6, 5, 2, None, ROPE_3D),     # 3 blocks, ragged last
    (6, 5, 2, 3, ROPE_3D),        # longer first block
    (1, 20, 6, None, ROPE_1D),    # 1-D RoPE
    (6, 4, 1, None, None),        # RoPE off, one-frame blocks
])
def test_backward_matches_finite_differences(tpf, frames, bf, f0, rope):
    N, d = frames * tpf, 8
    q, k, v, g = rand(41, N, d)
    dq, dk, dv = oracle.backward_head(q, k, v, g, tpf, bf, rope, first_block_frames=f0)
    rng = np.random.default_rng(42)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        checked = 0
        for _ in range(200):
            n, c = int(rng.integers(N)), int(rng.integers(d))
            if name != "v" and abs(x[n, c]) < 1e-3:
                continue                      # stay off ReLU's kink
            xp, xm = x.copy(), x.copy()
            xp[n, c] += h
            xm[n, c] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"], g, tpf, bf, rope, f0)
                  - loss(args_m["q"], args_m["k"], args_m["v"], g, tpf, bf, rope, f0)) / (2 * h)
            assert abs(fd - grad[n, c]) <= 1e-6 * max(1.0, abs(fd)), (name, n, c, fd, grad[n, c])
            checked += 1
            if checked == 25:
                break
        assert checked == 25


def test_backward_head_dim_32_matches_finite_differences():
    """The head dim of the workloads, 3-D RoPE split 8/12/12 on a 2 x 3 grid."""
    rope = {"split": (8, 12, 12), "grid": (2, 3), "base": 10000.0}
    tpf, frames, bf = 6, 4, 2
    q, k, v, g = rand(43, tpf * frames, 32)
    dq, dk, dv = oracle.backward_head(q, k, v, g, tpf, bf, rope)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for n, c in ((0, 0), (7, 13), (23, 31), (12, 20)):
            if name != "v" and abs(x[n, c]) < 1e-3:
                continue
            xs = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[n, c] += h
            xm[n, c] -= h
            lp = loss(*(xp if nm == name else xs[nm] for nm in "qkv"), g, tpf, bf, rope, None)
            lm = loss(*(xm if nm == name else xs[nm] for nm in "qkv"), g, tpf, bf, rope, None)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[n, c]) <= 1e-6 * max(1.0, abs(fd))


def test_backward_block_causality():
    """Output gradients of blocks before i do not reach dk, dv of block i; dq of a
    block depends on that block's output gradient only."""
    tpf, bf = 6, 2
    q, k, v, g = rand(44, 5 * bf * tpf, 8)
    L = bf * tpf
    a = oracle.backward_head(q, k, v, g, tpf, bf, ROPE_3D)
    g2 = g.copy()
    g2[:2 * L] = np.random.default_rng(45).standard_normal((2 * L, 8))
    b = oracle.backward_head(q, k, v, g2, tpf, bf, ROPE_3D)
    assert np.array_equal(a[1][2 * L:], b[1][2 * L:]) and np.array_equal(a[2][2 * L:], b[2][2 * L:])
    assert np.array_equal(a[0][2 * L:], b[0][2 * L:])
    assert not np.allclose(a[0][:2 * L], b[0][:2 * L])


def test_backward_linear_in_output_gradient():
    tpf, bf = 6, 2
    q, k, v, g = rand(46, 4 * bf * tpf, 8)
    a = oracle.backward_head(q, k, v, g, tpf, bf, ROPE_3D)
    b = oracle.backward_head(q, k, v, 2.5 * g, tpf, bf, ROPE_3D)
    z = oracle.backward_head(q, k, v, 0 * g, tpf, bf, ROPE_3D)
    for x, y, w in zip(a, b, z):
        assert np.allclose(2.5 * x, y, rtol=1e-12, atol=1e-14)
        assert np.all(w == 0.0)


def test_backward_batched_matches_heads():
    rng = np.random.default_rng(47)
    q, k, v, g = (rng.standard_normal((2, 24, 3, 8)) for _ in range(4))
    dq, dk, dv = oracle.backward(q, k, v, g, 6, 2, ROPE_3D)
    ref = oracle.backward_head(q[1, :, 2], k[1, :, 2], v[1, :, 2], g[1, :, 2], 6, 2, ROPE_3D)
    assert np.array_equal(dq[1, :, 2], ref[0]) and np.array_equal(dv[1, :, 2], ref[2])
