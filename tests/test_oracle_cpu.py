"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: an O(N^2)
masked form, exact rational arithmetic, the single-block formula in the layout
the pages print it in, a running-sum form, or an invariant of the method.
"""

from fractions import Fraction
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_qkv(seed, B, N, H, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, N, H, d)) * scale for _ in range(3))


ROPE_1D = {"split": (8, 0, 0), "grid": (1, 1), "base": 10000.0}
ROPE_3D = {"split": (2, 2, 4), "grid": (2, 3), "base": 100.0}


# ---------------------------------------------------------------- brute force (pin P1)

@pytest.mark.parametrize("tpf,frames,block_frames,rope", [
    (1, 24, 8, ROPE_1D),        # 3 whole blocks, 1-D RoPE over the token index
    (1, 23, 8, ROPE_1D),        # ragged last block
    (6, 5, 2, ROPE_3D),         # 3-D RoPE, 3 blocks, last one shorter
    (6, 4, 4, ROPE_3D),         # a single block
    (1, 9, 1, ROPE_1D),         # blocks of one token
    (6, 3, 1, None),            # RoPE off
])
def test_blocked_matches_brute_force(tpf, frames, block_frames, rope):
    q, k, v = rand_qkv(1, 2, frames * tpf, 2, 8)
    got = oracle.forward(q, k, v, tpf, block_frames, rope, eps=1e-8)
    ref = oracle.brute_force(q, k, v, tpf, block_frames, rope, eps=1e-8)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_brute_force_d32_tiny_shape():
    # the head dim of every workload, 1-D RoPE with the workload's split
    rope = {"split": (32, 0, 0), "grid": (1, 1), "base": 10000.0}
    q, k, v = rand_qkv(2, 1, 40, 1, 32)
    got = oracle.forward(q, k, v, 1, 16, rope)
    ref = oracle.brute_force(q, k, v, 1, 16, rope)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


# ------------------------------------------------ exact rational arithmetic (RoPE off)

def _fraction_reference(q, k, v, L, eps):
    """Block-causal ReLU linear attention evaluated exactly, token by token."""
    N, d = len(q), len(q[0])
    out = []
    for i in range(N):
        fq = [max(x, Fraction(0)) for x in q[i]]
        num = [Fraction(0)] * d
        den = Fraction(0)
        for j in range(N):
            if j // L > i // L:
                continue
            fk = [max(x, Fraction(0)) for x in k[j]]
            w = sum(a * b for a, b in zip(fk, fq))
            num = [n + w * vv for n, vv in zip(num, v[j])]
            den += w
        out.append([n / (den + eps) for n in num])
    return out


def test_exact_rational_small_integers():
    rng = np.random.default_rng(3)
    N, d, L = 7, 4, 3
    qi = rng.integers(-3, 4, (N, d))
    ki = rng.integers(-3, 4, (N, d))
    vi = rng.integers(-5, 6, (N, d))
    qi[:, 0] = np.abs(qi[:, 0]) + 1      # keep every normaliser positive
    ki[:, 0] = np.abs(ki[:, 0]) + 1
    eps = Fraction(1, 1000)
    ref = _fraction_reference([[Fraction(int(x)) for x in r] for r in qi],
                              [[Fraction(int(x)) for x in r] for r in ki],
                              [[Fraction(int(x)) for x in r] for r in vi], L, eps)
    got = oracle.forward(qi[None, :, None, :].astype(float), ki[None, :, None, :].astype(float),
                         vi[None, :, None, :].astype(float), 1, L, None, eps=float(eps))
    ref = np.array([[float(x) for x in r] for r in ref])
    assert np.allclose(got[0, :, 0], ref, rtol=1e-13, atol=1e-13)


def test_hand_worked_golden():
    """Values derived by hand in tests/golden/hand_example.json (see the derivation there)."""
    with open(os.path.join(HERE, "golden", "hand_example.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=float)[None, :, None, :]
    k = np.array(ex["k"], dtype=float)[None, :, None, :]
    v = np.array(ex["v"], dtype=float)[None, :, None, :]
    got = oracle.forward(q, k, v, 1, ex["block_tokens"], None, eps=ex["eps"])[0, :, 0]
    want = np.array([[Fraction(x).numerator / Fraction(x).denominator for x in row]
                     for row in ex["out"]])
    assert np.allclose(got, want, rtol=0, atol=1e-14)


# --------------------------------------- one block = the page's single-block formula (P2)

@pytest.mark.parametrize("rope", [None, ROPE_1D])
def test_single_block_equals_literal_formula(rope):
    q, k, v = rand_qkv(4, 2, 20, 3, 8)
    got = oracle.forward(q, k, v, 1, 20, rope, eps=1e-8)       # one block spans everything
    ref = oracle.lite_la_single_block(q, k, v, 1, rope, eps=1e-8)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# --------------------------------------------------------------------- invariants

def test_constant_v_gives_v_without_rope():
    """I1: RoPE off and v == c: out = c * D / (D + eps), i.e. c up to eps / D."""
    q, k, _ = rand_qkv(5, 1, 48, 2, 32)
    k[..., 0] = np.abs(k[..., 0]) + 0.5   # every token has a positive key sum ...
    q[..., 0] = np.abs(q[..., 0]) + 0.5   # ... and a positive query, so D > 0
    c = np.linspace(-2.0, 3.0, 32)
    v = np.broadcast_to(c, q.shape).copy()
    out = oracle.forward(q, k, v, 1, 16, None, eps=0.0)
    assert np.max(np.abs(out - v)) <= 1e-12 * np.max(np.abs(c))
    out_eps = oracle.forward(q, k, v, 1, 16, None, eps=1e-8)
    assert np.max(np.abs(out_eps - v)) <= 1e-6


def test_rope_breaks_constant_v_identity():
    """The numerator is rotated, the normaliser is not: with RoPE on, out != v in general."""
    q, k, _ = rand_qkv(6, 1, 48, 1, 8)
    k[..., 0] = np.abs(k[..., 0]) + 0.5
    q[..., 0] = np.abs(q[..., 0]) + 0.5
    v = np.ones_like(q)
    out = oracle.forward(q, k, v, 1, 16, ROPE_1D, eps=0.0)
    assert np.max(np.abs(out - v)) > 1e-3


@pytest.mark.parametrize("which", ["q", "k"])
def test_positive_scaling_invariance(which):
    """I2: phi is positively homogeneous, so scaling q or k by c > 0 cancels (eps = 0)."""
    q, k, v = rand_qkv(7, 1, 30, 2, 8)
    base = oracle.forward(q, k, v, 6, 2, ROPE_3D, eps=0.0)
    if which == "q":
        q = q * 3.7
    else:
        k = k * 0.21
    got = oracle.forward(q, k, v, 6, 2, ROPE_3D, eps=0.0)
    assert np.max(np.abs(got - base)) <= 1e-12 * np.max(np.abs(base))


def test_linear_in_v():
    """I3."""
    q, k, v1 = rand_qkv(8, 1, 30, 2, 8)
    _, _, v2 = rand_qkv(9, 1, 30, 2, 8)
    f = lambda v: oracle.forward(q, k, v, 6, 2, ROPE_3D)
    lhs = f(2.0 * v1 - 0.5 * v2)
    rhs = 2.0 * f(v1) - 0.5 * f(v2)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


def test_causality_later_blocks_do_not_leak():
    """I4: changing blocks > j leaves outputs of blocks <= j bit-identical."""
    q, k, v = rand_qkv(10, 1, 40, 2, 8)
    base = oracle.forward(q, k, v, 1, 10, ROPE_1D)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 20:] += 1.0
    k2[:, 20:] *= -3.0
    v2[:, 20:] = 7.0
    got = oracle.forward(q2, k2, v2, 1, 10, ROPE_1D)
    assert np.array_equal(got[:, :20], base[:, :20])
    assert not np.allclose(got[:, 20:], base[:, 20:])


def test_earlier_blocks_do_leak_forward():
    """Block-causal, not block-diagonal: changing block 0 changes every later block."""
    q, k, v = rand_qkv(11, 1, 30, 1, 8)
    base = oracle.forward(q, k, v, 1, 10, ROPE_1D)
    v2 = v.copy()
    v2[:, :10] += 1.0
    got = oracle.forward(q, k, v2, 1, 10, ROPE_1D)
    for s in (10, 20):
        assert not np.allclose(got[:, s:s + 10], base[:, s:s + 10])


def test_inside_block_is_not_token_causal():
    """Reading C1: a token sees later tokens of its own block."""
    q, k, v = rand_qkv(12, 1, 16, 1, 8)
    base = oracle.forward(q, k, v, 1, 16, None)
    v2 = v.copy()
    v2[:, 15] += 5.0
    got = oracle.forward(q, k, v2, 1, 16, None)
    assert not np.allclose(got[:, 0], base[:, 0])


@pytest.mark.parametrize("rope", [None, ROPE_1D])
def test_one_token_blocks_equal_running_sums(rope):
    """I5: blocks of one token == token-causal cumsum form."""
    q, k, v = rand_qkv(13, 2, 33, 2, 8)
    got = oracle.forward(q, k, v, 1, 1, rope)
    ref = oracle.token_causal_cumsum(q, k, v, 1, rope)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_zero_query_gives_zero_output():
    """Reading C10: phi(q) == 0 gives num = 0, den = eps, out = 0."""
    q, k, v = rand_qkv(14, 1, 12, 1, 8)
    q[:, 5] = -np.abs(q[:, 5])
    out = oracle.forward(q, k, v, 1, 4, ROPE_1D)
    assert np.all(out[:, 5] == 0.0)


# ---------------------------------------------------------------------- streaming

def test_streaming_equals_one_shot():
    """I6: 5 streamed blocks with the cache carried == one-shot over all frames."""
    tpf, bf, nblk = 6, 2, 5
    q, k, v = rand_qkv(15, 2, nblk * bf * tpf, 3, 8)
    ref = oracle.forward(q, k, v, tpf, bf, ROPE_3D)
    st = oracle.StreamState(2, 3, 8)
    L = bf * tpf
    outs = [oracle.stream_block(st, q[:, j * L:(j + 1) * L], k[:, j * L:(j + 1) * L],
                                v[:, j * L:(j + 1) * L], tpf, ROPE_3D) for j in range(nblk)]
    got = np.concatenate(outs, axis=1)
    assert st.frames_done == nblk * bf
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_streaming_without_save_leaves_cache():
    tpf, bf = 6, 2
    q, k, v = rand_qkv(16, 1, 3 * bf * tpf, 2, 8)
    L = bf * tpf
    st = oracle.StreamState(1, 2, 8)
    oracle.stream_block(st, q[:, :L], k[:, :L], v[:, :L], tpf, ROPE_3D)
    S0, z0, f0 = st.S.copy(), st.z.copy(), st.frames_done
    a = oracle.stream_block(st, q[:, L:2 * L], k[:, L:2 * L], v[:, L:2 * L], tpf, ROPE_3D, save=False)
    assert np.array_equal(st.S, S0) and np.array_equal(st.z, z0) and st.frames_done == f0
    b = oracle.stream_block(st, q[:, L:2 * L], k[:, L:2 * L], v[:, L:2 * L], tpf, ROPE_3D, save=True)
    assert np.array_equal(a, b)
    assert st.frames_done == f0 + bf


def test_global_time_shift_is_invisible():
    """I7: RoPE is relative, so one block read at frame offset 7 equals the same block at 0."""
    tpf, bf = 6, 3
    q, k, v = rand_qkv(17, 1, bf * tpf, 2, 8)
    st = oracle.StreamState(1, 2, 8)
    st.frames_done = 7
    got = oracle.stream_block(st, q, k, v, tpf, ROPE_3D)
    ref = oracle.forward(q, k, v, tpf, bf, ROPE_3D)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_streaming_with_reset_time_does_not_match():
    """I7 (negative): re-using t0 = 0 on every call is not the one-shot result."""
    tpf, bf, nblk = 6, 2, 3
    q, k, v = rand_qkv(18, 1, nblk * bf * tpf, 2, 8)
    ref = oracle.forward(q, k, v, tpf, bf, ROPE_3D)
    st = oracle.StreamState(1, 2, 8)
    L = bf * tpf
    outs = []
    for j in range(nblk):
        st.frames_done = 0
        outs.append(oracle.stream_block(st, q[:, j * L:(j + 1) * L], k[:, j * L:(j + 1) * L],
                                        v[:, j * L:(j + 1) * L], tpf, ROPE_3D))
    got = np.concatenate(outs, axis=1)
    assert np.max(np.abs(got - ref)) > 1e-6 * np.max(np.abs(ref))


def test_sampled_readout_matches_forward():
    """The sampled-output path used for full-size checks agrees with the full forward."""
    tpf, bf = 6, 2
    q, k, v = rand_qkv(19, 1, 5 * bf * tpf, 1, 8)
    ref = oracle.forward(q, k, v, tpf, bf, ROPE_3D)[0, :, 0]
    Sb, zb = oracle.block_states(k[0, :, 0], v[0, :, 0], tpf, bf, ROPE_3D)
    idx = np.array([0, 5, 13, 29, 47, 59])
    L = bf * tpf
    for n in idx:
        j = n // L
        got = oracle.readout_tokens(q[0, [n], 0], [n], Sb[j], zb[j], tpf, ROPE_3D)
        assert np.allclose(got[0], ref[n], rtol=1e-12, atol=1e-12)


def test_rel_err_metric():
    ref = np.array([3.0, -4.0])          # RMS = sqrt(12.5)
    got = np.array([3.5, -4.0])
    assert oracle.rel_err(got, ref) == pytest.approx(0.5 / np.sqrt(12.5))


# ------------------------------------------- first block longer than the others (N1)

@pytest.mark.parametrize("tpf,frames,block_frames,first,rope", [
    (6, 7, 2, 3, ROPE_3D),      # first block one frame longer: 3 + 2 + 2
    (6, 8, 2, 3, ROPE_3D),      # ... with a ragged last block: 3 + 2 + 2 + 1
    (1, 21, 4, 5, ROPE_1D),     # 1-D: 5 + 4 + 4 + 4 + 4
    (6, 5, 2, 1, ROPE_3D),      # first block shorter: 1 + 2 + 2
    (6, 3, 2, 4, ROPE_3D),      # first block covers the whole clip
])
def test_first_block_schedule_matches_brute_force(tpf, frames, block_frames, first, rope):
    q, k, v = rand_qkv(31, 2, frames * tpf, 2, 8)
    got = oracle.forward(q, k, v, tpf, block_frames, rope, first_block_frames=first)
    ref = oracle.brute_force(q, k, v, tpf, block_frames, rope, first_block_frames=first)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_first_block_schedule_bounds():
    assert oracle.block_bounds(17, 4, 5) == [(0, 5), (5, 9), (9, 13), (13, 17)]
    assert oracle.block_bounds(18, 4, 5) == [(0, 5), (5, 9), (9, 13), (13, 17), (17, 18)]
    assert oracle.block_bounds(3, 4, 5) == [(0, 3)]
    assert oracle.block_bounds(8, 4) == oracle.block_bounds(8, 4, 4) == [(0, 4), (4, 8)]


def test_first_block_equal_to_block_is_uniform():
    q, k, v = rand_qkv(32, 1, 7 * 6, 2, 8)
    a = oracle.forward(q, k, v, 6, 2, ROPE_3D)
    b = oracle.forward(q, k, v, 6, 2, ROPE_3D, first_block_frames=2)
    assert np.array_equal(a, b)


def test_first_block_spanning_clip_is_single_block_formula():
    """A first block holding every frame is the single-block formula as printed."""
    q, k, v = rand_qkv(33, 1, 4 * 6, 2, 8)
    got = oracle.forward(q, k, v, 6, 1, ROPE_3D, first_block_frames=4)
    ref = oracle.lite_la_single_block(q, k, v, 6, ROPE_3D)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_streaming_first_block_plus_one_equals_one_shot():
    """Streaming a 3-frame first block, then 2-frame blocks == one-shot with that schedule."""
    tpf, bf, first, frames = 6, 2, 3, 7
    q, k, v = rand_qkv(34, 2, frames * tpf, 2, 8)
    ref = oracle.forward(q, k, v, tpf, bf, ROPE_3D, first_block_frames=first)
    st = oracle.StreamState(2, 2, 8)
    outs, s = [], 0
    for f in (first, bf, bf):
        e = s + f * tpf
        outs.append(oracle.stream_block(st, q[:, s:e], k[:, s:e], v[:, s:e], tpf, ROPE_3D))
        s = e
    got = np.concatenate(outs, axis=1)
    assert st.frames_done == frames
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
