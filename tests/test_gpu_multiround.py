"""GPU parity of launches of many resident rounds, every element.

4 batch rows x 16 head groups x 32 blocks of 256 tokens make 2048 block-state
workgroups and 2048 readout workgroups, a few rounds of the chip's resident
slots, with a ragged last block (127 frames in blocks of 4) and a first block
of another length; head dims 32 and 64, bf16 and fp32 inputs, the backward,
and blocks streamed one at a time on top of the cache.  Every output element
is compared with the oracle (the full-size workloads compare sampled heads).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL_BF16, TOL_F32, device_inputs, err_bf16_out, to_f64_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL_BF16_IN_F32_GRAD = 1e-3     # bf16 inputs, fp32 gradients (hi/lo operand split inside)


@pytest.fixture(scope="module")
def lavr():
    import __graft_entry__
    __graft_entry__.ensure_built()
    from linear_attention_video_relu_amd import lavr
    return lavr


def W():
    from linear_attention_video_relu_amd import workloads
    return workloads


def say(*a):
    print(*a, flush=True)


def rounds_cfg(**kw):
    base = dict(index=300, B=4, H=32, head_dim=32, frames=127, tokens_per_frame=64, grid=(8, 8),
                block_frames=4, dtype="bf16", rope={"split": (8, 12, 12), "base": 10000.0},
                scale=1.0, outlier_frac=0.05, outlier_scale=8.0, name="rounds")
    base.update(kw)
    return base


def rope_for(lavr, cfg):
    return lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], DEV)


def oracle_fwd(cfg, arrs):
    w = W()
    return oracle.forward(*(w.to_f64(cfg, arrs[t]) for t in w.TENSORS), cfg["tokens_per_frame"],
                          cfg["block_frames"], w.oracle_rope(cfg),
                          first_block_frames=cfg.get("first_block_frames"))


@pytest.mark.parametrize("kw", [
    dict(),
    dict(first_block_frames=6),
    dict(head_dim=64, rope={"split": (16, 24, 24), "base": 10000.0}),
    dict(dtype="f32"),
])
def test_forward_many_rounds(lavr, kw):
    cfg = rounds_cfg(**kw)
    say(f"case many-round forward {kw}")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    ref = oracle_fwd(cfg, arrs)
    rope = rope_for(lavr, cfg)
    fb = cfg.get("first_block_frames")
    if cfg["dtype"] == "bf16":
        out32 = lavr.block_causal_forward(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                          first_block_frames=fb, out_dtype=torch.float32)
        out16 = lavr.block_causal_forward(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                          first_block_frames=fb)
        torch.cuda.synchronize()
        e32 = oracle.rel_err(to_f64_torch(out32), ref)
        e16 = err_bf16_out(to_f64_torch(out16), ref)
        say(f"  f32 out err {e32:.3e}, bf16 out err beyond rounding {e16:.3e}")
        assert e32 <= TOL_BF16 and e16 <= TOL_BF16
        # the bf16 output is the rounding of the fp32 one
        assert torch.equal(out16, out32.to(torch.bfloat16))
    else:
        out = lavr.block_causal_forward(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                        first_block_frames=fb)
        torch.cuda.synchronize()
        e = oracle.rel_err(to_f64_torch(out), ref)
        say(f"  f32 err {e:.3e}")
        assert e <= TOL_F32


def test_streaming_matches_many_round_launch(lavr):
    """Blocks streamed one at a time on top of the cache agree with the one-shot
    launch.  fp32 outputs: a streamed block is cut into more, shorter chunks
    (so that one block still fills the chip), so the two sum a block's state
    in other pieces and differ by rounding only; each is within ~1e-4 of the
    oracle (bf16 inputs, states and queries carried as hi + lo bf16 pairs), so
    they agree to 5e-4."""
    cfg = rounds_cfg(frames=128)
    say("case many-round one-shot vs streamed")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    bf, tpf = cfg["block_frames"], cfg["tokens_per_frame"]
    one = lavr.block_causal_forward(q, k, v, bf, tpf, rope, out_dtype=torch.float32)
    st = lavr.StreamState(cfg["B"], cfg["H"], device=DEV)
    parts = []
    L = bf * tpf
    for i in range(0, q.shape[1], L):
        parts.append(st.step(q[:, i:i + L].contiguous(), k[:, i:i + L].contiguous(),
                             v[:, i:i + L].contiguous(), tpf, rope, out_dtype=torch.float32))
    torch.cuda.synchronize()
    streamed = to_f64_torch(torch.cat(parts, dim=1))
    e = oracle.rel_err(streamed, to_f64_torch(one))
    say(f"  streamed vs one-shot rel err {e:.3e}")
    ref = oracle_fwd(cfg, arrs)
    e_s, e_o = oracle.rel_err(streamed, ref), oracle.rel_err(to_f64_torch(one), ref)
    say(f"  vs oracle: streamed {e_s:.3e}, one-shot {e_o:.3e}")
    assert e <= 5e-4
    assert e_s <= TOL_BF16 and e_o <= TOL_BF16


@pytest.mark.parametrize("kw", [dict(), dict(head_dim=64, rope={"split": (16, 24, 24), "base": 10000.0})])
def test_backward_many_rounds(lavr, kw):
    cfg = rounds_cfg(**kw)
    say(f"case many-round backward {kw}")
    w = W()
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    shape = (cfg["B"], w.n_tokens(cfg), cfg["H"], cfg["head_dim"])
    garr = w.f32_to_bf16_bits(np.random.default_rng([7, cfg["index"]]).standard_normal(shape, dtype=np.float32))
    g = w.to_torch(cfg, garr, DEV)
    rope = rope_for(lavr, cfg)
    grads = lavr.block_causal_backward(q, k, v, g, cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                       grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(*(w.to_f64(cfg, arrs[t]) for t in w.TENSORS), w.to_f64(cfg, garr),
                          cfg["tokens_per_frame"], cfg["block_frames"], w.oracle_rope(cfg))
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        e = oracle.rel_err(to_f64_torch(a), b)
        say(f"  {name} rel err {e:.3e}")
        assert e <= TOL_BF16_IN_F32_GRAD


def test_workspace_shared_across_shapes(lavr):
    """One workspace serves calls of different shapes in turn: a streamed block
    (one block, many short chunks), then a many-block forward and backward, then
    the streamed block again.  Every result equals the one from a fresh
    workspace bit for bit: no call depends on what an earlier call of another
    shape left in the workspace."""
    cfg = rounds_cfg(frames=32)
    say("case workspace shared across shapes")
    _, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    bf, tpf = cfg["block_frames"], cfg["tokens_per_frame"]
    B, H = cfg["B"], cfg["H"]
    g = torch.randn(q.shape, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV).to(q.dtype)
    L = bf * tpf
    blk = tuple(x[:, :L].contiguous() for x in (q, k, v))

    def streamed(ws):
        st = lavr.StreamState(B, H, device=DEV)
        return st.step(*blk, tpf, rope, out_dtype=torch.float32, workspace=ws)

    def one_shot(ws):
        out = lavr.block_causal_forward(q, k, v, bf, tpf, rope, out_dtype=torch.float32, workspace=ws)
        grads = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, grad_dtype=torch.float32, workspace=ws)
        return (out, *grads)

    need = max(lavr.backward_workspace_bytes(B, H, cfg["frames"], tpf, bf, rope=rope),
               lavr.workspace_bytes(B, H, bf, tpf, bf, rope=rope))
    ref_s = streamed(lavr.new_workspace(need, DEV))
    ref_o = one_shot(lavr.new_workspace(need, DEV))
    shared = lavr.new_workspace(need, DEV)
    got_s1 = streamed(shared)
    got_o = one_shot(shared)
    got_s2 = streamed(shared)
    torch.cuda.synchronize()
    assert torch.equal(got_s1, ref_s) and torch.equal(got_s2, ref_s)
    assert all(torch.equal(a, b) for a, b in zip(got_o, ref_o))


def test_rope_window_sized_workspace(lavr):
    """One token per frame, 1-D RoPE and blocks of 4096 frames: each block's
    pieces are cut short so that their rotary windows fit on chip.  A workspace
    of exactly the queried size (queried with the rotary description) runs, and
    the result matches the oracle."""
    cfg = dict(index=310, B=1, H=32, head_dim=32, frames=16384, tokens_per_frame=1, grid=(1, 1),
               block_frames=4096, dtype="bf16", rope={"split": (32, 0, 0), "base": 10000.0},
               scale=1.0, outlier_frac=0.0, outlier_scale=1.0, name="rope_window")
    say("case workspace sized with the rotary window (1-D RoPE, 4096-frame blocks)")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    bf, tpf = cfg["block_frames"], cfg["tokens_per_frame"]
    need = lavr.workspace_bytes(cfg["B"], cfg["H"], cfg["frames"], tpf, bf, rope=rope)
    assert need > lavr.workspace_bytes(cfg["B"], cfg["H"], cfg["frames"], tpf, bf)
    ws = lavr.new_workspace(need, DEV)[:need]
    out = lavr.block_causal_forward(q, k, v, bf, tpf, rope, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    e = oracle.rel_err(to_f64_torch(out), oracle_fwd(cfg, arrs))
    say(f"  f32 out err {e:.3e}")
    assert e <= TOL_BF16


def test_timed_forward_records_only_the_given_points(lavr):
    """la_block_causal_forward_timed writes the same output as the plain forward,
    bit for bit, whether it records all four points or only some (NULL entries
    are skipped), and the recorded points are in stream order."""
    import ctypes
    cfg = rounds_cfg(frames=32)
    say("case timed forward, all and some event points")
    _, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    bf, tpf = cfg["block_frames"], cfg["tokens_per_frame"]
    B, H, d = cfg["B"], cfg["H"], cfg["head_dim"]
    need = lavr.workspace_bytes(B, H, cfg["frames"], tpf, bf, rope=rope)
    ws = lavr.new_workspace(need, DEV)
    ref = lavr.block_causal_forward(q, k, v, bf, tpf, rope, workspace=ws)
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(4):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    code = lavr._dtype_code(q.dtype)
    try:
        for pick in ((0, 1, 2, 3), (2, 3)):
            out = torch.empty_like(q)
            marks = (ctypes.c_void_p * 4)(*(evs[i] if i in pick else None for i in range(4)))
            rc = lavr.lib.la_block_causal_forward_timed(
                *(ctypes.c_void_p(x.data_ptr()) for x in (q, k, v, out)), code, code, B, H, d,
                cfg["frames"], tpf, bf, 0, ctypes.byref(rope.desc), 1e-8,
                ctypes.c_void_p(ws.data_ptr()), need, stream, marks)
            assert rc == 0, lavr.status_string(rc)
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
            for a, b in zip(pick[:-1], pick[1:]):
                ms = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[a]),
                                               ctypes.c_void_p(evs[b])) == 0
                assert ms.value >= 0.0
    finally:
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))
