"""GPU: the replay forward (la_block_causal_forward_replay) equals streaming the
same clip block by block, bit for bit ("Block Causal Linear Attention",
happyin.space, "Integration Contract" and "Acceptance Checks": streaming must
reproduce the one-shot result), and matches the fp64 oracle."""

import pytest
import torch

import oracle
from helpers import TOL_BF16, device_inputs, err_bf16_out, oracle_head, to_f64_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


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


def rope_for(lavr, cfg):
    if cfg.get("rope") is None:
        return None
    return lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], DEV)


def small_cfg(**kw):
    base = dict(index=120, B=2, H=3, head_dim=32, frames=12, tokens_per_frame=60, grid=(6, 10),
                block_frames=3, dtype="bf16", rope={"split": (8, 12, 12), "base": 10000.0},
                scale=1.0, outlier_frac=0.05, outlier_scale=8.0, name="replay3d")
    base.update(kw)
    return base


def streamed(lavr, cfg, q, k, v, rope, out_dtype):
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    L = bf * tpf
    st = lavr.StreamState(cfg["B"], cfg["H"], head_dim=cfg["head_dim"], device=DEV)
    outs = []
    for j in range(cfg["frames"] // bf):
        sl = slice(j * L, (j + 1) * L)
        outs.append(st.step(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(), tpf, rope,
                            out_dtype=out_dtype))
    return torch.cat(outs, dim=1)


@pytest.mark.parametrize("over", [
    dict(),                                            # B=2, H=3 (a half-empty head group), 3-D RoPE
    dict(head_dim=64, H=2, rope={"split": (16, 24, 24), "base": 10000.0}),
    dict(dtype="f32", H=2),
    dict(frames=32, block_frames=2, B=1, H=4),         # sixteen blocks of two frames
    dict(rope=None, H=2),
])
def test_replay_equals_streaming_small(lavr, over):
    cfg = small_cfg(**over)
    say(f"case replay small {over}")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    for out_dtype in (q.dtype, torch.float32):
        one = lavr.block_causal_forward_replay(q, k, v, bf, tpf, rope, out_dtype=out_dtype)
        got = streamed(lavr, cfg, q, k, v, rope, out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(one, got), f"replay differs from streaming ({out_dtype})"
    ref = oracle.forward(*(W().to_f64(cfg, arrs[t]) for t in W().TENSORS), tpf, bf, W().oracle_rope(cfg))
    e = oracle.rel_err(to_f64_torch(one), ref)
    say(f"  fp32 out err {e:.3e}")
    assert e <= (1e-5 if cfg["dtype"] == "f32" else 1e-4)


def test_replay_full_size_streaming_workload(lavr):
    """The 40-block streaming workload (B=2, 70 heads, 3 frames of 30 x 52): the
    replay forward over 120 frames, one launch of many rounds, equals the 40
    streamed calls (one round each) bit for bit; sampled heads match the oracle."""
    w = W()
    cfg = w.workload("stream_bf16")
    say("case replay full-size stream_bf16")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = rope_for(lavr, cfg)
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    one = lavr.block_causal_forward_replay(q, k, v, bf, tpf, rope)
    got = streamed(lavr, cfg, q, k, v, rope, q.dtype)
    torch.cuda.synchronize()
    assert torch.equal(one, got)
    for b, h in [(0, 7), (1, 66)]:
        ref = oracle_head(cfg, arrs, b, h)
        e = err_bf16_out(one[b, :, h].float().cpu().numpy(), ref)
        say(f"  head ({b}, {h}) err {e:.3e}")
        assert e <= TOL_BF16
