"""Tensors past 4 GiB: the minute workload extended to 672 frames (1,048,320
tokens x 70 heads, 4.7 GB per bf16 tensor), through the forward, the fused
(B, N, 3, C) input (14 GB) and the backward, on sampled heads against the fp64
oracle.  The kernels address a chunk or tile with 32-bit offsets from 64-bit
bases; this is where a wrong base would show."""

import numpy as np
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


def say(*a):
    print(*a, flush=True)


def test_beyond_4gib(lavr):
    from linear_attention_video_relu_amd import workloads as W
    cfg = W.workload("minute_bf16", frames=672)
    B, H, d, N = cfg["B"], cfg["H"], cfg["head_dim"], W.n_tokens(cfg)
    assert B * N * H * d * 2 > 4 * 2 ** 30
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    say(f"case beyond 4 GiB: N={N}")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], DEV)
    out = lavr.block_causal_forward(q, k, v, bf, tpf, rope)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (0, 69)]:
        e = err_bf16_out(to_f64_torch(out[b, :, h]), oracle_head(cfg, arrs, b, h))
        say(f"  forward b={b} h={h} err {e:.3e}")
        assert e <= TOL_BF16

    # the same values through the fused layout (no weights): same plan, same sums
    qkv = torch.stack([t.reshape(B, N, H * d) for t in (q, k, v)], dim=2).contiguous()
    fused = lavr.block_causal_forward_qkv(qkv, H, bf, tpf, rope)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    del qkv, fused
    torch.cuda.empty_cache()

    # backward, bf16 gradients, on one sampled head
    gen = torch.Generator(device=DEV)
    gen.manual_seed(3)
    g = torch.randn(q.shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    dq, dk, dv = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    h = 41
    qh, kh, vh = (W.to_f64(cfg, arrs[t][0, :, h]) for t in W.TENSORS)
    gh = g[0, :, h].double().cpu().numpy()
    ref = oracle.backward_head(qh, kh, vh, gh, tpf, bf, W.oracle_rope(cfg))
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = oracle.rel_err(to_f64_torch(got[0, :, h]), want)
        say(f"  backward {name} h={h} err {e:.3e}")
        assert e <= 1e-3
    assert all(torch.isfinite(t).all().item() for t in (out, dq, dk, dv))
