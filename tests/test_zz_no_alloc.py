"""The allocation-free forward (la_block_causal_forward_noalloc, the library's
fixed per-GPU workspace) against la_block_causal_forward with a caller
workspace: two calls in a row, the second on a smaller input, then a third on
the first shape with fp32 output; each result equals the caller-workspace
forward's bit for bit, and sampled heads match the oracle."""

import pytest
import torch

import oracle
from helpers import TOL_BF16, device_inputs, err_bf16_out, to_f64_torch

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


def run_case(lavr, cfg, out_dtype=None, heads=(0,)):
    w = W()
    say(f"case no-alloc forward {cfg['name']} frames={cfg['frames']} H={cfg['H']} out={out_dtype}")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    rope = lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], DEV)
    bf, tpf = cfg["block_frames"], cfg["tokens_per_frame"]
    ref = lavr.block_causal_forward(q, k, v, bf, tpf, rope, out_dtype=out_dtype)
    out = torch.empty_like(ref)
    got = lavr.block_causal_forward_noalloc(q, k, v, bf, tpf, rope, out=out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert got is out
    assert torch.equal(got, ref)
    for h in heads:
        r = oracle.forward_head(*(w.to_f64(cfg, arrs[t][0, :, h]) for t in w.TENSORS), tpf, bf, w.oracle_rope(cfg))
        g = to_f64_torch(got[0, :, h])
        e = err_bf16_out(g, r) if got.dtype == torch.bfloat16 else oracle.rel_err(g, r)
        say(f"  head {h}: err {e:.3e}")
        assert e <= TOL_BF16


def test_noalloc_forward_two_calls_then_smaller(lavr):
    w = W()
    big = w.workload("clip480p_bf16")                    # 12 frames, 70 heads
    small = w.workload("clip480p_bf16", frames=3)         # one block of 3 frames
    run_case(lavr, big, heads=(0, 69))
    run_case(lavr, small, heads=(5,))
    run_case(lavr, big, out_dtype=torch.float32, heads=(33,))
