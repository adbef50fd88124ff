"""GPU parity of the cached temporal convolution (la_temporal_conv and
la_temporal_conv_stream_block) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL_BF16, TOL_F32, err_bf16_out, to_f64_torch

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


def inputs(seed, B, F, P, Ch, kt, dtype, bias=True):
    """x drawn through the seeded workload recipe, w and bias seeded float32."""
    w_ = W()
    x32, w, b = w_.draw_conv(seed, B, F * P, Ch, kt)
    x = torch.from_numpy(x32).to(DEV).to(dtype)
    host = x.double().cpu().numpy()                   # exact values of the dtype
    wt = torch.from_numpy(w).to(DEV)
    bt = torch.from_numpy(b).to(DEV) if bias else None
    return host, x, w.astype(np.float64), wt, (b.astype(np.float64) if bias else None), bt


def score(out, ref):
    got = to_f64_torch(out)
    return err_bf16_out(got, ref) if out.dtype == torch.bfloat16 else oracle.rel_err(got, ref)


@pytest.mark.parametrize("kt", [3, 2])
@pytest.mark.parametrize("shape", [
    dict(B=2, F=11, P=60, Ch=64, bf=3, f0=0),         # ragged last block
    dict(B=1, F=8, P=7, Ch=8, bf=8, f0=0),            # one block, one channel piece
    dict(B=1, F=13, P=33, Ch=136, bf=4, f0=5),        # first block of other length, odd pieces
    dict(B=3, F=5, P=1, Ch=2240, bf=1, f0=0),         # one-frame blocks, one token per frame
    dict(B=2, F=70, P=5, Ch=16, bf=4, f0=5),          # long call: 4 frame segments, starts mid-block
    dict(B=1, F=64, P=3, Ch=24, bf=7, f0=0),          # 4 segments of 16 frames over 7-frame blocks
])
@pytest.mark.parametrize("dtype,out_dtype", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                             (torch.float32, torch.float32)])
def test_tconv_small(lavr, kt, shape, dtype, out_dtype):
    B, F, P, Ch, bf, f0 = (shape[k] for k in ("B", "F", "P", "Ch", "bf", "f0"))
    say(f"case tconv kt={kt} {shape} {dtype}->{out_dtype}")
    host, x, w, wt, b, bt = inputs(1 + kt, B, F, P, Ch, kt, dtype)
    out = lavr.temporal_conv(x, wt, P, bf, bias=bt, first_block_frames=f0 or None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.temporal_conv(host, w, P, bf, bias=b, first_block_frames=f0 or None)
    e = score(out, ref)
    say(f"  err {e:.3e}")
    assert e <= (TOL_F32 if dtype == torch.float32 else TOL_BF16)
    if dtype == torch.bfloat16 and out_dtype == torch.float32:
        assert e <= 1e-6                             # three fp32 products per output


def test_tconv_no_bias_and_zero_input(lavr):
    host, x, w, wt, _, _ = inputs(7, 1, 6, 10, 32, 3, torch.bfloat16, bias=False)
    out = lavr.temporal_conv(x, wt, 10, 2, out_dtype=torch.float32)
    zero = lavr.temporal_conv(torch.zeros_like(x), wt, 10, 2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert oracle.rel_err(to_f64_torch(out), oracle.temporal_conv(host, w, 10, 2)) <= 1e-6
    assert torch.all(zero == 0).item()


@pytest.mark.parametrize("kt", [3, 2])
def test_tconv_streaming_equals_one_shot(lavr, kt):
    """Blocks streamed with a cache, each run twice with save=0 first, equal the
    one-shot result bit for bit, and the cache holds the last committed frame."""
    B, P, Ch, bf, nblk = 2, 30, 96, 3, 5
    say(f"case tconv streaming kt={kt}")
    host, x, w, wt, b, bt = inputs(11, B, bf * nblk, P, Ch, kt, torch.bfloat16)
    one = lavr.temporal_conv(x, wt, P, bf, bias=bt)
    st = lavr.ConvState(B, P, Ch, torch.bfloat16, DEV)
    L = bf * P
    parts = []
    for j in range(nblk):
        xb = x[:, j * L:(j + 1) * L].contiguous()
        trial = st.step(xb, wt, bias=bt, save=False)
        parts.append(st.step(xb, wt, bias=bt, save=True))
        torch.cuda.synchronize()
        assert torch.equal(trial, parts[-1])
    got = torch.cat(parts, dim=1)
    assert st.frames_done == bf * nblk
    assert torch.equal(got, one)
    assert torch.equal(st.last, x.view(B, bf * nblk, P, Ch)[:, -1])
    ref = oracle.temporal_conv(host, w, P, bf, bias=b)
    assert score(got, ref) <= TOL_BF16


def test_tconv_full_size(lavr):
    """The bench workload: 240 frames of 30 x 52 tokens, 2240 channels, blocks of
    8 frames; sampled token rows against the oracle, computed from the frames
    they need."""
    B, F, P, Ch, bf, kt = 1, 240, 1560, 2240, 8, 3
    say("case tconv full size")
    w_ = W()
    x32, w, b = w_.draw_conv(40, B, F * P, Ch, kt)
    x = torch.from_numpy(x32).to(DEV).to(torch.bfloat16)
    del x32
    out = lavr.temporal_conv(x, torch.from_numpy(w).to(DEV), P, bf, bias=torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    xs = x.view(B, F, P, Ch)
    rng = np.random.default_rng(5)
    frames = [0, 7, 8, 100, 119, 120, 239] + list(rng.integers(0, F, 5))
    worst = 0.0
    for f in frames:
        j0 = (f // bf) * bf                        # first frame of its block
        lo = max(j0 - 1, 0)
        hi = min(j0 + bf, F)
        seg = xs[:, lo:hi].double().cpu().numpy()
        cache = seg[:, 0] if j0 > 0 else None
        blk = seg[:, 1:] if j0 > 0 else seg
        ref = oracle.temporal_conv_block(blk, w.astype(np.float64), cache, b.astype(np.float64))[:, f - j0]
        got = out.view(B, F, P, Ch)[:, f].double().cpu().numpy()
        e = err_bf16_out(got, ref)
        worst = max(worst, e)
    say(f"  worst sampled-frame err {worst:.3e}")
    assert worst <= TOL_BF16
    assert torch.isfinite(out).all().item()
