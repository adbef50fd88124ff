"""GPU parity of the fused prologue: a (B, N, 3, C) q|k|v input with the q/k
RMSNorm over C, through la_block_causal_forward_qkv and la_stream_block_qkv,
against the fp64 oracle (oracle.forward_qkv, oracle.qk_rms_norm)."""

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL_BF16, TOL_F32, device_inputs, err_bf16_out, to_f64_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NORM_EPS = 1e-6


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
    base = dict(index=110, B=2, H=3, head_dim=32, frames=11, tokens_per_frame=60, grid=(6, 10),
                block_frames=3, dtype="bf16", rope={"split": (8, 12, 12), "base": 10000.0},
                scale=1.0, outlier_frac=0.05, outlier_scale=8.0, name="small3d_qkv")
    base.update(kw)
    return base


def fused(cfg):
    """Host fp64 fused array and the device (B, N, 3, C) tensor of a workload."""
    w = W()
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    B, N, H, d = q.shape
    qkv = torch.stack([t.reshape(B, N, H * d) for t in (q, k, v)], dim=2).contiguous()
    del q, k, v
    host = w.fuse_qkv(*(w.to_f64(cfg, arrs[t]) for t in w.TENSORS))
    return host, qkv


def weights(cfg, norm):
    """(host, device) weights for norm in {"both", "q", "k", "none"}."""
    w = W()
    out = {}
    for which, key in (("q", "q_gamma"), ("k", "k_gamma")):
        if norm in ("both", which):
            g = w.draw_norm_weight(cfg, key)
            out[key] = (g.astype(np.float64), torch.from_numpy(g).to(DEV))
        else:
            out[key] = (None, None)
    return out


def score(out, ref):
    got = to_f64_torch(out)
    if out.dtype == torch.bfloat16:
        return err_bf16_out(got, ref), oracle.rel_err(got, ref)
    e = oracle.rel_err(got, ref)
    return e, e


def run_small(lavr, cfg, norm, out_dtype=None):
    host, qkv = fused(cfg)
    wts = weights(cfg, norm)
    rope = rope_for(lavr, cfg)
    out = lavr.block_causal_forward_qkv(qkv, cfg["H"], cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                        q_gamma=wts["q_gamma"][1], k_gamma=wts["k_gamma"][1],
                                        norm_eps=NORM_EPS, out_dtype=out_dtype,
                                        first_block_frames=cfg.get("first_block_frames"))
    torch.cuda.synchronize()
    ref = oracle.forward_qkv(host, cfg["H"], cfg["tokens_per_frame"], cfg["block_frames"],
                             W().oracle_rope(cfg), q_gamma=wts["q_gamma"][0], k_gamma=wts["k_gamma"][0],
                             norm_eps=NORM_EPS, first_block_frames=cfg.get("first_block_frames"))
    return out, ref, qkv, wts, rope


@pytest.mark.parametrize("norm", ["both", "q", "k", "none"])
@pytest.mark.parametrize("kw", [
    dict(),                                              # odd head count, ragged last block
    dict(frames=12, block_frames=4, H=1, B=1),
    dict(head_dim=64, H=2, rope={"split": (16, 24, 24), "base": 10000.0}),
    dict(frames=7, block_frames=2, first_block_frames=3),
    dict(rope={"split": (6, 14, 12), "base": 10000.0}),  # odd pair counts
])
def test_fused_small_bf16(lavr, kw, norm):
    cfg = small_cfg(**kw)
    say(f"case fused small {kw} norm={norm}")
    for out_dtype in (None, torch.float32):
        out, ref, *_ = run_small(lavr, cfg, norm, out_dtype)
        e, plain = score(out, ref)
        say(f"  out {out.dtype}: err {e:.3e} (plain {plain:.3e})")
        assert e <= TOL_BF16
        if out.dtype == torch.float32:
            assert plain <= 1e-3     # fp32 output: the arithmetic alone, far inside the bf16 bound


@pytest.mark.parametrize("kw", [
    dict(dtype="f32"),
    dict(dtype="f32", head_dim=64, H=2, rope={"split": (16, 24, 24), "base": 10000.0}),
    dict(dtype="f32", frames=64, tokens_per_frame=1, grid=(1, 1), block_frames=16, H=2,
         rope={"split": (32, 0, 0), "base": 10000.0}),  # 1-D RoPE
])
def test_fused_small_f32(lavr, kw):
    cfg = small_cfg(**kw)
    say(f"case fused small f32 {kw}")
    out, ref, *_ = run_small(lavr, cfg, "both")
    e = oracle.rel_err(to_f64_torch(out), ref)
    say(f"  err {e:.3e}")
    assert e <= TOL_F32


def test_fused_without_norm_matches_split_inputs(lavr):
    """With no weights the fused input is only a layout: the result equals the
    plain forward on the split tensors, within one bf16 step."""
    cfg = small_cfg(frames=12)
    say("case fused layout vs split")
    host, qkv = fused(cfg)
    rope = rope_for(lavr, cfg)
    B, N, _, C = qkv.shape
    H, d = cfg["H"], cfg["head_dim"]
    q, k, v = (qkv[:, :, i].contiguous().view(B, N, H, d) for i in range(3))
    a = lavr.block_causal_forward_qkv(qkv, H, 3, cfg["tokens_per_frame"], rope, out_dtype=torch.float32)
    b = lavr.block_causal_forward(q, k, v, 3, cfg["tokens_per_frame"], rope, out_dtype=torch.float32)
    torch.cuda.synchronize()
    diff = (a - b).abs().max().item() / b.float().pow(2).mean().sqrt().item()
    say(f"  max diff / rms {diff:.3e}")
    assert diff <= 1e-5


def test_fused_zero_query_row(lavr):
    """A token whose q row is zero reads out zero through the norm (q_hat = 0)."""
    cfg = small_cfg(frames=6, B=1)
    say("case fused zero query row")
    host, qkv = fused(cfg)
    qkv[0, 17, 0] = 0
    host[0, 17, 0] = 0.0
    wts = weights(cfg, "both")
    rope = rope_for(lavr, cfg)
    out = lavr.block_causal_forward_qkv(qkv, cfg["H"], 3, cfg["tokens_per_frame"], rope,
                                        q_gamma=wts["q_gamma"][1], k_gamma=wts["k_gamma"][1],
                                        norm_eps=NORM_EPS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(out[0, 17] == 0).item()
    ref = oracle.forward_qkv(host, cfg["H"], cfg["tokens_per_frame"], 3, W().oracle_rope(cfg),
                             q_gamma=wts["q_gamma"][0], k_gamma=wts["k_gamma"][0], norm_eps=NORM_EPS)
    assert oracle.rel_err(to_f64_torch(out), ref) <= 1e-3


def test_fused_streaming_equals_one_shot(lavr):
    cfg = small_cfg(frames=12)
    say("case fused streaming")
    host, qkv = fused(cfg)
    wts = weights(cfg, "both")
    rope = rope_for(lavr, cfg)
    tpf = cfg["tokens_per_frame"]
    L = 3 * tpf
    st = lavr.StreamState(cfg["B"], cfg["H"], device=DEV)
    parts = [st.step_qkv(qkv[:, j * L:(j + 1) * L].contiguous(), tpf, rope, q_gamma=wts["q_gamma"][1],
                         k_gamma=wts["k_gamma"][1], norm_eps=NORM_EPS, out_dtype=torch.float32)
             for j in range(4)]
    torch.cuda.synchronize()
    assert st.frames_done == 12
    got = torch.cat(parts, dim=1)
    ost = oracle.StreamState(cfg["B"], cfg["H"], cfg["head_dim"])
    ref = np.concatenate([oracle.stream_block_qkv(ost, host[:, j * L:(j + 1) * L], cfg["H"], tpf,
                                                  W().oracle_rope(cfg), q_gamma=wts["q_gamma"][0],
                                                  k_gamma=wts["k_gamma"][0], norm_eps=NORM_EPS)
                          for j in range(4)], axis=1)
    e = oracle.rel_err(to_f64_torch(got), ref)
    say(f"  err {e:.3e}")
    assert e <= 1e-3
    one = lavr.block_causal_forward_qkv(qkv, cfg["H"], 3, tpf, rope, q_gamma=wts["q_gamma"][1],
                                        k_gamma=wts["k_gamma"][1], norm_eps=NORM_EPS,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (one - got).abs().max().item() <= 1e-4 * one.pow(2).mean().sqrt().item()


def oracle_fused_heads(cfg, wts, heads):
    """fp64 oracle outputs of sampled (b, h) slices of a full-size workload: the
    norm over each token's whole C channels (oracle.qk_rms_norm on full rows,
    chunk by chunk), then oracle.forward_head on the head's channels."""
    w = W()
    N, H, d = w.n_tokens(cfg), cfg["H"], cfg["head_dim"]
    sel = {}
    for t in w.TENSORS:
        cols = {}
        for s0 in range(0, N, 65536):
            s1 = min(N, s0 + 65536)
            x = w.to_f64(cfg, w.draw(cfg, t, (s0, s1)))          # (B, n, H, d)
            x = x.reshape(cfg["B"], s1 - s0, H * d)
            g = wts["q_gamma"][0] if t == "q" else wts["k_gamma"][0] if t == "k" else None
            if g is not None:
                x = oracle.qk_rms_norm(x, g, NORM_EPS)
            for b, h in heads:
                cols.setdefault((b, h), []).append(x[b, :, h * d:(h + 1) * d])
        sel[t] = {bh: np.concatenate(v, axis=0) for bh, v in cols.items()}
    return {bh: oracle.forward_head(sel["q"][bh], sel["k"][bh], sel["v"][bh], cfg["tokens_per_frame"],
                                    cfg["block_frames"], w.oracle_rope(cfg))
            for bh in heads}


@pytest.mark.parametrize("name,heads", [
    ("clip480p_bf16", [(0, 0), (0, 35), (0, 69)]),
    ("minute_bf16", [(0, 0), (0, 41)]),
])
def test_fused_full_size(lavr, name, heads):
    """The workload the benchmark times, fused and normalised, on sampled heads."""
    cfg = W().workload(name)
    say(f"case fused full-size {name}")
    qkv = fused_device_only(cfg)
    wts = weights(cfg, "both")
    rope = rope_for(lavr, cfg)
    out = lavr.block_causal_forward_qkv(qkv, cfg["H"], cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                        q_gamma=wts["q_gamma"][1], k_gamma=wts["k_gamma"][1],
                                        norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    del qkv
    refs = oracle_fused_heads(cfg, wts, heads)
    worst = 0.0
    for (b, h), ref in refs.items():
        got = to_f64_torch(out[b, :, h])
        e = err_bf16_out(got, ref)
        say(f"  {name} b={b} h={h} err {e:.3e} (plain {oracle.rel_err(got, ref):.3e})")
        worst = max(worst, e)
    assert worst <= TOL_BF16
    assert torch.isfinite(out).all().item()
    del out
    torch.cuda.empty_cache()


def fused_device_only(cfg):
    """Device (B, N, 3, C) tensor of a large workload without keeping host copies."""
    _, (q, k, v) = device_inputs(cfg, DEV)
    B, N, H, d = q.shape
    qkv = torch.stack([t.reshape(B, N, H * d) for t in (q, k, v)], dim=2).contiguous()
    del q, k, v
    torch.cuda.empty_cache()
    return qkv
