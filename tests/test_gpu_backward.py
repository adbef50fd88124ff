"""GPU parity of the backward (la_block_causal_backward) against the fp64 oracle backward."""

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


def small_cfg(**kw):
    base = dict(index=200, B=2, H=3, head_dim=32, frames=11, tokens_per_frame=60, grid=(6, 10),
                block_frames=3, dtype="bf16", rope={"split": (8, 12, 12), "base": 10000.0},
                scale=1.0, outlier_frac=0.05, outlier_scale=8.0, name="bw_small")
    base.update(kw)
    return base


def rope_for(lavr, cfg):
    if cfg.get("rope") is None:
        return None
    return lavr.RopeTable(cfg["rope"]["split"], cfg["grid"], cfg["frames"], cfg["rope"]["base"], DEV)


def draw_dout(cfg, seed=7):
    """A seeded output gradient with the inputs' shape and dtype."""
    w = W()
    shape = (cfg["B"], w.n_tokens(cfg), cfg["H"], cfg["head_dim"])
    x = np.random.default_rng([seed, cfg["index"]]).standard_normal(shape, dtype=np.float32)
    arr = w.f32_to_bf16_bits(x) if cfg["dtype"] == "bf16" else x
    return arr, w.to_torch(cfg, arr, DEV)


def oracle_grads(cfg, arrs, garr):
    w = W()
    q, k, v = (w.to_f64(cfg, arrs[t]) for t in w.TENSORS)
    g = w.to_f64(cfg, garr)
    return oracle.backward(q, k, v, g, cfg["tokens_per_frame"], cfg["block_frames"], w.oracle_rope(cfg),
                           first_block_frames=cfg.get("first_block_frames"))


def run(lavr, cfg, grad_dtype):
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    garr, g = draw_dout(cfg)
    grads = lavr.block_causal_backward(q, k, v, g, cfg["block_frames"], cfg["tokens_per_frame"],
                                       rope_for(lavr, cfg), grad_dtype=grad_dtype,
                                       first_block_frames=cfg.get("first_block_frames"))
    torch.cuda.synchronize()
    return [to_f64_torch(x) for x in grads], oracle_grads(cfg, arrs, garr)


@pytest.mark.parametrize("kw", [
    dict(),                                              # B=2, H=3 (a half-empty head pair), ragged last block
    dict(frames=12, block_frames=4, H=2, B=1),
    dict(frames=40, block_frames=3, H=2, B=1, tokens_per_frame=48, grid=(6, 8)),   # many tiles
    dict(rope={"split": (6, 14, 12), "base": 10000.0}),  # odd pair counts
    dict(frames=11, block_frames=3, first_block_frames=4),
    dict(rope=None),
    dict(head_dim=64, H=2, rope={"split": (16, 24, 24), "base": 10000.0}),          # one head per workgroup
    dict(head_dim=64, H=1, B=1, frames=40, block_frames=3, tokens_per_frame=48, grid=(6, 8),
         rope={"split": (14, 26, 24), "base": 10000.0}),                             # many groups, odd pairs
    dict(head_dim=64, H=2, rope=None, frames=7, block_frames=2, first_block_frames=3),
    dict(B=6, H=2, frames=7, block_frames=2),                                        # many batch rows
])
@pytest.mark.parametrize("grad", ["f32", "bf16"])
def test_backward_small_bf16_inputs(lavr, kw, grad):
    cfg = small_cfg(**kw)
    say(f"case backward {kw} grads={grad}")
    got, ref = run(lavr, cfg, torch.float32 if grad == "f32" else torch.bfloat16)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        if grad == "f32":
            e = oracle.rel_err(a, b)
            say(f"  {name} rel err {e:.3e}")
            assert e <= TOL_BF16_IN_F32_GRAD
        else:
            e = err_bf16_out(a, b)
            say(f"  {name} rel err beyond bf16 rounding {e:.3e}")
            assert e <= TOL_BF16


@pytest.mark.parametrize("split", [(8, 12, 12), (6, 14, 12), (16, 24, 24), (14, 26, 24)])
def test_backward_f32_inputs(lavr, split):
    d = sum(split)
    cfg = small_cfg(dtype="f32", rope={"split": split, "base": 10000.0}, head_dim=d, H=3 if d == 32 else 2)
    say(f"case backward f32 split {split}")
    got, ref = run(lavr, cfg, torch.float32)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        e = oracle.rel_err(a, b)
        say(f"  {name} rel err {e:.3e}")
        assert e <= 10 * TOL_F32


@pytest.mark.parametrize("d", [32, 64])
def test_backward_zero_queries_and_one_token_blocks(lavr, d):
    cfg = small_cfg(dtype="f32", frames=40, tokens_per_frame=1, grid=(1, 1), block_frames=1,
                    rope={"split": (d, 0, 0), "base": 10000.0}, B=1, H=2, head_dim=d)
    say(f"case backward one-token blocks, zero queries, d={d}")
    arrs, _ = device_inputs(cfg, DEV)
    arrs["q"][:, 7] = -np.abs(arrs["q"][:, 7])
    w = W()
    q, k, v = (w.to_torch(cfg, arrs[t], DEV) for t in w.TENSORS)
    garr, g = draw_dout(cfg)
    dq, dk, dv = lavr.block_causal_backward(q, k, v, g, 1, 1, rope_for(lavr, cfg))
    torch.cuda.synchronize()
    ref = oracle_grads(cfg, arrs, garr)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = oracle.rel_err(to_f64_torch(a), b)
        say(f"  {name} rel err {e:.3e}")
        assert e <= 10 * TOL_F32
    assert torch.all(dq[:, 7] == 0).item()
    assert torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()


def test_autograd_binding(lavr):
    cfg = small_cfg(frames=9)
    say("case autograd binding")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    garr, g = draw_dout(cfg)
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = lavr.block_causal_attention(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope_for(lavr, cfg))
    (out.float() * g.float()).sum().backward()
    torch.cuda.synchronize()
    ref = oracle_grads(cfg, arrs, garr)
    for name, t, b in zip(("dq", "dk", "dv"), (q, k, v), ref):
        e = err_bf16_out(to_f64_torch(t.grad), b)
        say(f"  {name} rel err beyond bf16 rounding {e:.3e}")
        assert e <= TOL_BF16


def test_autograd_fp32_upstream_gradient(lavr):
    """fp32 output from bf16 inputs: autograd hands the backward an fp32 upstream
    gradient, which is not rounded to bf16; the gradients (returned in bf16, the
    inputs' dtype) match the oracle's with an fp32 dout."""
    cfg = small_cfg(frames=9)
    say("case autograd, fp32 output and upstream gradient")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    shape = (cfg["B"], W().n_tokens(cfg), cfg["H"], cfg["head_dim"])
    g32 = np.random.default_rng([9, cfg["index"]]).standard_normal(shape).astype(np.float32)
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = lavr.block_causal_attention(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope_for(lavr, cfg),
                                      out_dtype=torch.float32)
    assert out.dtype == torch.float32
    (out * torch.from_numpy(g32).to(DEV)).sum().backward()
    torch.cuda.synchronize()
    w = W()
    ref = oracle.backward(*(w.to_f64(cfg, arrs[t]) for t in w.TENSORS), g32.astype(np.float64),
                          cfg["tokens_per_frame"], cfg["block_frames"], w.oracle_rope(cfg))
    for name, t, b in zip(("dq", "dk", "dv"), (q, k, v), ref):
        assert t.grad.dtype == torch.bfloat16
        e = err_bf16_out(to_f64_torch(t.grad), b)
        say(f"  {name} rel err beyond bf16 rounding {e:.3e}")
        assert e <= TOL_BF16


@pytest.mark.parametrize("d", [32, 64])
def test_backward_from_forward_matches(lavr, d):
    """Reusing the forward's block prefixes gives the recomputing backward's
    gradients bit for bit."""
    cfg = small_cfg(frames=10, head_dim=d, H=3 if d == 32 else 2,
                    rope={"split": (8, 12, 12) if d == 32 else (16, 24, 24), "base": 10000.0},
                    first_block_frames=4)
    say(f"case backward from forward d={d}")
    _, (q, k, v) = device_inputs(cfg, DEV)
    _, g = draw_dout(cfg)
    rope = rope_for(lavr, cfg)
    tpf, bf, f0 = cfg["tokens_per_frame"], cfg["block_frames"], cfg["first_block_frames"]
    need = lavr.backward_workspace_bytes(cfg["B"], cfg["H"], cfg["frames"], tpf, bf, head_dim=d,
                                         first_block_frames=f0, rope=rope)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    lavr.block_causal_forward(q, k, v, bf, tpf, rope, workspace=ws, first_block_frames=f0)
    a = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, first_block_frames=f0, workspace=ws,
                                   from_forward=True)
    b = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, first_block_frames=f0)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_backward_from_forward_foreign_workspace(lavr, grad_dtype):
    """The training path checks that its workspace holds the block prefixes of a
    matching forward: a workspace that a forward of another block schedule, of
    other k and v tensors or of the fused (B, N, 3, C) input wrote, or that no
    forward wrote, gives gradients that are NaN everywhere (a value check, the
    call itself succeeds); the matching workspace gives the recomputing
    backward's gradients bit for bit."""
    cfg = small_cfg(frames=9)
    say(f"case backward from forward, foreign workspaces, {grad_dtype}")
    _, (q, k, v) = device_inputs(cfg, DEV)
    _, g = draw_dout(cfg)
    rope = rope_for(lavr, cfg)
    tpf, bf = cfg["tokens_per_frame"], cfg["block_frames"]
    B, H, d = cfg["B"], cfg["H"], cfg["head_dim"]
    need = max(lavr.backward_workspace_bytes(B, H, cfg["frames"], tpf, bf, head_dim=d, rope=rope),
               lavr.backward_workspace_bytes(B, H, cfg["frames"], tpf, 1, head_dim=d, rope=rope),
               lavr.qkv_workspace_bytes(B, H, cfg["frames"], tpf, bf, d, rope=rope))

    def train(ws):
        out = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, grad_dtype=grad_dtype, workspace=ws,
                                         from_forward=True)
        torch.cuda.synchronize()
        return out

    ref = lavr.block_causal_backward(q, k, v, g, bf, tpf, rope, grad_dtype=grad_dtype)
    ws = lavr.new_workspace(need, DEV)
    lavr.block_causal_forward(q, k, v, bf, tpf, rope, workspace=ws)
    assert all(torch.equal(x, y) for x, y in zip(train(ws), ref))

    foreign = {}
    w1 = torch.zeros(need, dtype=torch.uint8, device=DEV)          # no forward wrote it
    foreign["unwritten"] = w1
    w2 = lavr.new_workspace(need, DEV)                              # another block schedule
    lavr.block_causal_forward(q, k, v, 1, tpf, rope, workspace=w2)
    foreign["other schedule"] = w2
    w3 = lavr.new_workspace(need, DEV)                              # other k and v tensors, same values
    lavr.block_causal_forward(q, k.clone(), v.clone(), bf, tpf, rope, workspace=w3)
    foreign["other tensors"] = w3
    w4 = lavr.new_workspace(need, DEV)                              # the fused-input forward
    qkv = torch.stack([t.reshape(B, -1, H * d) for t in (q, k, v)], dim=2).contiguous()
    lavr.block_causal_forward_qkv(qkv, H, bf, tpf, rope, workspace=w4)
    foreign["fused input"] = w4
    for name, wsx in foreign.items():
        grads = train(wsx)
        say(f"  {name}: all NaN {[bool(torch.isnan(x).all()) for x in grads]}")
        assert all(bool(torch.isnan(x).all()) for x in grads), name
    # the matching workspace still works after the failed calls
    lavr.block_causal_forward(q, k, v, bf, tpf, rope, workspace=ws)
    assert all(torch.equal(x, y) for x, y in zip(train(ws), ref))


def test_backward_deterministic(lavr):
    cfg = small_cfg(frames=9)
    _, (q, k, v) = device_inputs(cfg, DEV)
    _, g = draw_dout(cfg)
    rope = rope_for(lavr, cfg)
    a = [x.clone() for x in lavr.block_causal_backward(q, k, v, g, 3, cfg["tokens_per_frame"], rope)]
    b = lavr.block_causal_backward(q, k, v, g, 3, cfg["tokens_per_frame"], rope)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("d", [32, 64])
def test_backward_eps_zero_with_padded_groups(lavr, d):
    """eps = 0 with every query positive (den > 0 for every real token): groups
    past a chunk's end must add nothing to G, not 0 * inf."""
    cfg = small_cfg(frames=7, head_dim=d, H=2, rope=None, dtype="f32")
    say(f"case backward eps=0, d={d}")
    arrs, _ = device_inputs(cfg, DEV)
    arrs["q"] = np.abs(arrs["q"]) + 0.01
    w = W()
    q, k, v = (w.to_torch(cfg, arrs[t], DEV) for t in w.TENSORS)
    garr, g = draw_dout(cfg)
    grads = lavr.block_causal_backward(q, k, v, g, cfg["block_frames"], cfg["tokens_per_frame"], None, eps=0.0)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all().item() for t in grads)
    ref = oracle.backward(*(w.to_f64(cfg, arrs[t]) for t in w.TENSORS), garr, cfg["tokens_per_frame"],
                          cfg["block_frames"], None, eps=0.0)
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        e = oracle.rel_err(to_f64_torch(a), b)
        say(f"  {name} rel err {e:.3e}")
        assert e <= 10 * TOL_F32


@pytest.mark.parametrize("name,heads", [("clip480p_bf16", [(0, 0), (0, 35), (0, 69)]),
                                        ("clip480p_d64_bf16", [(0, 0), (0, 17), (0, 34)]),
                                        ("minute_bf16", [(0, 0), (0, 41)])])   # the timed backward's shape
def test_backward_full_size(lavr, name, heads):
    w = W()
    cfg = w.workload(name)
    say(f"case backward full-size {name}")
    arrs, (q, k, v) = device_inputs(cfg, DEV)
    garr, g = draw_dout(cfg)
    rope = rope_for(lavr, cfg)
    dq, dk, dv = lavr.block_causal_backward(q, k, v, g, cfg["block_frames"], cfg["tokens_per_frame"],
                                            rope, grad_dtype=torch.float32)
    # the training path (the forward's block prefixes reused) gives the same bits
    ws = lavr.new_workspace(lavr.backward_workspace_bytes(cfg["B"], cfg["H"], cfg["frames"], cfg["tokens_per_frame"],
                                                          cfg["block_frames"], head_dim=cfg["head_dim"],
                                                          rope=rope), DEV)
    lavr.block_causal_forward(q, k, v, cfg["block_frames"], cfg["tokens_per_frame"], rope, workspace=ws)
    again = lavr.block_causal_backward(q, k, v, g, cfg["block_frames"], cfg["tokens_per_frame"], rope,
                                       grad_dtype=torch.float32, workspace=ws, from_forward=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip((dq, dk, dv), again))
    for b_, h in heads:
        ref = oracle.backward_head(*(w.to_f64(cfg, arrs[t][b_, :, h]) for t in w.TENSORS),
                                   w.to_f64(cfg, garr[b_, :, h]), cfg["tokens_per_frame"],
                                   cfg["block_frames"], w.oracle_rope(cfg))
        for nm, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            e = oracle.rel_err(to_f64_torch(t[b_, :, h]), r)
            say(f"  b={b_} h={h} {nm} rel err {e:.3e}")
            assert e <= TOL_BF16_IN_F32_GRAD
    del dq, dk, dv, again, q, k, v, g, ws
    torch.cuda.empty_cache()
