"""GPU checks of the calling convention: the library keeps no global state and
only enqueues kernels on the caller's stream, so calls on two streams at once
give the same bits as the same calls one after the other, and a one-shot
forward or backward captured into a HIP graph replays to the eager result.
Inputs are seeded; both sides of every comparison are the HIP path (the
numbers themselves are checked against the oracle in the parity tests)."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
B, H, D, FRAMES, TPF, BF = 2, 6, 32, 11, 60, 3      # ragged last block, 3 head pairs
SPLIT, GRID = (8, 12, 12), (6, 10)


@pytest.fixture(scope="module")
def lavr():
    import __graft_entry__
    __graft_entry__.ensure_built()
    from linear_attention_video_relu_amd import lavr
    return lavr


def say(*a):
    print(*a, flush=True)


def inputs(seed, n=3):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return [torch.randn(B, FRAMES * TPF, H, D, device=DEV, generator=g).to(torch.bfloat16) for _ in range(n)]


def workspace(lavr, backward=False):
    f = lavr.backward_workspace_bytes if backward else lavr.workspace_bytes
    return torch.zeros(f(B, H, FRAMES, TPF, BF, head_dim=D), dtype=torch.uint8, device=DEV)


def test_two_streams_at_once(lavr):
    say("case forward on two streams at once")
    rope = lavr.RopeTable(SPLIT, GRID, FRAMES, 10000.0, DEV)
    xa, xb = inputs(1), inputs(2)
    ref_a = lavr.block_causal_forward(*xa, BF, TPF, rope)
    ref_b = lavr.block_causal_forward(*xb, BF, TPF, rope)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    wa, wb = workspace(lavr), workspace(lavr)
    oa, ob = torch.empty_like(ref_a), torch.empty_like(ref_b)
    s1.wait_stream(torch.cuda.current_stream(DEV))
    s2.wait_stream(torch.cuda.current_stream(DEV))
    for _ in range(4):
        with torch.cuda.stream(s1):
            lavr.block_causal_forward(*xa, BF, TPF, rope, out=oa, workspace=wa)
        with torch.cuda.stream(s2):
            lavr.block_causal_forward(*xb, BF, TPF, rope, out=ob, workspace=wb)
    torch.cuda.synchronize()
    assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


def test_forward_graph_replays(lavr):
    """Capture one forward, then replay it on new inputs copied into the captured
    buffers, with eager work and synchronisation between replays."""
    say("case forward captured in a graph")
    rope = lavr.RopeTable(SPLIT, GRID, FRAMES, 10000.0, DEV)
    q, k, v = inputs(3)
    ws = workspace(lavr)
    out = torch.empty_like(q)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):       # warm-up outside the capture
        lavr.block_causal_forward(q, k, v, BF, TPF, rope, out=out, workspace=ws)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lavr.block_causal_forward(q, k, v, BF, TPF, rope, out=out, workspace=ws)
    torch.cuda.synchronize()
    for seed in (4, 5, 6):
        nq, nk, nv = inputs(seed)
        ref = lavr.block_causal_forward(nq, nk, nv, BF, TPF, rope)   # eager, its own workspace
        torch.cuda.synchronize()
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay seed {seed}: equal {torch.equal(out, ref)}")
        assert torch.equal(out, ref)


def test_backward_graph_replays(lavr):
    """The training-path backward (forward and backward both captured) replays to
    the eager gradients."""
    say("case forward + backward captured in a graph")
    rope = lavr.RopeTable(SPLIT, GRID, FRAMES, 10000.0, DEV)
    q, k, v, g = inputs(7, 4)
    ws = workspace(lavr, backward=True)
    out = torch.empty_like(q)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        lavr.block_causal_forward(q, k, v, BF, TPF, rope, out=out, workspace=ws)
        lavr.block_causal_backward(q, k, v, g, BF, TPF, rope, grad_dtype=torch.float32, workspace=ws,
                                   from_forward=True)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lavr.block_causal_forward(q, k, v, BF, TPF, rope, out=out, workspace=ws)
        grads = lavr.block_causal_backward(q, k, v, g, BF, TPF, rope, grad_dtype=torch.float32,
                                           workspace=ws, from_forward=True)
    torch.cuda.synchronize()
    for seed in (8, 9):
        nq, nk, nv, ng = inputs(seed, 4)
        ref = lavr.block_causal_backward(nq, nk, nv, ng, BF, TPF, rope, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        for dst, src in zip((q, k, v, g), (nq, nk, nv, ng)):
            dst.copy_(src)
        for t in grads:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        same = [torch.equal(a, b) for a, b in zip(grads, ref)]
        say(f"  replay seed {seed}: dq, dk, dv equal {same}")
        assert all(same)
