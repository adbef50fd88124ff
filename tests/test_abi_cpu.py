"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes its buffers, and rejects bad arguments with the right
status before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lavr():
    import __graft_entry__
    __graft_entry__.ensure_built()
    from linear_attention_video_relu_amd import lavr
    return lavr


def header_functions():
    with open(os.path.join(ROOT, "include", "la_vr.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(lavr):
    names = header_functions()
    assert set(names) == set(lavr.EXPORTS), names
    raw = ctypes.CDLL(lavr.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_calls_only_enqueue_kernels():
    """The header promises that a call enqueues kernels only (so it can run under
    HIP graph capture): the library sources make no allocation, memset, copy or
    synchronisation call.  Only the timed forward takes events, bound to its
    kernels' dispatches by the one launch macro; no event is recorded between
    kernels."""
    src_dir = os.path.join(ROOT, "linear_attention_video_relu_amd", "csrc")
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipMemset\w*|hipMemcpy\w*|"
                        r"hipDeviceSynchronize|hipStreamSynchronize|hipEventSynchronize|hipStreamCreate\w*)\s*\(")
    events = ext = 0
    for name in sorted(os.listdir(src_dir)):
        if not name.endswith((".hip", ".cpp", ".h")):
            continue
        with open(os.path.join(src_dir, name)) as f:
            code = re.sub(r"//[^\n]*|/\*.*?\*/", "", f.read(), flags=re.S)
        assert not banned.search(code), (name, banned.search(code).group(0))
        events += len(re.findall(r"\bhipEventRecord\w*\s*\(", code))
        ext += len(re.findall(r"\bhipExtLaunchKernel\w*\s*\(", code))
    assert events == 0 and ext == 1


def test_version_and_status_strings(lavr):
    assert lavr.lib.la_version() == b"0.5.0"
    for code in range(5):
        assert lavr.status_string(code).startswith("LA_")
    assert "unknown" in lavr.status_string(99)


def test_rope_table_bytes(lavr):
    assert lavr.lib.rope_table_bytes(8, 12, 12, 240, 30, 52) == 8 * (240 * 4 + 30 * 6 + 52 * 6)
    assert lavr.lib.rope_table_bytes(32, 0, 0, 256, 1, 1) == 8 * 256 * 16
    assert lavr.lib.rope_table_bytes(7, 13, 12, 10, 30, 52) == 0     # odd section
    assert lavr.lib.rope_table_bytes(8, 12, 12, 0, 30, 52) == 0      # no frames


def test_workspace_bytes(lavr):
    # minute config: 30 blocks of 12480 tokens, 70 heads
    n = lavr.workspace_bytes(1, 70, 240, 1560, 8)
    rec = (32 * 32 + 32) * 4
    assert n >= 70 * 30 * rec            # at least the per-block prefix states
    assert n < 0.05 * 1 * 374400 * 70 * 32 * 2 * 4   # small next to q, k, v, out
    assert lavr.lib.la_workspace_bytes(1, 70, 48, 240, 1560, 8, 0, None) == 0   # head_dim 48 not built
    # the same channels as 35 heads of 64: records of 64 x 64 + 64 floats
    n64 = lavr.lib.la_workspace_bytes(1, 35, 64, 240, 1560, 8, 0, None)
    assert n64 >= 35 * 30 * (64 * 64 + 64) * 4
    assert lavr.lib.la_workspace_bytes(0, 70, 32, 240, 1560, 8, 0, None) == 0
    assert lavr.lib.la_workspace_bytes(1, 70, 32, 240, 1560, 8, -1, None) == 0  # bad first block
    # a first block of 9 frames: 1 + ceil(231 / 8) = 30 blocks, workspace at least as large
    assert lavr.workspace_bytes(1, 70, 240, 1560, 8, first_block_frames=9) >= 70 * 30 * rec
    assert lavr.workspace_bytes(1, 70, 240, 1560, 8, first_block_frames=8) == n


FAKE = 0x100000          # 16- and 256-byte aligned, never dereferenced: every call below fails validation


def call_forward(lavr, **kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, out=FAKE + 0x3000000,
                in_dt=lavr.LA_BF16, out_dt=lavr.LA_BF16, B=1, H=2, d=32, frames=4, tpf=6,
                bf=2, f0=0, rope=None, eps=1e-8, ws=FAKE + 0x4000000, ws_bytes=1 << 20)
    args.update(kw)
    return lavr.lib.la_block_causal_forward(
        ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["v"]),
        ctypes.c_void_p(args["out"]), args["in_dt"], args["out_dt"], args["B"], args["H"],
        args["d"], args["frames"], args["tpf"], args["bf"], args["f0"], args["rope"], args["eps"],
        ctypes.c_void_p(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1),                      # null pointer
    (dict(k=FAKE + 2), 1),               # misaligned
    (dict(B=0), 1),
    (dict(H=-1), 1),
    (dict(frames=0), 1),
    (dict(tpf=0), 1),
    (dict(bf=0), 1),
    (dict(f0=-2), 1),                    # negative first-block length
    (dict(d=48), 2),                     # head dims other than 32 and 64 are not built
    (dict(in_dt=7), 1),
    (dict(eps=-1.0), 1),
    (dict(eps=float("inf")), 1),
    (dict(ws_bytes=16), 1),              # workspace too small
    (dict(ws=FAKE + 8), 1),              # workspace misaligned
    (dict(out=FAKE + 0x1000000 + 64), 1),  # out overlaps k
])
def test_forward_rejects_bad_arguments(lavr, kw, code):
    assert call_forward(lavr, **kw) == code


def test_size_limits(lavr):
    """The documented maxima: 2^30 tokens per batch row, B <= 65535, B * H <= 2^24."""
    assert lavr.lib.la_workspace_bytes(1, 2, 32, 1 << 20, 1024, 2, 0, None) > 0          # N = 2^30 plans
    assert lavr.lib.la_workspace_bytes(1, 2, 32, (1 << 20) + 1, 1024, 2, 0, None) == 0   # one frame more does not
    assert call_forward(lavr, frames=(1 << 20) + 1, tpf=1024) == lavr.LA_ERR_UNSUPPORTED
    # at the maximum the plan is fine and the call fails only on the small workspace
    assert call_forward(lavr, frames=1 << 20, tpf=1024) == lavr.LA_ERR_INVALID_ARG
    assert call_forward(lavr, B=65536) == lavr.LA_ERR_UNSUPPORTED
    assert call_forward(lavr, B=4096, H=4097) == lavr.LA_ERR_UNSUPPORTED
    # N * tokens_per_frame reaches 2^42 (N = 2^27 tokens in frames of 2^15)
    assert lavr.lib.la_workspace_bytes(1, 2, 32, (1 << 12) - 1, 1 << 15, 2, 0, None) > 0
    assert lavr.lib.la_workspace_bytes(1, 2, 32, 1 << 12, 1 << 15, 2, 0, None) == 0


def rope_desc(lavr, **kw):
    r = lavr.LaRope()
    d = dict(table=FAKE + 0x5000000, d_t=8, d_h=12, d_w=12, max_frames=4, grid_h=2, grid_w=3)
    d.update(kw)
    for k_, v_ in d.items():
        setattr(r, k_, v_)
    return r


@pytest.mark.parametrize("kw", [
    dict(d_t=7, d_h=13),                 # odd section
    dict(d_t=8, d_h=12, d_w=10),         # sections do not sum to head_dim
    dict(grid_h=3),                      # grid does not match tokens per frame
    dict(max_frames=3),                  # frames past the table
    dict(table=FAKE + 0x5000000 + 4),    # misaligned table
])
def test_forward_rejects_bad_rope(lavr, kw):
    r = rope_desc(lavr, **kw)
    assert call_forward(lavr, rope=ctypes.byref(r)) == lavr.LA_ERR_INVALID_ARG


def test_replay_workspace_and_whole_blocks(lavr):
    """The replay forward plans every block as a streamed call of one block: on a
    clip of many blocks that is more, shorter chunks (a larger workspace than the
    plain forward's), and the clip must be whole blocks."""
    r = rope_desc(lavr, max_frames=120, grid_h=30, grid_w=52)
    plain = lavr.lib.la_workspace_bytes(2, 70, 32, 120, 1560, 3, 0, ctypes.byref(r))
    replay = lavr.lib.la_replay_workspace_bytes(2, 70, 32, 120, 1560, 3, ctypes.byref(r))
    assert replay > plain > 0
    # one block: the replay plan is the streamed one
    one = lavr.lib.la_workspace_bytes(2, 70, 32, 3, 1560, 3, 0, ctypes.byref(r))
    assert lavr.lib.la_replay_workspace_bytes(2, 70, 32, 3, 1560, 3, ctypes.byref(r)) == one
    assert lavr.lib.la_replay_workspace_bytes(2, 70, 32, 119, 1560, 3, ctypes.byref(r)) == 0
    assert lavr.lib.la_replay_workspace_bytes(2, 70, 32, 120, 1560, 0, ctypes.byref(r)) == 0
    rc = lavr.lib.la_block_causal_forward_replay(
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 0x1000000), ctypes.c_void_p(FAKE + 0x2000000),
        ctypes.c_void_p(FAKE + 0x3000000), lavr.LA_BF16, lavr.LA_BF16, 1, 2, 32, 5, 6, 2, None, 1e-8,
        ctypes.c_void_p(FAKE + 0x4000000), 1 << 30, None)
    assert rc == lavr.LA_ERR_INVALID_ARG          # 5 frames are not whole blocks of 2


def test_rope_table_pair_count_fits_32_bits(lavr):
    """The kernels index the rotary table's (cos, sin) pairs with 32-bit integers: a
    description of 2^31 pairs or more is refused by the planner (workspace query 0)."""
    def ws(max_frames):
        r = rope_desc(lavr, max_frames=max_frames, d_t=16, d_h=8, d_w=8)
        return lavr.lib.la_workspace_bytes(1, 2, 32, 4, 6, 2, 0, ctypes.byref(r))
    # 8 t pairs per frame plus 2 * 4 + 3 * 4 h/w pairs
    assert ws(1 << 27) > 0                                   # 2^30 + 20 pairs
    assert ws(((1 << 31) - 20) // 8) > 0                     # just below 2^31
    assert ws(((1 << 31) - 20) // 8 + 1) == 0                # 2^31 + 4
    assert ws(1 << 28) == 0


def test_forward_rejects_shared_memory(lavr):
    """The workspace may not share bytes with the tensors or the rotary table,
    nor the output with the table (checked before anything is launched)."""
    r = rope_desc(lavr)                  # table at FAKE + 0x5000000
    rp = ctypes.byref(r)
    assert call_forward(lavr, ws=FAKE, rope=rp) == 1                      # workspace over q
    assert call_forward(lavr, ws=FAKE + 0x3000000, rope=rp) == 1          # workspace over out
    assert call_forward(lavr, ws=FAKE + 0x5000000 - 256, rope=rp) == 1    # workspace over the table
    assert call_forward(lavr, out=FAKE + 0x5000000 - 64, rope=rp) == 1    # out over the table


def test_stream_block_rejects_shared_memory(lavr):
    st = lavr.LaState()
    st.S, st.z, st.B, st.H, st.head_dim, st.frames_done = FAKE, FAKE + 0x100000, 2, 4, 32, 0
    f = lavr.lib.la_stream_block
    vp = ctypes.c_void_p
    q, k, v, out = (FAKE + i * 0x1000000 for i in range(1, 5))
    ws = FAKE + 0x6000000

    def call(**kw):
        a = dict(q=q, k=k, v=v, out=out, ws=ws)
        a.update(kw)
        return f(ctypes.byref(st), vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["out"]), 1, 1, 2, 4, 32, 3, 6,
                 None, 1e-8, 1, vp(a["ws"]), 1 << 24, None)

    assert call(out=FAKE) == 1                   # out over the carried S
    assert call(ws=FAKE + 0x100000) == 1         # workspace over the carried z
    assert call(q=FAKE + 0x100000 - 64) == 1     # q over the carried S and z
    assert st.frames_done == 0


def test_backward_and_qkv_reject_shared_memory(lavr):
    assert call_backward(lavr, ws=FAKE + 0x3000000) == 1      # workspace over dout
    assert call_backward(lavr, ws=FAKE + 0x1000000) == 1      # workspace over k
    assert call_forward_qkv(lavr, ws=FAKE) == 1               # workspace over the fused rows
    assert call_forward_qkv(lavr, ws=FAKE + 0x5000000) == 1   # workspace over the q weights


def test_rope_table_build_rejects(lavr):
    r = lavr.LaRope()
    f = lavr.lib.rope_table_build
    ok = dict(dt=8, dh=12, dw=12, mf=4, gh=2, gw=3)
    assert f(ctypes.byref(r), ctypes.c_void_p(FAKE), 8, 32, 8, 12, 12, 4, 2, 3, 10000.0, None) == 1   # bytes
    assert f(ctypes.byref(r), ctypes.c_void_p(FAKE), 1 << 20, 48, 16, 16, 16, 4, 2, 3, 10000.0, None) == 2
    assert f(ctypes.byref(r), ctypes.c_void_p(FAKE), 1 << 20, 64, 8, 12, 12, 4, 2, 3, 10000.0, None) == 1
    assert f(ctypes.byref(r), ctypes.c_void_p(FAKE), 1 << 20, 32, 8, 12, 12, 4, 2, 3, -1.0, None) == 1
    assert f(ctypes.byref(r), ctypes.c_void_p(0), 1 << 20, 32, 8, 12, 12, 4, 2, 3, 10000.0, None) == 1
    assert f(None, ctypes.c_void_p(FAKE), 1 << 20, 32, 8, 12, 12, 4, 2, 3, 10000.0, None) == 1
    assert ok


def test_stream_block_state_checks(lavr):
    st = lavr.LaState()
    st.S, st.z, st.B, st.H, st.head_dim, st.frames_done = FAKE, FAKE + 0x100000, 2, 4, 32, 0
    f = lavr.lib.la_stream_block
    p = [ctypes.c_void_p(FAKE + i * 0x1000000) for i in range(1, 5)]
    ws = ctypes.c_void_p(FAKE + 0x6000000)
    # batch / heads / head_dim that differ from the state's
    assert f(ctypes.byref(st), *p, 1, 1, 1, 4, 32, 3, 6, None, 1e-8, 1, ws, 1 << 24, None) == 3
    assert f(ctypes.byref(st), *p, 1, 1, 2, 5, 32, 3, 6, None, 1e-8, 1, ws, 1 << 24, None) == 3
    # small workspace
    assert f(ctypes.byref(st), *p, 1, 1, 2, 4, 32, 3, 6, None, 1e-8, 1, ws, 64, None) == 1
    # frames past the rotary table at this offset
    st.frames_done = 3
    r = rope_desc(lavr, max_frames=5)
    assert f(ctypes.byref(st), *p, 1, 1, 2, 4, 32, 3, 6, ctypes.byref(r), 1e-8, 1, ws, 1 << 24, None) == 1
    st.S = 0
    assert f(ctypes.byref(st), *p, 1, 1, 2, 4, 32, 3, 6, None, 1e-8, 1, ws, 1 << 24, None) == 1
    assert st.frames_done == 3           # nothing committed by a rejected call


def test_state_init_rejects(lavr):
    st = lavr.LaState()
    f = lavr.lib.la_state_init
    assert f(ctypes.byref(st), ctypes.c_void_p(0), ctypes.c_void_p(FAKE), 1, 1, 32, None) == 1
    assert f(ctypes.byref(st), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 4), 1, 1, 32, None) == 1
    assert f(ctypes.byref(st), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 4096), 1, 1, 48, None) == 2
    assert f(ctypes.byref(st), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), 1, 1, 32, None) == 1  # overlap


def call_backward(lavr, **kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, g=FAKE + 0x3000000,
                dq=FAKE + 0x4000000, dk=FAKE + 0x5000000, dv=FAKE + 0x6000000,
                in_dt=lavr.LA_BF16, grad_dt=lavr.LA_BF16, B=1, H=2, d=32, frames=4, tpf=6,
                bf=2, f0=0, rope=None, eps=1e-8, ws=FAKE + 0x7000000, ws_bytes=1 << 20)
    args.update(kw)
    vp = ctypes.c_void_p
    return lavr.lib.la_block_causal_backward(
        vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]), vp(args["dq"]), vp(args["dk"]),
        vp(args["dv"]), args["in_dt"], args["grad_dt"], args["B"], args["H"], args["d"],
        args["frames"], args["tpf"], args["bf"], args["f0"], args["rope"], args["eps"],
        vp(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(g=0), 1),                          # null output gradient
    (dict(dk=FAKE + 0x5000000 + 4), 1),      # misaligned gradient
    (dict(dq=FAKE + 0x1000000 + 128), 1),    # dq overlaps k
    (dict(dv=FAKE + 0x5000000 + 64), 1),     # dv overlaps dk
    (dict(d=48), 2),
    (dict(grad_dt=5), 1),
    (dict(eps=-1.0), 1),
    (dict(ws_bytes=16), 1),
    (dict(bf=0), 1),
])
def test_backward_rejects_bad_arguments(lavr, kw, code):
    assert call_backward(lavr, **kw) == code


def test_backward_workspace_bytes(lavr):
    n = lavr.backward_workspace_bytes(1, 70, 240, 1560, 8)
    assert n > lavr.workspace_bytes(1, 70, 240, 1560, 8)     # plus the suffix records
    assert lavr.lib.la_backward_workspace_bytes(1, 35, 64, 240, 1560, 8, 0, None) > 0    # head dim 64 built
    assert lavr.lib.la_backward_workspace_bytes(1, 35, 48, 240, 1560, 8, 0, None) == 0


def call_forward_qkv(lavr, **kw):
    args = dict(qkv=FAKE, out=FAKE + 0x3000000, in_dt=lavr.LA_BF16, out_dt=lavr.LA_BF16, B=1, H=2,
                d=32, frames=4, tpf=6, bf=2, f0=0, rope=None, eps=1e-8, qg=FAKE + 0x5000000,
                kg=FAKE + 0x5001000, norm_eps=1e-6, ws=FAKE + 0x4000000, ws_bytes=1 << 20)
    args.update(kw)
    vp = ctypes.c_void_p
    return lavr.lib.la_block_causal_forward_qkv(
        vp(args["qkv"]), vp(args["out"]), args["in_dt"], args["out_dt"], args["B"], args["H"],
        args["d"], args["frames"], args["tpf"], args["bf"], args["f0"], args["rope"], args["eps"],
        vp(args["qg"]), vp(args["kg"]), args["norm_eps"], vp(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qkv=0), 1),                        # null input
    (dict(qkv=FAKE + 4), 1),                 # misaligned input
    (dict(out=FAKE + 3 * 24 * 64 * 2 - 64), 1),  # out overlaps the fused rows (3 * C per token)
    (dict(qg=FAKE + 0x5000000 + 4), 1),      # misaligned weight
    (dict(kg=FAKE + 0x3000000 + 16), 1),     # weight overlaps out
    (dict(norm_eps=0.0), 1),                 # a norm needs norm_eps > 0
    (dict(norm_eps=float("nan")), 1),
    (dict(d=48), 2),
    (dict(eps=-1.0), 1),
    (dict(ws_bytes=16), 1),
    (dict(bf=0), 1),
])
def test_forward_qkv_rejects_bad_arguments(lavr, kw, code):
    assert call_forward_qkv(lavr, **kw) == code


def test_qkv_workspace_bytes(lavr):
    # the forward's workspace plus two per-token scale arrays (q and k)
    base = lavr.workspace_bytes(1, 70, 240, 1560, 8)
    n = lavr.qkv_workspace_bytes(1, 70, 240, 1560, 8)
    assert n >= base + 2 * 374400 * 4
    assert n < base + 2 * 374400 * 4 + 1024
    assert lavr.lib.la_qkv_workspace_bytes(1, 70, 48, 240, 1560, 8, 0, None) == 0


def test_stream_block_qkv_state_checks(lavr):
    st = lavr.LaState()
    st.S, st.z, st.B, st.H, st.head_dim, st.frames_done = FAKE, FAKE + 0x100000, 2, 4, 32, 0
    f = lavr.lib.la_stream_block_qkv
    vp = ctypes.c_void_p
    qkv, out, ws = vp(FAKE + 0x1000000), vp(FAKE + 0x3000000), vp(FAKE + 0x6000000)
    g = vp(FAKE + 0x5000000)
    assert f(ctypes.byref(st), qkv, out, 1, 1, 1, 4, 32, 3, 6, None, 1e-8, g, g, 1e-6, 1, ws, 1 << 24, None) == 3
    assert f(ctypes.byref(st), qkv, out, 1, 1, 2, 4, 32, 3, 6, None, 1e-8, g, g, 1e-6, 1, ws, 64, None) == 1
    assert f(ctypes.byref(st), qkv, out, 1, 1, 2, 4, 32, 3, 6, None, 1e-8, g, None, -1.0, 1, ws, 1 << 24,
             None) == 1
    assert st.frames_done == 0


def call_tconv(lavr, **kw):
    args = dict(x=FAKE, y=FAKE + 0x1000000, in_dt=lavr.LA_BF16, out_dt=lavr.LA_BF16, B=1, frames=8,
                tpf=6, ch=64, bf=2, f0=0, kt=3, w=FAKE + 0x2000000, bias=FAKE + 0x2001000)
    args.update(kw)
    vp = ctypes.c_void_p
    return lavr.lib.la_temporal_conv(vp(args["x"]), vp(args["y"]), args["in_dt"], args["out_dt"], args["B"],
                                     args["frames"], args["tpf"], args["ch"], args["bf"], args["f0"],
                                     args["kt"], vp(args["w"]), vp(args["bias"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), 1),
    (dict(w=0), 1),                          # weights are required, bias is not
    (dict(y=FAKE + 8), 1),                   # misaligned
    (dict(ch=60), 1),                        # channels not a multiple of 8
    (dict(kt=4), 1),
    (dict(kt=1), 1),
    (dict(bf=0), 1),
    (dict(f0=-1), 1),
    (dict(frames=0), 1),
    (dict(y=FAKE + 512), 1),                 # y overlaps x
    (dict(w=FAKE + 0x1000000 + 32), 1),      # w overlaps y
    (dict(frames=1 << 20, tpf=1024, ch=2048), 2),   # a batch row past 4 GiB
])
def test_tconv_rejects_bad_arguments(lavr, kw, code):
    assert call_tconv(lavr, **kw) == code


def test_tconv_stream_state_checks(lavr):
    st = lavr.LaConvState()
    st.last, st.B, st.tokens_per_frame, st.channels, st.dtype, st.frames_done = FAKE, 2, 6, 64, 1, 0
    f = lavr.lib.la_temporal_conv_stream_block
    vp = ctypes.c_void_p
    x, y, w = vp(FAKE + 0x1000000), vp(FAKE + 0x2000000), vp(FAKE + 0x3000000)
    assert f(ctypes.byref(st), x, y, 1, 1, 3, 6, 64, 3, w, None, 1, None) == 3       # B differs
    assert f(ctypes.byref(st), x, y, 1, 2, 3, 6, 72, 3, w, None, 1, None) == 3       # channels differ
    assert f(ctypes.byref(st), x, vp(FAKE + 64), 1, 2, 3, 6, 64, 3, w, None, 1, None) == 1   # y over the cache
    assert f(ctypes.byref(st), x, y, 1, 2, 0, 6, 64, 3, w, None, 1, None) == 1       # no frames
    assert st.frames_done == 0
    assert lavr.lib.la_conv_state_init(ctypes.byref(st), vp(FAKE + 4), 1, 2, 6, 64, None) == 1


def test_workspace_query_plans_with_the_rotary_window(lavr):
    """A block's work is cut into pieces whose rotary window fits on chip; with
    one token per frame and long blocks (1-D RoPE over the token index) that
    takes more pieces than without RoPE, so the workspace queries take the
    rotary description.  Queried with it, the size is the one the call checks:
    a byte less is rejected, and the RoPE-off size is too small.  Placeholder
    device addresses: every call here returns before any HIP call."""
    B, H, d, frames, tpf, bf = 1, 70, 32, 16384, 1, 4096
    rope = lavr.LaRope(16, 32, 0, 0, frames, 1, 1)           # table address only read as a range
    with_rope = lavr.lib.la_workspace_bytes(B, H, d, frames, tpf, bf, 0, ctypes.byref(rope))
    without = lavr.lib.la_workspace_bytes(B, H, d, frames, tpf, bf, 0, None)
    assert with_rope > without > 0
    q, k, v, out, ws = (ctypes.c_void_p(i << 40) for i in range(1, 6))

    def fwd(nbytes):
        return lavr.lib.la_block_causal_forward(q, k, v, out, lavr.LA_BF16, lavr.LA_BF16, B, H, d, frames, tpf,
                                                bf, 0, ctypes.byref(rope), 1e-8, ws, nbytes, None)

    assert fwd(without) == lavr.LA_ERR_INVALID_ARG
    assert fwd(with_rope - 1) == lavr.LA_ERR_INVALID_ARG
    for query in (lavr.lib.la_backward_workspace_bytes, lavr.lib.la_qkv_workspace_bytes):
        assert query(B, H, d, frames, tpf, bf, 0, ctypes.byref(rope)) > query(B, H, d, frames, tpf, bf, 0, None)
    # a description the call would reject sizes to 0
    bad = lavr.LaRope(16, 30, 0, 0, frames, 1, 1)             # sections do not sum to head_dim
    assert lavr.lib.la_workspace_bytes(B, H, d, frames, tpf, bf, 0, ctypes.byref(bad)) == 0


def test_noalloc_forward_rejects_shapes_beyond_its_workspace(lavr):
    """The allocation-free forward's workspace is a fixed 64 MiB array: a shape
    that needs more (ten minute-length clips' worth of frames) is refused with
    LA_ERR_UNSUPPORTED before any HIP call (placeholder device addresses)."""
    B, H, d, frames, tpf, bf = 1, 70, 32, 2400, 1560, 8
    assert lavr.lib.la_workspace_bytes(B, H, d, frames, tpf, bf, 0, None) > 64 << 20
    q, k, v, out = (ctypes.c_void_p(i << 40) for i in range(1, 5))
    rc = lavr.lib.la_block_causal_forward_noalloc(q, k, v, out, lavr.LA_BF16, lavr.LA_BF16, B, H, d, frames, tpf,
                                                  bf, 0, None, 1e-8, None)
    assert rc == lavr.LA_ERR_UNSUPPORTED
    # argument checks come first, as for every call
    rc = lavr.lib.la_block_causal_forward_noalloc(None, k, v, out, lavr.LA_BF16, lavr.LA_BF16, 1, H, d, 240, tpf,
                                                  bf, 0, None, 1e-8, None)
    assert rc == lavr.LA_ERR_INVALID_ARG
