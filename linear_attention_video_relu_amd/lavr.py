"""ctypes binding of liblavr (include/la_vr.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  Torch supplies device memory and the current stream.  If the
library is not built this module raises ImportError on import; there is no
fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LAVR_LIBRARY may name another build of the same library (e.g. a tuning build).
LIB_PATH = os.environ.get("LAVR_LIBRARY") or os.path.join(_HERE, "liblavr.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_STATE_MISMATCH, LA_ERR_HIP = range(5)
LA_F32, LA_BF16 = 0, 1
HEAD_DIM = 32
EPS_DEFAULT = 1e-8
NORM_EPS_DEFAULT = 1e-6


class LaRope(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("d_t", ctypes.c_int), ("d_h", ctypes.c_int),
                ("d_w", ctypes.c_int), ("max_frames", ctypes.c_int), ("grid_h", ctypes.c_int),
                ("grid_w", ctypes.c_int)]


class LaState(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("z", ctypes.c_void_p), ("B", ctypes.c_int),
                ("H", ctypes.c_int), ("head_dim", ctypes.c_int), ("frames_done", ctypes.c_longlong)]


class LaConvState(ctypes.Structure):
    _fields_ = [("last", ctypes.c_void_p), ("B", ctypes.c_int), ("tokens_per_frame", ctypes.c_int),
                ("channels", ctypes.c_int), ("dtype", ctypes.c_int), ("frames_done", ctypes.c_longlong)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_vp, c_float, c_double = (ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.c_float, ctypes.c_double)
    sig = {
        "rope_table_bytes": (c_size, [c_int] * 6),
        "rope_table_build": (c_int, [ctypes.POINTER(LaRope), c_vp, c_size, c_int, c_int, c_int,
                                     c_int, c_int, c_int, c_int, c_double, c_vp]),
        "la_workspace_bytes": (c_size, [c_int] * 7 + [ctypes.POINTER(LaRope)]),
        "la_block_causal_forward": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                            c_int, c_int, c_int, c_int, c_int,
                                            ctypes.POINTER(LaRope), c_float, c_vp, c_size, c_vp]),
        "la_replay_workspace_bytes": (c_size, [c_int] * 6 + [ctypes.POINTER(LaRope)]),
        "la_block_causal_forward_replay": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                                   c_int, c_int, c_int, c_int,
                                                   ctypes.POINTER(LaRope), c_float, c_vp, c_size, c_vp]),
        "la_block_causal_forward_timed": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                                  c_int, c_int, c_int, c_int, c_int, c_int,
                                                  ctypes.POINTER(LaRope), c_float, c_vp, c_size,
                                                  c_vp, ctypes.POINTER(c_vp)]),
        "la_block_causal_forward_noalloc": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                                    c_int, c_int, c_int, c_int, c_int,
                                                    ctypes.POINTER(LaRope), c_float, c_vp]),
        "la_backward_workspace_bytes": (c_size, [c_int] * 7 + [ctypes.POINTER(LaRope)]),
        "la_block_causal_backward": (c_int, [c_vp] * 7 + [c_int] * 9 + [ctypes.POINTER(LaRope), c_float,
                                                                         c_vp, c_size, c_vp]),
        "la_block_causal_backward_from_forward": (c_int, [c_vp] * 7 + [c_int] * 9 +
                                                  [ctypes.POINTER(LaRope), c_float, c_vp, c_size, c_vp]),
        "la_qkv_workspace_bytes": (c_size, [c_int] * 7 + [ctypes.POINTER(LaRope)]),
        "la_block_causal_forward_qkv": (c_int, [c_vp, c_vp, c_int, c_int] + [c_int] * 7 +
                                        [ctypes.POINTER(LaRope), c_float, c_vp, c_vp, c_float, c_vp,
                                         c_size, c_vp]),
        "la_stream_block_qkv": (c_int, [ctypes.POINTER(LaState), c_vp, c_vp, c_int, c_int] + [c_int] * 5 +
                                [ctypes.POINTER(LaRope), c_float, c_vp, c_vp, c_float, c_int, c_vp,
                                 c_size, c_vp]),
        "la_temporal_conv": (c_int, [c_vp, c_vp] + [c_int] * 9 + [c_vp, c_vp, c_vp]),
        "la_conv_state_init": (c_int, [ctypes.POINTER(LaConvState), c_vp] + [c_int] * 4 + [c_vp]),
        "la_temporal_conv_stream_block": (c_int, [ctypes.POINTER(LaConvState), c_vp, c_vp] + [c_int] * 6 +
                                          [c_vp, c_vp, c_int, c_vp]),
        "la_state_init": (c_int, [ctypes.POINTER(LaState), c_vp, c_vp, c_int, c_int, c_int, c_vp]),
        "la_stream_block": (c_int, [ctypes.POINTER(LaState), c_vp, c_vp, c_vp, c_vp, c_int, c_int,
                                    c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(LaRope),
                                    c_float, c_int, c_vp, c_size, c_vp]),
        "la_status_string": (ctypes.c_char_p, [c_int]),
        "la_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()

EXPORTS = ("rope_table_bytes", "rope_table_build", "la_workspace_bytes", "la_block_causal_forward",
           "la_replay_workspace_bytes", "la_block_causal_forward_replay", "la_block_causal_forward_timed", "la_block_causal_forward_noalloc", "la_backward_workspace_bytes", "la_block_causal_backward",
           "la_block_causal_backward_from_forward",
           "la_qkv_workspace_bytes", "la_block_causal_forward_qkv", "la_stream_block_qkv",
           "la_temporal_conv", "la_conv_state_init", "la_temporal_conv_stream_block",
           "la_state_init", "la_stream_block", "la_status_string", "la_version")


def status_string(code):
    return lib.la_status_string(int(code)).decode()


def _check(code, what):
    if code == LA_OK:
        return
    msg = f"{what}: {status_string(code)}"
    if code == LA_ERR_HIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return LA_BF16
    if dt == torch.float32:
        return LA_F32
    raise ValueError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------- RoPE

class RopeTable:
    """Device rotary table built by rope_table_build, plus its la_rope description.

    split = (d_t, d_h, d_w) with d_t + d_h + d_w = the head dim (32 or 64), grid =
    (rows, cols) of a frame; max_frames rows of the t section.  A 1-D RoPE over the
    token index is split (head_dim, 0, 0), grid (1, 1).
    """

    def __init__(self, split, grid, max_frames, base=10000.0, device="cuda"):
        d_t, d_h, d_w = (int(s) for s in split)
        gh, gw = (int(g) for g in grid)
        nbytes = lib.rope_table_bytes(d_t, d_h, d_w, int(max_frames), gh, gw)
        if nbytes == 0:
            raise ValueError(f"invalid rotary table shape split={split} grid={grid} max_frames={max_frames}")
        self.device = torch.device(device)
        self.buffer = torch.empty(nbytes // 4, dtype=torch.float32, device=self.device)
        self.desc = LaRope()
        _check(lib.rope_table_build(ctypes.byref(self.desc), _ptr(self.buffer), nbytes, d_t + d_h + d_w,
                                    d_t, d_h, d_w, int(max_frames), gh, gw, float(base),
                                    _stream(self.device)), "rope_table_build")
        self.split, self.grid, self.max_frames, self.base = (d_t, d_h, d_w), (gh, gw), int(max_frames), float(base)


def _rope_ptr(rope):
    return ctypes.byref(rope.desc) if rope is not None else None


# ------------------------------------------------------------------ one-shot

def workspace_bytes(B, H, frames, tokens_per_frame, block_frames, head_dim=HEAD_DIM,
                    first_block_frames=0, rope=None):
    """Workspace bytes of a forward call (first_block_frames 0 = uniform blocks;
    rope: the RopeTable the call will use, or None)."""
    n = lib.la_workspace_bytes(int(B), int(H), int(head_dim), int(frames), int(tokens_per_frame),
                               int(block_frames), int(first_block_frames or 0), _rope_ptr(rope))
    if n == 0:
        raise ValueError("invalid shape for la_workspace_bytes")
    return n


def new_workspace(nbytes, device):
    """A workspace buffer of nbytes for the library's calls (no initial
    contents are needed)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


_ws_cache = {}


def _workspace(device, nbytes):
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = new_workspace(nbytes, device)
        _ws_cache[key] = buf
    return buf


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("q, k, v must be CUDA (HIP) tensors")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous (B, N, H, head_dim) tensors")
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")


def block_causal_forward(q, k, v, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                         out=None, out_dtype=None, workspace=None, first_block_frames=None):
    """One-shot block-causal forward.  q, k, v: (B, N, H, D) with D = 32 or 64,
    N = frames * tokens_per_frame.

    first_block_frames: frames of the first block (None = block_frames)."""
    _check_qkv(q, k, v)
    B, N, H, d = q.shape
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    frames = N // tokens_per_frame
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, N, H, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape and out_dtype on q's device")
    f0 = int(first_block_frames or 0)
    need = lib.la_workspace_bytes(B, H, d, frames, int(tokens_per_frame), int(block_frames), f0, _rope_ptr(rope))
    ws = _workspace(q.device, need) if workspace is None else workspace
    _check(lib.la_block_causal_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q.dtype),
                                       _dtype_code(out_dtype), B, H, d, frames,
                                       int(tokens_per_frame), int(block_frames), f0, _rope_ptr(rope),
                                       float(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(q.device)), "la_block_causal_forward")
    return out


def replay_workspace_bytes(B, H, frames, tokens_per_frame, block_frames, head_dim=HEAD_DIM, rope=None):
    """Workspace bytes of block_causal_forward_replay."""
    n = lib.la_replay_workspace_bytes(int(B), int(H), int(head_dim), int(frames), int(tokens_per_frame),
                                      int(block_frames), _rope_ptr(rope))
    if n == 0:
        raise ValueError("invalid shape for la_replay_workspace_bytes (whole blocks required)")
    return n


def block_causal_forward_replay(q, k, v, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                                out=None, out_dtype=None, workspace=None):
    """la_block_causal_forward_replay: the one-shot forward whose output equals,
    bit for bit, streaming the clip block by block with StreamState.step (save=True,
    from a fresh state).  The clip must be whole blocks of block_frames frames."""
    _check_qkv(q, k, v)
    B, N, H, d = q.shape
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    frames = N // tokens_per_frame
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, N, H, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape and out_dtype on q's device")
    need = replay_workspace_bytes(B, H, frames, tokens_per_frame, block_frames, d, rope)
    ws = _workspace(q.device, need) if workspace is None else workspace
    _check(lib.la_block_causal_forward_replay(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q.dtype),
                                              _dtype_code(out_dtype), B, H, d, frames,
                                              int(tokens_per_frame), int(block_frames), _rope_ptr(rope),
                                              float(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                              _stream(q.device)), "la_block_causal_forward_replay")
    return out


def block_causal_forward_noalloc(q, k, v, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT, *,
                                 out, out_dtype=None, first_block_frames=None):
    """la_block_causal_forward_noalloc: the one-shot forward with the library's
    fixed per-GPU workspace instead of a caller buffer.  `out` (contiguous, q's
    shape, out_dtype) is required, so that the call allocates nothing."""
    _check_qkv(q, k, v)
    B, N, H, d = q.shape
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape and out_dtype on q's device")
    _check(lib.la_block_causal_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q.dtype),
                                               _dtype_code(out_dtype), B, H, d, N // tokens_per_frame,
                                               int(tokens_per_frame), int(block_frames),
                                               int(first_block_frames or 0), _rope_ptr(rope), float(eps),
                                               _stream(q.device)), "la_block_causal_forward_noalloc")
    return out


# ------------------------------------------------------------ fused prologue

def qkv_workspace_bytes(B, H, frames, tokens_per_frame, block_frames, head_dim=HEAD_DIM,
                        first_block_frames=0, rope=None):
    n = lib.la_qkv_workspace_bytes(int(B), int(H), int(head_dim), int(frames), int(tokens_per_frame),
                                   int(block_frames), int(first_block_frames or 0), _rope_ptr(rope))
    if n == 0:
        raise ValueError("invalid shape for la_qkv_workspace_bytes")
    return n


def _check_fused(qkv, heads, q_gamma, k_gamma):
    if not isinstance(qkv, torch.Tensor) or qkv.device.type != "cuda":
        raise ValueError("qkv must be a CUDA (HIP) tensor")
    if qkv.dim() != 4 or qkv.shape[2] != 3 or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous (B, N, 3, C) tensor")
    C = qkv.shape[3]
    if C % heads:
        raise ValueError("C must be a multiple of heads")
    for g in (q_gamma, k_gamma):
        if g is None:
            continue
        if (not isinstance(g, torch.Tensor) or g.device != qkv.device or g.dtype != torch.float32
                or g.shape != (C,) or not g.is_contiguous()):
            raise ValueError("q_gamma / k_gamma must be contiguous float32 (C,) tensors on qkv's device")
    return C // heads


def _gptr(g):
    return None if g is None else _ptr(g)


def block_causal_forward_qkv(qkv, heads, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                             q_gamma=None, k_gamma=None, norm_eps=NORM_EPS_DEFAULT, out=None,
                             out_dtype=None, workspace=None, first_block_frames=None):
    """One-shot forward from the fused projection output qkv (B, N, 3, C): q, k, v
    rows in place, with q and/or k RMS-normalised over C when a weight is given.
    Returns out (B, N, heads, C // heads)."""
    d = _check_fused(qkv, heads, q_gamma, k_gamma)
    B, N = qkv.shape[0], qkv.shape[1]
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    frames = N // tokens_per_frame
    out_dtype = qkv.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, N, heads, d), dtype=out_dtype, device=qkv.device)
    elif (out.shape != (B, N, heads, d) or out.dtype != out_dtype or not out.is_contiguous()
          or out.device != qkv.device):
        raise ValueError("out must be a contiguous (B, N, heads, head_dim) tensor of out_dtype")
    f0 = int(first_block_frames or 0)
    need = lib.la_qkv_workspace_bytes(B, heads, d, frames, int(tokens_per_frame), int(block_frames), f0,
                                      _rope_ptr(rope))
    ws = _workspace(qkv.device, need) if workspace is None else workspace
    _check(lib.la_block_causal_forward_qkv(_ptr(qkv), _ptr(out), _dtype_code(qkv.dtype),
                                           _dtype_code(out_dtype), B, int(heads), d, frames,
                                           int(tokens_per_frame), int(block_frames), f0,
                                           _rope_ptr(rope), float(eps), _gptr(q_gamma), _gptr(k_gamma),
                                           float(norm_eps), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(qkv.device)), "la_block_causal_forward_qkv")
    return out


# ------------------------------------------------- cached temporal convolution

def _check_conv_args(x, w, bias):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous CUDA (B, N, channels) tensor")
    Ch = x.shape[2]
    if (not isinstance(w, torch.Tensor) or w.dtype != torch.float32 or w.dim() != 2 or w.shape[1] != Ch
            or w.shape[0] not in (2, 3) or not w.is_contiguous() or w.device != x.device):
        raise ValueError("w must be a contiguous float32 (kt, channels) tensor on x's device, kt 2 or 3")
    if bias is not None and (not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32
                             or bias.shape != (Ch,) or not bias.is_contiguous() or bias.device != x.device):
        raise ValueError("bias must be a contiguous float32 (channels,) tensor on x's device")
    return Ch, w.shape[0]


def temporal_conv(x, w, tokens_per_frame, block_frames, bias=None, first_block_frames=None, out=None,
                  out_dtype=None):
    """One-shot cached temporal convolution of x (B, N, channels); see la_temporal_conv."""
    Ch, kt = _check_conv_args(x, w, bias)
    B, N = x.shape[0], x.shape[1]
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, N, Ch), dtype=out_dtype, device=x.device)
    elif out.shape != x.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape and out_dtype")
    _check(lib.la_temporal_conv(_ptr(x), _ptr(out), _dtype_code(x.dtype), _dtype_code(out_dtype), B,
                                N // tokens_per_frame, int(tokens_per_frame), Ch, int(block_frames),
                                int(first_block_frames or 0), kt, _ptr(w), _gptr(bias), _stream(x.device)),
           "la_temporal_conv")
    return out


class ConvState:
    """Streaming cache of the temporal convolution (the last committed frame)."""

    def __init__(self, B, tokens_per_frame, channels, dtype=torch.bfloat16, device="cuda"):
        self.device = torch.device(device)
        self.last = torch.empty((B, tokens_per_frame, channels), dtype=dtype, device=self.device)
        self.desc = LaConvState()
        _check(lib.la_conv_state_init(ctypes.byref(self.desc), _ptr(self.last), _dtype_code(dtype), int(B),
                                      int(tokens_per_frame), int(channels), _stream(self.device)),
               "la_conv_state_init")

    @property
    def frames_done(self):
        return int(self.desc.frames_done)

    def step(self, x, w, bias=None, save=True, out=None, out_dtype=None):
        """One block (all of x's frames) against the cache; see la_temporal_conv_stream_block."""
        Ch, kt = _check_conv_args(x, w, bias)
        B, N = x.shape[0], x.shape[1]
        tpf = int(self.desc.tokens_per_frame)
        if N % tpf:
            raise ValueError("N must be a multiple of the cache's tokens_per_frame")
        out_dtype = x.dtype if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((B, N, Ch), dtype=out_dtype, device=x.device)
        _check(lib.la_temporal_conv_stream_block(ctypes.byref(self.desc), _ptr(x), _ptr(out),
                                                 _dtype_code(out_dtype), B, N // tpf, tpf, Ch, kt, _ptr(w),
                                                 _gptr(bias), int(bool(save)), _stream(x.device)),
               "la_temporal_conv_stream_block")
        return out


# ------------------------------------------------------------------ backward

def backward_workspace_bytes(B, H, frames, tokens_per_frame, block_frames, head_dim=HEAD_DIM,
                             first_block_frames=0, rope=None):
    n = lib.la_backward_workspace_bytes(int(B), int(H), int(head_dim), int(frames),
                                        int(tokens_per_frame), int(block_frames),
                                        int(first_block_frames or 0), _rope_ptr(rope))
    if n == 0:
        raise ValueError("invalid shape for la_backward_workspace_bytes")
    return n


def block_causal_backward(q, k, v, dout, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                          grad_dtype=None, first_block_frames=None, workspace=None, from_forward=False):
    """Gradients (dq, dk, dv) of sum(dout * block_causal_forward(q, k, v, ...)).

    from_forward=True: `workspace` is the one a block_causal_forward call with the
    same arguments filled (sized by backward_workspace_bytes) and the block
    states are not formed again (la_block_causal_backward_from_forward)."""
    _check_qkv(q, k, v)
    _check_qkv(q, k, dout)
    B, N, H, d = q.shape
    if N % tokens_per_frame:
        raise ValueError("N must be a multiple of tokens_per_frame")
    frames = N // tokens_per_frame
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    dq, dk, dv = (torch.empty((B, N, H, d), dtype=grad_dtype, device=q.device) for _ in range(3))
    f0 = int(first_block_frames or 0)
    need = lib.la_backward_workspace_bytes(B, H, d, frames, int(tokens_per_frame), int(block_frames), f0,
                                           _rope_ptr(rope))
    if need == 0:
        raise ValueError(f"backward not built for head dim {d} or invalid shape")
    if from_forward and workspace is None:
        raise ValueError("from_forward needs the forward's workspace")
    ws = _workspace(q.device, need) if workspace is None else workspace
    fn = lib.la_block_causal_backward_from_forward if from_forward else lib.la_block_causal_backward
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(q.dtype),
              _dtype_code(grad_dtype), B, H, d, frames, int(tokens_per_frame), int(block_frames), f0,
              _rope_ptr(rope), float(eps), _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)),
           "la_block_causal_backward")
    return dq, dk, dv


class BlockCausalAttention(torch.autograd.Function):
    """Autograd binding: forward through la_block_causal_forward into a workspace
    kept for the backward, backward through la_block_causal_backward_from_forward
    (the forward's block states reused; gradients in the input dtype)."""

    @staticmethod
    def forward(ctx, q, k, v, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                first_block_frames=None, out_dtype=None):
        q, k, v = (t.contiguous() for t in (q, k, v))
        B, N, H, d = q.shape
        need = backward_workspace_bytes(B, H, N // tokens_per_frame, tokens_per_frame, block_frames,
                                        head_dim=d, first_block_frames=first_block_frames, rope=rope)
        ws = new_workspace(need, q.device)
        out = block_causal_forward(q, k, v, block_frames, tokens_per_frame, rope, eps, workspace=ws,
                                   first_block_frames=first_block_frames, out_dtype=out_dtype)
        ctx.save_for_backward(q, k, v, ws)
        ctx.args = (block_frames, tokens_per_frame, rope, eps, first_block_frames)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, ws = ctx.saved_tensors
        bf, tpf, rope, eps, f0 = ctx.args
        dout = dout.contiguous()
        if dout.dtype == q.dtype:
            dq, dk, dv = block_causal_backward(q, k, v, dout, bf, tpf, rope, eps, first_block_frames=f0,
                                               workspace=ws, from_forward=True)
        else:
            # An upstream gradient wider than the inputs (fp32 for bf16 q, k, v)
            # is not rounded: the inputs are widened exactly and the gradients
            # are formed from fp32 operands, then returned in the inputs' dtype.
            w = [t.to(torch.float32) for t in (q, k, v)]
            dq, dk, dv = block_causal_backward(*w, dout.to(torch.float32), bf, tpf, rope, eps,
                                               grad_dtype=q.dtype, first_block_frames=f0)
        return dq, dk, dv, None, None, None, None, None, None


def block_causal_attention(q, k, v, block_frames, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                           first_block_frames=None, out_dtype=None):
    """Differentiable block-causal ReLU linear attention (see BlockCausalAttention).
    out_dtype: dtype of the output (default: the inputs'); an fp32 output of bf16
    inputs receives an fp32 upstream gradient, which the backward keeps in fp32."""
    return BlockCausalAttention.apply(q, k, v, block_frames, tokens_per_frame, rope, eps,
                                      first_block_frames, out_dtype)


# ----------------------------------------------------------------- streaming

class StreamState:
    """Constant-size (S, z) cache of one generation stream, on one device."""

    def __init__(self, B, H, head_dim=HEAD_DIM, device="cuda"):
        self.device = torch.device(device)
        self.S = torch.empty((B, H, head_dim, head_dim), dtype=torch.float32, device=self.device)
        self.z = torch.empty((B, H, head_dim), dtype=torch.float32, device=self.device)
        self.desc = LaState()
        _check(lib.la_state_init(ctypes.byref(self.desc), _ptr(self.S), _ptr(self.z), int(B), int(H),
                                 int(head_dim), _stream(self.device)), "la_state_init")

    @property
    def frames_done(self):
        return int(self.desc.frames_done)

    def snapshot(self):
        """Host copy of the full resumable state (S, z, frames_done)."""
        return self.S.cpu(), self.z.cpu(), self.frames_done

    def restore(self, snap):
        S, z, frames_done = snap
        self.S.copy_(S)
        self.z.copy_(z)
        self.desc.frames_done = int(frames_done)

    def step(self, q, k, v, tokens_per_frame, rope=None, eps=EPS_DEFAULT, save=True, out=None,
             out_dtype=None, workspace=None):
        """Run one block (all of q's tokens) against the cache; see la_stream_block."""
        _check_qkv(q, k, v)
        B, N, H, d = q.shape
        if N % tokens_per_frame:
            raise ValueError("N must be a multiple of tokens_per_frame")
        frames = N // tokens_per_frame
        out_dtype = q.dtype if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((B, N, H, d), dtype=out_dtype, device=q.device)
        elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor of q's shape and out_dtype")
        # (a caller's workspace is sized by the library's own check)
        ws = workspace if workspace is not None else _workspace(
            q.device, lib.la_workspace_bytes(B, H, d, frames, int(tokens_per_frame), frames, 0, _rope_ptr(rope)))
        _check(lib.la_stream_block(ctypes.byref(self.desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                   _dtype_code(q.dtype), _dtype_code(out_dtype), B, H, d, frames,
                                   int(tokens_per_frame), _rope_ptr(rope), float(eps), int(bool(save)),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)),
               "la_stream_block")
        return out

    def step_qkv(self, qkv, tokens_per_frame, rope=None, eps=EPS_DEFAULT, q_gamma=None, k_gamma=None,
                 norm_eps=NORM_EPS_DEFAULT, save=True, out=None, out_dtype=None, workspace=None):
        """step() from the fused projection output qkv (B, N, 3, C); see
        la_stream_block_qkv."""
        H = int(self.desc.H)
        d = _check_fused(qkv, H, q_gamma, k_gamma)
        B, N = qkv.shape[0], qkv.shape[1]
        if N % tokens_per_frame:
            raise ValueError("N must be a multiple of tokens_per_frame")
        frames = N // tokens_per_frame
        out_dtype = qkv.dtype if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((B, N, H, d), dtype=out_dtype, device=qkv.device)
        elif out.shape != (B, N, H, d) or out.dtype != out_dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous (B, N, H, head_dim) tensor of out_dtype")
        ws = workspace if workspace is not None else _workspace(
            qkv.device, lib.la_qkv_workspace_bytes(B, H, d, frames, int(tokens_per_frame), frames, 0,
                                                   _rope_ptr(rope)))
        _check(lib.la_stream_block_qkv(ctypes.byref(self.desc), _ptr(qkv), _ptr(out), _dtype_code(qkv.dtype),
                                       _dtype_code(out_dtype), B, H, d, frames, int(tokens_per_frame),
                                       _rope_ptr(rope), float(eps), _gptr(q_gamma), _gptr(k_gamma),
                                       float(norm_eps), int(bool(save)), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(qkv.device)),
               "la_stream_block_qkv")
        return out
