"""Named workloads and seeded synthetic inputs.

This module holds no arithmetic of the attention method: it only names the
problem shapes and draws seeded random inputs, so that the HIP path and the CPU
oracle can be fed the very same values.

Recipe (the same for every workload):
  * one numpy SeedSequence per (workload index, tensor, batch, token chunk),
    rooted at 42 (the only seed the LongSANA pull request prints);
  * standard-normal float32 draws times the workload's scale;
  * for keys with an outlier fraction p: an independent Bernoulli(p) mask per
    element, masked entries multiplied by the outlier factor after the draw;
  * bf16 workloads round the float32 draws to bf16 (round to nearest, ties to even);
  * B > 1 (conditional / unconditional) is simply independent draws per batch row;
  * the q/k norm weights of the fused prologue are 1 + 0.5 * N(0, 1) per channel.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

ROOT_SEED = 42
CHUNK_TOKENS = 4096

# Tensors drawn per workload, in a fixed order (their index enters the seed).
TENSORS = ("q", "k", "v")

ROPE_3D = {"split": (8, 12, 12), "base": 10000.0}
ROPE_3D_64 = {"split": (16, 24, 24), "base": 10000.0}

WORKLOADS = {
    # 1-D RoPE over the token index: one token per "frame", blocks of 64 tokens.
    "tiny_f32": dict(index=0, B=1, H=2, head_dim=32, frames=256, tokens_per_frame=1,
                     grid=(1, 1), block_frames=64, dtype="f32",
                     rope={"split": (32, 0, 0), "base": 10000.0}, scale=1.0,
                     outlier_frac=0.0, outlier_scale=1.0),
    "clip480p_bf16": dict(index=1, B=1, H=70, head_dim=32, frames=12, tokens_per_frame=1560,
                          grid=(30, 52), block_frames=3, dtype="bf16", rope=ROPE_3D,
                          scale=0.5, outlier_frac=0.0, outlier_scale=1.0),
    "clip720p_bf16": dict(index=2, B=2, H=70, head_dim=32, frames=21, tokens_per_frame=3600,
                          grid=(45, 80), block_frames=3, dtype="bf16", rope=ROPE_3D,
                          scale=1.0, outlier_frac=0.0, outlier_scale=1.0),
    # 40 calls of one 3-frame block each; "frames" is the whole streamed length.
    "stream_bf16": dict(index=3, B=2, H=70, head_dim=32, frames=120, tokens_per_frame=1560,
                        grid=(30, 52), block_frames=3, dtype="bf16", rope=ROPE_3D,
                        scale=1.0, outlier_frac=0.0, outlier_scale=1.0),
    "minute_bf16": dict(index=4, B=1, H=70, head_dim=32, frames=240, tokens_per_frame=1560,
                        grid=(30, 52), block_frames=8, dtype="bf16", rope=ROPE_3D,
                        scale=1.0, outlier_frac=0.05, outlier_scale=8.0),
    # The same 2240 channels as 35 heads of 64 (the pages name head dims 32 and
    # 64); the rotary split keeps the t:h:w = 8:12:12 proportions.
    "minute_d64_bf16": dict(index=5, B=1, H=35, head_dim=64, frames=240, tokens_per_frame=1560,
                            grid=(30, 52), block_frames=8, dtype="bf16", rope=ROPE_3D_64,
                            scale=1.0, outlier_frac=0.05, outlier_scale=8.0),
    "clip480p_d64_bf16": dict(index=6, B=1, H=35, head_dim=64, frames=12, tokens_per_frame=1560,
                              grid=(30, 52), block_frames=3, dtype="bf16", rope=ROPE_3D_64,
                              scale=0.5, outlier_frac=0.0, outlier_scale=1.0),
}


def workload(name, **overrides):
    """A copy of a named workload, with fields overridden (e.g. frames=6 for a short run)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def n_tokens(cfg):
    return cfg["frames"] * cfg["tokens_per_frame"]


def oracle_rope(cfg):
    """The RoPE description in the form the oracle takes (None when RoPE is off)."""
    if cfg.get("rope") is None:
        return None
    return {"split": tuple(cfg["rope"]["split"]), "grid": tuple(cfg["grid"]),
            "base": float(cfg["rope"]["base"])}


# ----------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


# ------------------------------------------------------------------------- drawing

def _draw_chunk(cfg, tensor_id, b, c, n0, n1):
    H, d = cfg["H"], cfg["head_dim"]
    ss = np.random.SeedSequence([ROOT_SEED, cfg["index"], tensor_id, b, c])
    rng = np.random.default_rng(ss)
    x = rng.standard_normal((n1 - n0, H, d), dtype=np.float32)
    if cfg["scale"] != 1.0:
        x *= np.float32(cfg["scale"])
    if TENSORS[tensor_id] == "k" and cfg["outlier_frac"] > 0.0:
        mask = rng.random((n1 - n0, H, d), dtype=np.float32) < np.float32(cfg["outlier_frac"])
        x[mask] *= np.float32(cfg["outlier_scale"])
    return x


def draw(cfg, tensor, token_range=None, threads=None):
    """Draw one tensor of the workload as (B, n, H, d).

    Returns uint16 bf16 bit patterns for bf16 workloads and float32 otherwise.
    token_range=(s, e) draws only those tokens (the values are the same as in a
    full draw, since every CHUNK_TOKENS-token chunk has its own seed).
    """
    tensor_id = TENSORS.index(tensor)
    N = n_tokens(cfg)
    s, e = (0, N) if token_range is None else token_range
    B, H, d = cfg["B"], cfg["H"], cfg["head_dim"]
    bf16 = cfg["dtype"] == "bf16"
    out = np.empty((B, e - s, H, d), dtype=np.uint16 if bf16 else np.float32)
    jobs = []
    for b in range(B):
        for c in range(s // CHUNK_TOKENS, (e + CHUNK_TOKENS - 1) // CHUNK_TOKENS):
            jobs.append((b, c))

    def one(job):
        b, c = job
        c0, c1 = c * CHUNK_TOKENS, min((c + 1) * CHUNK_TOKENS, N)
        x = _draw_chunk(cfg, tensor_id, b, c, c0, c1)
        lo, hi = max(c0, s), min(c1, e)
        x = x[lo - c0:hi - c0]
        out[b, lo - s:hi - s] = f32_to_bf16_bits(x) if bf16 else x

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if len(jobs) <= 1 or threads <= 1:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    return out


# Per-channel weights of the q/k RMSNorm prologue: 1 + 0.5 * N(0, 1) in float32
# (a few come out negative), one SeedSequence per weight vector.
NORM_WEIGHTS = ("q_gamma", "k_gamma")


def draw_norm_weight(cfg, which):
    """Seeded (C,) float32 weight vector of the q or k norm (C = H * head_dim)."""
    ss = np.random.SeedSequence([ROOT_SEED, cfg["index"], len(TENSORS) + NORM_WEIGHTS.index(which)])
    rng = np.random.default_rng(ss)
    return (1.0 + 0.5 * rng.standard_normal(cfg["H"] * cfg["head_dim"])).astype(np.float32)


def draw_conv(seed, B, N, Ch, kt):
    """Seeded inputs of the temporal convolution: x (B, N, Ch) standard normal
    float32, taps w (kt, Ch) and bias (Ch) as N(0, 1) / sqrt(kt) and 0.1 * N(0, 1)."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 1000 + seed]))
    x = rng.standard_normal((B, N, Ch), dtype=np.float32)
    w = (rng.standard_normal((kt, Ch)) / np.sqrt(kt)).astype(np.float32)
    b = (0.1 * rng.standard_normal(Ch)).astype(np.float32)
    return x, w, b


def fuse_qkv(q, k, v):
    """(B, N, H, d) q, k, v arrays -> one (B, N, 3, H * d) array with q | k | v rows."""
    B, N, H, d = q.shape
    return np.stack([a.reshape(B, N, H * d) for a in (q, k, v)], axis=2)


def to_f64(cfg, arr):
    """Exact float64 values of a drawn tensor."""
    return bf16_bits_to_f64(arr) if cfg["dtype"] == "bf16" else np.asarray(arr, dtype=np.float64)


def to_torch(cfg, arr, device):
    """Move a drawn tensor to torch on `device` (bf16 bit patterns become torch.bfloat16)."""
    import torch
    if cfg["dtype"] == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)
