"""Shared pieces of the test suite: inputs on the device, oracle slices, metrics."""

import numpy as np

import oracle
from linear_attention_video_relu_amd import workloads as W

BF16_UNIT_ROUNDOFF = 2.0 ** -8   # bf16 keeps 8 significant bits; RNE error <= 2^-8 |x|
TOL_BF16 = 2e-2                  # max |gpu - ref| / RMS(ref), bf16 inputs
TOL_F32 = 1e-5                   # same metric, fp32 inputs


def err_bf16_out(got, ref):
    """Parity metric for bf16 outputs: the output's own rounding (2^-8 |ref| per
    element) is allowed on top of the tolerance, since rounding the exact result
    to bf16 alone can exceed 2e-2 * RMS when max|out| > ~5 RMS."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(got - ref) - BF16_UNIT_ROUNDOFF * np.abs(ref)
    return float(max(0.0, np.max(excess))) / rms


def device_inputs(cfg, device):
    """Draw q, k, v of a workload; returns (host arrays dict, torch tensors tuple)."""
    arrs = {t: W.draw(cfg, t) for t in W.TENSORS}
    tens = tuple(W.to_torch(cfg, arrs[t], device) for t in W.TENSORS)
    return arrs, tens


def oracle_head(cfg, arrs, b, h, block_frames=None):
    """fp64 oracle output of one (batch, head) of a drawn workload: (N, 32)."""
    q, k, v = (W.to_f64(cfg, arrs[t][b, :, h]) for t in W.TENSORS)
    bf = cfg["block_frames"] if block_frames is None else block_frames
    return oracle.forward_head(q, k, v, cfg["tokens_per_frame"], bf, W.oracle_rope(cfg),
                               first_block_frames=cfg.get("first_block_frames"))


def to_f64_torch(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
